"""Pins of the oracle's FS-B forests ("FreeSolo" review, the two variants: a
forest over the whole prefix and one over the cells at or above the median
max norm; nodes with mean key, radius, max norm and min position; beam
search with the node score bounding the cell scores below; logsumexp re-rank
over the token keys of the reached cells).

- Node fields: brute force over each node's cells (numpy).
- Node score: it bounds every cell score below the node (the cell scores
  come from the pinned scores_one_row). For a one-cell node of radius 0 it
  equals that cell's score.
- Search: when the beam holds every node at every level, the reached set is
  every cell. The result is then the top K of each cell's logsumexp over its
  tokens, computed here with numpy."""
from __future__ import annotations

import numpy as np
import pytest

import oracle


def _inputs(seed, n, d=8, b=4, extra=3):
    rng = np.random.default_rng(seed)
    L = (n + extra) * b
    k = (np.round(rng.standard_normal((1, 2, L, d)) * 16) / 16).astype(np.float32)
    kb, mx, ce = oracle.block_summaries(k, b, nblocks=L // b)
    # equal norms are common: round the max norms
    mx = (np.round(mx * 2) / 2).astype(np.float32)
    q = rng.standard_normal((1, 2, 1, d)).astype(np.float32)
    return k, kb, mx, ce, q, L


def _subtree(l, j, F, m):
    span = F ** l
    return range(j * span, min((j + 1) * span, m))


@pytest.mark.parametrize("n,F", [(300, 4), (17, 16), (16, 16), (70, 4), (1, 4)])
def test_forest_node_fields_brute_force(n, F):
    k, kb, mx, ce, q, L = _inputs(120 + n, n)
    fo = oracle.forest_build(kb, mx, ce, n, F=F)
    for h in range(2):
        a = mx[0, h, :n]
        kk = (n + 1) // 2
        med = np.sort(a)[::-1][kk - 1]
        for f in range(2):
            m = int(fo["nmem"][0, h, f])
            mem = fo["members"][0, h, f, :m]
            want = np.arange(n) if f == 0 else np.nonzero(a >= med)[0]
            assert np.array_equal(mem, want) and np.all(fo["members"][0, h, f, m:] == -1)
            if f == 1:
                assert m >= kk
            # levels
            sizes, cur = [], m
            while cur > F:
                cur = -(-cur // F)
                sizes.append(cur)
            off = 0
            for l, cnt in enumerate(sizes, start=1):
                for j in range(cnt):
                    cells = mem[list(_subtree(l, j, F, m))]
                    keys = kb[0, h, cells].astype(np.float64)
                    mu = fo["mu"][0, h, f, off + j]
                    assert np.allclose(mu, keys.mean(axis=0), rtol=1e-6, atol=1e-7)
                    r = np.sqrt(((keys - mu.astype(np.float64)) ** 2).sum(axis=1)).max()
                    assert abs(fo["rad"][0, h, f, off + j] - r) <= 1e-6 * max(1.0, r)
                    assert fo["amax"][0, h, f, off + j] == mx[0, h, cells].max()
                    assert fo["pmin"][0, h, f, off + j] == ce[cells].min()
                off += cnt
            assert off == (oracle.forest_nodes(m, F))


def test_node_score_bounds_every_cell_below():
    n, F, b = 300, 4, 4
    k, kb, mx, ce, q, L = _inputs(131, n, b=b)
    fo = oracle.forest_build(kb, mx, ce, n, F=F)
    lam = np.array([0.7, 0.3], np.float32)
    sig = np.array([40.0, 9.0], np.float32)
    pos = L - 1
    for h in range(2):
        s = oracle.scores_one_row(q, kb, mx, ce, Hkv=2, b=b, q_pos0=pos, bidx=0, hs=h, row=0, prefix_mode=0,
                                  share_group=False, erf_lambda=lam, erf_sigma=sig)
        qh = q[0, h, 0].astype(np.float64)
        for f in range(2):
            m = int(fo["nmem"][0, h, f])
            mem = fo["members"][0, h, f, :m]
            sizes, cur = [], m
            while cur > F:
                cur = -(-cur // F)
                sizes.append(cur)
            off = 0
            for l, cnt in enumerate(sizes, start=1):
                for j in range(cnt):
                    v = off + j
                    u = oracle.node_score(qh, fo["mu"][0, h, f, v], fo["rad"][0, h, f, v], fo["amax"][0, h, f, v],
                                          fo["pmin"][0, h, f, v], lam=lam[h], sig=sig[h], pos=pos)
                    below = s[mem[list(_subtree(l, j, F, m))]]
                    assert u >= below.max() - 1e-9 * max(1.0, abs(u))
                off += cnt
        # a node of one cell and radius 0 scores exactly as that cell
        for c in (0, 7, n - 1):
            u = oracle.node_score(qh, kb[0, h, c].astype(np.float32), 0.0, mx[0, h, c], ce[c], lam=lam[h],
                                  sig=sig[h], pos=pos)
            assert abs(u - s[c]) <= 1e-12 * max(1.0, abs(s[c]))


@pytest.mark.parametrize("n,F,K", [(12, 4, 4), (16, 16, 3), (9, 4, 9)])
def test_full_beam_is_the_brute_force_rerank(n, F, K):
    """Beam of 16 with at most 16 candidates per level: every cell is reached,
    so the result is the top K of the per-cell logsumexp over its tokens."""
    b = 4
    k, kb, mx, ce, q, L = _inputs(140 + n, n, b=b)
    fo = oracle.forest_build(kb, mx, ce, n, F=F)
    lam = np.array([0.5, 0.5], np.float32)
    sig = np.array([20.0, 20.0], np.float32)
    r = oracle.forest_select(q, kb, mx, ce, k, fo, n, Hkv=2, b=b, K=K, q_pos0=L - 1, share_group=False,
                             erf_lambda=lam, erf_sigma=sig, F=F, Wb=16)
    d = q.shape[-1]
    for h in range(2):
        z = (k[0, h, :n * b].astype(np.float64).reshape(n, b, d) @ q[0, h, 0].astype(np.float64)) / np.sqrt(d)
        lse = np.log(np.exp(z - z.max(axis=1, keepdims=True)).sum(axis=1)) + z.max(axis=1)
        order = sorted(range(n), key=lambda c: (-lse[c], c))[:min(K, n)]
        want = np.full(K, -1, np.int32)
        want[:len(order)] = sorted(order)
        assert np.array_equal(r["idx"][0, h, 0], want)


def test_cell_token_lse_closed_forms():
    """The re-rank score of a cell (logsumexp over its b token keys of
    qhat.k/sqrt(d)) on keys with closed forms: b identical keys give
    s + log b; a cell of two distinct keys, each b/2 times, gives
    log((b/2)(e^s1 + e^s2)); with a shared group qhat is the heads' mean."""
    d, b = 4, 8
    q = np.array([[[[1.0, -0.5, 2.0, 0.25]], [[3.0, 0.5, 0.0, -0.25]]]], np.float32)     # [1, 2, 1, d]
    k1 = np.array([0.5, 1.0, -1.0, 2.0], np.float32)
    k2 = np.array([-2.0, 0.25, 1.5, 0.0], np.float32)
    k = np.zeros((1, 1, 3 * b, d), np.float32)
    k[0, 0, 0:b] = k1
    k[0, 0, b:2 * b:2] = k1
    k[0, 0, b + 1:2 * b:2] = k2
    k[0, 0, 2 * b:] = k2
    for hs in (0, 1):
        qh = q[0, hs, 0].astype(np.float64)
        s1, s2 = qh @ k1 / 2.0, qh @ k2 / 2.0                     # sqrt(d) = 2
        got = oracle.cell_token_lse(q, k, Hkv=1, b=b, bidx=0, hs=hs, row=0, ncells=3)
        assert got[0] == pytest.approx(s1 + np.log(b), abs=1e-13)
        assert got[1] == pytest.approx(np.log(b / 2 * (np.exp(s1) + np.exp(s2))), abs=1e-13)
        assert got[2] == pytest.approx(s2 + np.log(b), abs=1e-13)
    qm = q[0, :, 0].astype(np.float64).mean(axis=0)
    got = oracle.cell_token_lse(q, k, Hkv=1, b=b, bidx=0, hs=0, row=0, ncells=1, share_group=True)
    assert got[0] == pytest.approx(qm @ k1 / 2.0 + np.log(b), abs=1e-13)


def test_cell_token_lse_ranks_like_the_full_beam_search():
    """With at most 16 cells a forest scores its cells directly and the beam of
    16 reaches every cell, so the selection is the top K of the per-cell
    re-rank scores that cell_token_lse writes out."""
    n, K, b = 16, 5, 4
    k, kb, mx, ce, q, L = _inputs(777, n, b=b)
    fo = oracle.forest_build(kb, mx, ce, n, F=16)
    pos = L - 1
    ora = oracle.forest_select(q, kb, mx, ce, k, fo, n, Hkv=2, b=b, K=K, q_pos0=pos, F=16, Wb=16)
    for hs in range(2):
        s = oracle.cell_token_lse(q, k, Hkv=2, b=b, bidx=0, hs=hs, row=0, ncells=n)
        want, _, _, _, _ = oracle.select_from_scores(s, K, gate=False)
        assert np.array_equal(ora["idx"][0, hs, 0], want)
