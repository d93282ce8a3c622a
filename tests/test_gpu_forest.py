"""GPU parity of the FS-B forests ("FreeSolo" review, the two variants):
sparse_forest_build against the oracle's forests, and sparse_forest_select
against the oracle's beam search and re-rank. Members and counts must be
bit-exact, max norms and min positions too. Means must be bit-exact (the same
fp64 sums, child by child); radii may differ by rounding (fused products).
Selection must be index-exact except where a cut's score margin is below
1e-6. One FS-B decode step is also checked end to end."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_summaries_amd import ops
from block_sparse_attention_summaries_amd.inputs import config, make_inputs
from tests.gpu_util import check_indices, dev, host, rel_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _build(cfg, x, n):
    b = cfg["b"]
    kb, mx, ce = oracle.block_summaries(x["k"], b, nblocks=x["L"] // b)
    fo = oracle.forest_build(kb, mx, ce, n)
    fg = ops.sparse_forest_build(dev(kb), dev(mx), dev(ce), n)
    torch.cuda.synchronize()
    fg = {k: host(v) for k, v in fg.items()}
    assert np.array_equal(fg["nmem"], fo["nmem"])
    assert np.array_equal(fg["members"], fo["members"])
    assert np.array_equal(fg["amax"], fo["amax"]) and np.array_equal(fg["pmin"], fo["pmin"])
    assert np.array_equal(fg["mu"], fo["mu"])
    assert np.allclose(fg["rad"], fo["rad"], rtol=1e-6, atol=0)
    return kb, mx, ce, fo, fg


@pytest.mark.parametrize("over,n", [
    (dict(n=16384, Hq=2, Hkv=2, seed=151), 512),            # three levels (512 -> 32 -> 2)
    (dict(n=4096, Hq=2, Hkv=2, seed=152), 17),              # two level-1 nodes
    (dict(n=4096, Hq=2, Hkv=2, seed=153), 16),              # cells only
    (dict(n=4096, Hq=2, Hkv=2, seed=154), 1),
    (dict(n=4096, Hq=2, Hkv=1, d=128, dtype="f32", seed=155), 100),
    (dict(n=524288, Hq=1, Hkv=1, seed=156), 16384),         # 512K tokens: 16384 cells, 1092 nodes
])
def test_forest_build_parity(over, n):
    cfg = config("prefill_cells", **over)
    _say(f"[forest build] {over} n={n}")
    x = make_inputs(cfg) if over["n"] < 524288 else _keys_only(cfg)
    _build(cfg, x, n)


def _keys_only(cfg):
    """Seeded keys of the workload without the (large) query and value arrays."""
    from block_sparse_attention_summaries_amd.inputs import _normal
    rng = np.random.Generator(np.random.PCG64(cfg["seed"]))
    return dict(L=cfg["n"], k=_normal(rng, (cfg["B"], cfg["Hkv"], cfg["n"], cfg["d"]), cfg["dtype"]))


def _select_case(cfg, x, nrows, share_group=False):
    b, qb, K, L = cfg["b"], cfg["qblock"], cfg["K"], x["L"]
    q0 = L - nrows                              # rows of the last query block
    assert q0 // qb == (L - 1) // qb
    n = (qb * (q0 // qb)) // b
    kb, mx, ce, fo, fg = _build(cfg, x, n)
    q = np.ascontiguousarray(x["q"][:, :, q0:])
    Hsel = cfg["Hkv"] if share_group else cfg["Hq"]
    lam = np.ascontiguousarray(x["erf_lambda"][:Hsel])
    sig = np.ascontiguousarray(x["erf_sigma"][:Hsel])
    ora = oracle.forest_select(q, kb, mx, ce, x["k"], fo, n, Hkv=cfg["Hkv"], b=b, K=K, q_pos0=q0,
                               share_group=share_group, erf_lambda=lam, erf_sigma=sig)
    forest = {k: dev(v) for k, v in fo.items()}
    idx, keff = ops.sparse_forest_select(dev(q), dev(kb), dev(mx), dev(ce), dev(x["k"]), forest, n,
                                         Hkv=cfg["Hkv"], b=b, K=K, q_pos0=q0, prefix_mode=1, qblock=qb,
                                         share_group=share_group, erf_lambda=dev(lam), erf_sigma=dev(sig))
    torch.cuda.synchronize()
    idx = host(idx)
    ex = check_indices(idx, ora, _rerank_fn(q, x["k"], cfg, n, share_group))
    assert np.array_equal(host(keff), np.minimum(K, np.sum(ora["idx"] >= 0, axis=-1)))
    return ex, (kb, mx, ce, fo, n, q0, ora, idx)


def _rerank_fn(q, k, cfg, n, share_group):
    """Scores for the gap rule of the forest selection: each prefix cell's
    re-rank score (logsumexp over its token keys).  A row whose oracle cut
    margin is below 1e-6 may end on another set, but every cell it keeps must
    re-rank within 1e-6 of the oracle's K-th."""
    def score_fn(pos):
        return oracle.cell_token_lse(q, k, Hkv=cfg["Hkv"], b=cfg["b"], bidx=pos[0], hs=pos[1], row=pos[2],
                                     ncells=n, share_group=share_group)
    return score_fn


@pytest.mark.parametrize("over,nrows,share_group", [
    (dict(n=16384, Hq=2, Hkv=2, seed=157), 128, False),
    (dict(n=8192, Hq=8, Hkv=2, seed=158), 64, True),          # group mean
    (dict(n=4096, Hq=2, Hkv=2, d=128, dtype="f32", K=6, seed=159), 32, False),
    (dict(n=2048, Hq=2, Hkv=2, b=16, K=4, seed=160), 100, False),
])
def test_forest_select_parity(over, nrows, share_group):
    cfg = config("prefill_cells", **over)
    _say(f"[forest select] {over} rows={nrows} share_group={share_group}")
    x = make_inputs(cfg)
    ex, _ = _select_case(cfg, x, nrows, share_group)
    _say(f"  exempt rows {ex}")


def test_fsb_decode_step_end_to_end():
    """One FS-B decode step at n = 65536 (2048 cells): forests, beam search,
    re-rank, then the two-branch attention; GPU chain against the oracle."""
    cfg = config("prefill_cells", n=65536, Hq=2, Hkv=2, seed=161)
    x = make_inputs(cfg)
    ex, (kb, mx, ce, fo, n, q0, ora, idx) = _select_case(cfg, x, 1)
    assert np.array_equal(idx, ex.idx)
    b, qb, K = cfg["b"], cfg["qblock"], cfg["K"]
    q1 = np.ascontiguousarray(x["q"][:, :, q0:])
    akw = dict(b=b, K=K, q_pos0=q0, share_group=False, local=1, window=cfg["window"], prefix_mode=1, qblock=qb)
    o_o, _ = oracle.attn_fwd(q1, x["k"], x["v"], ex.idx, None, alpha=x["alpha"], **akw)
    o, _ = ops.sparse_attn_fwd(dev(q1), dev(x["k"]), dev(x["v"]), dev(idx), None, alpha=dev(x["alpha"]), **akw)
    torch.cuda.synchronize()
    e = rel_err(host(o), o_o)
    _say(f"  o rel err {e:.2e}")
    assert e <= 2e-2


def test_fsb_decode_512k_full_size():
    """The FS-B decode step as the benchmark times it: forests over the 16384
    prefix cells of a 512K context, 16 heads, d = 64, one query after the last
    full cell; beam search, re-rank and the two-branch attention against the
    oracle."""
    cfg = config("prefill_cells", kind="cell_decode", n=524288, seed=163)
    _say("[fsb decode] 512K full size, 16 heads")
    x = make_inputs(cfg)
    b, qb, K, L, q0 = cfg["b"], cfg["qblock"], cfg["K"], x["L"], x["q_pos0"]
    n = (qb * (q0 // qb)) // b
    kb, mx, ce, fo, fg = _build(cfg, x, n)
    lam, sig = x["erf_lambda"], x["erf_sigma"]
    ora = oracle.forest_select(x["q"], kb, mx, ce, x["k"], fo, n, Hkv=cfg["Hkv"], b=b, K=K, q_pos0=q0,
                               share_group=False, erf_lambda=lam, erf_sigma=sig)
    forest = {k: dev(v) for k, v in fo.items()}
    kd, vd, qd = dev(x["k"]), dev(x["v"]), dev(x["q"])
    idx, keff = ops.sparse_forest_select(qd, dev(kb), dev(mx), dev(ce), kd, forest, n, Hkv=cfg["Hkv"], b=b, K=K,
                                         q_pos0=q0, prefix_mode=1, qblock=qb, share_group=False,
                                         erf_lambda=dev(lam), erf_sigma=dev(sig))
    akw = dict(b=b, K=K, q_pos0=q0, share_group=False, local=1, window=cfg["window"], prefix_mode=1, qblock=qb)
    o, _ = ops.sparse_attn_fwd(qd, kd, vd, idx, None, alpha=dev(x["alpha"]), **akw)
    torch.cuda.synchronize()
    idx = host(idx)
    ex = check_indices(idx, ora, _rerank_fn(x["q"], x["k"], cfg, n, False))
    _say(f"  exempt rows {ex}")
    assert np.array_equal(host(keff), np.minimum(K, np.sum(ora["idx"] >= 0, axis=-1)))
    o_o, _ = oracle.attn_fwd(x["q"], x["k"], x["v"], ex.idx, None, alpha=x["alpha"], **akw)
    for h in range(cfg["Hq"]):
        e = rel_err(host(o)[:, h:h + 1], o_o[:, h:h + 1])
        assert e <= 2e-2, (h, e)

