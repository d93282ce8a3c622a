"""GPU parity of the FS-L fixed-state path ("FreeSolo" review, the two
variants): sparse_retain_cells against the oracle's kept set (bit-exact,
including equal norms), sparse_score_select_subset against the oracle's
selection inside the kept set (index-exact up to the K-boundary gap rule,
gates to 1e-4), and one FS-L decode step end to end: summaries, kept set,
selection in it, then the two-branch attention (selected cells + window,
alpha mix)."""
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


@pytest.mark.parametrize("B,Hkv,ncand,W,P,levels", [
    (2, 3, 200, 8, 64, 5),          # many equal norms
    (2, 3, 200, 8, 64, 100000),
    (1, 4, 16384, 8, 64, 100000),   # 512K tokens of 32-token cells
    (1, 2, 16384, 8, 64, 3),
    (1, 2, 73, 8, 64, 4), (1, 2, 72, 8, 64, 4), (1, 2, 40, 8, 64, 4), (1, 2, 5, 8, 64, 4),
    (1, 2, 0, 8, 64, 4), (2, 2, 1000, 0, 64, 9), (2, 2, 1000, 16, 32, 9), (1, 1, 777, 192, 64, 50),
])
def test_retain_cells_parity(B, Hkv, ncand, W, P, levels):
    rng = np.random.default_rng(ncand + 31 * W + P + levels)
    ccap = max(ncand, 1) + 3
    a = (rng.integers(0, levels, size=(B, Hkv, ccap)) / 8.0).astype(np.float32)
    a[:, :, ncand:] = 1e9                        # cells past the prefix must never be kept
    cells_o, count_o = oracle.retain_cells(a, ncand=ncand, W=W, P=P)
    cells, count = ops.sparse_retain_cells(dev(a), ncand, W, P)
    torch.cuda.synchronize()
    assert np.array_equal(host(count), count_o)
    assert np.array_equal(host(cells), cells_o)


def _fs_case(cfg, x, share_group, gate, rows_q=None, q_pos0=0):
    """Kept set (oracle summaries and retention) and the selection inside it,
    GPU against oracle."""
    b, qb, K = cfg["b"], cfg["qblock"], cfg["K"]
    Hsel = cfg["Hkv"] if share_group else cfg["Hq"]
    q = x["q"] if rows_q is None else rows_q
    L = x["L"]
    kb, mx, ce = oracle.block_summaries(x["k"], b, nblocks=L // b)
    ncand = (qb * ((q_pos0 + q.shape[2] - 1) // qb)) // b
    cells, count = oracle.retain_cells(mx, ncand=ncand, W=8, P=64)
    kw = dict(Hkv=cfg["Hkv"], b=b, K=K, q_pos0=q_pos0, gate=gate, prefix_mode=1, qblock=qb,
              share_group=share_group)
    lam = np.ascontiguousarray(x["erf_lambda"][:Hsel])
    sig = np.ascontiguousarray(x["erf_sigma"][:Hsel])
    ora = oracle.score_select_subset(q, kb, mx, ce, cells, count, erf_lambda=lam, erf_sigma=sig, **kw)
    idx, logg, keff = ops.sparse_score_select_subset(dev(q), dev(kb), dev(mx), dev(ce), dev(cells), dev(count),
                                                     erf_lambda=dev(lam), erf_sigma=dev(sig), **kw)
    torch.cuda.synchronize()
    idx, keff = host(idx), host(keff)

    def score_fn(pos):
        # the row's scores on its kept candidate cells; every other cell is
        # not a candidate of the subset selection
        s = oracle.scores_one_row(q, kb, mx, ce, Hkv=cfg["Hkv"], b=b, q_pos0=q_pos0, bidx=pos[0], hs=pos[1],
                                  row=pos[2], prefix_mode=1, qblock=qb, share_group=share_group,
                                  erf_lambda=lam, erf_sigma=sig)
        kvh = pos[1] if share_group else pos[1] // (cfg["Hq"] // cfg["Hkv"])
        kept = cells[pos[0], kvh, :count[pos[0], kvh]]
        out = np.full(s.shape, -np.inf)
        kept = kept[(kept >= 0) & (kept < s.shape[0])]
        out[kept] = s[kept]
        return out

    ex = check_indices(idx, ora, score_fn)
    assert np.array_equal(keff, ora["k_eff"])
    if gate:
        d = np.abs(host(logg).astype(np.float64) - ex.logg)
        assert d.max(initial=0.0) <= 1e-4 * max(1.0, np.abs(ex.logg).max())
    return ex, (kb, mx, ce, cells, count, ora)


@pytest.mark.parametrize("over,share_group,gate", [
    (dict(n=4096, Hq=4, Hkv=4, seed=94), False, False),         # the FreeSolo geometry: erf bias, no gate
    (dict(n=3000, Hq=8, Hkv=2, seed=95), True, True),           # group mean, gate, ragged
    (dict(n=2048, Hq=4, Hkv=2, d=128, K=8, seed=96), False, True),
    (dict(n=2048, Hq=2, Hkv=2, dtype="f32", seed=97), False, True),
])
def test_select_subset_parity(over, share_group, gate):
    cfg = config("prefill_cells", **over)
    _say(f"[select subset] {over} share_group={share_group} gate={gate}")
    x = make_inputs(cfg)
    ex, _ = _fs_case(cfg, x, share_group, gate)
    _say(f"  exempt rows {ex}")


def test_fsl_decode_step_end_to_end():
    """One FS-L decode step at n = 65536 (2048 cells): kept set, top K inside
    it, then attention over the selected cells plus the window, mixed with
    alpha; GPU chain against the oracle chain."""
    cfg = config("prefill_cells", n=65536, Hq=4, Hkv=4, seed=98)
    x = make_inputs(cfg)
    pos = x["L"] - 1
    _fsl_step(cfg, x, np.ascontiguousarray(x["q"][:, :, pos:pos + 1]), pos)


def test_fsl_decode_512k_full_size():
    """The FS-L decode step as the benchmark times it: 512K tokens (16384
    cells), 16 heads, d = 64, one query after the last full cell."""
    cfg = config("prefill_cells", kind="cell_decode", n=524288, seed=99)
    _say("[fsl decode] 512K full size, 16 heads")
    x = make_inputs(cfg)
    _fsl_step(cfg, x, x["q"], x["q_pos0"])


def _fsl_step(cfg, x, q1, pos):
    b, qb, K = cfg["b"], cfg["qblock"], cfg["K"]
    ex, (kb, mx, ce, cells_o, count_o, ora) = _fs_case(cfg, x, False, False, rows_q=q1, q_pos0=pos)
    ncand = (qb * (pos // qb)) // b
    akw = dict(b=b, K=K, q_pos0=pos, share_group=False, local=1, window=cfg["window"], prefix_mode=1, qblock=qb)
    # the oracle's attention on the oracle's selection, or on the GPU's where
    # a row with a K-boundary gap below 1e-6 took another valid top-K
    o_o, _ = oracle.attn_fwd(q1, x["k"], x["v"], ex.idx, None, alpha=x["alpha"], **akw)
    # GPU chain from the keys: summaries, kept set, selection, attention
    kd, vd, qd = dev(x["k"]), dev(x["v"]), dev(q1)
    kb_g, mx_g, ce_g = ops.sparse_block_summaries(kd, b)
    cells, count = ops.sparse_retain_cells(mx_g, ncand, 8, 64)
    idx, _, _ = ops.sparse_score_select_subset(qd, kb_g, mx_g, ce_g, cells, count, Hkv=cfg["Hkv"], b=b, K=K,
                                               q_pos0=pos, gate=False, prefix_mode=1, qblock=qb, share_group=False,
                                               erf_lambda=dev(x["erf_lambda"]), erf_sigma=dev(x["erf_sigma"]))
    o, _ = ops.sparse_attn_fwd(qd, kd, vd, idx, None, alpha=dev(x["alpha"]), **akw)
    torch.cuda.synchronize()
    assert np.array_equal(host(cells), cells_o) and np.array_equal(host(count), count_o)
    assert np.array_equal(host(idx), ex.idx)
    e = rel_err(host(o), o_o)
    _say(f"  o rel err {e:.2e}")
    assert e <= 2e-2
