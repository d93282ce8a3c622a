"""GPU parity of the optional fp8 block summaries of the decode scorer (OCP
E4M3, one fp32 scale = amax / 448 per block):

- sparse_quantize_summaries_fp8: codes and scales bit-exact against the
  oracle (bf16 and fp32 summaries, a zero block, a block range, the 512K
  summaries in full);
- sparse_dequantize_summaries_fp8 (the scorer's own decode): every one of
  the 256 codes, times several scales, bit-exact against the exact rebuild
  rounded to fp32;
- decode steps whose scorer reads the codes: selection against the oracle
  scoring the exactly rebuilt summaries (index-exact up to the K-boundary gap
  rule, log gates to 1e-4), output against the oracle's attention over that
  selection, and the one-call step bit-identical to the two calls."""
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

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("d", [64, 128])
def test_dequantize_every_code(d):
    codes = np.tile(np.arange(256, dtype=np.uint8), 8).reshape(-1, d)          # every code, 8 times
    scales = np.resize(np.array([1.0, 0.3712, 3.1e-3, 0.0, -2.5], np.float32), codes.shape[0])
    got = host(ops.sparse_dequantize_summaries_fp8(dev(codes), dev(scales)))
    want = oracle.dequantize_fp8(codes, scales).astype(np.float32)   # the exact product, rounded to fp32
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


@pytest.mark.parametrize("name,over", [
    ("tiny_decode", {}),
    ("decode_32k", {}),
    ("decode_32k", dict(d=64, dtype="f32", n=4096, Hq=8, Hkv=4, seed=21)),
])
def test_quantize_parity(name, over):
    cfg = config(name, **over)
    x = make_inputs(cfg)
    b = cfg["b"]
    kb, _, _ = oracle.block_summaries(x["k"], b, nblocks=x["L"] // b)
    kb[:, :, 3] = 0                                  # a block of zeros
    codes_o, sc_o = oracle.quantize_fp8(kb)
    codes_g, sc_g = ops.sparse_quantize_summaries_fp8(dev(kb))
    torch.cuda.synchronize()
    assert np.array_equal(host(sc_g).view(np.uint32), sc_o.view(np.uint32))
    assert np.array_equal(host(codes_g), codes_o)
    assert np.all(sc_o[:, :, 3] == 0) and np.all(codes_o[:, :, 3] == 0)


def test_quantize_range_only():
    cfg = config("decode_32k", n=4096)
    x = make_inputs(cfg)
    b = cfg["b"]
    kb, _, _ = oracle.block_summaries(x["k"], b, nblocks=x["L"] // b)
    codes_o, sc_o = oracle.quantize_fp8(kb, first=5, num=4)
    codes = torch.full(kb.shape, 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full(kb.shape[:3], -1.0, dtype=torch.float32, device="cuda")
    ops.sparse_quantize_summaries_fp8(dev(kb), first_block=5, num_blocks=4, codes=codes, scales=scales)
    c, s = host(codes), host(scales)
    assert np.array_equal(c[:, :, 5:9], codes_o[:, :, 5:9]) and np.array_equal(s[:, :, 5:9], sc_o[:, :, 5:9])
    out = np.ones(kb.shape[2], bool)
    out[5:9] = False
    assert np.all(c[:, :, out] == 0xAB) and np.all(s[:, :, out] == -1.0)


def test_quantize_full_512k():
    cfg = config("decode_512k")
    _say("[fp8 quantize] decode_512k full size")
    x = make_inputs(cfg)
    b = cfg["b"]
    kb, _, _ = oracle.block_summaries(x["k"], b, nblocks=x["L"] // b)
    codes_o, sc_o = oracle.quantize_fp8(kb)
    codes_g, sc_g = ops.sparse_quantize_summaries_fp8(dev(kb))
    torch.cuda.synchronize()
    assert np.array_equal(host(sc_g).view(np.uint32), sc_o.view(np.uint32))
    assert np.array_equal(host(codes_g), codes_o)


def _fp8_decode(cfg, x):
    K, b, L = cfg["K"], cfg["b"], x["L"]
    nblk = L // b
    q_pos0, gate, sg = x["q_pos0"], cfg["gate"], cfg["share_group"]
    proj = x.get("proj_w")
    kw = dict(Hkv=cfg["Hkv"], b=b, K=K, q_pos0=q_pos0, gate=gate, share_group=sg)
    kb_o, mx_o, ce_o = oracle.block_summaries(x["k"], b, nblocks=nblk)
    codes_o, sc_o = oracle.quantize_fp8(kb_o)
    ora = oracle.score_select(x["q"], oracle.dequantize_fp8(codes_o, sc_o), mx_o, ce_o, proj_w=proj, **kw)
    o_o, _ = oracle.attn_fwd(x["q"], x["k"], x["v"], ora["idx"], ora["logg"] if gate else None, b=b, K=K,
                             q_pos0=q_pos0, share_group=sg)
    ref = oracle.score_select(x["q"], kb_o, mx_o, ce_o, proj_w=proj, **kw)      # the same step in dtype
    qd, kd, vd = dev(x["q"]), dev(x["k"]), dev(x["v"])
    pw = None if proj is None else dev(proj)
    kb_g, mx_g, ce_g = ops.sparse_block_summaries(kd, b)
    codes_g, sc_g = ops.sparse_quantize_summaries_fp8(kb_g)
    idx, logg, keff = ops.sparse_score_select(qd, codes_g, mx_g, ce_g, proj_w=pw, kbar_scale=sc_g, **kw)
    o, lse = ops.sparse_attn_fwd(qd, kd, vd, idx, logg if gate else None, b=b, K=K, q_pos0=q_pos0, share_group=sg)
    f = ops.sparse_decode_step(qd, codes_g, mx_g, ce_g, kd, vd, proj_w=pw, kbar_scale=sc_g, **kw)
    torch.cuda.synchronize()
    idx, keff, o, lse = host(idx), host(keff), host(o), host(lse)
    kb_r = oracle.dequantize_fp8(codes_o, sc_o)
    ex = check_indices(idx, ora, lambda p: oracle.scores_one_row(
        x["q"], kb_r, mx_o, ce_o, Hkv=cfg["Hkv"], b=b, q_pos0=q_pos0, bidx=p[0], hs=p[1], row=p[2],
        share_group=sg, proj_w=proj))
    assert np.array_equal(keff, ora["k_eff"])
    if gate:
        dl = np.abs(host(logg).astype(np.float64) - ex.logg)
        assert dl.max(initial=0.0) <= 1e-4 * max(1.0, np.abs(ex.logg).max())
    if ex.alt:
        o_o, _ = oracle.attn_fwd(x["q"], x["k"], x["v"], ex.idx, ex.logg if gate else None, b=b, K=K,
                                 q_pos0=q_pos0, share_group=sg)
    for bi in range(cfg["B"]):
        for h in range(cfg["Hq"]):
            e = rel_err(o[bi:bi + 1, h:h + 1], o_o[bi:bi + 1, h:h + 1])
            assert e <= TOL[cfg["dtype"]], (bi, h, e)
    fi, fl, fk, fo, fs = (None if t is None else host(t) for t in f)
    assert np.array_equal(fi, idx) and np.array_equal(fk, keff) and np.array_equal(fo, o) and np.array_equal(fs, lse)
    if gate:
        assert np.array_equal(fl, host(logg))
    # how much of the selection in dtype the fp8 summaries keep (reported, not a bar)
    keep = np.mean([len(set(a[a >= 0]) & set(r[r >= 0])) / max(1, (r >= 0).sum())
                    for a, r in zip(ora["idx"].reshape(-1, K), ref["idx"].reshape(-1, K))])
    return ex, keep


@pytest.mark.parametrize("name,over", [
    ("decode_32k", {}),
    ("decode_32k", dict(n=4096, t=33, share_group=False, Hq=8, Hkv=8, seed=22)),
    ("decode_512k", dict(n=65536, seed=23)),                 # projection W
    ("decode_32k", dict(d=64, dtype="f32", n=4096, Hq=8, Hkv=4, proj=True, seed=24)),
    ("tiny_decode", dict(gate=True, seed=25)),
])
def test_fp8_decode_parity(name, over):
    cfg = config(name, **over)
    _say(f"[fp8 decode] {name} {over}")
    ex, keep = _fp8_decode(cfg, make_inputs(cfg))
    _say(f"  exempt rows {ex}; selection kept vs the summaries in dtype {keep:.3f}")


def test_fp8_decode_512k_full_size():
    cfg = config("decode_512k")
    _say("[fp8 decode] decode_512k full size")
    ex, keep = _fp8_decode(cfg, make_inputs(cfg))
    _say(f"  exempt rows {ex}; selection kept vs the summaries in dtype {keep:.3f}")
