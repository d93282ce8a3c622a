"""GPU parity of the selector-side backward (sparse_select_bwd): the gate
gradient dg carried through log g = s - LSE(s) into q and the block summaries
("SAS" review, "How it works" step 5; §4.2.2 softmax gate), against the fp64
oracle on the same seeded inputs, the oracle's summaries and its selection.

Tolerance: 2e-2 of the largest magnitude per (batch, head) slice, the bar of
the other bf16 backward outputs.  The kernel recomputes the scores from q_hat
rounded to bf16 and feeds ds to bf16 MFMAs (split hi + lo for dq, one bf16
for dkbar); the oracle works in fp64 throughout."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_summaries_amd import ops
from block_sparse_attention_summaries_amd.inputs import bf16_bits_to_f32, config, f32_to_bf16_bits, make_inputs
from tests.gpu_util import dev, host, rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _gate_grads(shape, seed):
    """Seeded stand-in for the dg that sparse_attn_bwd hands over."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(shape, dtype=np.float32)


def _case(cfg, x, *, share_group, q_pos0=0, kv_slice=None, seed=900, proj=False, with_dk=False):
    """Run oracle and GPU on rows q_pos0.. of the inputs; kv_slice = (batch,
    kv head) restricts both to one selection group (the heads are
    independent), which keeps the full-size oracle run short.  proj: through
    the learned projection W (dW checked too); with_dk: dk += dkbar / b on a
    seeded dk."""
    b, K, Hkv = cfg["b"], cfg["K"], cfg["Hkv"]
    G = cfg["Hq"] // Hkv
    q, k = x["q"][:, :, q_pos0:], x["k"]
    if kv_slice is not None:
        bi, kh = kv_slice
        q = q[bi:bi + 1, kh * G:kh * G + G]
        k = k[bi:bi + 1, kh:kh + 1]
        Hkv = 1
    q, k = np.ascontiguousarray(q), np.ascontiguousarray(k)
    B, Hq, nq, _ = q.shape
    L = k.shape[2]
    Hsel = Hkv if share_group else Hq
    W = x["proj_w"] if proj else None
    kw = dict(Hkv=Hkv, b=b, K=K, q_pos0=q_pos0, share_group=share_group)
    kb, mx, ce = oracle.block_summaries(k, b, nblocks=L // b)
    ora = oracle.score_select(q, kb, mx, ce, gate=True, proj_w=W, **kw)
    dg = _gate_grads((B, Hsel, nq, K), seed)
    res = oracle.select_bwd(q, kb, ora["idx"], dg, proj_w=W, **kw)
    dq_o, dkb_o = res[0], res[1]
    dk_in = dk_g = None
    if with_dk:
        rng = np.random.Generator(np.random.PCG64(seed + 1))
        dk_in = f32_to_bf16_bits(rng.standard_normal(k.shape, dtype=np.float32) * np.float32(0.01))
        dk_g = dev(dk_in)
    dq, dkb, dw = ops.sparse_select_bwd(dev(q), dev(kb), dev(mx), dev(ce), dev(ora["idx"]),
                                        dev(ora["logg"].astype(np.float32)), dev(dg), gate=True, dk=dk_g,
                                        proj_w=None if W is None else dev(W), **kw)
    torch.cuda.synchronize()
    dq, dkb = host(dq), host(dkb)
    e_dq, e_dk = rel_err(dq, dq_o), rel_err(dkb, dkb_o)
    msg = f"  dq {e_dq:.2e} dkbar {e_dk:.2e}"
    if proj:
        e_dw = rel_err(host(dw)[None, None], res[2][None, None])
        msg += f" dW {e_dw:.2e}"
        assert e_dw <= TOL, e_dw
    if with_dk:
        want = bf16_bits_to_f32(dk_in).astype(np.float64) + oracle.mean_bwd(dkb_o, b, L)
        e_k = rel_err(host(dk_g), want)
        msg += f" dk {e_k:.2e}"
        assert e_k <= TOL, e_k
        # tokens past the last summary are untouched
        ncap = kb.shape[2]
        assert np.array_equal(host(dk_g)[:, :, ncap * b:], dk_in[:, :, ncap * b:])
    _say(msg)
    # rows without candidates and summaries that are no row's candidate get 0
    first = max(0, b - q_pos0)
    assert not np.any(dq[:, :, :min(first, nq)])
    ncand_max = (q_pos0 + nq - 1) // b
    assert not np.any(dkb[:, :, ncand_max:])
    assert e_dq <= TOL and e_dk <= TOL, (e_dq, e_dk)


@pytest.mark.parametrize("over,share_group", [
    (dict(B=2, n=1024, Hq=8, Hkv=2, K=8, seed=61), True),                    # G = 4, d = 128
    (dict(B=1, n=1000, Hq=4, Hkv=4, K=5, seed=62), False),                   # ragged, per-head selection
    (dict(B=1, n=700, Hq=4, Hkv=2, b=32, d=64, K=8, seed=63), True),         # d = 64, b = 32, ragged
    (dict(B=1, n=640, Hq=8, Hkv=1, b=16, K=32, seed=64), True),              # G = 8, K = 32, b = 16
    (dict(B=1, n=900, Hq=4, Hkv=2, b=32, d=64, K=3, seed=65), False),        # G = 2 per head, d = 64
])
def test_select_bwd_parity(over, share_group):
    cfg = config("train", **over)
    _say(f"[select bwd] {over} share_group={share_group}")
    _case(cfg, make_inputs(cfg), share_group=share_group)


def test_select_bwd_rows_after_offset():
    """Rows at positions q_pos0.. of a longer cache (chunked training rows)."""
    cfg = config("train", B=1, n=1536, Hq=4, Hkv=2, K=6, seed=66)
    _case(cfg, make_inputs(cfg), share_group=True, q_pos0=600)


def test_select_bwd_keys_with_common_offset():
    """Keys with a large shared offset: the summaries differ only slightly, so
    dq comes from heavy cancellation in sum_c ds_c kbar_c (ds sums to zero)."""
    cfg = config("train", B=1, n=1024, Hq=4, Hkv=2, K=8, seed=67)
    x = make_inputs(cfg)
    x["k"] = f32_to_bf16_bits(bf16_bits_to_f32(x["k"]) + np.float32(4.0))
    _case(cfg, x, share_group=True)


def test_select_bwd_full_size_one_slice():
    """Full training workload (8192 rows, 128 blocks, d = 128, K = 16), one
    (batch, kv head) selection group."""
    cfg = config("train")
    _say("[select bwd] full size, slice b=2 kvh=3")
    _case(cfg, make_inputs(cfg), share_group=True, kv_slice=(2, 3))


@pytest.mark.parametrize("over,share_group", [
    (dict(B=1, n=1024, Hq=8, Hkv=2, K=8, seed=68, proj=True), True),               # d = 128
    (dict(B=2, n=700, Hq=4, Hkv=2, b=32, d=64, K=6, seed=69, proj=True), False),    # d = 64, ragged
])
def test_select_bwd_through_projection(over, share_group):
    """Learned projection ktilde = W kbar: dq, dkbar = W^T dktilde and dW."""
    cfg = config("train", **over)
    _say(f"[select bwd proj] {over} share_group={share_group}")
    _case(cfg, make_inputs(cfg), share_group=share_group, proj=True)


@pytest.mark.parametrize("over,proj", [
    (dict(B=1, n=1000, Hq=4, Hkv=2, K=5, seed=70), False),                # 1000 = 15 blocks + 40 tokens
    (dict(B=1, n=640, Hq=4, Hkv=1, b=32, d=64, K=4, seed=71, proj=True), True),
])
def test_select_bwd_into_keys_through_the_mean(over, proj):
    """dk += dkbar / b over the tokens of each summarised block; tokens of
    the open tail block are left as they were."""
    cfg = config("train", **over)
    _say(f"[select bwd dk] {over}")
    _case(cfg, make_inputs(cfg), share_group=True, proj=proj, with_dk=True)
