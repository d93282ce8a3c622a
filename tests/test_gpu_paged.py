"""GPU parity of the paged decode path (sparse_block_summaries_paged,
sparse_decode_step_paged): the K / V caches are scattered into page pools in a
seeded random page order ("SAS" review, inference setup: paged KV cache), the
oracle runs on the contiguous caches the pages describe, and the paged results
must pass the same checks and equal the contiguous GPU path bit for bit."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_summaries_amd import ops
from block_sparse_attention_summaries_amd.inputs import config, f32_to_bf16_bits, make_inputs
from tests.gpu_util import dev, host, rel_err
from tests.test_gpu_parity import _check_decode_chain

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _paginate(caches, b, seed, spare_pages=5, spare_cols=3):
    """Scatter [B, Hkv, L, d] caches into pools [num_pages, Hkv, b, d] in a
    seeded random page order; the unused pages and the tail of a partial
    last block hold seeded noise; table columns past the blocks are -1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, Hkv, L, d = caches[0].shape
    nblk = (L + b - 1) // b
    npages = B * nblk + spare_pages
    order = rng.permutation(npages).astype(np.int32)
    table = np.full((B, nblk + spare_cols), -1, np.int32)
    table[:, :nblk] = order[:B * nblk].reshape(B, nblk)
    spare = order[B * nblk:]
    pools = []
    for x in caches:
        def noise(shape):
            z = rng.standard_normal(shape, dtype=np.float32)
            return f32_to_bf16_bits(z) if x.dtype == np.uint16 else z
        pool = np.empty((npages, Hkv, b, d), dtype=x.dtype)
        pool[spare] = noise((len(spare), Hkv, b, d))
        full = L // b
        blocks = x[:, :, :full * b, :].reshape(B, Hkv, full, b, d).transpose(0, 2, 1, 3, 4)
        pool[table[:, :full].reshape(-1)] = blocks.reshape(B * full, Hkv, b, d)
        if full < nblk:                                    # partial last block
            n = L - full * b
            for bi in range(B):
                pg = table[bi, full]
                pool[pg] = noise((Hkv, b, d))
                pool[pg, :, :n, :] = x[bi, :, full * b:, :]
        pools.append(pool)
    return pools, table, npages


def _decode_paged(cfg, x, seed):
    b, L, K = cfg["b"], x["L"], cfg["K"]
    nblk_full = L // b
    q_pos0 = x["q_pos0"]
    gate = cfg["gate"]
    proj = x.get("proj_w")
    kw = dict(Hkv=cfg["Hkv"], b=b, K=K, q_pos0=q_pos0, gate=gate, share_group=cfg["share_group"])
    kb_o, mx_o, ce_o = oracle.block_summaries(x["k"], b, nblocks=nblk_full, ccap=max(nblk_full, 1))
    ora = oracle.score_select(x["q"], kb_o, mx_o, ce_o, proj_w=proj, **kw)
    o_o, lse_o = oracle.attn_fwd(x["q"], x["k"], x["v"], ora["idx"], ora["logg"] if gate else None,
                                 b=b, K=K, q_pos0=q_pos0, share_group=cfg["share_group"])
    (kp, vp), table, npages = _paginate([x["k"], x["v"]], b, seed)
    qd, kpd, vpd, td = dev(x["q"]), dev(kp), dev(vp), dev(table)
    pw = None if proj is None else dev(proj)
    ccap = max(nblk_full, 1)
    kb, mx, ce = ops.sparse_block_summaries_paged(kpd, td, L, b, num_blocks=nblk_full, ccap=ccap)
    idx, logg, keff, o, lse = ops.sparse_decode_step_paged(qd, kb, mx, ce, kpd, vpd, td, L, proj_w=pw, **kw)
    # the contiguous path on the same inputs
    kd, vd = dev(x["k"]), dev(x["v"])
    kb_c, mx_c, ce_c = ops.sparse_block_summaries(kd, b, num_blocks=nblk_full, ccap=ccap)
    c_idx, c_logg, c_keff, c_o, c_lse = ops.sparse_decode_step(qd, kb_c, mx_c, ce_c, kd, vd, proj_w=pw, **kw)
    torch.cuda.synchronize()

    def score_fn(pos):
        return oracle.scores_one_row(x["q"], kb_o, mx_o, ce_o, Hkv=cfg["Hkv"], b=b, q_pos0=q_pos0, bidx=pos[0],
                                     hs=pos[1], row=pos[2], share_group=cfg["share_group"], proj_w=proj)

    def oracle_attn(idx_a, logg_a):
        return oracle.attn_fwd(x["q"], x["k"], x["v"], idx_a, logg_a if gate else None, b=b, K=K, q_pos0=q_pos0,
                               share_group=cfg["share_group"])[0]

    r = dict(ora=ora, o_o=o_o, lse_o=lse_o, score_fn=score_fn, oracle_attn=oracle_attn)
    paged = dict(idx=host(idx), logg=None if logg is None else host(logg), keff=host(keff), o=host(o),
                 lse=host(lse), kb=host(kb), mx=host(mx))
    contig = dict(idx=host(c_idx), logg=None if c_logg is None else host(c_logg), keff=host(c_keff),
                  o=host(c_o), lse=host(c_lse))
    return r, paged, contig, (kb_o, mx_o)


@pytest.mark.parametrize("name,over", [
    ("decode_32k", dict(n=8192, seed=81)),                                   # bf16, merge folded in
    ("decode_32k", dict(n=4096, t=17, K=8, seed=82)),                        # partial current block
    ("decode_32k", dict(n=4096, b=32, K=12, share_group=False, Hq=8, Hkv=8, seed=83)),
    ("decode_512k", dict(n=65536, seed=84)),                                 # projection, K = 32
    ("tiny_decode", dict(t=40, seed=85)),                                    # fp32: two-call path
])
def test_paged_decode_step_parity(name, over):
    cfg = config(name, **over)
    _say(f"[paged decode] {name} {over}")
    x = make_inputs(cfg)
    r, paged, contig, (kb_o, mx_o) = _decode_paged(cfg, x, seed=over["seed"] + 1000)
    # summaries through the pages: bit-exact
    assert np.array_equal(paged["kb"], kb_o)
    assert np.array_equal(paged["mx"], mx_o)
    ex = _check_decode_chain(cfg, r, paged)
    for key in ("idx", "keff", "o", "lse"):
        assert np.array_equal(paged[key], contig[key]), key
    if cfg["gate"]:
        assert np.array_equal(paged["logg"], contig["logg"])
    _say(f"  exempt rows {ex}")


def test_paged_summary_of_unmapped_block_is_zero():
    """A block whose page id lies outside the pool reads as zero keys (no
    access outside the pool); the other blocks are unaffected."""
    cfg = config("decode_32k", n=2048, seed=86)
    x = make_inputs(cfg)
    b, L = cfg["b"], x["L"]
    (kp,), table, npages = _paginate([x["k"]], b, seed=87)
    table[0, 5] = npages + 7
    table[0, 9] = -3
    kb, mx, _ = ops.sparse_block_summaries_paged(dev(kp), dev(table), L, b)
    torch.cuda.synchronize()
    kb, mx = host(kb), host(mx)
    kb_o, mx_o, _ = oracle.block_summaries(x["k"], b, nblocks=L // b)
    bad = np.zeros(kb.shape[2], bool)
    bad[[5, 9]] = True
    assert not np.any(kb[:, :, bad]) and not np.any(mx[:, :, bad])
    assert np.array_equal(kb[:, :, ~bad], kb_o[:, :, ~bad]) and np.array_equal(mx[:, :, ~bad], mx_o[:, :, ~bad])


def test_paged_decode_512k_full_size():
    """The full 512K decode workload (8193 pages of 64 tokens per kv head)."""
    cfg = config("decode_512k")
    _say("[paged decode] decode_512k full size")
    x = make_inputs(cfg)
    r, paged, contig, (kb_o, mx_o) = _decode_paged(cfg, x, seed=88)
    assert np.array_equal(paged["kb"], kb_o) and np.array_equal(paged["mx"], mx_o)
    ex = _check_decode_chain(cfg, r, paged)
    for key in ("idx", "keff", "o", "lse"):
        assert np.array_equal(paged[key], contig[key]), key
    _say(f"  exempt rows {ex}")


def test_paged_decode_with_unmapped_selected_block():
    """A selected block whose page id lies outside the pool is attended as
    empty: the selection (from the summaries the caller passes) is unchanged,
    and o / lse equal the oracle's attention with that block left out of every
    head's selection."""
    cfg = config("decode_32k", n=4096, K=8, seed=88)
    _say("[paged decode] unmapped selected block")
    x = make_inputs(cfg)
    b, L, K = cfg["b"], x["L"], cfg["K"]
    nblk_full = L // b
    kw = dict(Hkv=cfg["Hkv"], b=b, K=K, q_pos0=x["q_pos0"], gate=cfg["gate"], share_group=cfg["share_group"])
    (kp, vp), table, npages = _paginate([x["k"], x["v"]], b, seed=89)
    qd, kpd, vpd = dev(x["q"]), dev(kp), dev(vp)
    kb, mx, ce = ops.sparse_block_summaries(dev(x["k"]), b, num_blocks=nblk_full, ccap=nblk_full)
    idx0, logg0, _, _, _ = ops.sparse_decode_step_paged(qd, kb, mx, ce, kpd, vpd, dev(table), L, **kw)
    torch.cuda.synchronize()
    idx0 = host(idx0)
    c_drop = int(idx0[0, 0, 0, 0])
    assert 0 <= c_drop < nblk_full
    table[0, c_drop] = npages + 3
    idx1, logg1, _, o1, lse1 = ops.sparse_decode_step_paged(qd, kb, mx, ce, kpd, vpd, dev(table), L, **kw)
    torch.cuda.synchronize()
    idx1, logg1 = host(idx1), host(logg1)
    assert np.array_equal(idx1, idx0)
    idx_kept = np.where(idx1 == c_drop, -1, idx1).astype(np.int32)
    o_ref, lse_ref = oracle.attn_fwd(x["q"], x["k"], x["v"], idx_kept, logg1.astype(np.float64), b=b, K=K,
                                     q_pos0=x["q_pos0"], share_group=cfg["share_group"])
    err = rel_err(host(o1), o_ref)
    assert err <= 2e-2, err
    assert np.abs(host(lse1) - lse_ref).max() <= 2e-1
    _say(f"  block {c_drop} unmapped: o rel err {err:.2e}")
