"""Full-size checks over every row (GPU).

The oracle computes the full-size prefill and training workloads on sampled
rows or slices only (its cost grows with rows x candidates x d in fp64).
These tests cover every row with properties that hold at any size, computed
by torch on the device from inputs the library does not touch:

- prefill_cells selection: recomputing every (row, candidate) score in fp64
  ("FreeSolo" review, "How it works": q.kbar / sqrt(d) plus the erf position
  bias), the returned set of each row is a valid top-K: K_eff = min(K,
  candidates) distinct candidates in ascending order, -1 after them, and no
  candidate left out scores above a kept one by more than the 1e-6 gap under
  which several sets are correct;
- prefill_cells attention: every row's output equals an fp32 dense
  evaluation of the two branches on the returned selection (routed cells;
  window (i - w, i]) mixed by alpha_h;
- training: forward outputs and lse and the backward gradients dq, dk, dv
  and dg of every (batch, kv head) slice equal torch autograd of the dense
  masked attention ("SAS" review §4.1 Eq. 4, §4.3 Eq. 9: current block plus
  the selected blocks, log-gate bias) on the oracle's selection.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_summaries_amd import ops
from block_sparse_attention_summaries_amd.inputs import config, make_inputs
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _rel(got: torch.Tensor, want: torch.Tensor) -> float:
    return float((got - want).abs().max() / want.abs().max().clamp_min(1e-30))


def test_prefill_cells_every_row():
    cfg = config("prefill_cells")
    _say("[every row] prefill_cells")
    x = make_inputs(cfg)
    b, qb, K, w, d, H = cfg["b"], cfg["qblock"], cfg["K"], cfg["window"], cfg["d"], cfg["Hq"]
    L = x["L"]
    lam = np.ascontiguousarray(x["erf_lambda"][:H])
    sig = np.ascontiguousarray(x["erf_sigma"][:H])
    qd, kd, vd = dev(x["q"]), dev(x["k"]), dev(x["v"])
    kb, mx, ce = ops.sparse_block_summaries(kd, b)
    kw = dict(Hkv=H, b=b, K=K, q_pos0=0, gate=False, prefix_mode=1, qblock=qb, share_group=False)
    idx, _, keff = ops.sparse_score_select(qd, kb, mx, ce, erf_lambda=dev(lam), erf_sigma=dev(sig), **kw)
    akw = dict(b=b, K=K, q_pos0=0, share_group=False, local=1, window=w, prefix_mode=1, qblock=qb)
    o, _ = ops.sparse_attn_fwd(qd, kd, vd, idx, None, alpha=dev(x["alpha"]), **akw)
    torch.cuda.synchronize()

    dv_ = qd.device
    rows = torch.arange(L, device=dv_)
    ncand = (qb * (rows // qb)) // b                       # cells before the row's query block
    C = int(ncand.max())
    cells = torch.arange(C, device=dv_)
    alpha = torch.from_numpy(np.ascontiguousarray(x["alpha"])).to(dv_)
    R = 2048
    worst_sel, worst_o = 0.0, 0.0
    for h in range(H):
        kbar = kb[0, h, :C].double()
        an = mx[0, h, :C].double()
        pc = ce.reshape(-1)[:C].double()
        k_h, v_h = kd[0, h].float(), vd[0, h].float()
        for r0 in range(0, L, R):
            r1 = min(L, r0 + R)
            ir = rows[r0:r1]
            nc = ncand[r0:r1]
            # ---- selection: a valid top-K of the fp64 scores
            q64 = qd[0, h, r0:r1].double()
            s = q64 @ kbar.T / math.sqrt(d)
            s = s + float(lam[h]) * an[None, :] * torch.special.erf(
                (ir[:, None].double() - pc[None, :]) / (2.0 * float(sig[h])))
            valid = cells[None, :] < nc[:, None]
            s = s.masked_fill(~valid, float("-inf"))
            sel = idx[0, h, r0:r1].long()
            ke = torch.minimum(nc, torch.full_like(nc, K))
            assert torch.equal(keff[0, h, r0:r1].long(), ke), h
            slot = torch.arange(K, device=dv_)[None, :]
            used = slot < ke[:, None]
            assert bool(((sel >= 0) == used).all()), h                       # -1 exactly past K_eff
            assert bool(((sel < nc[:, None]) | ~used).all()), h              # candidates only
            assert bool(((sel[:, 1:] > sel[:, :-1]) | ~used[:, 1:]).all()), h   # ascending, distinct
            # unused slots land on a dummy column past the candidates
            kept = torch.zeros((r1 - r0, C + 1), dtype=torch.bool, device=dv_)
            kept.scatter_(1, torch.where(used, sel, C), used)
            kept = kept[:, :C]
            s_kept = s.masked_fill(~kept, float("inf")).min(dim=1).values
            s_left = s.masked_fill(kept, float("-inf")).max(dim=1).values
            chk = (ke > 0) & (nc > ke)
            if bool(chk.any()):
                gap = (s_left - s_kept)[chk]
                worst_sel = max(worst_sel, float(gap.max()))
                assert float(gap.max()) <= 1e-6, (h, float(gap.max()))
            # ---- attention: routed cells (branch L) and window (branch S), fp32
            q32 = qd[0, h, r0:r1].float()
            okc = used & (sel >= 0)
            keys = (sel.clamp(min=0)[:, :, None] * b + torch.arange(b, device=dv_)[None, None, :]).reshape(r1 - r0, -1)
            kk, vv = k_h[keys], v_h[keys]                                     # [R, K b, d]
            z = torch.bmm(kk, q32[:, :, None]).squeeze(-1) / math.sqrt(d)
            z = z.masked_fill(~okc.repeat_interleave(b, dim=1), float("-inf"))
            has = okc.any(dim=1)
            p = torch.softmax(z.masked_fill(~has[:, None], 0.0), dim=-1) * has[:, None]
            o_l = torch.bmm(p[:, None, :], vv).squeeze(1)
            j0 = max(0, r0 - w + 1)
            jj = torch.arange(j0, r1, device=dv_)
            zs = q32 @ k_h[j0:r1].T / math.sqrt(d)
            band = (jj[None, :] <= ir[:, None]) & (jj[None, :] > ir[:, None] - w)
            ps = torch.softmax(zs.masked_fill(~band, float("-inf")), dim=-1)
            o_s = ps @ v_h[j0:r1]
            ref = alpha[h] * o_l + (1.0 - alpha[h]) * o_s
            e = _rel(o[0, h, r0:r1].float(), ref)
            worst_o = max(worst_o, e)
            assert e <= TOL_BF16, (h, r0, e)
    _say(f"  {L} rows x {H} heads: largest kept-vs-left score excess {worst_sel:.2e}, o rel err {worst_o:.2e}")


def test_train_every_slice():
    cfg = config("train")
    _say("[every row] train: forward and backward of every (batch, kv head) slice")
    x = make_inputs(cfg)
    B, Hq, Hkv, d, b, K = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["b"], cfg["K"]
    G = Hq // Hkv
    L = x["L"]
    nblk = L // b
    kw = dict(Hkv=Hkv, b=b, K=K, q_pos0=0, gate=True, share_group=True)
    kb_o, mx_o, ce_o = oracle.block_summaries(x["k"], b, nblocks=nblk)
    ora = oracle.score_select(x["q"], kb_o, mx_o, ce_o, **kw)
    qd, kd, vd, dod = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["dout"])
    idx = dev(ora["idx"])
    lg = dev(ora["logg"].astype(np.float32))
    akw = dict(b=b, K=K, q_pos0=0, share_group=True)
    o, lse = ops.sparse_attn_fwd(qd, kd, vd, idx, lg, **akw)
    dq, dk, dv, dg = ops.sparse_attn_bwd(qd, kd, vd, idx, lg, o, dod, lse, **akw)
    torch.cuda.synchronize()

    dv_ = qd.device
    i = torch.arange(L, device=dv_)
    jb = i // b
    cur = (jb[None, :] == jb[:, None]) & (i[None, :] <= i[:, None])       # the row's current block, causal
    worst = {}
    for bi in range(B):
        for kh in range(Hkv):
            hq = slice(kh * G, kh * G + G)
            sel = idx[bi, kh].long()
            ok = (sel >= 0) & (sel < jb[:, None])
            q = qd[bi, hq].float().requires_grad_()
            k = kd[bi, kh].float().requires_grad_()
            v = vd[bi, kh].float().requires_grad_()
            lgt = lg[bi, kh].clone().requires_grad_()
            # unused slots land on a dummy column past the blocks
            slot_col = torch.where(ok, sel, nblk)
            bias_blk = torch.zeros((L, nblk + 1), device=dv_).scatter(1, slot_col, lgt * ok)[:, :nblk]
            allow_blk = torch.zeros((L, nblk + 1), dtype=torch.bool, device=dv_).scatter(1, slot_col, ok)[:, :nblk]
            allow = allow_blk[:, jb] | cur
            z = torch.matmul(q, k.T.contiguous()) / math.sqrt(d) + bias_blk[:, jb][None]
            z = z.masked_fill(~allow[None], float("-inf"))
            lse_ref = torch.logsumexp(z, dim=-1)
            out = torch.matmul(torch.softmax(z, dim=-1), v)
            (out * dod[bi, hq].float()).sum().backward()
            dg_ref = (lgt.grad * torch.exp(-lgt)).masked_fill(~ok, 0.0)
            errs = dict(o=_rel(o[bi, hq].float(), out.detach()),
                        lse=float((lse[bi, hq] - lse_ref.detach()).abs().max()),
                        dq=_rel(dq[bi, hq].float(), q.grad), dk=_rel(dk[bi, kh].float(), k.grad),
                        dv=_rel(dv[bi, kh].float(), v.grad), dg=_rel(dg[bi, kh].float(), dg_ref))
            for n_, e in errs.items():
                worst[n_] = max(worst.get(n_, 0.0), e)
            assert max(errs[n_] for n_ in ("o", "dq", "dk", "dv", "dg")) <= TOL_BF16, (bi, kh, errs)
            assert errs["lse"] <= 10 * TOL_BF16, (bi, kh, errs)
            del q, k, v, lgt, z, out, lse_ref, bias_blk, allow_blk, allow
    _say("  worst over 32 slices: " + ", ".join(f"{n_} {e:.2e}" for n_, e in worst.items()))
