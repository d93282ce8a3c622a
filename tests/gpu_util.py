"""Helpers for the GPU parity tests: move the seeded numpy inputs to the
device, compare results with the oracle, and the index-match rule with the
K-boundary gap exemption."""
from __future__ import annotations

import numpy as np
import torch

from block_sparse_attention_summaries_amd.inputs import bf16_bits_to_f32

GAP_EXEMPT = 1e-6


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy (fp32 / bf16 bits as uint16 / int32) -> device tensor, same bytes."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy with the same bytes (bf16 -> uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def rel_err(x: np.ndarray, y: np.ndarray, lead: int = 2) -> float:
    """max over (batch, head) slices of ||x - y||_inf / max(||y||_inf, 1e-30)."""
    x = as_f64(x) if x.dtype != np.float64 else x
    y = as_f64(y) if y.dtype != np.float64 else y
    xs = x.reshape(int(np.prod(x.shape[:lead])), -1)
    ys = y.reshape(int(np.prod(y.shape[:lead])), -1)
    num = np.abs(xs - ys).max(axis=1)
    den = np.maximum(np.abs(ys).max(axis=1), 1e-30)
    return float((num / den).max())


def check_indices(gpu_idx, ora, score_fn=None):
    """Selected indices must equal the oracle's, except in rows whose oracle
    K-boundary gap is below 1e-6; there the GPU set must still be a valid
    top-K within 1e-6 of the oracle's scores (checked with score_fn(pos) ->
    (b, h, r) score vector when given).  Returns the number of exempted rows."""
    oi = ora["idx"]
    gap = ora["gap"]
    assert gpu_idx.shape == oi.shape, (gpu_idx.shape, oi.shape)
    diff = np.any(gpu_idx != oi, axis=-1)
    exempt = gap < GAP_EXEMPT
    bad = diff & ~exempt
    if bad.any():
        where = np.argwhere(bad)[:5]
        msg = [f"{tuple(w)}: gpu {gpu_idx[tuple(w)]} oracle {oi[tuple(w)]} gap {gap[tuple(w)]}" for w in where]
        raise AssertionError(f"{int(bad.sum())} rows select different blocks:\n" + "\n".join(msg))
    n_ex = int((diff & exempt).sum())
    if score_fn is not None:
        for w in np.argwhere(diff & exempt):
            s = score_fn(tuple(w))
            ke = int(ora["k_eff"][tuple(w)])
            o_sel = [c for c in oi[tuple(w)] if c >= 0]
            g_sel = [c for c in gpu_idx[tuple(w)] if c >= 0]
            assert len(g_sel) == ke == len(o_sel)
            kth = min(s[c] for c in o_sel)
            assert all(s[c] >= kth - GAP_EXEMPT for c in g_sel)
    return n_ex
