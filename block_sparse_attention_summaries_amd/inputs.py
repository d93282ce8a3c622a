"""Seeded synthetic inputs shaped like the pages' workloads.

This module is the only code shared by the HIP path's tests/benchmark and the
CPU oracle.  It draws random numbers and rounds fp32 draws to bf16 (nearest
even) so both sides see identical bytes; it holds none of the method's
arithmetic (no summaries, scores, selection or attention).

Workloads (the pages give no datasets for these shapes; seeded N(0, 1) draws
stand in for them):
  tiny_decode     1 head, d=64, fp32, n=4096, b=64, K=8, one query, gate off
  decode_32k      32 q / 8 kv heads, d=128, bf16, n=32768, b=64, K=16, 1% outlier
                  keys scaled x8, softmax log gate on
  decode_512k     as decode_32k with n=524288, K=32 and a 128x128 fp32 selector
                  projection W ~ N(0, 1/128)
  prefill_cells   16 heads, d=64, bf16, n=16384, cells of 32, query blocks of 128,
                  K=4 cells, window 512, lambda_h, alpha_h ~ U(0,1), sigma_h = 512
  train           batch 4, n=8192, 32 q / 8 kv heads, d=128, bf16, b=64, K=16,
                  gate on, upstream gradient dO ~ N(0, 1)
Decode context: L = n + t tokens with the current block full by default
(t = b), the query at position L - 1.  kind="cell_decode" (a prefill_cells
geometry) gives one query after n + b tokens, as the FS-L / FS-B decode
steps take it.
"""
from __future__ import annotations

import copy

import numpy as np

CONFIGS = {
    "tiny_decode": dict(kind="decode", B=1, Hq=1, Hkv=1, d=64, dtype="f32", n=4096, b=64,
                        K=8, t=64, gate=False, share_group=True, outlier_p=0.0,
                        proj=False, seed=1),
    "decode_32k": dict(kind="decode", B=1, Hq=32, Hkv=8, d=128, dtype="bf16", n=32768, b=64,
                       K=16, t=64, gate=True, share_group=True, outlier_p=0.01,
                       outlier_scale=8.0, proj=False, seed=2),
    "decode_512k": dict(kind="decode", B=1, Hq=32, Hkv=8, d=128, dtype="bf16", n=524288, b=64,
                        K=32, t=64, gate=True, share_group=True, outlier_p=0.0,
                        proj=True, seed=3),
    "prefill_cells": dict(kind="prefill", B=1, Hq=16, Hkv=16, d=64, dtype="bf16", n=16384,
                          b=32, qblock=128, K=4, window=512, sigma=512.0, gate=False,
                          share_group=False, seed=4),
    "train": dict(kind="train", B=4, Hq=32, Hkv=8, d=128, dtype="bf16", n=8192, b=64, K=16,
                  gate=True, share_group=True, seed=5),
}


def config(name: str, **overrides) -> dict:
    """A copy of a named workload with some fields replaced (smaller sizes for
    parity cases)."""
    c = copy.deepcopy(CONFIGS[name])
    c.update(overrides)
    c["name"] = name
    return c


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16, nearest even, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, dtype, chunk_rows=1 << 22, scale_rows=None):
    """N(0,1) draws in fp32 (generated in chunks to bound host memory), rounded
    to bf16 when dtype == 'bf16'.  scale_rows (optional, same leading shape
    without the last axis) multiplies whole rows before rounding."""
    *lead, d = shape
    nrows = int(np.prod(lead)) if lead else 1
    out = np.empty((nrows, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    sr = None if scale_rows is None else scale_rows.reshape(nrows)
    for r0 in range(0, nrows, chunk_rows):
        r1 = min(nrows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0, d), dtype=np.float32)
        if sr is not None:
            x *= sr[r0:r1, None]
        out[r0:r1] = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return out.reshape(shape)


def make_inputs(cfg: dict) -> dict:
    """Seeded inputs for a workload dict (see CONFIGS).  Arrays are numpy:
    fp32, or uint16 bf16 bit patterns when cfg['dtype'] == 'bf16'."""
    rng = np.random.Generator(np.random.PCG64(cfg["seed"]))
    B, Hq, Hkv, d, dt = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["dtype"]
    out = {}
    if cfg["kind"] == "decode":
        L = cfg["n"] + cfg.get("t", cfg["b"])
        nq = 1
        q_pos0 = L - 1
    elif cfg["kind"] == "cell_decode":           # one query after n + b tokens (cell-routing decode)
        L = cfg["n"] + cfg["b"]
        nq = 1
        q_pos0 = L - 1
    else:
        L = cfg["n"]
        nq = L
        q_pos0 = 0
    out["L"], out["nq"], out["q_pos0"] = L, nq, q_pos0
    out["q"] = _normal(rng, (B, Hq, nq, d), dt)
    scale = None
    if cfg.get("outlier_p", 0.0) > 0.0:
        mask = rng.random((B, Hkv, L), dtype=np.float32) < cfg["outlier_p"]
        scale = np.where(mask, np.float32(cfg["outlier_scale"]), np.float32(1.0)).astype(np.float32)
    out["k"] = _normal(rng, (B, Hkv, L, d), dt, scale_rows=scale)
    out["v"] = _normal(rng, (B, Hkv, L, d), dt)
    if cfg.get("proj"):
        out["proj_w"] = (rng.standard_normal((d, d), dtype=np.float32)
                         * np.float32(1.0 / np.sqrt(d))).astype(np.float32)
    if cfg["kind"] in ("prefill", "cell_decode"):
        out["erf_lambda"] = rng.random((Hq,), dtype=np.float32)
        out["erf_sigma"] = np.full((Hq,), cfg["sigma"], dtype=np.float32)
        out["alpha"] = rng.random((Hq,), dtype=np.float32)
    if cfg["kind"] == "train":
        out["dout"] = _normal(rng, (B, Hq, nq, d), dt)
    return out


def decode_queries(cfg: dict, count: int, seed_offset: int = 1000) -> np.ndarray:
    """`count` further independent query vectors [count, B, Hq, 1, d] for
    benchmarks that rotate queries between decode steps."""
    rng = np.random.Generator(np.random.PCG64(cfg["seed"] + seed_offset))
    return _normal(rng, (count, cfg["B"], cfg["Hq"], 1, cfg["d"]), cfg["dtype"])
