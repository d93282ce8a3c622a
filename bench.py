"""Benchmark: decode attention step at 512K context on one MI355X, plus prefill
tokens/s (cell routing, n = 16384), the FS-L fixed-state and FS-B forest
decode steps at 512K (fsl_decode_us_per_step, fsb_decode_us_per_step) and
training tokens/s.

One decode step = the hot path for one query token of one layer:
  score + softmax log gate + top-K select over all C = 8192 block summaries,
  then exact attention over the current block + the K = 32 selected blocks for
  all 32 query heads, in one sparse_decode_step call (the same outputs as
  sparse_score_select then sparse_attn_fwd; its top-K merge runs inside the
  attention workgroups), plus, on every b-th step, the summary of the block
  that closes (sparse_block_summaries).  The two-call sequence is timed the
  same way for comparison (unfused_us_per_step), and so is the step over the
  same caches scattered into page pools (paged_us_per_step) and the step whose
  scorer reads fp8 (E4M3) summaries with per-block scales (fp8_summaries; on
  closing steps the new block is also quantized).  The 32K decode workload
runs as configured as well (decode_32k: K = 16, 1 % outlier keys, no
projection).
Steps rotate over 16 layers' KV caches (2.15 GB each) and 64 query vectors so
that every step reads its summaries and selected K/V cold from HBM, as a
multi-layer decoder would.  Inputs are resident in HBM before timing starts.
The steps are captured once in a HIP graph and replayed (the pages measured
decode with graph replay); that replay is the timed region.  Per-kernel
durations for the roofline come from the same steps run once more eagerly,
each kernel launched with start/stop events attached to its dispatch
(spa_profile_next_call), i.e. the kernel's own begin/end timestamps.

Prints one JSON line.  Only N = 1 GPU is supported.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_sparse_attention_summaries_amd import ops  # noqa: E402
from block_sparse_attention_summaries_amd.inputs import config, decode_queries, make_inputs  # noqa: E402

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0         # dense bf16 MFMA, vendor figure
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_512k_hbm_counters.json")
CSRC = os.path.join(ROOT, "block_sparse_attention_summaries_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# sources the decode kernels are built from (the HBM counters are tied to them)
DECODE_SOURCES = ("attn.hip", "decode_merge.h", "decode_step.hip", "decode_tile.h", "select.hip", "spa_device.h",
                  "spa_launch.h")


def source_hash():
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime already loaded by torch."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self):
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.made.append(ev)
        return ev

    def elapsed(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy_all(self):
        for ev in self.made:
            self.hip.hipEventDestroy(ev)
        self.made = []


# the kernels of one decode step, in launch order: the one-call step (bf16 or
# fp8 summaries), and the select + attend pair
STEP_KERNELS = [("score", "decode_score_kernel"), ("step", "decode_step_kernel")]
TWO_CALL_KERNELS = [("chunk", "decode_chunk_kernel"), ("merge", "decode_merge_kernel"),
                    ("partial", "decode_attn_partial_kernel"), ("combine", "decode_combine_kernel")]


# ---------------------------------------------------------------- decode workload
class DecodeWorkload:
    """Layers of a 512K-token KV cache with their block summaries, rotating
    queries, and preallocated outputs/workspaces for graph capture."""

    def __init__(self, cfg, n_layers, n_queries, host_layer0):
        self.cfg = cfg
        B, Hq, Hkv, d, b = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["b"]
        x = host_layer0
        self.L, self.pos = x["L"], x["q_pos0"]
        self.ccap = self.L // b
        self.C = self.pos // b                      # historical candidates of the query
        self.K, self.b = cfg["K"], b
        g = torch.Generator(device="cuda")
        proj = x.get("proj_w") is not None
        self.k, self.v = [dev(x["k"])], [dev(x["v"])]
        self.w = [dev(x["proj_w"]) if proj else None]
        for layer in range(1, n_layers):
            g.manual_seed(cfg["seed"] * 1000 + layer)
            kf = torch.randn((B, Hkv, self.L, d), generator=g, device="cuda")
            if cfg.get("outlier_p", 0.0) > 0.0:
                # the same outlier rule as layer 0: whole keys scaled before rounding
                hit = torch.rand((B, Hkv, self.L, 1), generator=g, device="cuda") < cfg["outlier_p"]
                kf = torch.where(hit, kf * cfg["outlier_scale"], kf)
            self.k.append(kf.to(torch.bfloat16))
            self.v.append(torch.randn((B, Hkv, self.L, d), generator=g, device="cuda").to(torch.bfloat16))
            self.w.append(torch.randn((d, d), generator=g, device="cuda") / float(np.sqrt(d)) if proj else None)
        self.q = dev(decode_queries(cfg, n_queries))  # [nQ, B, Hq, 1, d]
        self.kbar, self.mx, self.ce = [], [], []
        for layer in range(n_layers):
            kb, mx, ce = ops.sparse_block_summaries(self.k[layer], b, num_blocks=self.ccap - 1,
                                                    ccap=self.ccap)
            self.kbar.append(kb)
            self.mx.append(mx)
            self.ce.append(ce)
        self.idx = torch.empty((B, Hkv, 1, self.K), dtype=torch.int32, device="cuda")
        self.logg = torch.empty((B, Hkv, 1, self.K), dtype=torch.float32, device="cuda")
        self.keff = torch.empty((B, Hkv, 1), dtype=torch.int32, device="cuda")
        self.o = torch.empty((B, Hq, 1, d), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
        self.ws_sel = ops.Workspace()
        self.ws_att = ops.Workspace()
        self.ws_dec = ops.Workspace()
        torch.cuda.synchronize()

    def close_block(self, layer):
        """Summary of the block that just closed (the current block, now full)."""
        ops.sparse_block_summaries(self.k[layer], self.b, first_block=self.ccap - 1, num_blocks=1,
                                   kbar=self.kbar[layer], max_norm=self.mx[layer], centre=self.ce[layer])

    def select(self, layer, qi):
        ops.sparse_score_select(self.q[qi], self.kbar[layer], self.mx[layer], self.ce[layer],
                                Hkv=self.cfg["Hkv"], b=self.b, K=self.K, q_pos0=self.pos, gate=True,
                                proj_w=self.w[layer], idx=self.idx, logg=self.logg, k_eff=self.keff,
                                workspace=self.ws_sel)

    def attend(self, layer, qi):
        ops.sparse_attn_fwd(self.q[qi], self.k[layer], self.v[layer], self.idx, self.logg, b=self.b,
                            K=self.K, q_pos0=self.pos, o=self.o, lse=self.lse, workspace=self.ws_att)

    def make_paged(self):
        """The same caches scattered into page pools [pages, Hkv, b, d] in a
        seeded random page order, with the block table (benchmark setup)."""
        B, Hkv, d, b = self.cfg["B"], self.cfg["Hkv"], self.cfg["d"], self.b
        nblk = self.L // b
        g = torch.Generator(device="cuda")
        g.manual_seed(self.cfg["seed"] * 7919)
        perm = torch.randperm(B * nblk, generator=g, device="cuda")
        self.table = perm.to(torch.int32).view(B, nblk).contiguous()
        self.kp, self.vp = [], []
        for layer in range(len(self.k)):
            for src, dst in ((self.k[layer], self.kp), (self.v[layer], self.vp)):
                pool = torch.empty((B * nblk, Hkv, b, d), dtype=src.dtype, device="cuda")
                pool[perm] = src.view(B, Hkv, nblk, b, d).permute(0, 2, 1, 3, 4).reshape(B * nblk, Hkv, b, d)
                dst.append(pool)
        self.ws_pag = ops.Workspace()
        torch.cuda.synchronize()

    def make_fp8(self):
        """fp8 (E4M3) copies of every layer's summaries with per-block scales."""
        self.codes8, self.scale8 = [], []
        for layer in range(len(self.kbar)):
            c, sc = ops.sparse_quantize_summaries_fp8(self.kbar[layer])
            self.codes8.append(c)
            self.scale8.append(sc)
        self.ws_f8 = ops.Workspace()
        torch.cuda.synchronize()

    def close_block_fp8(self, layer):
        self.close_block(layer)
        ops.sparse_quantize_summaries_fp8(self.kbar[layer], first_block=self.ccap - 1, num_blocks=1,
                                          codes=self.codes8[layer], scales=self.scale8[layer])

    def decode_fp8(self, layer, qi):
        ops.sparse_decode_step(self.q[qi], self.codes8[layer], self.mx[layer], self.ce[layer], self.k[layer],
                               self.v[layer], Hkv=self.cfg["Hkv"], b=self.b, K=self.K, q_pos0=self.pos, gate=True,
                               proj_w=self.w[layer], idx=self.idx, logg=self.logg, k_eff=self.keff, o=self.o,
                               lse=self.lse, workspace=self.ws_f8, kbar_scale=self.scale8[layer])

    def close_block_paged(self, layer):
        ops.sparse_block_summaries_paged(self.kp[layer], self.table, self.L, self.b, first_block=self.ccap - 1,
                                         num_blocks=1, kbar=self.kbar[layer], max_norm=self.mx[layer],
                                         centre=self.ce[layer])

    def decode_paged(self, layer, qi):
        ops.sparse_decode_step_paged(self.q[qi], self.kbar[layer], self.mx[layer], self.ce[layer], self.kp[layer],
                                     self.vp[layer], self.table, self.L, Hkv=self.cfg["Hkv"], b=self.b, K=self.K,
                                     q_pos0=self.pos, gate=True, proj_w=self.w[layer], idx=self.idx,
                                     logg=self.logg, k_eff=self.keff, o=self.o, lse=self.lse,
                                     workspace=self.ws_pag)

    def decode(self, layer, qi, pos=None):
        ops.sparse_decode_step(self.q[qi], self.kbar[layer], self.mx[layer], self.ce[layer], self.k[layer],
                               self.v[layer], Hkv=self.cfg["Hkv"], b=self.b, K=self.K,
                               q_pos0=self.pos if pos is None else pos, gate=True, proj_w=self.w[layer],
                               idx=self.idx, logg=self.logg, k_eff=self.keff, o=self.o, lse=self.lse,
                               workspace=self.ws_dec)

    def two_calls_at(self, layer, qi, pos):
        """The select + attend pair at query position pos."""
        ops.sparse_score_select(self.q[qi], self.kbar[layer], self.mx[layer], self.ce[layer],
                                Hkv=self.cfg["Hkv"], b=self.b, K=self.K, q_pos0=pos, gate=True,
                                proj_w=self.w[layer], idx=self.idx, logg=self.logg, k_eff=self.keff,
                                workspace=self.ws_sel)
        ops.sparse_attn_fwd(self.q[qi], self.k[layer], self.v[layer], self.idx, self.logg, b=self.b,
                            K=self.K, q_pos0=pos, o=self.o, lse=self.lse, workspace=self.ws_att)

    def selected_kv_bytes(self):
        c = self.cfg
        t = self.pos - (self.pos // self.b) * self.b + 1    # tokens of the current block
        keff = min(self.K, self.C)
        kv = c["B"] * c["Hkv"] * (keff * self.b + t) * c["d"] * 2 * 2   # K and V, bf16
        qo = c["B"] * c["Hq"] * c["d"] * 2 * 2 + c["B"] * c["Hkv"] * self.K * 8
        return kv + qo

    def scoring_bytes(self, fp8=False):
        c = self.cfg
        row = c["d"] + 4 if fp8 else c["d"] * 2          # codes + scale, or the bf16 summary
        w = c["d"] * c["d"] * 4 if self.w[0] is not None else 0
        return c["B"] * c["Hkv"] * self.C * row + w + c["B"] * c["Hq"] * c["d"] * 2


def run_decode(args):
    cfg = config("decode_512k")
    t0 = time.time()
    x = make_inputs(cfg)
    log(f"[bench] host inputs for {cfg['name']} in {time.time() - t0:.1f}s")
    wl = DecodeWorkload(cfg, args.layers, args.queries, x)
    log(f"[bench] {args.layers} layers of L={wl.L} resident; C={wl.C} candidates, K={wl.K}")

    # summaries of a whole 512K cache (prefill-time work), timed eagerly
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for layer in range(args.layers):
        ops.sparse_block_summaries(wl.k[layer], wl.b, num_blocks=wl.ccap, ccap=wl.ccap,
                                   kbar=wl.kbar[layer], max_norm=wl.mx[layer], centre=wl.ce[layer])
    e1.record()
    torch.cuda.synchronize()
    summ_ms = e0.elapsed_time(e1) / args.layers
    summ_bytes = cfg["B"] * cfg["Hkv"] * (wl.ccap * wl.b * cfg["d"] * 2 + wl.ccap * (cfg["d"] * 2 + 4))

    # warm-up (eager), also builds the workspaces
    for s in range(args.warmup):
        wl.decode(s % args.layers, s % args.queries)
        wl.select(s % args.layers, s % args.queries)
        wl.attend(s % args.layers, s % args.queries)
    torch.cuda.synchronize()

    steps = args.steps
    stream = torch.cuda.Stream()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed_graph(one_step, close=wl.close_block):
        """Capture `steps` decode steps in one graph, replay once untimed
        (upload), then time one replay of the whole sequence."""
        graph = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            graph.capture_begin()
            for s in range(steps):
                layer, qi = s % args.layers, s % args.queries
                if s % wl.b == wl.b - 1:
                    close(layer)
                one_step(layer, qi)
            graph.capture_end()
        torch.cuda.current_stream().wait_stream(stream)
        graph.replay()
        torch.cuda.synchronize()
        g0.record()
        graph.replay()
        g1.record()
        torch.cuda.synchronize()
        return g0.elapsed_time(g1)

    def per_kernel(one_step, close, names):
        """Per-kernel durations over the same steps (eager), from each kernel's
        own dispatch timestamps (start/stop events attached to its launch);
        `names` lists (short name, kernel) in launch order."""
        hip = HipEvents()
        n = len(names)
        EvArr = ctypes.c_void_p * (2 * n)
        evs = [EvArr(*[hip.create() for _ in range(2 * n)]) for _ in range(steps)]
        lib = ops.lib()
        for s in range(steps):
            layer, qi = s % args.layers, s % args.queries
            if s % wl.b == wl.b - 1:
                close(layer)
            lib.spa_profile_next_call(evs[s], n)
            one_step(layer, qi)
        torch.cuda.synchronize()
        out = {short: np.array([hip.elapsed(evs[s][2 * i], evs[s][2 * i + 1]) for s in range(steps)])
               for i, (short, _) in enumerate(names)}
        hip.destroy_all()
        return out

    def step_latencies(pairs, reps):
        """Device time of each of `reps` one-step graph replays, one graph per
        (layer, query) pair, taken in turn.  A spin kernel first lets the host
        queue every replay before the device reaches it, so each pair of
        events brackets device work only."""
        graphs = []
        for layer, qi in pairs:
            g = torch.cuda.CUDAGraph()
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                g.capture_begin()
                wl.decode(layer, qi)
                g.capture_end()
            torch.cuda.current_stream().wait_stream(stream)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda._sleep(20_000_000)
        ev[0].record()
        for r in range(reps):
            graphs[r % len(graphs)].replay()
            ev[r + 1].record()
        torch.cuda.synchronize()
        t = np.array([ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]) * 1e3
        del graphs
        return dict(median_us=round(float(np.median(t)), 3), p99_us=round(float(np.percentile(t, 99)), 3),
                    mean_us=round(float(t.mean()), 3), replays=reps, graphs=len(pairs))

    # timed region: the one-call decode step
    total_ms = timed_graph(wl.decode)

    def two_calls(layer, qi):
        wl.select(layer, qi)
        wl.attend(layer, qi)
    unfused_ms = paged_ms = fp8_ms = None
    fp8_k_ms = None
    if not args.skip_variants:
        unfused_ms = timed_graph(two_calls)
        # the same steps with fp8 summaries (the scorer reads codes + scales)
        wl.make_fp8()
        for s in range(4):
            wl.decode_fp8(s % args.layers, s % args.queries)
        fp8_ms = timed_graph(wl.decode_fp8, close=wl.close_block_fp8)
        fp8_k_ms = per_kernel(wl.decode_fp8, wl.close_block_fp8, STEP_KERNELS)
        # the same steps over a paged cache (random page order)
        wl.make_paged()
        for s in range(4):
            wl.decode_paged(s % args.layers, s % args.queries)
        paged_ms = timed_graph(wl.decode_paged, close=wl.close_block_paged)

    k_ms = per_kernel(wl.decode, wl.close_block, STEP_KERNELS)
    # per-step latency distribution: cold (16 layers' caches in turn) and warm
    # (one layer, one query)
    dist = {"cold": step_latencies([(i % args.layers, i % args.queries) for i in range(16)], args.replays),
            "warm": step_latencies([(0, 0)], args.replays)}
    sweep = run_decode_sweep(wl, args, stream) if not args.skip_variants else None

    # the summary of a closing block (once per b steps): timed alone, so that
    # its share per step is known whatever --steps is
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(32):
        wl.close_block(s % args.layers)
    e1.record()
    torch.cuda.synchronize()
    close_us = e0.elapsed_time(e1) * 1e3 / 32

    # a hot-cache variant (one layer, one query) for context
    hot = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        hot.capture_begin()
        for s in range(64):
            wl.decode(0, 0)
        hot.capture_end()
    torch.cuda.current_stream().wait_stream(stream)
    hot.replay()
    torch.cuda.synchronize()
    g0.record()
    hot.replay()
    g1.record()
    torch.cuda.synchronize()
    hot_us = g0.elapsed_time(g1) * 1e3 / 64

    floor_us = latency_floor_us(stream, steps, len(k_ms))
    return dict(wl=wl, cfg=cfg, x=x, total_ms=total_ms, unfused_ms=unfused_ms, paged_ms=paged_ms, k_ms=k_ms,
                fp8_ms=fp8_ms, fp8_k_ms=fp8_k_ms, dist=dist, sweep=sweep, close_us=close_us,
                summ_ms=summ_ms, summ_bytes=summ_bytes, hot_us=hot_us, floor_us=floor_us)


def run_decode_32k(args, steps=256):
    """The 32K decode workload as configured (32 q / 8 kv heads, K = 16, 1 %
    outlier keys x8, log gate on, no projection) over 16 layers and rotating
    queries: one-call steps replayed as one graph, µs per step, and the
    selected K/V rate over the step kernel's event-timed duration."""
    cfg = config("decode_32k")
    wl = DecodeWorkload(cfg, args.layers, args.queries, make_inputs(cfg))
    for s in range(8):
        wl.decode(s % args.layers, s % args.queries)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        g.capture_begin()
        for s in range(steps):
            wl.decode(s % args.layers, s % args.queries)
        g.capture_end()
    torch.cuda.current_stream().wait_stream(stream)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    del g
    hip = HipEvents()
    lib = ops.lib()
    nk = len(STEP_KERNELS)
    evs = [(ctypes.c_void_p * (2 * nk))(*[hip.create() for _ in range(2 * nk)]) for _ in range(64)]
    for s in range(64):
        lib.spa_profile_next_call(evs[s], nk)
        wl.decode(s % args.layers, s % args.queries)
    torch.cuda.synchronize()
    kern = {n: round(float(np.mean([hip.elapsed(ev[2 * i], ev[2 * i + 1]) for ev in evs])) * 1e3, 3)
            for i, (n, _) in enumerate(STEP_KERNELS)}
    hip.destroy_all()
    kv = wl.selected_kv_bytes()
    return dict(us_per_step=round(us, 3), context=wl.L, candidates=wl.C, K=wl.K, kernels_us=kern,
                selected_kv_bytes=kv, selected_kv_gbps=round(kv / (kern["step"] * 1e-6) / 1e9, 1))


def run_decode_sweep(wl, args, stream, contexts=(32768, 65536, 131072, 262144, 524288), steps=64):
    """The decode step at shorter contexts over the same caches (the query at
    the same offset in its block): µs per step of the one-call step (graph
    replay of `steps` steps over the layers in turn) and the per-kernel split
    of the select + attend pair: selection (chunk scores + merge) and
    attention (partials + combine)."""
    off = wl.pos % wl.b
    hip = HipEvents()
    out = []
    for ctx in contexts:
        pos = ctx + off
        for s in range(4):
            wl.decode(s % args.layers, 0, pos)
            wl.two_calls_at(s % args.layers, 0, pos)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            g.capture_begin()
            for s in range(steps):
                wl.decode(s % args.layers, s % args.queries, pos)
            g.capture_end()
        torch.cuda.current_stream().wait_stream(stream)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        step_us = e0.elapsed_time(e1) * 1e3 / steps
        del g
        k1 = {n: [] for n, _ in STEP_KERNELS}
        k2 = {n: [] for n, _ in TWO_CALL_KERNELS}
        lib = ops.lib()
        for s in range(steps):
            layer, qi = s % args.layers, s % args.queries
            ev1 = (ctypes.c_void_p * 4)(*[hip.create() for _ in range(4)])
            lib.spa_profile_next_call(ev1, 2)
            wl.decode(layer, qi, pos)
            ev_sel = (ctypes.c_void_p * 4)(*[hip.create() for _ in range(4)])
            ev_att = (ctypes.c_void_p * 4)(*[hip.create() for _ in range(4)])
            lib.spa_profile_next_call(ev_sel, 2)
            ops.sparse_score_select(wl.q[qi], wl.kbar[layer], wl.mx[layer], wl.ce[layer], Hkv=wl.cfg["Hkv"],
                                    b=wl.b, K=wl.K, q_pos0=pos, gate=True, proj_w=wl.w[layer], idx=wl.idx,
                                    logg=wl.logg, k_eff=wl.keff, workspace=wl.ws_sel)
            lib.spa_profile_next_call(ev_att, 2)
            ops.sparse_attn_fwd(wl.q[qi], wl.k[layer], wl.v[layer], wl.idx, wl.logg, b=wl.b, K=wl.K, q_pos0=pos,
                                o=wl.o, lse=wl.lse, workspace=wl.ws_att)
            k1["score"].append((ev1, 0))
            k1["step"].append((ev1, 1))
            k2["chunk"].append((ev_sel, 0))
            k2["merge"].append((ev_sel, 1))
            k2["partial"].append((ev_att, 0))
            k2["combine"].append((ev_att, 1))
        torch.cuda.synchronize()

        def mean_us(lst):
            return float(np.mean([hip.elapsed(ev[2 * i], ev[2 * i + 1]) for ev, i in lst])) * 1e3
        ks = {n: mean_us(v) for n, v in k1.items()}
        kt = {n: mean_us(v) for n, v in k2.items()}
        out.append(dict(context=ctx, candidates=pos // wl.b, step_us=round(step_us, 3),
                        score_kernel_us=round(ks["score"], 3), step_kernel_us=round(ks["step"], 3),
                        two_call_selection_us=round(kt["chunk"] + kt["merge"], 3),
                        two_call_attention_us=round(kt["partial"] + kt["combine"], 3)))
        log(f"[bench] sweep {out[-1]}")
    hip.destroy_all()
    return out


def load_latency_ns(nbytes, steps, seed=11):
    """Round-trip latency of one dependent load (ns) with the chased list
    spread over nbytes: a random cyclic order of one entry per 256 bytes.  A
    list of at most 2^18 entries is walked once in full first (resident in L2,
    or in the MALL once it outgrows L2); a longer one is timed cold, after a
    768 MiB write that evicts it from the MALL."""
    n = nbytes // 4
    stride = 64
    m = n // stride
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    perm = torch.randperm(m, generator=g, device="cuda")
    nxt = torch.zeros(n, dtype=torch.int32, device="cuda")
    nxt[perm * stride] = (torch.roll(perm, -1) * stride).to(torch.int32)
    start = int(perm[0].item()) * stride
    del perm
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    if m <= 1 << 18:
        ops.sparse_probe_load_chase(nxt, m, start=start, out=out)
    else:
        flush = torch.empty(768 << 20, dtype=torch.uint8, device="cuda")
        flush.fill_(1)
        del flush
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    ops.sparse_probe_load_chase(nxt, steps, start=start, out=out)
    e1.record()
    torch.cuda.synchronize()
    ns = e0.elapsed_time(e1) * 1e6 / steps
    del nxt
    torch.cuda.empty_cache()
    return ns


def latency_floor_us(stream, steps, n_kernels):
    """Graph replay of `steps` x n_kernels dependent 256-workgroup kernels that
    do next to nothing (the library's workspace fill of 1 MiB): the launch and
    dependency cost a decode step of that many kernels pays before moving any
    bytes."""
    buf = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    lib = ops.lib()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        g.capture_begin()
        for _ in range(n_kernels * steps):
            lib.sparse_workspace_init(ctypes.c_void_p(buf.data_ptr()), buf.numel(),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        g.capture_end()
    torch.cuda.current_stream().wait_stream(stream)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


# ---------------------------------------------------------------- prefill / training
def run_prefill(reps):
    cfg = config("prefill_cells")
    x = make_inputs(cfg)
    b, qb, K = cfg["b"], cfg["qblock"], cfg["K"]
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    lam, sig, alpha = dev(x["erf_lambda"]), dev(x["erf_sigma"]), dev(x["alpha"])
    ws1, ws2 = ops.Workspace(), ops.Workspace()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    times = []
    kb, mx, ce = ops.sparse_block_summaries(k, b)      # output buffers, rewritten in full by every call

    def once():
        # a spin kernel ahead of the timed calls lets the host queue them all,
        # so the events time the GPU work, not Python's launch overhead
        torch.cuda._sleep(1_000_000)
        ev[0].record()
        ops.sparse_block_summaries(k, b, kbar=kb, max_norm=mx, centre=ce)
        ev[1].record()
        idx, _, _ = ops.sparse_score_select(q, kb, mx, ce, Hkv=cfg["Hkv"], b=b, K=K, q_pos0=0, gate=False,
                                            prefix_mode=1, qblock=qb, share_group=False,
                                            erf_lambda=lam, erf_sigma=sig, workspace=ws1)
        ev[2].record()
        ops.sparse_attn_fwd(q, k, v, idx, None, b=b, K=K, q_pos0=0, share_group=False, local=1,
                            window=cfg["window"], alpha=alpha, prefix_mode=1, qblock=qb, workspace=ws2)
        ev[3].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(3)]

    once()
    for _ in range(reps):
        times.append(once())
    t = np.median(np.array(times), axis=0)
    n = x["L"]
    # algorithmic work: 2d flops per causal (query, cell) score; 4d per (q, k) pair
    scores = sum((qb * (i // qb)) // b for i in range(n)) * cfg["Hq"]      # causal (query, cell) pairs
    # attention: 4d flops per (query, key) pair of branch L (K cells of b keys
    # once there are that many candidates) and of the window
    routed = sum(min(cfg["K"], (qb * (i // qb)) // b) * b for i in range(n))
    window = sum(min(cfg["window"], i + 1) for i in range(n))
    attn_gflop = 4 * cfg["d"] * (routed + window) * cfg["Hq"] / 1e9
    return dict(ms=dict(summaries=t[0], score_select=t[1], attention=t[2]),
                tokens_per_s=n / (t.sum() * 1e-3), score_gflop=2 * cfg["d"] * scores / 1e9, attn_gflop=attn_gflop)


def run_train(reps):
    cfg = config("train")
    x = make_inputs(cfg)
    b, K = cfg["b"], cfg["K"]
    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["dout"])
    ws = [ops.Workspace() for _ in range(4)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    times = []

    kb, mx, ce = ops.sparse_block_summaries(k, b)      # output buffers, rewritten in full by every call

    def once():
        torch.cuda._sleep(1_000_000)                   # the host queues the calls ahead of the GPU
        ev[0].record()
        ops.sparse_block_summaries(k, b, kbar=kb, max_norm=mx, centre=ce)
        idx, logg, _ = ops.sparse_score_select(q, kb, mx, ce, Hkv=cfg["Hkv"], b=b, K=K, q_pos0=0,
                                               gate=True, workspace=ws[0])
        ev[1].record()
        o, lse = ops.sparse_attn_fwd(q, k, v, idx, logg, b=b, K=K, q_pos0=0, workspace=ws[1])
        ev[2].record()
        _, dk, _, dg = ops.sparse_attn_bwd(q, k, v, idx, logg, o, do, lse, b=b, K=K, q_pos0=0,
                                          workspace=ws[2])
        ev[3].record()
        # selector side: dg through the gate into q and the summaries, and
        # through the block means into dk
        ops.sparse_select_bwd(q, kb, mx, ce, idx, logg, dg, dk=dk, Hkv=cfg["Hkv"], b=b, K=K, q_pos0=0,
                              gate=True, workspace=ws[3])
        ev[4].record()
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(4)]

    once()
    for _ in range(reps):
        times.append(once())
    t = np.median(np.array(times), axis=0)
    tokens = cfg["B"] * x["L"]
    # kept (query, key) pairs: the causal part of the current block plus the
    # K_eff = min(K, blocks before it) selected blocks; fwd 4d flops per pair,
    # bwd 10d algorithmic (S, dP, dV, dQ, dK once each), 14d as executed (the
    # dq and the dk/dv kernels each recompute S and dP)
    n = x["L"]
    pairs = sum(i % b + 1 + min(K, i // b) * b for i in range(n)) * cfg["B"] * cfg["Hq"]
    return dict(ms=dict(select=t[0], fwd=t[1], bwd=t[2], select_bwd=t[3]), tokens_per_s=tokens / (t.sum() * 1e-3),
                fwd_tflop=4 * cfg["d"] * pairs / 1e12, bwd_tflop=10 * cfg["d"] * pairs / 1e12,
                bwd_exec_tflop=14 * cfg["d"] * pairs / 1e12)


def run_sas_fwd_long(n=32768, reps=3):
    """SAS forward (selection, then attention) on one sequence of n tokens with
    the train workload's heads (32 query / 8 kv, d = 128, b = 64, K = 16,
    gate on); device-side seeded N(0, 1) bf16 inputs.  At this length a row
    tile's union of selections is ~15x the kept blocks, so the attention runs
    block-major (selected blocks as per-(row, slot) partials)."""
    cfg = config("train")
    Hq, Hkv, d, b, K = cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["b"], cfg["K"]
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg["seed"] * 7919 + n)
    q = torch.randn((1, Hq, n, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((1, Hkv, n, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((1, Hkv, n, d), generator=g, device="cuda").to(torch.bfloat16)
    kb, mx, ce = ops.sparse_block_summaries(k, b)
    idx, logg, _ = ops.sparse_score_select(q, kb, mx, ce, Hkv=Hkv, b=b, K=K, q_pos0=0, gate=True)
    ws = ops.Workspace()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps + 1):
        torch.cuda._sleep(1_000_000)
        e0.record()
        ops.sparse_attn_fwd(q, k, v, idx, logg, b=b, K=K, q_pos0=0, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts[1:]))
    pairs = sum(i % b + 1 + min(K, i // b) * b for i in range(n)) * Hq
    return dict(ms=ms, tflop=4 * d * pairs / 1e12)


def run_fsl_decode(steps, n_layers=4, n_queries=32):
    """FS-L decode at 512K tokens with the cell-routing head geometry (16
    heads, d = 64, 32-token cells, query blocks of 128, K = 4, window 512):
    per step the selection inside the kept set (W = 8 recent cells + P = 64 of
    largest max key norm) and the two-branch attention; when a cell closes,
    its summary and the new kept set.  Layers and queries rotate as in the
    main decode benchmark; graph replay is the timed region."""
    cfg = config("prefill_cells")
    B, H, d, b, qb, K, w = 1, cfg["Hq"], cfg["d"], cfg["b"], cfg["qblock"], cfg["K"], cfg["window"]
    W, P = 8, 64
    L = 524288 + b
    pos = L - 1
    ncand = (qb * (pos // qb)) // b
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg["seed"] * 104729)
    ks = [torch.randn((B, H, L, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(n_layers)]
    vs = [torch.randn((B, H, L, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(n_layers)]
    qs = torch.randn((n_queries, B, H, 1, d), generator=g, device="cuda").to(torch.bfloat16)
    lam = torch.rand((H,), generator=g, device="cuda")
    sig = torch.full((H,), cfg["sigma"], device="cuda")
    alpha = torch.rand((H,), generator=g, device="cuda")
    summ = [ops.sparse_block_summaries(k, b) for k in ks]
    kept = [ops.sparse_retain_cells(mx, ncand, W, P) for (_, mx, _) in summ]
    idx = torch.empty((B, H, 1, K), dtype=torch.int32, device="cuda")
    keff = torch.empty((B, H, 1), dtype=torch.int32, device="cuda")
    o = torch.empty((B, H, 1, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, 1), dtype=torch.float32, device="cuda")
    akw = dict(b=b, K=K, q_pos0=pos, share_group=False, local=1, window=w, prefix_mode=1, qblock=qb)

    def step(s):
        layer, qi = s % n_layers, s % n_queries
        kb, mx, ce = summ[layer]
        cells, count = kept[layer]
        if s % b == b - 1:          # a cell closes: its summary, then the kept set
            nblk = L // b
            ops.sparse_block_summaries(ks[layer], b, first_block=nblk - 1, num_blocks=1, kbar=kb, max_norm=mx,
                                       centre=ce)
            ops.sparse_retain_cells(mx, ncand, W, P, cells=cells, count=count)
        ops.sparse_score_select_subset(qs[qi], kb, mx, ce, cells, count, Hkv=H, b=b, K=K, q_pos0=pos, gate=False,
                                       prefix_mode=1, qblock=qb, share_group=False, erf_lambda=lam,
                                       erf_sigma=sig, idx=idx, k_eff=keff)
        ops.sparse_attn_fwd(qs[qi], ks[layer], vs[layer], idx, None, alpha=alpha, o=o, lse=lse, **akw)

    for s in range(8):
        step(s)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        graph.capture_begin()
        for s in range(steps):
            step(s)
        graph.capture_end()
    torch.cuda.current_stream().wait_stream(stream)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    # the kept-set update alone (once per closing cell)
    e0.record()
    for _ in range(16):
        ops.sparse_retain_cells(summ[0][1], ncand, W, P, cells=kept[0][0], count=kept[0][1])
    e1.record()
    torch.cuda.synchronize()
    retain_us = e0.elapsed_time(e1) * 1e3 / 16

    # FS-B on the same caches: forests over the prefix cells (once per query
    # block), then per step the beam search + re-rank and the same attention
    forests = [ops.sparse_forest_build(kb, mx, ce, ncand) for (kb, mx, ce) in summ]
    torch.cuda.synchronize()
    e0.record()
    for layer in range(n_layers):
        kb, mx, ce = summ[layer]
        ops.sparse_forest_build(kb, mx, ce, ncand, forest=forests[layer])
    e1.record()
    torch.cuda.synchronize()
    build_us = e0.elapsed_time(e1) * 1e3 / n_layers

    def fsb_step(s):
        layer, qi = s % n_layers, s % n_queries
        kb, mx, ce = summ[layer]
        ops.sparse_forest_select(qs[qi], kb, mx, ce, ks[layer], forests[layer], ncand, Hkv=H, b=b, K=K,
                                 q_pos0=pos, prefix_mode=1, qblock=qb, share_group=False, erf_lambda=lam,
                                 erf_sigma=sig, idx=idx, k_eff=keff)
        ops.sparse_attn_fwd(qs[qi], ks[layer], vs[layer], idx, None, alpha=alpha, o=o, lse=lse, **akw)

    for s in range(4):
        fsb_step(s)
    torch.cuda.synchronize()
    graph2 = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        graph2.capture_begin()
        for s in range(steps):
            fsb_step(s)
        graph2.capture_end()
    torch.cuda.current_stream().wait_stream(stream)
    graph2.replay()
    torch.cuda.synchronize()
    e0.record()
    graph2.replay()
    e1.record()
    torch.cuda.synchronize()
    fsb_us = e0.elapsed_time(e1) * 1e3 / steps
    del ks, vs
    return dict(us_per_step=us, retain_us=retain_us, cells=ncand, fsb_us=fsb_us, forest_build_us=build_us)


# ---------------------------------------------------------------- CPU oracle baseline
def run_cpu_baseline(res, seconds):
    """The fp64 oracle's decode step (score + gate + top-K + attention) on the
    host for layer 0 of the same workload, rotating the same queries."""
    import oracle
    cfg, x, wl = res["cfg"], res["x"], res["wl"]
    b, K, pos = cfg["b"], cfg["K"], x["q_pos0"]
    t0 = time.time()
    kb, mx, ce = oracle.block_summaries(x["k"], b, nblocks=wl.ccap)
    log(f"[bench] oracle summaries of layer 0 in {time.time() - t0:.1f}s")
    qs = decode_queries(cfg, 64)
    n = 0
    t0 = time.time()
    while time.time() - t0 < seconds:
        qn = np.ascontiguousarray(qs[n % 64])
        sel = oracle.score_select(qn, kb, mx, ce, Hkv=cfg["Hkv"], b=b, K=K, q_pos0=pos, gate=True,
                                  proj_w=x["proj_w"])
        oracle.attn_fwd(qn, x["k"], x["v"], sel["idx"], sel["logg"], b=b, K=K, q_pos0=pos)
        n += 1
    dt = time.time() - t0
    # the same step at shorter contexts (the query earlier in the same cache):
    # the fitted exponent of time against context length
    ctx, ts = [], []
    for lg in range(15, 20):                     # 32K .. 512K tokens before the current block
        p_ctx = (1 << lg) + b - 1
        if p_ctx >= x["L"]:
            break
        m, t1 = 0, time.time()
        while m < 2 or time.time() - t1 < seconds / 10:
            qn = np.ascontiguousarray(qs[m % 64])
            sel = oracle.score_select(qn, kb, mx, ce, Hkv=cfg["Hkv"], b=b, K=K, q_pos0=p_ctx, gate=True,
                                      proj_w=x["proj_w"])
            oracle.attn_fwd(qn, x["k"], x["v"], sel["idx"], sel["logg"], b=b, K=K, q_pos0=p_ctx)
            m += 1
        ctx.append(p_ctx + 1)
        ts.append((time.time() - t1) / m)
    expo = float(np.polyfit(np.log(ctx), np.log(ts), 1)[0])
    return dict(value=dt / n * 1e6, unit="us/step", cores=oracle.num_threads(), kind="oracle",
                sample=f"{n} decode steps of layer 0 (512K context, 8 kv heads, C=8192, K=32), "
                       f"rotating 64 queries; block summaries precomputed",
                context_scaling={"contexts": ctx, "us_per_step": [round(t * 1e6, 1) for t in ts],
                                 "fitted_exponent": round(expo, 3)})


def measure_device_peaks():
    """Measured references next to the vendor peaks: a 1 GiB device copy
    (read + write bytes per second) and a bf16 8192^3 GEMM (torch / hipBLASLt)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    a = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    bm = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)

    def best(fn, reps=5):
        fn()
        out = []
        for _ in range(reps):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            out.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        return min(out)

    t_copy = best(lambda: dst.copy_(src))
    t_gemm = best(lambda: torch.mm(a, bm))
    res = {"hbm_copy_gbps": round(2 * src.numel() * 2 / t_copy / 1e9, 1),
           "bf16_gemm_tflops": round(2 * 8192 ** 3 / t_gemm / 1e12, 1),
           "vendor_hbm_gbps": HBM_PEAK_GBPS, "vendor_bf16_tflops": BF16_PEAK_TFLOPS}
    del src, dst, a, bm
    torch.cuda.empty_cache()
    return res


def hbm_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, if it was taken on the current kernel sources."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    try:
        c = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    if c.get("source_sha") != source_hash() or kernel not in c.get("kernels", {}):
        return None
    return c["kernels"][kernel]["traffic_bytes"]


COPY_BYTES = 256 << 20


def calibrate_copy():
    """One plain device-to-device copy of COPY_BYTES, for scaling the HBM
    byte counters of a rocprofv3 --pmc run."""
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def _read_pmc_rows(path, counter):
    """(kernel name, dispatch id, value in KiB, grid size) of every dispatch of
    a rocprofv3 counter_collection.csv for one counter."""
    import csv
    out = []
    with open(path) as fh:
        for row in csv.DictReader(fh):
            name = row.get("Kernel_Name") or row.get("Kernel-Name") or ""
            cname = row.get("Counter_Name") or row.get("Counter-Name") or ""
            if cname != counter:
                continue
            did = int(row.get("Dispatch_Id") or row.get("Dispatch-Id") or 0)
            grid = int(row.get("Grid_Size") or row.get("Grid-Size") or 0)
            out.append((name, did, float(row.get("Counter_Value") or row.get("Counter-Value") or 0.0), grid))
    return out


def write_counters(fetch_csv, write_csv):
    """profiles/decode_512k_hbm_counters.json from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE) of `bench.py --calibrate-copy ...`.  The
    calibration is the device copy whose WRITE_SIZE is nearest COPY_BYTES (the
    runs hold other copies of other sizes); a kernel's figures are the means
    over its dispatches at the 512K workload, the largest grid it was launched
    with (the same run also times the 32K decode workload)."""
    fetch = _read_pmc_rows(fetch_csv, "FETCH_SIZE")
    write = _read_pmc_rows(write_csv, "WRITE_SIZE")
    copy_key = "copyBuffer"          # the runtime's device-to-device copy kernel
    kib = COPY_BYTES / 1024.0
    cw = [(abs(v - kib), did, v) for n, did, v, _ in write if copy_key in n]
    if not cw:
        raise SystemExit("no copy kernel found in the counter files")
    _, cal_id, cal_w = min(cw)
    cf = [v for n, did, v, _ in fetch if copy_key in n and did == cal_id]
    if not cf:
        raise SystemExit("the calibration copy is missing from the FETCH_SIZE run")

    def mean_of(rows, key):
        sel = [(v, g) for n, _, v, g in rows if key in n]
        if not sel:
            return None
        gmax = max(g for _, g in sel)
        vals = [v for v, g in sel if g == gmax]
        return sum(vals) / len(vals)

    out = {"source_sha": source_hash(), "copy_bytes": COPY_BYTES, "copy_dispatch": cal_id,
           "copy_fetch_kib": cf[0], "copy_write_kib": cal_w,
           "fetch_scale": kib / cf[0], "write_scale": kib / cal_w, "kernels": {}}
    out["copy_scale"] = 1.0
    for kname in [k for _, k in STEP_KERNELS + TWO_CALL_KERNELS]:
        f, w = mean_of(fetch, kname), mean_of(write, kname)
        if f is not None and w is not None:
            out["kernels"][kname] = {"fetch_kib": f, "write_kib": w,
                                     "traffic_bytes": f * 1024 * out["fetch_scale"] + w * 1024 * out["write_scale"]}
    with open(COUNTERS_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--layers", type=int, default=16)
    ap.add_argument("--queries", type=int, default=64)
    ap.add_argument("--replays", type=int, default=256,
                    help="one-step graph replays for the per-step median and p99 (cold and warm)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--skip-variants", action="store_true",
                    help="time only the one-call decode step (no two-call or paged comparison); for profiling")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 256 MiB device copy (for scaling rocprofv3 byte counters)")
    ap.add_argument("--only-prefill", action="store_true",
                    help="run only the prefill_cells pipeline --steps times and print its figures; for profiling")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM counters file from two rocprofv3 --pmc CSVs and exit")
    args = ap.parse_args()
    if args.write_counters:
        write_counters(*args.write_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        sys.exit("bench.py measures one GPU only: the method has no cross-GPU exchange on this path "
                 "(see the sharding note in the design document); run with --gpus 1")
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    ops.lib()
    if args.only_prefill:
        if args.calibrate_copy:
            calibrate_copy()
        pf = run_prefill(args.steps)
        print(json.dumps({"prefill_tokens_per_s": round(pf["tokens_per_s"], 1),
                          "prefill_ms": {k: round(float(v), 4) for k, v in pf["ms"].items()}}))
        return

    res = run_decode(args)
    if args.calibrate_copy:
        calibrate_copy()
    wl, steps = res["wl"], args.steps
    us_per_step = res["total_ms"] * 1e3 / steps
    att_bytes, sel_bytes = wl.selected_kv_bytes(), wl.scoring_bytes()
    heads = wl.cfg["B"] * wl.cfg["Hkv"]
    nch = (wl.C + 255) // 256
    d = wl.cfg["d"]
    ntiles = (wl.K + 1) * ((wl.b + 31) // 32)
    # algorithmic bytes per launch.  The scorer: the summaries, W and q, then
    # the scores it hands on (one fp32 per candidate, the chunks' (max, sum)
    # and the group maxima).  The step kernel: the selected K and V, the
    # scores read once per head, and the split-K partials written and read
    # once (the other workgroups of a head re-read the scores from L2).
    score_io = heads * (wl.C * 4 + nch * (8 + 16))
    kbytes = {
        "score": sel_bytes + score_io,
        "step": att_bytes + score_io + 2 * heads * ntiles * 4 * (d + 2) * 4,
    }
    kern = {}
    for k, v in res["k_ms"].items():
        us = float(v.mean() * 1e3)
        kern[k] = dict(kernel=dict(STEP_KERNELS)[k], us=us, p50_us=float(np.median(v) * 1e3),
                       p99_us=float(np.percentile(v, 99) * 1e3), bytes=kbytes[k],
                       gbps=kbytes[k] / (us * 1e-6) / 1e9)
    dom = max(kern, key=lambda n: kern[n]["us"])
    # the roofline of the dominant kernel on the bytes the method must move
    # there: the selected K and V (what the selected-KV rate reports)
    achieved = att_bytes / (kern[dom]["us"] * 1e-6) / 1e9 if dom == "step" else kern[dom]["gbps"]
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4),
                    traffic=hbm_traffic(kern[dom]["kernel"]), kernel=kern[dom]["kernel"],
                    algorithmic_bytes=att_bytes if dom == "step" else kern[dom]["bytes"],
                    launch_us=round(kern[dom]["us"], 3))
    lat = {"l2": load_latency_ns(1 << 20, 20000), "mall": load_latency_ns(64 << 20, 20000),
           "hbm": load_latency_ns(2 << 30, 20000)}
    log(f"[bench] dependent-load latency ns: {lat}")
    out = {
        "metric": "decode attn µs/step + selected-KV HBM GB/s at 512K ctx; prefill tokens/s",
        "value": round(us_per_step, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["total_ms"] / steps, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 K/V/q, N(0,1/128) fp32 selector projection)",
        "config": {"workload": "decode_512k", "batch": 1, "context": wl.L - 1, "q_heads": 32,
                   "kv_heads": 8, "head_dim": 128, "block": wl.b, "K": wl.K, "gate": "softmax_log",
                   "layers_rotated": args.layers, "queries_rotated": args.queries, "graph_replay": True},
        "selected_kv_gbps": round(att_bytes / (kern["step"]["us"] * 1e-6) / 1e9, 1),
        "step_latency_us": res["dist"],
        "decode_sweep": res["sweep"],
        "unfused_us_per_step": None if res["unfused_ms"] is None else round(res["unfused_ms"] * 1e3 / steps, 3),
        "paged_us_per_step": None if res["paged_ms"] is None else round(res["paged_ms"] * 1e3 / steps, 3),
        "fp8_summaries": None if res["fp8_ms"] is None else {
            "us_per_step": round(res["fp8_ms"] * 1e3 / steps, 3),
            "kernels_us": {k: round(float(np.mean(v)) * 1e3, 3) for k, v in res["fp8_k_ms"].items()},
            "scoring_bytes": wl.scoring_bytes(fp8=True),
        },
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kern.items()},
        "hot_cache_us_per_step": round(res["hot_us"], 3),
        # the timed steps include a block close every b steps only when
        # --steps reaches b; the close alone and its share per step:
        "block_close_us": round(res["close_us"], 3),
        "closes_in_timed_steps": steps // wl.b,
        "us_per_step_with_amortised_close": round(
            (res["total_ms"] * 1e3 - (steps // wl.b) * res["close_us"]) / steps + res["close_us"] / wl.b, 3),
        "summaries_512k_ms": round(res["summ_ms"], 3),
        "summaries_gbps": round(res["summ_bytes"] / (res["summ_ms"] * 1e-3) / 1e9, 1),
        "roofline": roofline,
        # t >= (launch + dependency cost of the step's kernels) + (the chain of
        # dependent loads at the measured latencies) + (all bytes at peak).
        # The chain: W and q (HBM); u from the workgroup that formed it, then
        # the scores (MALL: written moments before on another XCD); the K/V
        # tile (HBM); the arrival count, then the partials (MALL); the output
        # (HBM)
        "latency_floor": {
            "kernels_per_step": len(kern),
            "kernel_chain_step_us": round(res["floor_us"], 3),
            "load_latency_ns": {k: round(v, 1) for k, v in lat.items()},
            "dependent_loads": {"hbm": 3, "mall": 4},
            "bytes_at_peak_us": round(sum(k["bytes"] for k in kern.values()) / (HBM_PEAK_GBPS * 1e3), 3),
            "bound_us": round(res["floor_us"] + (3 * lat["hbm"] + 4 * lat["mall"]) * 1e-3
                              + sum(k["bytes"] for k in kern.values()) / (HBM_PEAK_GBPS * 1e3), 3),
        },
    }
    # the 32K decode workload as configured (K = 16, outlier keys, no projection)
    out["decode_32k"] = run_decode_32k(args)
    if not args.no_prefill:
        pf = run_prefill(3)
        out["prefill_tokens_per_s"] = round(pf["tokens_per_s"], 1)
        out["prefill_ms"] = {k: round(v, 3) for k, v in pf["ms"].items()}
        out["prefill_score_mfma_frac"] = round(pf["score_gflop"] / (pf["ms"]["score_select"] * 1e-3)
                                               / (BF16_PEAK_TFLOPS * 1e3), 5)
        fsl = run_fsl_decode(256)
        out["fsl_decode_us_per_step"] = round(fsl["us_per_step"], 3)
        out["fsl_retain_us"] = round(fsl["retain_us"], 3)
        out["fsb_decode_us_per_step"] = round(fsl["fsb_us"], 3)
        out["fsb_forest_build_us"] = round(fsl["forest_build_us"], 3)
        tr = run_train(2)
        out["train_tokens_per_s"] = round(tr["tokens_per_s"], 1)
        out["train_ms"] = {k: round(v, 3) for k, v in tr["ms"].items()}
        sl = run_sas_fwd_long()
        out["sas_fwd_32k_ms"] = round(sl["ms"], 3)
        out["sas_fwd_32k_mfma_frac"] = round(sl["tflop"] / (sl["ms"] * 1e-3) / BF16_PEAK_TFLOPS, 5)
        # algorithmic flops / time / dense bf16 peak (the kernels also execute
        # masked tile work: the union of a row tile's selections)
        out["mfma_frac"] = {
            "prefill_attention": round(pf["attn_gflop"] / (pf["ms"]["attention"] * 1e-3) / (BF16_PEAK_TFLOPS * 1e3), 5),
            "train_fwd": round(tr["fwd_tflop"] / (tr["ms"]["fwd"] * 1e-3) / BF16_PEAK_TFLOPS, 5),
            "train_bwd": round(tr["bwd_tflop"] / (tr["ms"]["bwd"] * 1e-3) / BF16_PEAK_TFLOPS, 5),
            "train_bwd_executed": round(tr["bwd_exec_tflop"] / (tr["ms"]["bwd"] * 1e-3) / BF16_PEAK_TFLOPS, 5)}
    out["device_peaks_measured"] = measure_device_peaks()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = run_cpu_baseline(res, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
