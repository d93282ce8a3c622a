"""GPU test of sparse_decode_step_noalloc (the decode step for callers that
cannot allocate device memory): through the C ABI, its outputs must equal
those of sparse_decode_step (workspace argument, same kernels) bit for bit,
on two calls in a row, the second on a smaller input, and again on the first
input (the library's scratch keeps the last call's contents)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from block_sparse_attention_summaries_amd import ops
from block_sparse_attention_summaries_amd.inputs import config, make_inputs
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def _step(cfg, x, noalloc):
    b, K, pos = cfg["b"], cfg["K"], x["q_pos0"]
    kw = dict(Hkv=cfg["Hkv"], b=b, K=K, q_pos0=pos, gate=cfg["gate"], share_group=cfg["share_group"])
    qd, kd, vd = dev(x["q"]), dev(x["k"]), dev(x["v"])
    kb, mx, ce = ops.sparse_block_summaries(kd, b, num_blocks=x["L"] // b, ccap=max(x["L"] // b, 1))
    pw = None if x.get("proj_w") is None else dev(x["proj_w"])
    f = ops.sparse_decode_step_noalloc if noalloc else ops.sparse_decode_step
    out = f(qd, kb, mx, ce, kd, vd, proj_w=pw, **kw)
    torch.cuda.synchronize()
    return [None if t is None else host(t) for t in out]


CASES = [("decode_512k", dict(n=65536, seed=201)),                    # projection, K = 32, 8 kv heads
         ("decode_32k", dict(n=4096, Hq=8, Hkv=2, K=8, t=17, seed=202)),  # smaller: 2 kv heads, partial block
         ("decode_512k", dict(n=65536, seed=201))]


def test_noalloc_decode_step_equals_workspace_step():
    for name, over in CASES:
        cfg = config(name, **over)
        print(f"[noalloc decode] {name} {over}", file=sys.stderr, flush=True)
        x = make_inputs(cfg)
        want = _step(cfg, x, noalloc=False)
        got = _step(cfg, x, noalloc=True)
        for key, w, g in zip(("idx", "logg", "k_eff", "o", "lse"), want, got):
            if w is None:
                assert g is None, key
                continue
            assert g.shape == w.shape and np.array_equal(g.view(np.uint8), w.view(np.uint8)), key
