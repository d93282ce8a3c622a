"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every entry point declared in include/sparse_attn.h, and rejects invalid
arguments with the documented status codes before launching anything."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from block_sparse_attention_summaries_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced (validation fails first)
FAKE_ODD = ctypes.c_void_p(0x10001)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)))


def test_library_exports_every_declared_symbol():
    lib = ops.lib()
    names = declared_functions()
    assert set(names) == set(ops.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.sparse_abi_version() == 2 and lib.spa_abi_version() == 2
    # the four entry points and the helpers under the names the boundary
    # specifies, the entry points typed spa_status
    text = open(HEADER).read()
    for n in ("sparse_block_summaries", "sparse_score_select", "sparse_attn_fwd", "sparse_attn_bwd"):
        assert re.search(r"^spa_status " + n + r"\(", text, flags=re.M), n
    for n in ("sparse_workspace_bytes", "sparse_last_error", "sparse_abi_version"):
        assert n in names, n


def _sel(**kw):
    a = ops.SelectArgs(q=FAKE, dtype=1, B=1, Hq=32, Hkv=8, nq=1, d=128, q_pos0=32831, kbar=FAKE,
                       max_norm=FAKE, centre=FAKE, ccap=513, b=64, prefix_mode=0, qblock=128,
                       share_group=1, proj_w=None, erf_lambda=None, erf_sigma=None, K=16, gate=1,
                       idx=FAKE, logg=FAKE, k_eff=None)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _attn(**kw):
    a = ops.AttnArgs(q=FAKE, k=FAKE, v=FAKE, dtype=1, B=1, Hq=32, Hkv=8, nq=1, d=128, L=32832,
                     q_pos0=32831, b=64, prefix_mode=0, qblock=128, idx=FAKE, logg=FAKE, K=16,
                     share_group=1, local=0, window=0, alpha=None, o=FAKE, lse=FAKE)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _select_status(a, ws=None, n=0):
    return ops.lib().sparse_score_select(ctypes.byref(a), ws, n, None)


def _attn_status(a, ws=None, n=0):
    return ops.lib().sparse_attn_fwd(ctypes.byref(a), ws, n, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), ops.SPA_ERR_INVALID_ARG),
    (dict(idx=None), ops.SPA_ERR_INVALID_ARG),
    (dict(q=FAKE_ODD), ops.SPA_ERR_INVALID_ARG),
    (dict(d=96), ops.SPA_ERR_UNSUPPORTED),
    (dict(dtype=7), ops.SPA_ERR_UNSUPPORTED),
    (dict(b=48), ops.SPA_ERR_UNSUPPORTED),
    (dict(b=256), ops.SPA_ERR_UNSUPPORTED),
    (dict(K=0), ops.SPA_ERR_UNSUPPORTED),
    (dict(K=65), ops.SPA_ERR_UNSUPPORTED),
    (dict(Hq=30), ops.SPA_ERR_INVALID_ARG),          # G does not divide
    (dict(Hq=8 * 16), ops.SPA_ERR_UNSUPPORTED),      # G = 16
    (dict(logg=None), ops.SPA_ERR_INVALID_ARG),      # gate on needs logg
    (dict(gate=3), ops.SPA_ERR_INVALID_ARG),
    (dict(ccap=100), ops.SPA_ERR_INVALID_ARG),       # candidates beyond kbar
    (dict(erf_lambda=FAKE), ops.SPA_ERR_INVALID_ARG),  # sigma missing
    (dict(prefix_mode=1, qblock=100), ops.SPA_ERR_INVALID_ARG),
    (dict(nq=0), ops.SPA_ERR_INVALID_ARG),
])
def test_select_rejects_invalid_arguments(kw, code):
    assert _select_status(_sel(**kw)) == code
    assert ops.lib().sparse_last_error().decode() != ""


def test_select_workspace_too_small():
    a = _sel()
    need = ops.lib().sparse_workspace_bytes(ops.SPA_OP_SCORE_SELECT, ctypes.byref(a))
    # decode path: 512 candidates -> 8 heads x 2 chunks of 256 blocks x K keys + (m, l) per chunk
    assert need == 256 * ((8 * 2 * 16 * 8 + 255) // 256) + 256 * ((8 * 2 * 8 + 255) // 256)
    assert _select_status(a, None, 0) == ops.SPA_ERR_WORKSPACE
    assert _select_status(a, FAKE, need - 1) == ops.SPA_ERR_WORKSPACE


def test_select_rows_erf_workspace():
    """Many bf16 rows with the erf term keep one fp32 and one fp64 filter table
    per selection head in the workspace (160 KiB each); without the erf term
    the row selection needs none."""
    rows = dict(nq=16384, q_pos0=0, Hq=16, Hkv=16, d=64, ccap=512, b=32, prefix_mode=1, qblock=128,
                share_group=0, K=4, gate=0, logg=None)
    a = _sel(**rows, erf_lambda=FAKE, erf_sigma=FAKE)
    need = ops.lib().sparse_workspace_bytes(ops.SPA_OP_SCORE_SELECT, ctypes.byref(a))
    assert need == 16 * (8192 * 4 + 16384 * 8)
    assert _select_status(a, None, 0) == ops.SPA_ERR_WORKSPACE
    assert _select_status(a, FAKE, need - 256) == ops.SPA_ERR_WORKSPACE
    plain = _sel(**rows)
    assert ops.lib().sparse_workspace_bytes(ops.SPA_OP_SCORE_SELECT, ctypes.byref(plain)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(v=None), ops.SPA_ERR_INVALID_ARG),
    (dict(o=None), ops.SPA_ERR_INVALID_ARG),
    (dict(q_pos0=32832), ops.SPA_ERR_INVALID_ARG),   # row beyond L
    (dict(local=1), ops.SPA_ERR_UNSUPPORTED),         # no window, no alpha
    (dict(window=512), ops.SPA_ERR_UNSUPPORTED),      # window without alpha / local
    (dict(d=32), ops.SPA_ERR_UNSUPPORTED),
    (dict(b=24), ops.SPA_ERR_UNSUPPORTED),
])
def test_attn_rejects_invalid_arguments(kw, code):
    assert _attn_status(_attn(**kw)) == code


def test_attn_workspace_sizes():
    a = _attn()
    need = ops.lib().sparse_workspace_bytes(ops.SPA_OP_ATTN_FWD, ctypes.byref(a))
    # decode split-K: 8 heads x 17 tiles x 4 q heads x (128 acc floats) + (m, l)
    acc = 8 * 17 * 4 * 128 * 4
    ml = 8 * 17 * 4 * 8
    assert need == 256 * ((acc + 255) // 256) + 256 * ((ml + 255) // 256)
    assert _attn_status(a, None, 0) == ops.SPA_ERR_WORKSPACE
    pre = _attn(nq=8192, q_pos0=0, L=8192)
    assert ops.lib().sparse_workspace_bytes(ops.SPA_OP_ATTN_FWD, ctypes.byref(pre)) == 0
    # backward: D_i per (head, row); the bf16 MFMA path adds one selection bit
    # per (selection head, block, row): 8 heads x 128 blocks x 256 words
    dbuf = 32 * 8192 * 4
    assert ops.lib().sparse_workspace_bytes(ops.SPA_OP_ATTN_BWD, ctypes.byref(pre)) == dbuf + 8 * 128 * 256 * 4
    pre32 = _attn(nq=8192, q_pos0=0, L=8192, dtype=0)
    assert ops.lib().sparse_workspace_bytes(ops.SPA_OP_ATTN_BWD, ctypes.byref(pre32)) == dbuf


def test_bwd_rejects_unsupported_modes():
    lib = ops.lib()
    a = _attn(nq=256, q_pos0=0, L=256, local=1, window=64, alpha=FAKE)
    assert lib.sparse_attn_bwd(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                               None) == ops.SPA_ERR_UNSUPPORTED
    a = _attn(nq=256, q_pos0=0, L=256, b=128)
    assert lib.sparse_attn_bwd(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                               None) == ops.SPA_ERR_UNSUPPORTED
    a = _attn(nq=256, q_pos0=0, L=256)
    assert lib.sparse_attn_bwd(ctypes.byref(a), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                               None) == ops.SPA_ERR_INVALID_ARG


def _grads(**kw):
    g = ops.SelectGrads(dg=FAKE, dq=FAKE, dkbar=FAKE, dproj_w=None, dk=None, L=0)
    for k, v in kw.items():
        setattr(g, k, v)
    return g


def test_select_bwd_rejects_unsupported_modes():
    lib = ops.lib()

    def st(a, g=None, n=1 << 20):
        g = _grads() if g is None else g
        return lib.sparse_select_bwd(ctypes.byref(a), ctypes.byref(g), FAKE, n, None)
    base = dict(nq=8192, q_pos0=0, ccap=128)
    assert st(_sel(**base, gate=0, logg=None)) == ops.SPA_ERR_UNSUPPORTED
    assert st(_sel(**base, dtype=0)) == ops.SPA_ERR_UNSUPPORTED
    assert st(_sel(**base, prefix_mode=1, qblock=128)) == ops.SPA_ERR_UNSUPPORTED
    assert st(_sel(**base, erf_lambda=FAKE, erf_sigma=FAKE)) == ops.SPA_ERR_UNSUPPORTED
    assert st(_sel(**base), _grads(dg=None)) == ops.SPA_ERR_INVALID_ARG
    assert st(_sel(**base), _grads(dq=FAKE_ODD)) == ops.SPA_ERR_INVALID_ARG
    assert st(_sel(**base, proj_w=FAKE)) == ops.SPA_ERR_INVALID_ARG          # dproj_w missing
    assert st(_sel(**base), _grads(dproj_w=FAKE)) == ops.SPA_ERR_INVALID_ARG  # no projection
    assert st(_sel(**base), _grads(dk=FAKE, L=128 * 64 - 1)) == ops.SPA_ERR_INVALID_ARG
    assert st(_sel(**base), _grads(dk=FAKE_ODD, L=8192)) == ops.SPA_ERR_INVALID_ARG
    a = _sel(**base)
    rows = 8 * 8192
    # one (LSE, sum_S p dg) pair per (batch, selection head, row), q_hat (bf16)
    # per row, and 16 row shares of dkbar (4 candidate tiles x 8 heads = 32
    # workgroups per share)
    shares = 16 * 8 * 128 * 128 * 4
    need = lib.sparse_workspace_bytes(ops.SPA_OP_SELECT_BWD, ctypes.byref(a))
    assert need == rows * 8 + rows * 128 * 2 + shares
    assert st(a, n=need - 1) == ops.SPA_ERR_WORKSPACE
    # one head per selection: no q_hat copy
    a1 = _sel(**base, share_group=0)
    rows1 = 32 * 8192
    assert lib.sparse_workspace_bytes(ops.SPA_OP_SELECT_BWD, ctypes.byref(a1)) == rows1 * 8 + shares
    # with the projection: u (bf16) and r (fp32) per row instead, + 256 dW partials
    ap = _sel(**base, proj_w=FAKE)
    assert lib.sparse_workspace_bytes(ops.SPA_OP_SELECT_BWD, ctypes.byref(ap)) == \
        rows * 8 + shares + rows * 128 * 2 + rows * 128 * 4 + 256 * 128 * 128 * 4


def test_decode_step_validation_and_workspace():
    lib = ops.lib()
    sel, att = _sel(), _attn()
    da = ops.DecodeArgs(select=ctypes.pointer(sel), attn=ctypes.pointer(att))
    need = lib.sparse_workspace_bytes(ops.SPA_OP_DECODE_STEP, ctypes.byref(da))
    need_sel = lib.sparse_workspace_bytes(ops.SPA_OP_SCORE_SELECT, ctypes.byref(sel))
    need_att = lib.sparse_workspace_bytes(ops.SPA_OP_ATTN_FWD, ctypes.byref(att))
    # the one-call scorer's u block (16 KiB at offset 0, u [8, 128] as
    # ready-marked 64-bit words), scores [8 heads, 2 chunks, 256] fp32, chunk
    # (max, sum exp) and group maxima, or the two-call selection's scratch
    # after the same block, whichever is larger; then split-K partials and one
    # arrival counter per selection head
    r256 = lambda x: 256 * ((x + 255) // 256)
    scorer = 16384 + r256(8 * 2 * 256 * 4) + r256(8 * 2 * 8) + r256(8 * 2 * 4 * 4)
    assert need == r256(max(scorer, 16384 + need_sel)) + need_att + 256
    assert lib.sparse_decode_step(ctypes.byref(da), FAKE, need - 1, None) == ops.SPA_ERR_WORKSPACE

    def status(s, a):
        d = ops.DecodeArgs(select=ctypes.pointer(s), attn=ctypes.pointer(a))
        return lib.sparse_decode_step(ctypes.byref(d), FAKE, 1 << 30, None)
    assert status(_sel(), _attn(K=8)) == ops.SPA_ERR_INVALID_ARG                  # different K
    assert status(_sel(), _attn(idx=FAKE_ODD)) == ops.SPA_ERR_INVALID_ARG         # not select's idx
    assert status(_sel(), _attn(q=ctypes.c_void_p(0x20000))) == ops.SPA_ERR_INVALID_ARG
    assert status(_sel(nq=2, q_pos0=32830), _attn(nq=2, q_pos0=32830)) == ops.SPA_ERR_UNSUPPORTED
    assert status(_sel(), _attn(local=1, window=64, alpha=FAKE)) == ops.SPA_ERR_UNSUPPORTED
    assert lib.sparse_decode_step(None, FAKE, 1 << 30, None) == ops.SPA_ERR_INVALID_ARG


def test_decode_step_noalloc_rejects_before_launch():
    """The no-alloc step validates like sparse_decode_step and refuses a step
    whose scratch exceeds the library's array, before any HIP call."""
    lib = ops.lib()
    cap = 8 << 20                                   # SPA_NOALLOC_SCRATCH_BYTES
    # 64 sequences x 8 kv heads, K = 64: the split-K partials alone exceed it
    sel = _sel(B=64, K=64, q_pos0=(1 << 20) + 63, ccap=1 << 14)
    att = _attn(B=64, K=64, q_pos0=(1 << 20) + 63, L=(1 << 20) + 64)
    da = ops.DecodeArgs(select=ctypes.pointer(sel), attn=ctypes.pointer(att))
    assert lib.sparse_workspace_bytes(ops.SPA_OP_DECODE_STEP, ctypes.byref(da)) > cap
    assert lib.sparse_decode_step_noalloc(ctypes.byref(da), None) == ops.SPA_ERR_WORKSPACE
    assert "scratch" in lib.sparse_last_error().decode()
    # the decode_32k step fits
    da = ops.DecodeArgs(select=ctypes.pointer(_sel()), attn=ctypes.pointer(_attn()))
    assert lib.sparse_workspace_bytes(ops.SPA_OP_DECODE_STEP, ctypes.byref(da)) <= cap
    assert lib.sparse_decode_step_noalloc(None, None) == ops.SPA_ERR_INVALID_ARG
    bad = ops.DecodeArgs(select=ctypes.pointer(_sel()), attn=ctypes.pointer(_attn(K=8)))
    assert lib.sparse_decode_step_noalloc(ctypes.byref(bad), None) == ops.SPA_ERR_INVALID_ARG


def test_summaries_rejects_invalid_arguments():
    lib = ops.lib()
    f = lib.sparse_block_summaries
    assert f(None, 1, 1, 8, 4096, 128, 64, 0, 64, 64, FAKE, FAKE, None, None) == ops.SPA_ERR_INVALID_ARG
    assert f(FAKE, 1, 1, 8, 4096, 128, 64, 0, 65, 65, FAKE, FAKE, None, None) == ops.SPA_ERR_INVALID_ARG
    assert f(FAKE, 1, 1, 8, 4096, 128, 64, 0, 64, 63, FAKE, FAKE, None, None) == ops.SPA_ERR_INVALID_ARG
    assert f(FAKE, 1, 1, 8, 4096, 100, 64, 0, 64, 64, FAKE, FAKE, None, None) == ops.SPA_ERR_UNSUPPORTED
    assert f(FAKE, 1, 1, 8, 4096, 128, 64, 0, 0, 64, FAKE, FAKE, None, None) == ops.SPA_OK  # nothing to do
    assert ops.lib().sparse_last_error().decode() == ""


@pytest.mark.parametrize("kw,code", [
    (dict(kbar_scale=FAKE, nq=2, q_pos0=32830), ops.SPA_ERR_UNSUPPORTED),    # rows path
    (dict(kbar_scale=FAKE, prefix_mode=1), ops.SPA_ERR_UNSUPPORTED),
    (dict(kbar_scale=FAKE, erf_lambda=FAKE, erf_sigma=FAKE), ops.SPA_ERR_UNSUPPORTED),
])
def test_fp8_summaries_only_on_the_decode_scorer(kw, code):
    assert _select_status(_sel(**kw)) == code
    assert "fp8" in ops.lib().sparse_last_error().decode()
    # the one-row decode scorer takes them (workspace check comes next)
    assert _select_status(_sel(kbar_scale=FAKE)) == ops.SPA_ERR_WORKSPACE


def test_fp8_quantize_and_dequantize_reject_invalid_arguments():
    L = ops.lib()
    q = L.sparse_quantize_summaries_fp8
    assert q(None, 1, 1, 8, 16, 128, 0, 16, FAKE, FAKE, None) == ops.SPA_ERR_INVALID_ARG
    assert q(FAKE, 1, 1, 8, 16, 128, 0, 16, FAKE_ODD, FAKE, None) == ops.SPA_ERR_INVALID_ARG
    assert q(FAKE, 1, 1, 8, 16, 128, 8, 9, FAKE, FAKE, None) == ops.SPA_ERR_INVALID_ARG      # past ccap
    assert q(FAKE, 1, 1, 8, 16, 96, 0, 16, FAKE, FAKE, None) == ops.SPA_ERR_UNSUPPORTED
    assert q(FAKE, 5, 1, 8, 16, 128, 0, 16, FAKE, FAKE, None) == ops.SPA_ERR_UNSUPPORTED
    assert q(FAKE, 1, 1, 8, 16, 128, 3, 0, FAKE, FAKE, None) == ops.SPA_OK                   # nothing to do
    dq = L.sparse_dequantize_summaries_fp8
    assert dq(FAKE, FAKE, 4, 96, FAKE, None) == ops.SPA_ERR_UNSUPPORTED
    assert dq(None, FAKE, 4, 128, FAKE, None) == ops.SPA_ERR_INVALID_ARG
    assert dq(FAKE, FAKE, -1, 128, FAKE, None) == ops.SPA_ERR_INVALID_ARG
    assert dq(FAKE, FAKE, 0, 128, FAKE, None) == ops.SPA_OK


def test_load_chase_probe_rejects_invalid_arguments():
    lib = ops.lib()
    out = FAKE
    for n, steps in ((3, 10), (0, 10), (1 << 33, 10), (1024, 0)):
        assert lib.sparse_probe_load_chase(FAKE, n, steps, 0, out, None) == -1, (n, steps)
        assert b"sparse_probe_load_chase" in lib.sparse_last_error() or b"n =" in lib.sparse_last_error() \
            or b"steps" in lib.sparse_last_error()
    assert lib.sparse_probe_load_chase(None, 1024, 10, 0, out, None) == -1


def test_workspace_clears_the_decode_flags_after_other_calls():
    """A Workspace handed to another entry point and then to a decode step
    has the step's u block (ready-marked words) zeroed first (host buffer, no GPU)."""
    ws = ops.Workspace(device="cpu")
    buf, _ = ws.get(1 << 16, ops.SPA_OP_SCORE_SELECT)
    buf.fill_(7)
    buf, _ = ws.get(1 << 16, ops.SPA_OP_DECODE_STEP)
    assert int(buf[:ops.SPA_DECODE_FLAG_BYTES].sum()) == 0
    assert int(buf[ops.SPA_DECODE_FLAG_BYTES]) == 7          # the rest is left as it is
    buf[:ops.SPA_DECODE_FLAG_BYTES].fill_(3)                 # decode steps keep it (they restore it)
    buf, _ = ws.get(1 << 16, ops.SPA_OP_DECODE_STEP)
    assert int(buf[0]) == 3
    assert ops.SPA_DECODE_FLAG_BYTES == 16384
