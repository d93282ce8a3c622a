"""Thin Python binding of libsparse_attn.so (C ABI in include/sparse_attn.h).

Argument marshalling only: PyTorch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing or its call fails, these
functions raise.

Function names match the C entry points: sparse_block_summaries,
sparse_score_select, sparse_attn_fwd, sparse_attn_bwd, sparse_select_bwd,
sparse_decode_step.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_attn.so")

SPA_OK, SPA_ERR_INVALID_ARG, SPA_ERR_UNSUPPORTED, SPA_ERR_HIP, SPA_ERR_WORKSPACE = 0, -1, -2, -3, -4
SPA_DTYPE_F32, SPA_DTYPE_BF16 = 0, 1
SPA_PREFIX_CURRENT_BLOCK, SPA_PREFIX_QUERY_BLOCK = 0, 1
SPA_GATE_NONE, SPA_GATE_SOFTMAX_LOG = 0, 1
SPA_LOCAL_CURRENT_BLOCK, SPA_LOCAL_NONE = 0, 1
SPA_OP_SCORE_SELECT, SPA_OP_ATTN_FWD, SPA_OP_ATTN_BWD, SPA_OP_SELECT_BWD, SPA_OP_DECODE_STEP = 1, 2, 3, 4, 5

EXPORTED = ["sparse_abi_version", "sparse_last_error", "spa_abi_version", "spa_profile_next_call", "spa_last_error",
            "sparse_block_summaries", "sparse_score_select",
            "sparse_attn_fwd", "sparse_attn_bwd", "sparse_select_bwd", "sparse_decode_step", "sparse_decode_step_noalloc",
            "sparse_block_summaries_paged", "sparse_decode_step_paged", "sparse_retain_cells",
            "sparse_score_select_subset", "sparse_forest_nodes", "sparse_forest_workspace_bytes",
            "sparse_forest_build", "sparse_forest_select", "sparse_quantize_summaries_fp8",
            "sparse_dequantize_summaries_fp8", "sparse_workspace_bytes", "sparse_workspace_init",
            "sparse_probe_load_chase"]

_vp, _i, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
ABI_VERSION = 2               # layout of the argument structs below


class SelectArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("dtype", _i), ("B", _i), ("Hq", _i), ("Hkv", _i), ("nq", _i), ("d", _i),
                ("q_pos0", _i64), ("kbar", _vp), ("max_norm", _vp), ("centre", _vp), ("ccap", _i64),
                ("b", _i), ("prefix_mode", _i), ("qblock", _i), ("share_group", _i), ("proj_w", _vp),
                ("erf_lambda", _vp), ("erf_sigma", _vp), ("K", _i), ("gate", _i), ("idx", _vp),
                ("logg", _vp), ("k_eff", _vp), ("kbar_scale", _vp)]


class SelectGrads(ctypes.Structure):
    _fields_ = [("dg", _vp), ("dq", _vp), ("dkbar", _vp), ("dproj_w", _vp), ("dk", _vp), ("L", _i64)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("dtype", _i), ("B", _i), ("Hq", _i), ("Hkv", _i),
                ("nq", _i), ("d", _i), ("L", _i64), ("q_pos0", _i64), ("b", _i), ("prefix_mode", _i),
                ("qblock", _i), ("idx", _vp), ("logg", _vp), ("K", _i), ("share_group", _i),
                ("local", _i), ("window", _i), ("alpha", _vp), ("o", _vp), ("lse", _vp)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("select", ctypes.POINTER(SelectArgs)), ("attn", ctypes.POINTER(AttnArgs))]


class KvPages(ctypes.Structure):
    _fields_ = [("block_table", _vp), ("table_stride", _i64), ("num_pages", _i64)]


class Forest(ctypes.Structure):
    _fields_ = [("members", _vp), ("nmem", _vp), ("mu", _vp), ("rad", _vp), ("amax", _vp), ("pmin", _vp)]


class SpaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libsparse_attn error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load libsparse_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name in ("sparse_abi_version", "spa_abi_version"):
            getattr(L, name).restype = _i
            getattr(L, name).argtypes = []
        L.spa_profile_next_call.restype = _i
        L.spa_profile_next_call.argtypes = [ctypes.POINTER(_vp), _i]
        for name in ("sparse_last_error", "spa_last_error"):
            getattr(L, name).restype = ctypes.c_char_p
            getattr(L, name).argtypes = []
        L.sparse_block_summaries.restype = _i
        L.sparse_block_summaries.argtypes = [_vp, _i, _i, _i, _i64, _i, _i, _i64, _i64, _i64, _vp, _vp,
                                             _vp, _vp]
        L.sparse_score_select.restype = _i
        L.sparse_score_select.argtypes = [ctypes.POINTER(SelectArgs), _vp, _sz, _vp]
        L.sparse_attn_fwd.restype = _i
        L.sparse_attn_fwd.argtypes = [ctypes.POINTER(AttnArgs), _vp, _sz, _vp]
        L.sparse_attn_bwd.restype = _i
        L.sparse_attn_bwd.argtypes = [ctypes.POINTER(AttnArgs), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _sz, _vp]
        L.sparse_select_bwd.restype = _i
        L.sparse_select_bwd.argtypes = [ctypes.POINTER(SelectArgs), ctypes.POINTER(SelectGrads), _vp, _sz, _vp]
        L.sparse_decode_step.restype = _i
        L.sparse_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _vp, _sz, _vp]
        L.sparse_decode_step_noalloc.restype = _i
        L.sparse_decode_step_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
        L.sparse_block_summaries_paged.restype = _i
        L.sparse_block_summaries_paged.argtypes = [_vp, _i, _i, _i, _i64, _i, _i, ctypes.POINTER(KvPages), _i64,
                                                   _i64, _i64, _vp, _vp, _vp, _vp]
        L.sparse_decode_step_paged.restype = _i
        L.sparse_decode_step_paged.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(KvPages), _vp, _sz, _vp]
        L.sparse_retain_cells.restype = _i
        L.sparse_retain_cells.argtypes = [_vp, _i, _i, _i64, _i64, _i, _i, _vp, _vp, _vp]
        L.sparse_score_select_subset.restype = _i
        L.sparse_score_select_subset.argtypes = [ctypes.POINTER(SelectArgs), _vp, _vp, _i, _vp]
        L.sparse_forest_nodes.restype = _i64
        L.sparse_forest_nodes.argtypes = [_i64]
        L.sparse_forest_workspace_bytes.restype = _sz
        L.sparse_forest_workspace_bytes.argtypes = [_i, _i, _i, _i64]
        L.sparse_forest_build.restype = _i
        L.sparse_forest_build.argtypes = [_vp, _i, _vp, _vp, _i, _i, _i, _i64, _i64, ctypes.POINTER(Forest), _vp,
                                          _sz, _vp]
        L.sparse_forest_select.restype = _i
        L.sparse_forest_select.argtypes = [ctypes.POINTER(SelectArgs), _vp, _i64, ctypes.POINTER(Forest), _i64, _vp]
        L.sparse_quantize_summaries_fp8.restype = _i
        L.sparse_quantize_summaries_fp8.argtypes = [_vp, _i, _i, _i, _i64, _i, _i64, _i64, _vp, _vp, _vp]
        L.sparse_dequantize_summaries_fp8.restype = _i
        L.sparse_dequantize_summaries_fp8.argtypes = [_vp, _vp, _i64, _i, _vp, _vp]
        L.sparse_workspace_bytes.restype = _sz
        L.sparse_workspace_bytes.argtypes = [_i, _vp]
        L.sparse_workspace_init.restype = _i
        L.sparse_workspace_init.argtypes = [_vp, _sz, _vp]
        L.sparse_probe_load_chase.restype = _i
        L.sparse_probe_load_chase.argtypes = [_vp, _i64, _i, ctypes.c_uint32, _vp, _vp]
        if L.sparse_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.sparse_abi_version()}, this binding needs "
                               f"{ABI_VERSION}: rebuild it with __graft_entry__.build()")
        _lib = L
    return _lib


def _check(code):
    if code != SPA_OK:
        raise SpaError(code, lib().sparse_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return SPA_DTYPE_BF16
    if t.dtype == torch.float32:
        return SPA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors passed to libsparse_attn must be contiguous")


SPA_DECODE_FLAG_BYTES = 16384     # the decode step's ready-marked words at the workspace's start


class Workspace:
    """A zero-initialised device buffer reused across calls (grown on demand).
    Calls that share one Workspace must not overlap in time.  A decode step
    after another entry point's call clears the step's u block (ready-marked words) first."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None
        self.last_op = None

    def get(self, nbytes, op=None):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            n = (nbytes + 255) // 256 * 256
            self.buf = torch.zeros(n, dtype=torch.uint8, device=self.device)
        elif op == SPA_OP_DECODE_STEP and self.last_op not in (None, SPA_OP_DECODE_STEP):
            self.buf[:min(SPA_DECODE_FLAG_BYTES, self.buf.numel())].zero_()
        self.last_op = 0 if op is None else op
        return self.buf, self.buf.numel()


_default_ws = {}


def _ws(workspace, op, args, device):
    need = lib().sparse_workspace_bytes(op, ctypes.byref(args))
    if need == 0:          # none needed (invalid arguments are reported by the call itself)
        return None, 0
    if workspace is None:
        key = (str(device), op)
        workspace = _default_ws.setdefault(key, Workspace(device))
    buf, size = workspace.get(need, op)
    return buf, size


def sparse_block_summaries(k, b, first_block=0, num_blocks=None, ccap=None, kbar=None,
                           max_norm=None, centre=None, stream=None):
    """Summaries of full blocks [first_block, first_block + num_blocks) of
    k [B, Hkv, L, d]: mean key (k dtype), max key norm (fp32), centre (fp32).
    Outputs are allocated when not given (kbar [B,Hkv,ccap,d], max_norm
    [B,Hkv,ccap], centre [ccap])."""
    _contig(k, kbar, max_norm, centre)
    B, Hkv, L, d = k.shape
    if num_blocks is None:
        num_blocks = L // b - first_block
    if ccap is None:
        ccap = kbar.shape[2] if kbar is not None else first_block + num_blocks
    if kbar is None:
        kbar = torch.zeros((B, Hkv, ccap, d), dtype=k.dtype, device=k.device)
    if max_norm is None:
        max_norm = torch.zeros((B, Hkv, ccap), dtype=torch.float32, device=k.device)
    if centre is None:
        centre = torch.zeros((ccap,), dtype=torch.float32, device=k.device)
    _check(lib().sparse_block_summaries(_p(k), _dtype(k), B, Hkv, L, d, b, first_block, num_blocks,
                                        ccap, _p(kbar), _p(max_norm), _p(centre), _stream(stream)))
    return kbar, max_norm, centre


def sparse_quantize_summaries_fp8(kbar, first_block=0, num_blocks=None, codes=None, scales=None, stream=None):
    """fp8 (OCP E4M3) block summaries of kbar [B, Hkv, ccap, d] for blocks
    [first_block, first_block + num_blocks): codes uint8 [B, Hkv, ccap, d] and
    per-block scales fp32 [B, Hkv, ccap] (allocated zeroed when not given)."""
    _contig(kbar, codes, scales)
    B, Hkv, ccap, d = kbar.shape
    if num_blocks is None:
        num_blocks = ccap - first_block
    if codes is None:
        codes = torch.zeros((B, Hkv, ccap, d), dtype=torch.uint8, device=kbar.device)
    if scales is None:
        scales = torch.zeros((B, Hkv, ccap), dtype=torch.float32, device=kbar.device)
    _check(lib().sparse_quantize_summaries_fp8(_p(kbar), _dtype(kbar), B, Hkv, ccap, d, first_block, num_blocks,
                                               _p(codes), _p(scales), _stream(stream)))
    return codes, scales


def sparse_dequantize_summaries_fp8(codes, scales, out=None, stream=None):
    """The fp32 summaries the decode scorer reads: scales * decode(codes)."""
    _contig(codes, scales, out)
    d = codes.shape[-1]
    if out is None:
        out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _check(lib().sparse_dequantize_summaries_fp8(_p(codes), _p(scales), codes.numel() // d, d, _p(out),
                                                 _stream(stream)))
    return out


def select_args(q, kbar, max_norm, centre, *, Hkv, b, K, q_pos0, gate=True, prefix_mode=0,
                qblock=128, share_group=True, proj_w=None, erf_lambda=None, erf_sigma=None,
                idx=None, logg=None, k_eff=None, kbar_scale=None):
    """kbar_scale: None, or the per-block scales of fp8 summaries (kbar then
    holds the uint8 codes of sparse_quantize_summaries_fp8)."""
    _contig(q, kbar, max_norm, centre, proj_w, erf_lambda, erf_sigma, idx, logg, k_eff, kbar_scale)
    B, Hq, nq, d = q.shape
    Hsel = Hkv if share_group else Hq
    dev = q.device
    if idx is None:
        idx = torch.empty((B, Hsel, nq, K), dtype=torch.int32, device=dev)
    if logg is None and gate:
        logg = torch.empty((B, Hsel, nq, K), dtype=torch.float32, device=dev)
    if k_eff is None:
        k_eff = torch.empty((B, Hsel, nq), dtype=torch.int32, device=dev)
    a = SelectArgs(q=_p(q), dtype=_dtype(q), B=B, Hq=Hq, Hkv=Hkv, nq=nq, d=d, q_pos0=q_pos0,
                   kbar=_p(kbar), max_norm=_p(max_norm), centre=_p(centre), ccap=kbar.shape[2], b=b,
                   prefix_mode=prefix_mode, qblock=qblock, share_group=int(bool(share_group)),
                   proj_w=_p(proj_w), erf_lambda=_p(erf_lambda), erf_sigma=_p(erf_sigma), K=K,
                   gate=int(bool(gate)), idx=_p(idx), logg=_p(logg), k_eff=_p(k_eff),
                   kbar_scale=_p(kbar_scale))
    return a, (idx, logg, k_eff)


def sparse_score_select(q, kbar, max_norm, centre, *, workspace=None, stream=None, **kw):
    """Scores + softmax log gate + top-K for every row of q [B, Hq, nq, d].
    Returns (idx [B,Hsel,nq,K] int32, logg fp32 or None, k_eff int32)."""
    a, outs = select_args(q, kbar, max_norm, centre, **kw)
    buf, size = _ws(workspace, SPA_OP_SCORE_SELECT, a, q.device)
    _check(lib().sparse_score_select(ctypes.byref(a), _p(buf), size, _stream(stream)))
    return outs


def attn_args(q, k, v, idx, logg, *, b, K, q_pos0, share_group=True, local=0, window=0,
              alpha=None, prefix_mode=0, qblock=128, o=None, lse=None):
    _contig(q, k, v, idx, logg, alpha, o, lse)
    B, Hq, nq, d = q.shape
    _, Hkv, L, _ = k.shape
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, nq), dtype=torch.float32, device=q.device)
    a = AttnArgs(q=_p(q), k=_p(k), v=_p(v), dtype=_dtype(q), B=B, Hq=Hq, Hkv=Hkv, nq=nq, d=d, L=L,
                 q_pos0=q_pos0, b=b, prefix_mode=prefix_mode, qblock=qblock, idx=_p(idx),
                 logg=_p(logg), K=K, share_group=int(bool(share_group)), local=local, window=window,
                 alpha=_p(alpha), o=_p(o), lse=_p(lse))
    return a, (o, lse)


def sparse_attn_fwd(q, k, v, idx, logg, *, workspace=None, stream=None, **kw):
    """Exact softmax attention over the current block + selected blocks (or the
    routed-cell branch mixed with a window).  Returns (o, lse)."""
    a, outs = attn_args(q, k, v, idx, logg, **kw)
    buf, size = _ws(workspace, SPA_OP_ATTN_FWD, a, q.device)
    _check(lib().sparse_attn_fwd(ctypes.byref(a), _p(buf), size, _stream(stream)))
    return outs


def sparse_attn_bwd(q, k, v, idx, logg, o, dout, lse, *, dq=None, dk=None, dv=None, dg=None,
                    workspace=None, stream=None, **kw):
    """Backward of sparse_attn_fwd (current block + selected blocks with the log
    gate).  Returns (dq, dk, dv, dg)."""
    _contig(o, dout, lse, dq, dk, dv, dg)
    a, _ = attn_args(q, k, v, idx, logg, o=o, lse=lse, **kw)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dg is None:
        dg = torch.empty(idx.shape, dtype=torch.float32, device=q.device)
    buf, size = _ws(workspace, SPA_OP_ATTN_BWD, a, q.device)
    _check(lib().sparse_attn_bwd(ctypes.byref(a), _p(o), _p(dout), _p(lse), _p(dq), _p(dk), _p(dv),
                                 _p(dg), _p(buf), size, _stream(stream)))
    return dq, dk, dv, dg


def sparse_select_bwd(q, kbar, max_norm, centre, idx, logg, dg, *, dq=None, dkbar=None, dproj_w=None, dk=None,
                      workspace=None, stream=None, **kw):
    """Selector side of the backward: dg [B,Hsel,nq,K] (from sparse_attn_bwd)
    through log g = s - LSE(s) into q, kbar and (with proj_w) the projection;
    with dk [B,Hkv,L,d] given, dk += dkbar / b over each summarised block.
    Takes the arguments of the sparse_score_select call that produced idx /
    logg.  Returns (dq, dkbar, dproj_w), fp32 (dproj_w None without proj_w)."""
    _contig(dg, dq, dkbar, dproj_w, dk)
    a, _ = select_args(q, kbar, max_norm, centre, idx=idx, logg=logg, **kw)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dq is None else dq
    dkbar = torch.empty(kbar.shape, dtype=torch.float32, device=q.device) if dkbar is None else dkbar
    if dproj_w is None and kw.get("proj_w") is not None:
        d = q.shape[-1]
        dproj_w = torch.empty((d, d), dtype=torch.float32, device=q.device)
    g = SelectGrads(dg=_p(dg), dq=_p(dq), dkbar=_p(dkbar), dproj_w=_p(dproj_w), dk=_p(dk),
                    L=0 if dk is None else dk.shape[2])
    buf, size = _ws(workspace, SPA_OP_SELECT_BWD, a, q.device)
    _check(lib().sparse_select_bwd(ctypes.byref(a), ctypes.byref(g), _p(buf), size, _stream(stream)))
    return dq, dkbar, dproj_w


def sparse_decode_step(q, kbar, max_norm, centre, k, v, *, Hkv, b, K, q_pos0, gate=True, share_group=True,
                       proj_w=None, idx=None, logg=None, k_eff=None, o=None, lse=None, workspace=None,
                       stream=None, kbar_scale=None):
    """One decode step (nq = 1): score + gate + top-K over the summaries, then
    attention over the current block and the selected blocks.  Returns
    (idx, logg, k_eff, o, lse).  With kbar_scale the summaries are fp8 codes."""
    sa, (idx, logg, k_eff) = select_args(q, kbar, max_norm, centre, Hkv=Hkv, b=b, K=K, q_pos0=q_pos0, gate=gate,
                                         share_group=share_group, proj_w=proj_w, idx=idx, logg=logg,
                                         k_eff=k_eff, kbar_scale=kbar_scale)
    aa, (o, lse) = attn_args(q, k, v, idx, logg, b=b, K=K, q_pos0=q_pos0, share_group=share_group, o=o,
                             lse=lse)
    da = DecodeArgs(select=ctypes.pointer(sa), attn=ctypes.pointer(aa))
    buf, size = _ws(workspace, SPA_OP_DECODE_STEP, da, q.device)
    _check(lib().sparse_decode_step(ctypes.byref(da), _p(buf), size, _stream(stream)))
    return idx, logg, k_eff, o, lse


def sparse_decode_step_noalloc(q, kbar, max_norm, centre, k, v, *, Hkv, b, K, q_pos0, gate=True, share_group=True,
                               proj_w=None, idx=None, logg=None, k_eff=None, o=None, lse=None, stream=None,
                               kbar_scale=None):
    """sparse_decode_step with the library's own device scratch instead of a
    workspace (no device allocation by the library; outputs allocated here
    when not given).  Returns (idx, logg, k_eff, o, lse)."""
    sa, (idx, logg, k_eff) = select_args(q, kbar, max_norm, centre, Hkv=Hkv, b=b, K=K, q_pos0=q_pos0, gate=gate,
                                         share_group=share_group, proj_w=proj_w, idx=idx, logg=logg,
                                         k_eff=k_eff, kbar_scale=kbar_scale)
    aa, (o, lse) = attn_args(q, k, v, idx, logg, b=b, K=K, q_pos0=q_pos0, share_group=share_group, o=o,
                             lse=lse)
    da = DecodeArgs(select=ctypes.pointer(sa), attn=ctypes.pointer(aa))
    _check(lib().sparse_decode_step_noalloc(ctypes.byref(da), _stream(stream)))
    return idx, logg, k_eff, o, lse


def _pages(block_table, num_pages):
    return KvPages(block_table=_p(block_table), table_stride=block_table.shape[-1], num_pages=num_pages)


def sparse_block_summaries_paged(k_pages, block_table, L, b, first_block=0, num_blocks=None, ccap=None, kbar=None,
                                 max_norm=None, centre=None, stream=None):
    """sparse_block_summaries over a paged key cache: k_pages [num_pages, Hkv, b, d],
    block_table [B, table_stride] int32, L logical tokens per batch row."""
    _contig(k_pages, block_table, kbar, max_norm, centre)
    npages, Hkv, pb, d = k_pages.shape
    assert pb == b, "a page holds one block of b tokens"
    B = block_table.shape[0]
    if num_blocks is None:
        num_blocks = L // b - first_block
    if ccap is None:
        ccap = kbar.shape[2] if kbar is not None else first_block + num_blocks
    if kbar is None:
        kbar = torch.zeros((B, Hkv, ccap, d), dtype=k_pages.dtype, device=k_pages.device)
    if max_norm is None:
        max_norm = torch.zeros((B, Hkv, ccap), dtype=torch.float32, device=k_pages.device)
    if centre is None:
        centre = torch.zeros((ccap,), dtype=torch.float32, device=k_pages.device)
    pg = _pages(block_table, npages)
    _check(lib().sparse_block_summaries_paged(_p(k_pages), _dtype(k_pages), B, Hkv, L, d, b, ctypes.byref(pg),
                                              first_block, num_blocks, ccap, _p(kbar), _p(max_norm), _p(centre),
                                              _stream(stream)))
    return kbar, max_norm, centre


def sparse_decode_step_paged(q, kbar, max_norm, centre, k_pages, v_pages, block_table, L, *, Hkv, b, K, q_pos0,
                             gate=True, share_group=True, proj_w=None, idx=None, logg=None, k_eff=None, o=None,
                             lse=None, workspace=None, stream=None):
    """sparse_decode_step over a paged cache (pools [num_pages, Hkv, b, d],
    block_table [B, table_stride] int32, L logical tokens).  Returns
    (idx, logg, k_eff, o, lse)."""
    _contig(k_pages, v_pages, block_table)
    sa, (idx, logg, k_eff) = select_args(q, kbar, max_norm, centre, Hkv=Hkv, b=b, K=K, q_pos0=q_pos0, gate=gate,
                                         share_group=share_group, proj_w=proj_w, idx=idx, logg=logg,
                                         k_eff=k_eff)
    aa, (o, lse) = attn_args(q, k_pages, v_pages, idx, logg, b=b, K=K, q_pos0=q_pos0, share_group=share_group,
                             o=o, lse=lse)
    aa.L = L
    da = DecodeArgs(select=ctypes.pointer(sa), attn=ctypes.pointer(aa))
    pg = _pages(block_table, k_pages.shape[0])
    buf, size = _ws(workspace, SPA_OP_DECODE_STEP, da, q.device)
    _check(lib().sparse_decode_step_paged(ctypes.byref(da), ctypes.byref(pg), _p(buf), size, _stream(stream)))
    return idx, logg, k_eff, o, lse


def sparse_retain_cells(max_norm, ncand, W, P, cells=None, count=None, stream=None):
    """FS-L kept set of every (batch, kv head) from max_norm [B, Hkv, ccap]:
    the W most recent of the ncand prefix cells plus the P older cells of
    largest max key norm.  Returns (cells [B, Hkv, W + P] int32, count [B, Hkv])."""
    _contig(max_norm, cells, count)
    B, Hkv, ccap = max_norm.shape
    if cells is None:
        cells = torch.empty((B, Hkv, W + P), dtype=torch.int32, device=max_norm.device)
    if count is None:
        count = torch.empty((B, Hkv), dtype=torch.int32, device=max_norm.device)
    _check(lib().sparse_retain_cells(_p(max_norm), B, Hkv, ccap, ncand, W, P, _p(cells), _p(count),
                                     _stream(stream)))
    return cells, count


def sparse_score_select_subset(q, kbar, max_norm, centre, cells, count, *, stream=None, **kw):
    """sparse_score_select restricted to the kept cells (cells, count from
    sparse_retain_cells).  Returns (idx, logg or None, k_eff)."""
    _contig(cells, count)
    a, outs = select_args(q, kbar, max_norm, centre, **kw)
    _check(lib().sparse_score_select_subset(ctypes.byref(a), _p(cells), _p(count), cells.shape[-1],
                                            _stream(stream)))
    return outs


def sparse_forest_build(kbar, max_norm, centre, n, forest=None, workspace=None, stream=None):
    """FS-B forests of every (batch, kv head) over the n prefix cells (summaries
    as sparse_block_summaries writes them).  Returns a dict of the forest arrays
    (members, nmem, mu, rad, amax, pmin); node arrays get one zero slot when a
    forest has no internal node (n <= 16)."""
    _contig(kbar, max_norm, centre)
    B, Hkv, ccap, d = kbar.shape
    NN = max(int(lib().sparse_forest_nodes(n)), 1)
    dev_ = kbar.device
    if forest is None:
        forest = dict(members=torch.empty((B, Hkv, 2, n), dtype=torch.int32, device=dev_),
                      nmem=torch.empty((B, Hkv, 2), dtype=torch.int32, device=dev_),
                      mu=torch.zeros((B, Hkv, 2, NN, d), dtype=torch.float32, device=dev_),
                      rad=torch.zeros((B, Hkv, 2, NN), dtype=torch.float32, device=dev_),
                      amax=torch.zeros((B, Hkv, 2, NN), dtype=torch.float32, device=dev_),
                      pmin=torch.zeros((B, Hkv, 2, NN), dtype=torch.float32, device=dev_))
    fo = Forest(**{k: _p(v) for k, v in forest.items()})
    need = lib().sparse_forest_workspace_bytes(B, Hkv, d, n)
    if workspace is None:
        workspace = _default_ws.setdefault((str(dev_), "forest"), Workspace(dev_))
    buf, size = workspace.get(need)
    _check(lib().sparse_forest_build(_p(kbar), _dtype(kbar), _p(max_norm), _p(centre), B, Hkv, d, ccap, n,
                                     ctypes.byref(fo), _p(buf), size, _stream(stream)))
    return forest


def sparse_forest_select(q, kbar, max_norm, centre, k, forest, n, *, stream=None, **kw):
    """Per-query top K cells by the beam search of both forests and the
    logsumexp re-rank over the token keys k [B, Hkv, L, d].  Returns
    (idx, k_eff)."""
    kw.setdefault("gate", False)
    a, (idx, _, k_eff) = select_args(q, kbar, max_norm, centre, **kw)
    fo = Forest(**{key: _p(v) for key, v in forest.items()})
    _check(lib().sparse_forest_select(ctypes.byref(a), _p(k), k.shape[2], ctypes.byref(fo), n, _stream(stream)))
    return idx, k_eff


def sparse_probe_load_chase(next_idx, steps, start=0, out=None, stream=None):
    """Measurement aid: one lane follows the cyclic index list next_idx (int32
    on the device, length a power of two) for `steps` dependent loads; time
    the call with events for the memory level's round-trip latency.  Returns
    out (one int32: the last index)."""
    if out is None:
        out = torch.empty(1, dtype=torch.int32, device=next_idx.device)
    _check(lib().sparse_probe_load_chase(_p(next_idx), next_idx.numel(), steps, start, _p(out), _stream(stream)))
    return out

