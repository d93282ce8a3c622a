"""Plain fp64 CPU oracle for block-sparse causal attention with learned block
selection: summaries -> scores -> softmax log gate -> top-K -> exact softmax
attention -> backward with the log-gate gradient.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library (``block_sparse_attention_summaries_amd``); the only thing
both sides use is the seeded input generator module, which holds none of the
method's arithmetic.

The arithmetic lives in ``oracle.c`` (plain loops, fp64); this module only
compiles it with gcc and marshals numpy arrays through ctypes.  Every function
cites the page passage it follows in ``oracle.c``.

Parity pins (see ``tests/test_oracle_pins.py``): the SAS worked example, dense
causal attention via torch's SDPA when every block is selected, an
independently built dense block mask (gate == 1), brute-force subset
enumeration, central finite differences and torch autograd for the backward,
the FreeSolo reductions (lambda = 0, alpha in {0, 1}), and summary identities.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


P = ctypes.c_void_p
I = ctypes.c_int
I64 = ctypes.c_int64


def _declare(lib):
    lib.orc_round_bf16.argtypes = [ctypes.c_double]
    lib.orc_round_bf16.restype = ctypes.c_uint16
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = I
    lib.orc_block_summaries.argtypes = [P, I, I, I, I64, I, I, I64, I64, P, P, P]
    lib.orc_block_summaries.restype = None
    lib.orc_fp8_decode.argtypes = [ctypes.c_uint8]
    lib.orc_fp8_decode.restype = ctypes.c_double
    lib.orc_fp8_encode.argtypes = [ctypes.c_float]
    lib.orc_fp8_encode.restype = ctypes.c_uint8
    lib.orc_quantize_fp8.argtypes = [P, I, I, I, I64, I, I64, I64, P, P]
    lib.orc_quantize_fp8.restype = None
    lib.orc_dequantize_fp8.argtypes = [P, P, I64, I, P]
    lib.orc_dequantize_fp8.restype = None
    lib.orc_num_candidates.argtypes = [I64, I, I, I]
    lib.orc_num_candidates.restype = I64
    lib.orc_select_from_scores.argtypes = [P, I64, I, I, P, P, P, P]
    lib.orc_select_from_scores.restype = I
    lib.orc_score_select.argtypes = [P, I, I, I, I, I, I, I64, P, I, P, P, I64, I, I, I, I,
                                     P, P, P, I, I, P, I64, P, P, P, P, P]
    lib.orc_score_select.restype = None
    lib.orc_scores_one_row.argtypes = [P, I, I, I, I, I, I, I64, P, I, P, P, I64, I, I, I, I,
                                       P, P, P, I, I, I64, P]
    lib.orc_scores_one_row.restype = None
    lib.orc_attn_fwd.argtypes = [P, P, P, I, I, I, I, I, I, I64, I64, I, I, I, P, P, I, I, I, I,
                                 P, P, I64, P, P]
    lib.orc_attn_fwd.restype = None
    lib.orc_retain_cells.restype = None
    lib.orc_retain_cells.argtypes = [P, I, I, I64, I64, I, I, P, P]
    lib.orc_score_select_subset.restype = None
    lib.orc_score_select_subset.argtypes = [P, I, I, I, I, I, I, I64, P, I, P, P, I64, I, I, I, I, P, P, P, P,
                                            I, I, I, P, P, P, P]
    lib.orc_forest_nodes.restype = I64
    lib.orc_forest_nodes.argtypes = [I64, I]
    lib.orc_forest_build.restype = None
    lib.orc_forest_build.argtypes = [P, I, P, P, I, I, I, I64, I64, I, P, P, P, P, P, P]
    lib.orc_forest_select.restype = None
    lib.orc_forest_select.argtypes = [P, I, I, I, I, I, I, I64, P, I, P, P, I64, P, I64, I, I, P, P, P, P, P, P,
                                      P, P, I64, I, I, I, P, P]
    lib.orc_node_score.restype = ctypes.c_double
    lib.orc_node_score.argtypes = [P, ctypes.c_double, P, ctypes.c_float, ctypes.c_float, ctypes.c_float, I,
                                   ctypes.c_double, ctypes.c_double, ctypes.c_double, I]
    lib.orc_select_bwd.restype = None
    lib.orc_select_bwd.argtypes = [P, I, I, I, I, I, I, I64, P, I, I64, I, I, I, P, P, P, P, P, P]
    lib.orc_attn_bwd.argtypes = [P, P, P, P, I, I, I, I, I, I, I64, I64, I, P, P, I, I, I64,
                                 P, P, P, P]
    lib.orc_attn_bwd.restype = None
    lib.orc_cell_token_lse.restype = None
    lib.orc_cell_token_lse.argtypes = [P, I, I, I, I, I, I, P, I, I64, I, I, I, I, I64, I64, P]


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle takes float32, float64 or bf16 bit patterns (uint16), got {a.dtype}")


def num_threads() -> int:
    return int(_load().orc_num_threads())


def round_bf16(x: float) -> int:
    """bf16 bit pattern of x rounded to nearest even (the oracle's rounding)."""
    return int(_load().orc_round_bf16(float(x)))


def num_candidates(i: int, b: int, prefix_mode: int = 0, qblock: int = 128) -> int:
    return int(_load().orc_num_candidates(int(i), int(b), int(prefix_mode), int(qblock)))


def block_summaries(k: np.ndarray, b: int, nblocks: int | None = None, ccap: int | None = None):
    """k [B, Hkv, L, d] (float32 or bf16 bits) -> kbar [B,Hkv,ccap,d] (same dtype),
    max_norm [B,Hkv,ccap] fp32, centre [ccap] fp32."""
    lib = _load()
    B, Hkv, L, d = k.shape
    if nblocks is None:
        nblocks = L // b
    if ccap is None:
        ccap = nblocks
    kbar = np.zeros((B, Hkv, ccap, d), dtype=k.dtype)
    mx = np.zeros((B, Hkv, ccap), dtype=np.float32)
    centre = np.zeros((ccap,), dtype=np.float32)
    lib.orc_block_summaries(_ptr(k), _dtype_code(k), B, Hkv, L, d, b, nblocks, ccap,
                            _ptr(kbar), _ptr(mx), _ptr(centre))
    return kbar, mx, centre


def fp8_decode(code: int) -> float:
    """Value of one OCP E4M3 code (NaN for S.1111.111)."""
    return float(_load().orc_fp8_decode(int(code)))


def fp8_encode(y: float) -> int:
    """Nearest E4M3 code to the fp32 value y (ties to the even code, held at
    +-448, sign kept)."""
    return int(_load().orc_fp8_encode(float(np.float32(y))))


def quantize_fp8(kbar: np.ndarray, first: int = 0, num: int | None = None):
    """fp8 block summaries: kbar [B, Hkv, ccap, d] (float32 or bf16 bits) ->
    codes [B, Hkv, ccap, d] uint8, scales [B, Hkv, ccap] fp32 for blocks
    [first, first + num) (zeros elsewhere): per block scale = amax / 448, codes
    = E4M3(kbar * (448 / amax)), single-precision scale arithmetic."""
    lib = _load()
    B, Hkv, ccap, d = kbar.shape
    if num is None:
        num = ccap - first
    kbar = np.ascontiguousarray(kbar)
    codes = np.zeros((B, Hkv, ccap, d), np.uint8)
    scales = np.zeros((B, Hkv, ccap), np.float32)
    lib.orc_quantize_fp8(_ptr(kbar), _dtype_code(kbar), B, Hkv, ccap, d, int(first), int(num),
                         _ptr(codes), _ptr(scales))
    return codes, scales


def dequantize_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The summaries the scorer reads, exact in fp64: scale_c * decode(code)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    out = np.zeros(codes.shape, np.float64)
    d = codes.shape[-1]
    _load().orc_dequantize_fp8(_ptr(codes), _ptr(scales), codes.size // d, d, _ptr(out))
    return out


def select_from_scores(s, K: int, gate: bool = True):
    """Top-K + softmax log gate of one score vector.  Returns
    (idx[K] int32 ascending, -1 padded; logg[K]; k_eff; gap; lse)."""
    lib = _load()
    s = np.ascontiguousarray(np.asarray(s, dtype=np.float64))
    idx = np.zeros((K,), np.int32)
    logg = np.zeros((K,), np.float64)
    gap = ctypes.c_double(0.0)
    lse = ctypes.c_double(0.0)
    ke = lib.orc_select_from_scores(_ptr(s), s.shape[0], K, int(bool(gate)), _ptr(idx),
                                    _ptr(logg), ctypes.byref(gap), ctypes.byref(lse))
    return idx, logg, int(ke), gap.value, lse.value


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def score_select(q, kbar, max_norm, centre, *, Hkv, b, K, q_pos0, gate=True,
                 prefix_mode=0, qblock=128, share_group=True, proj_w=None,
                 erf_lambda=None, erf_sigma=None, rows=None):
    """Scores + gate + top-K for query rows of q [B, Hq, nq, d].
    Returns dict(idx [B,Hsel,nq,K] int32, logg fp64, k_eff int32, gap fp64,
    lse fp64 [B,Hsel,nq]).  With ``rows`` only those rows are filled."""
    lib = _load()
    B, Hq, nq, d = q.shape
    ccap = kbar.shape[2]
    Hsel = Hkv if share_group else Hq
    idx = np.full((B, Hsel, nq, K), -1, np.int32)
    logg = np.zeros((B, Hsel, nq, K), np.float64)
    keff = np.zeros((B, Hsel, nq), np.int32)
    gap = np.zeros((B, Hsel, nq), np.float64)
    lse = np.zeros((B, Hsel, nq), np.float64)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    max_norm = _f32(max_norm)
    centre = _f32(centre)
    proj_w, erf_lambda, erf_sigma = _f32(proj_w), _f32(erf_lambda), _f32(erf_sigma)
    lib.orc_score_select(_ptr(q), _dtype_code(q), B, Hq, Hkv, nq, d, int(q_pos0), _ptr(kbar),
                         _dtype_code(kbar), _ptr(max_norm), _ptr(centre), ccap, b,
                         int(prefix_mode), int(qblock), int(bool(share_group)), _ptr(proj_w),
                         _ptr(erf_lambda), _ptr(erf_sigma), K, int(bool(gate)), _ptr(rows_a),
                         0 if rows_a is None else rows_a.shape[0], _ptr(idx), _ptr(logg),
                         _ptr(keff), _ptr(gap), _ptr(lse))
    return dict(idx=idx, logg=logg, k_eff=keff, gap=gap, lse=lse)


def scores_one_row(q, kbar, max_norm, centre, *, Hkv, b, q_pos0, bidx, hs, row,
                   prefix_mode=0, qblock=128, share_group=True, proj_w=None,
                   erf_lambda=None, erf_sigma=None):
    """Full candidate score vector (fp64) of one row and one selection head."""
    lib = _load()
    B, Hq, nq, d = q.shape
    ccap = kbar.shape[2]
    ncand = num_candidates(q_pos0 + row, b, prefix_mode, qblock)
    s = np.zeros((max(ncand, 1),), np.float64)
    max_norm = _f32(max_norm)
    centre = _f32(centre)
    proj_w, erf_lambda, erf_sigma = _f32(proj_w), _f32(erf_lambda), _f32(erf_sigma)
    lib.orc_scores_one_row(_ptr(q), _dtype_code(q), B, Hq, Hkv, nq, d, int(q_pos0), _ptr(kbar),
                           _dtype_code(kbar), _ptr(max_norm), _ptr(centre), ccap, b,
                           int(prefix_mode), int(qblock), int(bool(share_group)), _ptr(proj_w),
                           _ptr(erf_lambda), _ptr(erf_sigma), int(bidx), int(hs), int(row),
                           _ptr(s))
    return s[:ncand]


def attn_fwd(q, k, v, idx, logg, *, b, K, q_pos0, share_group=True, local=0,
             window=0, alpha=None, prefix_mode=0, qblock=128, rows=None):
    """Exact softmax attention over the kept keys.  local 0 = current block kept,
    1 = none; window/alpha select the two-branch mix.  Returns (o fp64
    [B,Hq,nq,d], lse fp64 [B,Hq,nq]); with ``rows`` only those rows are filled."""
    lib = _load()
    B, Hq, nq, d = q.shape
    _, Hkv, L, _ = k.shape
    assert k.dtype == q.dtype == v.dtype
    o = np.zeros((B, Hq, nq, d), np.float64)
    lse = np.zeros((B, Hq, nq), np.float64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    logg_a = None if logg is None else np.ascontiguousarray(logg, dtype=np.float64)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    alpha = _f32(alpha)
    lib.orc_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, nq, d, L,
                     int(q_pos0), b, int(prefix_mode), int(qblock), _ptr(idx), _ptr(logg_a),
                     K, int(bool(share_group)), int(local), int(window), _ptr(alpha),
                     _ptr(rows_a), 0 if rows_a is None else rows_a.shape[0], _ptr(o), _ptr(lse))
    return o, lse


def attn_bwd(q, k, v, dout, idx, logg, *, b, K, q_pos0, share_group=True, kv_slice=-1):
    """Backward of the current-block + selected-blocks attention with the log
    gate.  Returns (dq, dk, dv, dg) in fp64; dg [B, Hsel, nq, K].  kv_slice
    (= batch*Hkv + kv_head) restricts the work to one (batch, kv head) pair."""
    lib = _load()
    B, Hq, nq, d = q.shape
    _, Hkv, L, _ = k.shape
    Hsel = Hkv if share_group else Hq
    dq = np.zeros((B, Hq, nq, d), np.float64)
    dk = np.zeros((B, Hkv, L, d), np.float64)
    dv = np.zeros((B, Hkv, L, d), np.float64)
    dg = np.zeros((B, Hsel, nq, K), np.float64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    logg_a = None if logg is None else np.ascontiguousarray(logg, dtype=np.float64)
    lib.orc_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _dtype_code(q), B, Hq, Hkv, nq, d,
                     L, int(q_pos0), b, _ptr(idx), _ptr(logg_a), K, int(bool(share_group)),
                     int(kv_slice), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg))
    return dq, dk, dv, dg


def retain_cells(max_norm, *, ncand, W, P):
    """FS-L kept set per (batch, kv head): the W most recent of the ncand prefix
    cells plus the P older cells of largest max key norm.  Returns (cells
    [B, Hkv, W + P] ascending, -1 padded; count [B, Hkv])."""
    lib = _load()
    mx = _f32(max_norm)
    B, Hkv, ccap = mx.shape
    cells = np.full((B, Hkv, W + P), -1, np.int32)
    count = np.zeros((B, Hkv), np.int32)
    lib.orc_retain_cells(_ptr(mx), B, Hkv, ccap, int(ncand), int(W), int(P), _ptr(cells), _ptr(count))
    return cells, count


def score_select_subset(q, kbar, max_norm, centre, cells, count, *, Hkv, b, K, q_pos0, gate=True,
                        prefix_mode=0, qblock=128, share_group=True, erf_lambda=None, erf_sigma=None):
    """score_select restricted to the kept cells of each kv head (cells, count
    as retain_cells returns them).  Returns dict(idx, logg, k_eff, gap)."""
    lib = _load()
    B, Hq, nq, d = q.shape
    ccap = kbar.shape[2]
    Hsel = Hkv if share_group else Hq
    cells = np.ascontiguousarray(cells, dtype=np.int32)
    count = np.ascontiguousarray(count, dtype=np.int32)
    idx = np.full((B, Hsel, nq, K), -1, np.int32)
    logg = np.zeros((B, Hsel, nq, K), np.float64)
    keff = np.zeros((B, Hsel, nq), np.int32)
    gap = np.zeros((B, Hsel, nq), np.float64)
    max_norm, centre = _f32(max_norm), _f32(centre)
    erf_lambda, erf_sigma = _f32(erf_lambda), _f32(erf_sigma)
    lib.orc_score_select_subset(_ptr(q), _dtype_code(q), B, Hq, Hkv, nq, d, int(q_pos0), _ptr(kbar),
                                _dtype_code(kbar), _ptr(max_norm), _ptr(centre), ccap, b, int(prefix_mode),
                                int(qblock), int(bool(share_group)), _ptr(erf_lambda), _ptr(erf_sigma),
                                _ptr(cells), _ptr(count), cells.shape[-1], K, int(bool(gate)), _ptr(idx),
                                _ptr(logg), _ptr(keff), _ptr(gap))
    return dict(idx=idx, logg=logg, k_eff=keff, gap=gap)


FOREST_FANOUT = 16
FOREST_BEAM = 16


def forest_nodes(n, F=FOREST_FANOUT):
    """Internal nodes of a forest over n member cells."""
    return int(_load().orc_forest_nodes(int(n), int(F)))


def forest_build(kbar, max_norm, centre, n, F=FOREST_FANOUT):
    """FS-B forests of every (batch, kv head) over the n prefix cells: the
    whole prefix (forest 0) and the cells at or above the median max norm
    (forest 1).  Returns dict(members [B,Hkv,2,n] int32 (-1 padded), nmem
    [B,Hkv,2], mu [B,Hkv,2,NN,d] fp32, rad / amax / pmin [B,Hkv,2,NN] fp32)."""
    lib = _load()
    B, Hkv, ccap, d = kbar.shape
    NN = forest_nodes(n, F)
    out = dict(members=np.full((B, Hkv, 2, max(n, 1)), -1, np.int32), nmem=np.zeros((B, Hkv, 2), np.int32),
               mu=np.zeros((B, Hkv, 2, max(NN, 1), d), np.float32), rad=np.zeros((B, Hkv, 2, max(NN, 1)), np.float32),
               amax=np.zeros((B, Hkv, 2, max(NN, 1)), np.float32), pmin=np.zeros((B, Hkv, 2, max(NN, 1)), np.float32))
    mx, ce = _f32(max_norm), _f32(centre)
    lib.orc_forest_build(_ptr(kbar), _dtype_code(kbar), _ptr(mx), _ptr(ce), B, Hkv, d, ccap, int(n), int(F),
                         _ptr(out["members"]), _ptr(out["nmem"]), _ptr(out["mu"]), _ptr(out["rad"]),
                         _ptr(out["amax"]), _ptr(out["pmin"]))
    return out


def forest_select(q, kbar, max_norm, centre, k, forest, n, *, Hkv, b, K, q_pos0, share_group=False,
                  erf_lambda=None, erf_sigma=None, F=FOREST_FANOUT, Wb=FOREST_BEAM):
    """Beam search of both forests, then the logsumexp re-rank over token keys
    of the reached cells; top K ascending.  Returns dict(idx, gap) with gap the
    smallest score margin at any cut (beam levels and the final top K)."""
    assert F <= 16 and Wb <= 16
    lib = _load()
    B, Hq, nq, d = q.shape
    ccap = kbar.shape[2]
    L = k.shape[2]
    Hsel = Hkv if share_group else Hq
    idx = np.full((B, Hsel, nq, K), -1, np.int32)
    gap = np.zeros((B, Hsel, nq), np.float64)
    mx, ce = _f32(max_norm), _f32(centre)
    lam, sig = _f32(erf_lambda), _f32(erf_sigma)
    f = {key: np.ascontiguousarray(v) for key, v in forest.items()}
    lib.orc_forest_select(_ptr(q), _dtype_code(q), B, Hq, Hkv, nq, d, int(q_pos0), _ptr(kbar), _dtype_code(kbar),
                          _ptr(mx), _ptr(ce), ccap, _ptr(k), L, b, int(bool(share_group)), _ptr(lam), _ptr(sig),
                          _ptr(f["members"]), _ptr(f["nmem"]), _ptr(f["mu"]), _ptr(f["rad"]), _ptr(f["amax"]),
                          _ptr(f["pmin"]), int(n), int(F), int(Wb), K, _ptr(idx), _ptr(gap))
    return dict(idx=idx, gap=gap)


def cell_token_lse(q, k, *, Hkv, b, bidx, hs, row, ncells, share_group=False):
    """Re-rank score of cells 0..ncells-1 for one row and selection head: the
    logsumexp over each cell's b token keys of qhat.k/sqrt(d) (fp64)."""
    lib = _load()
    B, Hq, nq, d = q.shape
    L = k.shape[2]
    assert k.dtype == q.dtype and ncells * b <= L
    out = np.zeros((max(int(ncells), 1),), np.float64)
    lib.orc_cell_token_lse(_ptr(q), _dtype_code(q), B, Hq, Hkv, nq, d, _ptr(k), _dtype_code(k), L, b,
                           int(bool(share_group)), int(bidx), int(hs), int(row), int(ncells), _ptr(out))
    return out[:ncells]


def node_score(q_hat, mu, rad, amax, pmin, *, lam, sig, pos, with_erf=True):
    """U of one node for one query vector q_hat (fp64)."""
    qh = np.ascontiguousarray(q_hat, dtype=np.float64)
    m = np.ascontiguousarray(mu, dtype=np.float32)
    return float(_load().orc_node_score(_ptr(qh), float(np.sqrt((qh * qh).sum())), _ptr(m), float(rad),
                                        float(amax), float(pmin), qh.shape[0], float(lam), float(sig),
                                        float(pos), int(bool(with_erf))))


def select_bwd(q, kbar, idx, dg, *, Hkv, b, K, q_pos0, share_group=True, proj_w=None):
    """Selector-side backward: the gate gradient dg [B, Hsel, nq, K] (w.r.t. g)
    through log g = s - LSE(s) into q (dq [B, Hq, nq, d]) and the block
    summaries (dkbar [B, Hkv, ccap, d]), fp64.  Current-block candidates, no
    erf term.  With the projection proj_w [d, d] (fp32, ktilde = W kbar) also
    returns dW [d, d]: (dq, dkbar, dW)."""
    lib = _load()
    B, Hq, nq, d = q.shape
    ccap = kbar.shape[2]
    dq = np.zeros((B, Hq, nq, d), np.float64)
    dkbar = np.zeros((B, Hkv, ccap, d), np.float64)
    dW = np.zeros((d, d), np.float64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    dg = np.ascontiguousarray(dg, dtype=np.float64)
    W = None if proj_w is None else np.ascontiguousarray(proj_w, dtype=np.float32)
    lib.orc_select_bwd(_ptr(q), _dtype_code(q), B, Hq, Hkv, nq, d, int(q_pos0), _ptr(kbar),
                       _dtype_code(kbar), ccap, b, int(bool(share_group)), K, _ptr(W), _ptr(idx),
                       _ptr(dg), _ptr(dq), _ptr(dkbar), _ptr(dW))
    if W is None:
        return dq, dkbar
    return dq, dkbar, dW


def mean_bwd(dkbar, b, L):
    """Gradient of the block mean kbar_c = (1/b) sum_{j in block c} k_j with
    respect to the keys ([SAS] §3, the mean-key summary): dk_j = dkbar_c / b
    for each token j of block c < ccap, 0 for tokens past ccap * b.  fp64
    [B, Hkv, L, d].  The rounding of kbar to the key dtype is passed straight
    through."""
    B, Hkv, ccap, d = dkbar.shape
    assert ccap * b <= L
    dk = np.zeros((B, Hkv, L, d), np.float64)
    for c in range(ccap):
        dk[:, :, c * b:(c + 1) * b, :] = np.asarray(dkbar[:, :, c:c + 1, :], np.float64) / b
    return dk
