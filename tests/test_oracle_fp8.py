"""Pins of the oracle's fp8 block summaries (OCP 8-bit floating point, E4M3
with no infinities; per-block scale amax / 448).

- Decode of all 256 codes against torch's float8_e4m3fn (an independent
  library implementation of the same format), NaN codes included.
- Encode (nearest, ties to the even code) against torch's conversion for
  every magnitude below the first overflow midpoint (464), on random values,
  every representable value and every midpoint between neighbours; values at
  or past 448 are held at 448 (torch gives NaN past 464, the scale rule never
  reaches it).
- Quantization: the largest magnitude of a block maps to code +-448, zero
  blocks give scale 0 and zero codes, and the rebuilt summary is within half
  a step of the input (relative 2^-4 for normal codes, 2^-10 scale absolute
  for subnormal ones).
- The scorer's fp64 loader: fp32 summaries passed as fp64 score identically."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_match_torch():
    got = np.array([oracle.fp8_decode(c) for c in range(256)])
    want = _torch_decode(np.arange(256))
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


def _finite_values():
    v = np.array([oracle.fp8_decode(c) for c in range(0x7F)])
    assert np.all(np.diff(v) > 0)               # strictly increasing over the finite codes
    return v


def test_encode_matches_torch_below_overflow():
    v = _finite_values()
    mids = (v[:-1] + v[1:]) / 2                  # exact in fp32: neighbours differ in <= 5 bits
    rng = np.random.default_rng(7)
    rnd = np.concatenate([rng.uniform(0, 464, 3000), np.exp(rng.uniform(np.log(1e-4), np.log(463.9), 3000))])
    ys = np.concatenate([v, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                         np.nextafter(mids.astype(np.float32), np.float32(np.inf)), rnd]).astype(np.float32)
    ys = ys[ys < 464]
    ys = np.concatenate([ys, -ys])
    got = np.array([oracle.fp8_encode(y) for y in ys], np.uint8)
    assert np.array_equal(got, _torch_encode(ys))


@pytest.mark.parametrize("y,code", [(448.0, 0x7E), (455.9, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (-600.0, 0xFE),
                                    (-0.0, 0x80), (-2.0 ** -11, 0x80), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02)])
def test_encode_saturation_and_signed_zero(y, code):
    assert oracle.fp8_encode(y) == code


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_scale_rule_and_error_bound(dtype):
    rng = np.random.default_rng(11)
    kb = (rng.standard_normal((2, 3, 9, 64)) * np.exp(rng.uniform(-6, 3, (2, 3, 9, 1)))).astype(np.float32)
    kb[0, 1, 4] = 0.0                            # a zero block
    kb[1, 2, 7, 5] = -kb[1, 2, 7].__abs__().max() * 2   # negative largest magnitude
    if dtype == "bf16":
        kb = np.array([oracle.round_bf16(float(x)) for x in kb.ravel()], np.uint16).reshape(kb.shape)
        kf = (kb.astype(np.uint32) << 16).view(np.float32)
    else:
        kf = kb
    codes, scales = oracle.quantize_fp8(kb, first=1, num=7)
    assert np.all(codes[:, :, [0, 8]] == 0) and np.all(scales[:, :, [0, 8]] == 0)
    assert scales[0, 1, 4] == 0 and np.all(codes[0, 1, 4] == 0)
    amax = np.abs(kf).max(axis=-1)
    live = (amax > 0)
    live[:, :, [0, 8]] = False
    assert np.array_equal(scales[live], (amax[live] / np.float32(448)).astype(np.float32))
    # the largest magnitude of each block is +-448
    arg = np.abs(kf).argmax(axis=-1)
    top = np.take_along_axis(codes, arg[..., None], -1)[..., 0]
    assert np.all((top[live] & 0x7F) == 0x7E)
    assert np.all((top[live] >> 7) == (np.take_along_axis(kf, arg[..., None], -1)[..., 0][live] < 0))
    deq = oracle.dequantize_fp8(codes, scales)
    x = kf.astype(np.float64)
    err = np.abs(deq - x)
    s = scales.astype(np.float64)[..., None]
    normal = np.abs(deq) >= s * 2.0 ** -6
    # half a step in the scaled domain, plus |x| |scale * inv - 1| (two single-precision roundings)
    bound = np.where(normal, 2.0 ** -4 * np.abs(x), 2.0 ** -10 * s) + 2.0 ** -21 * np.abs(x)
    assert np.all(err[live] <= bound[live])


def test_fp64_summaries_score_like_fp32():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, nq, d, b, K = 1, 4, 2, 3, 64, 64, 4
    q = rng.standard_normal((B, Hq, nq, d)).astype(np.float32)
    kb = rng.standard_normal((B, Hkv, 20, d)).astype(np.float32)
    kw = dict(Hkv=Hkv, b=b, K=K, q_pos0=20 * b - 1, gate=True, share_group=True)
    a = oracle.score_select(q, kb, None, None, **kw)
    c = oracle.score_select(q, kb.astype(np.float64), None, None, **kw)
    assert np.array_equal(a["idx"], c["idx"]) and np.array_equal(a["logg"], c["logg"])
