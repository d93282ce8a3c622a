// spa_device.h -- device helpers shared by the gfx950 kernels of libsparse_attn:
// element decoding, rounding, orderable score keys and wave-level (64 lane)
// bitonic networks.  Device code only; no host logic lives here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spa {

constexpr int kWave = 64;  // CDNA wavefront width

// ------------------------------------------------------------- element types
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_float(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// fp64 -> bf16, round to nearest even, without double rounding: first round
// the double to fp32 with round-to-odd (truncate, then set the sticky bit if
// anything was cut), which keeps enough bits (24 >= 8 + 2) for the second,
// nearest-even rounding to 8 significant bits to be exact (Boldo & Melquiond,
// "Emulation of FMA and correctly rounded sums: proved algorithms using
// rounding to odd", 2008).
__device__ __forceinline__ uint16_t double_to_bf16_rne(double x) {
  float t = __double2float_rz(x);
  uint32_t u = __float_as_uint(t);
  if (static_cast<double>(t) != x) u |= 1u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte load
  __device__ __forceinline__ static float to_float(float x) { return x; }
  __device__ __forceinline__ static float from_float(float x) { return x; }
  __device__ __forceinline__ static float from_double(double x) { return __double2float_rn(x); }
  // unpack a 16-byte vector into kVec floats
  __device__ __forceinline__ static void unpack(const uint4& v, float* out) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  }
};

template <>
struct Elem<bf16_t> {
  static constexpr int kVec = 8;
  __device__ __forceinline__ static float to_float(bf16_t x) { return bf16_to_float(x.bits); }
  __device__ __forceinline__ static bf16_t from_float(float x) { return bf16_t{float_to_bf16_rne(x)}; }
  __device__ __forceinline__ static bf16_t from_double(double x) { return bf16_t{double_to_bf16_rne(x)}; }
  __device__ __forceinline__ static void unpack(const uint4& v, float* out) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

template <typename T>
__device__ __forceinline__ float ld_f(const T* p) {
  return Elem<T>::to_float(*p);
}

// ------------------------------------------------------- XCD-aware order
// Dispatch places workgroup w (linear, x fastest) on XCD w % 8, and each XCD
// has its own L2.  Renumbering w so that XCD x runs one contiguous range of
// logical workgroups (x per + min(x, rem) onward) lets neighbouring tiles,
// which read the same keys, share that L2.  A bijection of [0, total).
__device__ __forceinline__ uint32_t xcd_swizzle(uint32_t w, uint32_t total) {
  constexpr uint32_t kXcds = 8;
  const uint32_t per = total / kXcds, rem = total % kXcds;
  const uint32_t x = w % kXcds, s = w / kXcds;
  return x * per + (x < rem ? x : rem) + s;
}

// (blockIdx.x, blockIdx.y) of this workgroup's logical position under xcd_swizzle.
__device__ __forceinline__ uint2 xcd_block_xy() {
  const uint32_t w = blockIdx.y * gridDim.x + blockIdx.x;
  const uint32_t l = xcd_swizzle(w, gridDim.x * gridDim.y);
  return make_uint2(l % gridDim.x, l / gridDim.x);
}

// As xcd_block_xy with x counted from the last: where x is a causal row tile
// (work growing with x), every XCD starts on its longest tiles.
__device__ __forceinline__ uint2 xcd_block_xy_last_first() {
  const uint2 v = xcd_block_xy();
  return make_uint2(gridDim.x - 1 - v.x, v.y);
}

// ------------------------------------------------------- fp8 summaries
// OCP 8-bit floating point, E4M3 without infinities: sign, 4 exponent bits
// biased by 7, 3 mantissa bits; exponent field 0 holds m/8 2^-6; S.1111.111
// is NaN, so 448 = 1.75 2^8 is the largest finite magnitude.
//
// Nearest code to y, ties to the even code, magnitudes at or past 448 held
// at 448, the sign kept.  A normal magnitude a in [2^e, 2^(e+1)) has quantum
// 2^(e-3): a 2^(3-e) lies in [8, 16) and rounds (to even) to an integer r;
// code = ((e + 7) << 3) + r - 8, a carry to r = 16 landing on the next
// exponent's first code.  Below 2^-6 the quantum is 2^-9 and code = rint(a 2^9).
__device__ __forceinline__ uint32_t fp8_e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | static_cast<uint32_t>(rintf(a * 512.0f));   // exact power-of-two scale
  const int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xFFu) - 127;
  const int r = static_cast<int>(rintf(ldexpf(a, 3 - e)));
  return sign | static_cast<uint32_t>(((e + 7) << 3) + r - 8);
}

// 16 E4M3 codes of a 16-byte vector (byte j of word w is element 4w + j) to
// fp32, exact (hardware conversion, two codes per instruction).
__device__ __forceinline__ void fp8_e4m3_unpack16(const uint4& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), true);
    out[4 * i] = lo[0];
    out[4 * i + 1] = lo[1];
    out[4 * i + 2] = hi[0];
    out[4 * i + 3] = hi[1];
  }
}

// --------------------------------------------------------------- score keys
// A 64-bit key that orders (score desc, index asc) as an unsigned integer:
// high word = order-preserving image of the fp32 score, low word = ~index.
// Key 0 is below every real key and marks "no candidate".
__device__ __forceinline__ uint32_t orderable_f32(float f) {
  if (f == 0.0f) f = 0.0f;  // +0 and -0 compare equal
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable_f32(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t make_key(float score, int32_t index) {
  return (static_cast<uint64_t>(orderable_f32(score)) << 32) |
         static_cast<uint64_t>(~static_cast<uint32_t>(index));
}
__device__ __forceinline__ int32_t key_index(uint64_t key) {
  return static_cast<int32_t>(~static_cast<uint32_t>(key & 0xFFFFFFFFull));
}
__device__ __forceinline__ float key_score(uint64_t key) {
  return from_orderable_f32(static_cast<uint32_t>(key >> 32));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  lo = __shfl_xor(lo, mask, kWave);
  hi = __shfl_xor(hi, mask, kWave);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  lo = __shfl(lo, src, kWave);
  hi = __shfl(hi, src, kWave);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Sort one key per lane across the wave, descending (lane 0 = largest).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t key, int lane) {
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      uint64_t other = shfl_xor_u64(key, j);
      bool desc = (lane & k) == 0;
      bool lower = (lane & j) == 0;
      uint64_t hi = key > other ? key : other;
      uint64_t lo = key > other ? other : key;
      key = (lower == desc) ? hi : lo;
    }
  }
  return key;
}

// Given two descending wave lists a (this lane's element a[lane]) and
// b_rev = b[63 - lane], return the descending list of the 64 largest keys of
// a U b.  max(a[i], b[63-i]) is bitonic and holds the top 64; a bitonic merge
// sorts it.
__device__ __forceinline__ uint64_t wave_merge_top_desc(uint64_t a, uint64_t b_rev, int lane) {
  uint64_t key = a > b_rev ? a : b_rev;
#pragma unroll
  for (int j = kWave >> 1; j > 0; j >>= 1) {
    uint64_t other = shfl_xor_u64(key, j);
    bool lower = (lane & j) == 0;
    uint64_t hi = key > other ? key : other;
    uint64_t lo = key > other ? other : key;
    key = lower ? hi : lo;
  }
  return key;
}

// Ascending sort of one 32-bit value per lane.
__device__ __forceinline__ uint32_t wave_sort_asc_u32(uint32_t key, int lane) {
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      uint32_t other = __shfl_xor(key, j, kWave);
      bool asc = (lane & k) == 0;
      bool lower = (lane & j) == 0;
      uint32_t hi = key > other ? key : other;
      uint32_t lo = key > other ? other : key;
      key = (lower == asc) ? lo : hi;
    }
  }
  return key;
}

// ------------------------------------------------------- lane exchanges (VALU)
// v from lane (lane ^ M), without going through LDS: DPP row permutes for
// M = 1, 2, 4, 8 (xor 4 = xor 3 then xor 7; xor 8 = xor 7 then xor 15) and the
// gfx950 permlane16/32 swaps for M = 16, 32.
template <int M>
__device__ __forceinline__ uint32_t xor_lanes(uint32_t v) {
  if constexpr (M == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);            // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);            // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    const uint32_t t = __builtin_amdgcn_mov_dpp(v, 0x1B, 0xF, 0xF, false); // quad_perm [3,2,1,0]
    return __builtin_amdgcn_mov_dpp(t, 0x141, 0xF, 0xF, false);           // row_half_mirror
  } else if constexpr (M == 8) {
    const uint32_t t = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
    return __builtin_amdgcn_mov_dpp(t, 0x140, 0xF, 0xF, false);           // row_mirror
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (__lane_id() & 16) ? r[0] : r[1];
  } else {
    static_assert(M == 32, "xor distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (__lane_id() & 32) ? r[0] : r[1];
  }
}
template <int M>
__device__ __forceinline__ float xor_lanes_f(float v) {
  return __uint_as_float(xor_lanes<M>(__float_as_uint(v)));
}

// One compare-exchange stage of a bitonic network over the wave's lanes:
// lane pairs (l, l ^ J); the lower lane keeps the larger key when desc.
template <int J>
__device__ __forceinline__ uint32_t bitonic_cx_u32(uint32_t key, bool desc, int lane) {
  const uint32_t other = xor_lanes<J>(key);
  const bool lower = (lane & J) == 0;
  const uint32_t hi = key > other ? key : other;
  const uint32_t lo = key > other ? other : key;
  return (lower == desc) ? hi : lo;
}

// Sort one 32-bit key per lane across the wave, descending (lane 0 =
// largest), with DPP / permlane exchanges only.
__device__ __forceinline__ uint32_t wave_sort_desc_u32(uint32_t key) {
  const int lane = static_cast<int>(__lane_id());
#define SPA_CX(K, J) key = bitonic_cx_u32<J>(key, (lane & (K)) == 0, lane)
  SPA_CX(2, 1);
  SPA_CX(4, 2); SPA_CX(4, 1);
  SPA_CX(8, 4); SPA_CX(8, 2); SPA_CX(8, 1);
  SPA_CX(16, 8); SPA_CX(16, 4); SPA_CX(16, 2); SPA_CX(16, 1);
  SPA_CX(32, 16); SPA_CX(32, 8); SPA_CX(32, 4); SPA_CX(32, 2); SPA_CX(32, 1);
  SPA_CX(64, 32); SPA_CX(64, 16); SPA_CX(64, 8); SPA_CX(64, 4); SPA_CX(64, 2); SPA_CX(64, 1);
#undef SPA_CX
  return key;
}

// ----------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xor_lanes_f<32>(v));
  v = fmaxf(v, xor_lanes_f<16>(v));
  v = fmaxf(v, xor_lanes_f<8>(v));
  v = fmaxf(v, xor_lanes_f<4>(v));
  v = fmaxf(v, xor_lanes_f<2>(v));
  return fmaxf(v, xor_lanes_f<1>(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += xor_lanes_f<32>(v);
  v += xor_lanes_f<16>(v);
  v += xor_lanes_f<8>(v);
  v += xor_lanes_f<4>(v);
  v += xor_lanes_f<2>(v);
  return v + xor_lanes_f<1>(v);
}
// Sum over aligned groups of G lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 64) v += xor_lanes_f<32>(v);
  if constexpr (G >= 32) v += xor_lanes_f<16>(v);
  if constexpr (G >= 16) v += xor_lanes_f<8>(v);
  if constexpr (G >= 8) v += xor_lanes_f<4>(v);
  if constexpr (G >= 4) v += xor_lanes_f<2>(v);
  if constexpr (G >= 2) v += xor_lanes_f<1>(v);
  return v;
}

// Workgroup barrier that orders LDS only: outstanding global loads stay in
// flight across it (a plain __syncthreads also waits for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS ordering among the lanes of one wave (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------- hand-off between workgroups
// Agent-scope relaxed atomic stores and loads are write-through / coherent
// accesses (sc1): a value stored this way is visible to every XCD once the
// store completes, and a load this way never returns a stale L2 copy.  A
// workgroup publishes its results with publish_* , waits for them to
// complete (wait_published), and only then counts itself done with an
// agent-scope atomic; the workgroup that sees the last count reads the
// results with acquire_* loads.  This is the release / acquire pattern
// without the L2 write-back (buffer_wbl2) and invalidation a fence would do,
// valid because every value handed over travels through these accesses.
__device__ __forceinline__ void publish_u64(void* p, uint64_t v) {
  __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_u32(void* p, uint32_t v) {
  __hip_atomic_store(static_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_f2(void* p, float a, float b) {
  publish_u64(p, (static_cast<uint64_t>(__float_as_uint(b)) << 32) | __float_as_uint(a));
}
__device__ __forceinline__ uint64_t acquire_u64(const void* p) {
  return __hip_atomic_load(static_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 acquire_f2(const void* p) {
  const uint64_t u = acquire_u64(p);
  return make_float2(__uint_as_float(static_cast<uint32_t>(u)), __uint_as_float(static_cast<uint32_t>(u >> 32)));
}
__device__ __forceinline__ float acquire_f32(const void* p) {
  return __uint_as_float(
      __hip_atomic_load(static_cast<const uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// Wait until this thread's stores (and loads) have completed.
__device__ __forceinline__ void wait_published() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ uint32_t count_arrival(uint32_t* ctr) {
  return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Number of set bits of a wave-uniform mask held by lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u)));
}

// erf in fp64 to within 3e-14 (absolute) with few live registers:
// |x| < 2.5: the positive-term series erf(x) = 2/sqrt(pi) exp(-x^2)
//   sum_n 2^n x^(2n+1) / (1 3 5 ... (2n+1)) (Abramowitz & Stegun 7.1.6), 33 terms;
// 2.5 <= |x| < 6: the continued fraction for erfc (A&S 7.1.14), 20 levels,
//   evaluated from the tail as one numerator/denominator pair;
// |x| >= 6: +-1 (erfc(6) < 2.2e-17).
__device__ __forceinline__ double erf_exact(double x) {
  const double ax = fabs(x);
  if (ax >= 6.0) return copysign(1.0, x);
  const double g = exp(-ax * ax);
  double r;
  if (ax < 2.5) {
    const double y = 2.0 * ax * ax;
    double t = ax, s = ax;
#pragma unroll
    for (int n = 1; n <= 32; ++n) {
      t *= y * (1.0 / (2 * n + 1));
      s += t;
    }
    r = 1.1283791670955126 * g * s;               // 2 / sqrt(pi)
  } else {
    double num = ax, den = 1.0;
#pragma unroll
    for (int k = 20; k >= 1; --k) {
      const double nn = fma(ax, num, 0.5 * k * den);
      den = num;
      num = nn;
    }
    r = 1.0 - g * den / (1.7724538509055159 * num);  // sqrt(pi)
  }
  return copysign(r, x);
}

// ------------------------------------------------------- fp64 top-k of a wave
__device__ __forceinline__ uint64_t orderable_f64(double v) {
  if (v == 0.0) v = 0.0;                       // +0 and -0 compare equal
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// Top `want` of the wave's 4 x 64 (score, slot) pairs (slot = i * 64 + lane,
// ok marks the valid ones), higher score first, lower slot on ties: a bitwise
// search for the threshold over the scores' orderable bits below the common
// prefix of the smallest and largest (ballot counts, stopping once the kept
// set is decided), then every pair above it and the first ones equal to it in
// slot order.  Sets taken[], returns how many.
__device__ __forceinline__ int wave_top_f64x4(const double (&sc)[4], const bool (&ok)[4], int want, bool (&taken)[4]) {
  uint64_t key[4];
  int nv = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    key[i] = ok[i] ? orderable_f64(sc[i]) : 0ull;
    nv += __popcll(__ballot(ok[i]));
  }
  const int kk = nv < want ? nv : want;
  uint64_t t = ~0ull;
  if (kk > 0) {
    // every valid key shares the common prefix of the smallest and largest
    uint64_t lo = ~0ull, hi = 0ull;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ok[i]) {
        lo = key[i] < lo ? key[i] : lo;
        hi = key[i] > hi ? key[i] : hi;
      }
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
      const uint64_t ol = __shfl_xor(lo, o), oh = __shfl_xor(hi, o);
      lo = ol < lo ? ol : lo;
      hi = oh > hi ? oh : hi;
    }
    const int top = lo == hi ? -1 : 63 - __clzll(static_cast<long long>(lo ^ hi));
    t = top < 0 ? hi : (hi & ~((2ull << top) - 1ull));
    for (int bit = top; bit >= 0; --bit) {
      const uint64_t cand = t | (1ull << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) cnt += __popcll(__ballot(key[i] >= cand));
      if (cnt >= kk) {
        t = cand;
        if (cnt == kk) break;
      }
    }
  }
  int ngt = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) ngt += __popcll(__ballot(key[i] > t));
  const int need = kk - ngt;
  int eq_seen = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t eq = __ballot(key[i] == t && key[i] != 0ull);
    taken[i] = key[i] > t || (key[i] == t && key[i] != 0ull && eq_seen + lanes_below(eq) < need);
    eq_seen += __popcll(eq);
  }
  return kk;
}

// ------------------------------------------- k-th largest of a workgroup
// Workgroups of 1024 threads holding kRegs keys each in registers (cell
// j * 1024 + tid in key[j], 0 past the n cells); cells beyond the registers
// are read from `a` (fp32, through orderable_f32).  Returns the largest t
// with at least kr (1 <= kr <= n) keys at or above it: a bitwise search below
// the common prefix of the smallest and largest key, counts summed over the
// workgroup from ballots, stopping once exactly kr keys are at or above the
// candidate.  s_part: 2 x 16 ints, s_lohi: 2 x 16 words of LDS.
constexpr int kWgThreads = 1024;
constexpr int kWgWaves = kWgThreads / kWave;

template <int kRegs>
__device__ inline uint32_t wg_kth_largest_f32(const uint32_t (&key)[kRegs], const float* __restrict__ a, int64_t n,
                                              int kr, int* s_part, uint32_t* s_lohi) {
  constexpr int64_t kSpan = static_cast<int64_t>(kWgThreads) * kRegs;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  uint32_t lo = ~0u, hi = 0u;
#pragma unroll
  for (int j = 0; j < kRegs; ++j) {
    if (j * kWgThreads + tid < n) {
      lo = key[j] < lo ? key[j] : lo;
      hi = key[j] > hi ? key[j] : hi;
    }
  }
  for (int64_t c = kSpan + tid; c < n; c += kWgThreads) {
    const uint32_t kv = orderable_f32(a[c]);
    lo = kv < lo ? kv : lo;
    hi = kv > hi ? kv : hi;
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    const uint32_t ol = __shfl_xor(lo, o), oh = __shfl_xor(hi, o);
    lo = ol < lo ? ol : lo;
    hi = oh > hi ? oh : hi;
  }
  if (lane == 0) {
    s_lohi[wave] = lo;
    s_lohi[kWgWaves + wave] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWgWaves; ++w) {
    lo = s_lohi[w] < lo ? s_lohi[w] : lo;
    hi = s_lohi[kWgWaves + w] > hi ? s_lohi[kWgWaves + w] : hi;
  }
  uint32_t t = hi;                             // every key equal: hi is the threshold
  if (lo != hi) {
    const int top = 31 - __clz(lo ^ hi);       // highest bit where the keys differ
    t = hi & ~((2u << top) - 1u);              // the common prefix: every key is at or above it
    for (int bit = top, it = 0; bit >= 0; --bit, ++it) {
      const uint32_t cand = t | (1u << bit);
      int cnt = 0;                             // wave-uniform: ballot counts
#pragma unroll
      for (int j = 0; j < kRegs; ++j) cnt += __popcll(__ballot(key[j] >= cand));
      for (int64_t c0 = kSpan; c0 < n; c0 += kWgThreads) {
        const int64_t c = c0 + tid;
        cnt += __popcll(__ballot(c < n && orderable_f32(a[c < n ? c : n - 1]) >= cand));
      }
      if (lane == 0) s_part[(it & 1) * kWgWaves + wave] = cnt;
      __syncthreads();
      int tot = 0;
#pragma unroll
      for (int w = 0; w < kWgWaves; ++w) tot += s_part[(it & 1) * kWgWaves + w];
      if (tot >= kr) {
        t = cand;
        if (tot == kr) break;
      }
    }
  }
  __syncthreads();                             // s_part / s_lohi free for the caller
  return t;
}



// Top-k threshold of the wave's NV x 64 keys: returns t with
// count(key > t) <= k <= count(key >= t), so that the keys > t plus the
// first k - count(key > t) keys == t are exactly a top k (0xFFFFFFFF if
// k == 0).  Bitwise search from the top bit; each step counts with ballots,
// so the count never leaves the scalar unit.  The search stops as soon as
// count(key >= t) == k (the kept set is then decided), and when lo <= T <= hi
// is known for the k-th largest key T, it starts below their common top bits.
// Keys equal to 0 never count.
template <int NV>
__device__ __forceinline__ uint32_t wave_kth_largest(const uint32_t (&key)[NV], int k, uint32_t lo = 0u,
                                                     uint32_t hi = 0xFFFFFFFFu) {
  if (k <= 0) return 0xFFFFFFFFu;
  const uint32_t diff = lo ^ hi;
  if (diff == 0u) return lo;
  const int top = 31 - __builtin_clz(diff);
  uint32_t t = lo & ~((2u << top) - 1u);   // common prefix of lo and hi (top == 31: nothing)
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) cnt += __popcll(__ballot(key[i] >= cand));
    if (cnt >= k) {
      t = cand;
      if (cnt == k) break;
    }
  }
  return t;
}

// Largest key of the wave (0 if none).
template <int NV>
__device__ __forceinline__ uint32_t wave_max_key(const uint32_t (&key)[NV]) {
  uint32_t m = key[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) m = key[i] > m ? key[i] : m;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off));
    m = o > m ? o : m;
  }
  return m;
}

// Online-softmax combine of (m, l) pairs: result represents l e^m.
__device__ __forceinline__ void ml_combine(float& m, float& l, float m2, float l2) {
  float mm = fmaxf(m, m2);
  if (mm == -INFINITY) {
    m = mm;
    l = 0.f;
    return;
  }
  l = l * __expf(m - mm) + l2 * __expf(m2 - mm);
  m = mm;
}

// ------------------------------------------------------ per-lane top-K lists
// (score, index) pairs; better = higher score, then lower index.
template <typename S>
__device__ __forceinline__ bool sel_better(S s1, int i1, S s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

// Insert (s, c) into a list sorted best-first (caller checked it qualifies).
// Branch-free: with w[t] = "(s, c) beats entry t" (false up to the insertion
// point, true after it), slot t keeps its entry, takes (s, c), or takes entry
// t - 1; every slot is decided independently of the others.
template <typename S, int KMAX>
__device__ __forceinline__ void topk_push(S (&ts)[KMAX], int (&ti)[KMAX], S s, int c) {
  bool w[KMAX];
#pragma unroll
  for (int t = 0; t < KMAX; ++t) w[t] = sel_better(s, c, ts[t], ti[t]);
#pragma unroll
  for (int t = KMAX - 1; t > 0; --t) {
    const S up_s = w[t - 1] ? ts[t - 1] : s;
    const int up_i = w[t - 1] ? ti[t - 1] : c;
    ts[t] = w[t] ? up_s : ts[t];
    ti[t] = w[t] ? up_i : ti[t];
  }
  ts[0] = w[0] ? s : ts[0];
  ti[0] = w[0] ? c : ti[0];
}

// The same for a candidate that arrives after every held entry in index
// order, so a tie keeps the held entry (plain score comparisons).
template <typename S, int KMAX>
__device__ __forceinline__ void topk_push_later(S (&ts)[KMAX], int (&ti)[KMAX], S s, int c) {
  bool w[KMAX];
#pragma unroll
  for (int t = 0; t < KMAX; ++t) w[t] = s > ts[t];
#pragma unroll
  for (int t = KMAX - 1; t > 0; --t) {
    const S up_s = w[t - 1] ? ts[t - 1] : s;
    const int up_i = w[t - 1] ? ti[t - 1] : c;
    ts[t] = w[t] ? up_s : ts[t];
    ti[t] = w[t] ? up_i : ti[t];
  }
  ts[0] = w[0] ? s : ts[0];
  ti[0] = w[0] ? c : ti[0];
}

// Sort a bitonic list best-first (Batcher's half-cleaner cascade).
template <typename S, int N>
__device__ __forceinline__ void bitonic_clean_best_first(S (&ts)[N], int (&ti)[N]) {
#pragma unroll
  for (int j = N / 2; j > 0; j >>= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if ((i & j) == 0 && sel_better(ts[i + j], ti[i + j], ts[i], ti[i])) {
        const S xs = ts[i]; ts[i] = ts[i + j]; ts[i + j] = xs;
        const int xi = ti[i]; ti[i] = ti[i + j]; ti[i + j] = xi;
      }
    }
  }
}

// Sort by ascending index (Batcher's bitonic sorting network; indices distinct
// apart from the 0x7FFFFFFF fill).
template <typename S, int N>
__device__ __forceinline__ void sort_by_index(S (&ts)[N], int (&ti)[N]) {
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int l = i ^ j;
        if (l > i && ((ti[i] > ti[l]) == ((i & k) == 0))) {
          const S xs = ts[i]; ts[i] = ts[l]; ts[l] = xs;
          const int xi = ti[i]; ti[i] = ti[l]; ti[l] = xi;
        }
      }
    }
  }
}

}  // namespace spa
