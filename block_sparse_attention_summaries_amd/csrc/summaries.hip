// summaries.hip -- block / cell summaries of the key cache on gfx950.
//
// Per (batch, kv head, full block c): mean key (exact fp64 sum, rounded to
// nearest even in the key dtype), max L2 key norm (fp64, rounded to fp32) and
// centre position c b + (b-1)/2.  ("SAS" review §3 Eq. 3: pooled block
// summaries read by the selector; "FreeSolo" review, "How it works": mean
// key, centre position and max key norm of each cell.)
//
// HBM-bound streaming reduction: one wave per block, 16-byte coalesced loads
// (a block of b rows x d elements is one contiguous span), fp64 column sums
// in registers, a cross-lane sum of squares per row and lane exchanges for the
// column sums.
//
// Optional fp8 summaries for the decode scorer (half the scoring bytes):
// quantize_fp8_kernel turns block rows of kbar into OCP E4M3 codes with one
// fp32 scale per block (amax / 448; codes of kbar * (448 / amax), nearest,
// ties to even), one wave per row; dequantize_fp8_kernel rebuilds fp32
// summaries through the same decode the scorer uses.
#include "spa_device.h"
#include "spa_launch.h"

namespace spa {

// With a page table, block c of (batch, kv head) is page table[batch * tstride
// + c] of the pool [npages, Hkv, b, d]; an unmapped page (id outside the
// pool) reads as zero keys.
//
// One wave per block, four per workgroup: kLPR lanes cover a key row with
// 16-byte loads and a pass covers kRPW rows; the loads of kChunk passes are
// in flight together.  A lane sums its column slice over its rows in fp64;
// each row's sum of squares is added over the row's lanes and the largest is
// kept (the norm is its square root, taken once: sqrt and the rounding to
// fp32 are monotone); at the end the column sums are added across the row
// groups by lane exchanges (every sum is exact in fp64 for key values within
// 2^40 of each other, so the order does not change the mean).
template <int M>
__device__ __forceinline__ double xor_lanes_d(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint64_t r = (static_cast<uint64_t>(xor_lanes<M>(static_cast<uint32_t>(u >> 32))) << 32) |
                     xor_lanes<M>(static_cast<uint32_t>(u));
  return __longlong_as_double(static_cast<long long>(r));
}

template <typename T, int D>
__global__ __launch_bounds__(256) void block_summaries_kernel(
    const T* __restrict__ k, int Hkv, int64_t L, int b, int64_t first_block, int64_t num_blocks,
    int64_t ccap, T* __restrict__ kbar, float* __restrict__ max_norm, float* __restrict__ centre,
    const int32_t* __restrict__ table, int64_t tstride, int64_t npages) {
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kLPR = D / kVec;                // lanes covering one key row
  constexpr int kRPW = kWave / kLPR;            // rows per pass of a wave
  constexpr int kChunk = 8;                     // passes with their loads in flight together
  static_assert(kLPR <= kWave, "row must fit in one wave");

  const int lane = threadIdx.x % kWave;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (blk >= num_blocks) return;                // whole wave leaves
  const int64_t c = first_block + blk;
  const int64_t bh = blockIdx.y;
  const int cg = lane % kLPR;                   // which kVec columns
  const int rg = lane / kLPR;                   // which row of a pass
  const T* base = k + (bh * L + c * b) * D;
  int nrows = b;
  if (table != nullptr) {
    const int64_t pg = table[(bh / Hkv) * tstride + c];
    const bool mapped = pg >= 0 && pg < npages;
    base = k + ((mapped ? pg : 0) * Hkv + bh % Hkv) * b * D;
    nrows = mapped ? b : 0;
  }

  double acc[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i) acc[i] = 0.0;
  double best2 = 0.0;                           // largest row sum of squares
  for (int r0 = 0; r0 < nrows; r0 += kRPW * kChunk) {
    uint4 raw[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int r = r0 + u * kRPW + rg;
      raw[u] = r < nrows ? *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(r) * D + cg * kVec)
                         : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (r0 + u * kRPW >= nrows) break;        // the same for every lane: nrows is a multiple of kRPW
      float x[kVec];
      Elem<T>::unpack(raw[u], x);
      double ss = 0.0;
#pragma unroll
      for (int i = 0; i < kVec; ++i) {
        const double xd = static_cast<double>(x[i]);
        acc[i] += xd;
        ss = fma(xd, xd, ss);
      }
      // sum of squares over the lanes of this row (aligned groups of kLPR)
      if constexpr (kLPR >= 32) ss += xor_lanes_d<16>(ss);
      if constexpr (kLPR >= 16) ss += xor_lanes_d<8>(ss);
      ss += xor_lanes_d<4>(ss);
      ss += xor_lanes_d<2>(ss);
      ss += xor_lanes_d<1>(ss);
      best2 = ss > best2 ? ss : best2;
    }
  }
  // column sums over the row groups
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    if constexpr (kLPR <= 8) acc[i] += xor_lanes_d<8>(acc[i]);
    if constexpr (kLPR <= 16) acc[i] += xor_lanes_d<16>(acc[i]);
    acc[i] += xor_lanes_d<32>(acc[i]);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const double o = __shfl_xor(best2, m, kWave);
    best2 = o > best2 ? o : best2;
  }
  const float best = __double2float_rn(sqrt(best2));

  const int64_t out = bh * ccap + c;
  if (rg == 0) {
#pragma unroll
    for (int i = 0; i < kVec; ++i)
      kbar[out * D + cg * kVec + i] = Elem<T>::from_double(acc[i] * (1.0 / static_cast<double>(b)));
  }
  if (lane == 0) {
    max_norm[out] = best;
    if (centre != nullptr && bh == 0)
      centre[c] = static_cast<float>(static_cast<double>(c) * b + 0.5 * (b - 1));
  }
}

template <typename T, int D>
static hipError_t launch_summaries_t(const SummaryLaunch& p, hipStream_t st) {
  dim3 grid(static_cast<unsigned>((p.num_blocks + 3) / 4), static_cast<unsigned>(p.B * p.Hkv));
  return launch(true, block_summaries_kernel<T, D>, grid, dim3(256), st, static_cast<const T*>(p.k),
                p.Hkv, p.L, p.b, p.first_block, p.num_blocks, p.ccap, static_cast<T*>(p.kbar),
                p.max_norm, p.centre, p.pages.table, p.pages.tstride, p.pages.npages);
}

hipError_t launch_block_summaries(const SummaryLaunch& p, hipStream_t st) {
  if (p.dtype == 1) {
    return p.d == 64 ? launch_summaries_t<bf16_t, 64>(p, st) : launch_summaries_t<bf16_t, 128>(p, st);
  }
  return p.d == 64 ? launch_summaries_t<float, 64>(p, st) : launch_summaries_t<float, 128>(p, st);
}

// One wave per (batch, kv head, block) row: the row's largest magnitude, then
// scale = amax / 448 and codes of x (448 / amax), both quotients correctly
// rounded in single precision; a zero row gets scale 0 and zero codes.
template <typename T, int D>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const T* __restrict__ kbar, int64_t ccap,
                                                           int64_t first, int64_t num, int64_t rows_total,
                                                           uint8_t* __restrict__ codes, float* __restrict__ scales) {
  constexpr int kPer = D / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;   // (bh, block) in the range
  if (r >= rows_total) return;                  // whole wave leaves
  const int64_t bh = r / num, c = first + r % num;
  const int64_t row = (bh * ccap + c) * D;
  float x[kPer];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    x[i] = ld_f(kbar + row + i * kWave + lane);
    amax = fmaxf(amax, fabsf(x[i]));
  }
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const bool zero = amax == 0.f;
  const float inv = zero ? 0.f : __fdiv_rn(448.0f, amax);
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    codes[row + i * kWave + lane] = static_cast<uint8_t>(zero ? 0u : fp8_e4m3_encode(__fmul_rn(x[i], inv)));
  if (lane == 0) scales[bh * ccap + c] = zero ? 0.f : __fdiv_rn(amax, 448.0f);
}

// One thread per 16 codes: out = scale * decode(code) (single-precision product).
__global__ __launch_bounds__(256) void dequantize_fp8_kernel(const uint8_t* __restrict__ codes,
                                                             const float* __restrict__ scales, int64_t rows,
                                                             int d, float* __restrict__ out) {
  const int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = d / 16;
  if (v >= rows * per_row) return;
  const float s = scales[v / per_row];
  float x[16];
  fp8_e4m3_unpack16(reinterpret_cast<const uint4*>(codes)[v], x);
  float4* o = reinterpret_cast<float4*>(out) + v * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = make_float4(__fmul_rn(x[4 * i], s), __fmul_rn(x[4 * i + 1], s), __fmul_rn(x[4 * i + 2], s),
                       __fmul_rn(x[4 * i + 3], s));
}

template <typename T, int D>
static hipError_t launch_quantize_t(const void* kbar, int B, int Hkv, int64_t ccap, int64_t first, int64_t num,
                                    uint8_t* codes, float* scales, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(B) * Hkv * num;
  return launch(true, quantize_fp8_kernel<T, D>, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), st,
                static_cast<const T*>(kbar), ccap, first, num, rows, codes, scales);
}

hipError_t launch_quantize_fp8(const void* kbar, int dtype, int B, int Hkv, int64_t ccap, int d, int64_t first,
                               int64_t num, uint8_t* codes, float* scales, hipStream_t st) {
  if (dtype == kDtypeBf16)
    return d == 64 ? launch_quantize_t<bf16_t, 64>(kbar, B, Hkv, ccap, first, num, codes, scales, st)
                   : launch_quantize_t<bf16_t, 128>(kbar, B, Hkv, ccap, first, num, codes, scales, st);
  return d == 64 ? launch_quantize_t<float, 64>(kbar, B, Hkv, ccap, first, num, codes, scales, st)
                 : launch_quantize_t<float, 128>(kbar, B, Hkv, ccap, first, num, codes, scales, st);
}

hipError_t launch_dequantize_fp8(const uint8_t* codes, const float* scales, int64_t rows, int d, float* out,
                                 hipStream_t st) {
  const int64_t n = rows * (d / 16);
  return launch(true, dequantize_fp8_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), st, codes,
                scales, rows, d, out);
}

}  // namespace spa
