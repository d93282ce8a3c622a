// decode_tile.h -- split-K attention pieces of the decode step (one query
// row) shared by the two-call path (attn.hip) and the one-call step
// (decode_step.hip): the partial of one 64-key bf16 K / V tile for the G query
// heads of a group, and the combine of a selection head's partials inside the
// kernel that wrote them.
//
// Keys of the tile are attended with z_j = q_h.k_j / sqrt(d) + bias (bias =
// log g of the selected block, 0 for the current block; "SAS" review §4.1
// Eq. 4, §4.3 Eq. 9); the partial of head h is (m_h, l_h, acc_h) with
// m_h = max_j z_j, l_h = sum_j exp(z_j - m_h), acc_h = sum_j exp(z_j - m_h) v_j.
#pragma once

#include "spa_device.h"

namespace spa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 dbf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float dfloatx4_t;

constexpr int kTileTok = 64;      // keys per decode tile
constexpr int kMaxTiles = 130;    // (K + 1) * tiles per unit for K <= 64, b <= 128

__device__ __forceinline__ dbf16x8_t dec_bf16x8(uint4 v) { return __builtin_bit_cast(dbf16x8_t, v); }

// Partial of one tile of ntok (1..64) keys: kt / vt point at the tile's first
// key row ([ntok, D] bf16, rows contiguous), q at query head 0 of the group
// (HPW heads, rows of D).  Wave w takes keys 16w .. 16w + 15:
//  - S^T = K Q^T with v_mfma_f32_16x16x32_bf16: lane l feeds K row 16w + l%16,
//    columns 32j + 8(l/16) .. +7 straight from memory as the A operand, and
//    query head l%16 (zero for l%16 >= HPW) as B; it gets back the scores of
//    keys 16w + 4(l/16) + i (i < 4) for head l%16.
//  - the softmax max and sum of a head reduce over the lanes holding it
//    (xor 16 and 32) and over the four waves through LDS;
//  - P V on the vector units: lane (g = l/16, c = l%16) holds V rows
//    16w + 4g + i, columns c D/16 .. +D/16, and reads each head's
//    probabilities of those rows from lane 16g + h; the sums over g are
//    reduce-scattered (xor 32, xor 16: lane g keeps the g-th quarter of its
//    columns) and the waves' sums added in wave order through LDS.
// Writes ws_ml[obase + h] and ws_acc[(obase + h) D ..]; kPublish: with
// agent-scope write-through stores (read back in the same kernel).
template <int D, int HPW, bool kPublish>
__device__ __forceinline__ void tile_partial_bf16(const bf16_t* __restrict__ q, const bf16_t* __restrict__ kt,
                                                  const bf16_t* __restrict__ vt, int ntok, float bias,
                                                  float* __restrict__ ws_acc, float2* __restrict__ ws_ml,
                                                  int64_t obase) {
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(HPW == 1 || HPW == 2 || HPW == 4 || HPW == 8, "heads per group");
  constexpr int kKB = D / 32;        // MFMA k-blocks of 32
  constexpr int kVE = D / 16;        // V columns per lane (8 or 4)
  constexpr int kQE = kVE / 4;       // columns per lane after the reduce-scatter
  __shared__ float s_m[4][16];
  __shared__ float s_l[4][16];
  __shared__ __align__(16) float s_acc[4][HPW][D];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = lane >> 4, c = lane & 15;

  // loads: K (A operand), the group's queries (B operand), V rows
  const int krow = 16 * wave + c;
  const int kr = krow < ntok ? krow : ntok - 1;
  uint4 ka[kKB], qb[kKB];
  const int hq = c < HPW ? c : 0;
#pragma unroll
  for (int j = 0; j < kKB; ++j) {
    ka[j] = *reinterpret_cast<const uint4*>(kt + static_cast<int64_t>(kr) * D + 32 * j + 8 * g);
    qb[j] = *reinterpret_cast<const uint4*>(q + static_cast<int64_t>(hq) * D + 32 * j + 8 * g);
  }
  uint32_t vw[4][kVE / 2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int vrow = 16 * wave + 4 * g + i;
    const int vr = vrow < ntok ? vrow : ntok - 1;
    const bf16_t* src = vt + static_cast<int64_t>(vr) * D + c * kVE;
    if constexpr (kVE == 8) {
      const uint4 x = *reinterpret_cast<const uint4*>(src);
      vw[i][0] = x.x; vw[i][1] = x.y; vw[i][2] = x.z; vw[i][3] = x.w;
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(src);
      vw[i][0] = x.x; vw[i][1] = x.y;
    }
  }
  if (c >= HPW) {
#pragma unroll
    for (int j = 0; j < kKB; ++j) qb[j] = make_uint4(0u, 0u, 0u, 0u);
  }

  // scores of keys 16 wave + 4 g + i, head c
  dfloatx4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kKB; ++j) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dec_bf16x8(ka[j]), dec_bf16x8(qb[j]), st, 0, 0, 0);
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  float z[4];
  float mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = 16 * wave + 4 * g + i;
    z[i] = key < ntok ? st[i] * scale + bias : -INFINITY;
    mloc = fmaxf(mloc, z[i]);
  }
  mloc = fmaxf(mloc, xor_lanes_f<16>(mloc));
  mloc = fmaxf(mloc, xor_lanes_f<32>(mloc));
  if (g == 0) s_m[wave][c] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_m[0][c], s_m[1][c]), fmaxf(s_m[2][c], s_m[3][c]));
  float p[4];
  float lloc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = z[i] == -INFINITY ? 0.f : __expf(z[i] - M);
    lloc += p[i];
  }
  lloc += xor_lanes_f<16>(lloc);
  lloc += xor_lanes_f<32>(lloc);

  // P V for the lane's four rows and kVE columns, every head of the group
  float acc[HPW][kVE];
#pragma unroll
  for (int h = 0; h < HPW; ++h)
#pragma unroll
    for (int e = 0; e < kVE; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float vf[kVE];
#pragma unroll
    for (int e = 0; e < kVE / 2; ++e) {
      vf[2 * e] = __uint_as_float(vw[i][e] << 16);
      vf[2 * e + 1] = __uint_as_float(vw[i][e] & 0xFFFF0000u);
    }
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      const float ph = __shfl(p[i], 16 * g + h, kWave);
#pragma unroll
      for (int e = 0; e < kVE; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
    }
  }
  // reduce-scatter over g: xor 32 keeps columns [0, kVE/2) for g < 2, then
  // xor 16 keeps the lane's quarter g
  float r2[HPW][kVE / 2];
  const bool hi32 = (g & 2) != 0;
#pragma unroll
  for (int h = 0; h < HPW; ++h)
#pragma unroll
    for (int e = 0; e < kVE / 2; ++e) {
      const float mine = hi32 ? acc[h][kVE / 2 + e] : acc[h][e];
      const float other = hi32 ? acc[h][e] : acc[h][kVE / 2 + e];
      r2[h][e] = mine + xor_lanes_f<32>(other);
    }
  const bool hi16 = (g & 1) != 0;
#pragma unroll
  for (int h = 0; h < HPW; ++h)
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      const float mine = hi16 ? r2[h][kQE + e] : r2[h][e];
      const float other = hi16 ? r2[h][e] : r2[h][kQE + e];
      s_acc[wave][h][c * kVE + g * kQE + e] = mine + xor_lanes_f<16>(other);
    }
  if (g == 0) s_l[wave][c] = lloc;
  __syncthreads();

  // the tile's partial: waves added in order
  if (tid < HPW) {
    const float m = fmaxf(fmaxf(s_m[0][tid], s_m[1][tid]), fmaxf(s_m[2][tid], s_m[3][tid]));
    const float l = ((s_l[0][tid] + s_l[1][tid]) + s_l[2][tid]) + s_l[3][tid];
    if constexpr (kPublish)
      publish_f2(ws_ml + obase + tid, m, l);
    else
      ws_ml[obase + tid] = make_float2(m, l);
  }
  constexpr int kOut = HPW * D;
  for (int x = 2 * tid; x < kOut; x += 512) {
    const int h = x / D, e = x % D;
    const float a0 = ((s_acc[0][h][e] + s_acc[1][h][e]) + s_acc[2][h][e]) + s_acc[3][h][e];
    const float a1 = ((s_acc[0][h][e + 1] + s_acc[1][h][e + 1]) + s_acc[2][h][e + 1]) + s_acc[3][h][e + 1];
    float* dst = ws_acc + (obase + h) * D + e;
    if constexpr (kPublish) {
      publish_f2(dst, a0, a1);
    } else {
      dst[0] = a0;
      dst[1] = a1;
    }
  }
}

// Split-K combine of one selection head's partials inside the kernel that
// wrote them (their last workgroup): wave w merges query heads w, w + 4, ...
// of the group.  Per output column the same arithmetic in the same order as
// decode_combine_kernel: M = max_t m_t, w_t = exp(m_t - M),
// o = sum_t w_t acc_t / sum_t w_t l_t, lse = M + log sum_t w_t l_t.  The
// partials were published with agent-scope stores and are read the same way;
// every load of a head is issued before the first is used.
template <typename T, int D, int HPW>
__device__ __forceinline__ void combine_partials(const float* __restrict__ ws_acc, const float2* __restrict__ ws_ml,
                                                 int bh, int bi, int hs, int G, int Hq, int share_group,
                                                 int ntiles, T* __restrict__ o, float* __restrict__ lse) {
  constexpr int kCPL = D / kWave;
  constexpr int kBatch = 36;       // tiles whose partials are in flight at once
  __shared__ float s_w[4][kMaxTiles];
  __shared__ float s_l[4][kMaxTiles];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t base = static_cast<int64_t>(bh) * ntiles * HPW;   // partial (tile t, head hh) at base + t*HPW + hh
  for (int hh = wave; hh < HPW; hh += 4) {
    float lsum = 0.f, acc[kCPL];
#pragma unroll
    for (int cc = 0; cc < kCPL; ++cc) acc[cc] = 0.f;
    float M = -INFINITY;
    for (int t0 = 0; t0 < ntiles; t0 += kBatch) {
      // this batch's partials, then (first batch) the (m, l) pairs of every tile
      float part[kBatch][kCPL];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int t = t0 + u < ntiles ? t0 + u : ntiles - 1;
        const float* src = ws_acc + (base + t * HPW + hh) * D + kCPL * lane;
        if constexpr (kCPL == 2) {
          const float2 a = acquire_f2(src);
          part[u][0] = a.x;
          part[u][1] = a.y;
        } else {
          part[u][0] = acquire_f32(src);
        }
      }
      if (t0 == 0) {
        float mloc = -INFINITY;
        for (int t = lane; t < ntiles; t += kWave) {
          const float2 ml = acquire_f2(ws_ml + base + t * HPW + hh);
          s_w[wave][t] = ml.x;
          s_l[wave][t] = ml.y;
          mloc = fmaxf(mloc, ml.x);
        }
        M = wave_max(mloc);
        for (int t = lane; t < ntiles; t += kWave) {
          const float mt = s_w[wave][t];
          s_w[wave][t] = (M == -INFINITY || mt == -INFINITY) ? 0.f : __expf(mt - M);
        }
        wave_lds_sync();
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (t0 + u < ntiles) {
          const float w = s_w[wave][t0 + u];
          lsum = fmaf(s_l[wave][t0 + u], w, lsum);
#pragma unroll
          for (int cc = 0; cc < kCPL; ++cc) acc[cc] = fmaf(part[u][cc], w, acc[cc]);
        }
      }
    }
    const int hq = share_group ? hs * G + hh : hs;
    const int64_t orow = static_cast<int64_t>(bi) * Hq + hq;   // one query row
#pragma unroll
    for (int cc = 0; cc < kCPL; ++cc)
      o[orow * D + kCPL * lane + cc] = Elem<T>::from_float(lsum > 0.f ? acc[cc] / lsum : 0.f);
    if (lane == 0 && lse != nullptr) lse[orow] = lsum > 0.f ? M + __logf(lsum) : -INFINITY;
    wave_lds_sync();
  }
}

}  // namespace spa
