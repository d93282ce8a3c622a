// attn.hip -- exact softmax attention over the kept keys, forward and
// backward, on gfx950.
//
// Keys of a query row at position i:
//   branch L: the current block {j : floor(j/b) = floor(i/b), j <= i} (when
//             kept) plus every selected unit, each selected logit biased by its
//             log gate ("SAS" review §4.1 Eq. 4, §4.3 Eq. 9; "Monodratic" news
//             page: guaranteed local block + exact causal softmax on the set);
//   branch S: the window i - w < j <= i, mixed o = alpha o_L + (1 - alpha) o_S
//             ("FreeSolo" review, "How it works").
// Backward (SAS branch): D = do.o, dS = p (do.v - D), dq, dk, dv and the
// inner-gate gradient dg_m = sum_{j in B_m} dS_j / g_m ("SAS" review §4.2.2
// Eq. 5), summed over the query heads that share a selection.
//
// Decode (one query row): split-K over the K+1 kept blocks.  One workgroup per
// (selection head, kept block, 64-token tile) stages the K and V tile in LDS
// once for all G query heads of the group (GQA-shared gather), writes an
// online-softmax partial (m, l, acc); a combine kernel (one workgroup per
// query head) merges the partials.
// Rows (prefill / training): one wave per (query head, row) streaming its key
// segments 64 keys at a time with an online softmax.
#include <type_traits>

#include "decode_merge.h"
#include "decode_tile.h"
#include "spa_device.h"
#include "spa_launch.h"

namespace spa {


// ======================================================== decode: split-K

// Online-softmax partial of one K/V tile for the HPW query heads of a group:
// loads the tile into LDS once, then scores, (m, l) and acc per head.  All
// global loads are unconditional (rows past ntok are clamped to the last
// valid row and masked out of the softmax).
// kPublish: the partial is stored with agent-scope write-through stores (it
// is read back in the same kernel by the head's last workgroup).
template <typename T, int D, int HPW, bool kPublish = false>
__device__ __forceinline__ void tile_partial(const T* __restrict__ q, const T* __restrict__ kt,
                                             const T* __restrict__ vt, int bi, int hs, int G, int Hq,
                                             int share_group, int ntok, float bias, float* __restrict__ ws_acc,
                                             float2* __restrict__ ws_ml, int64_t obase) {
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kVPR = D / kVec;                     // 16-byte vectors per row
  constexpr int kPadRow = D + kVec;                  // padded LDS row (elements)
  constexpr int kIters = kTileTok * kVPR / 256;
  constexpr int kQIters = (HPW * D + 255) / 256;
  constexpr int kCPL = D / kWave;                    // output columns per lane
  __shared__ __align__(16) T s_k[kTileTok * kPadRow];
  __shared__ __align__(16) T s_v[kTileTok * D];
  __shared__ float s_q[HPW][D];
  __shared__ float s_p[HPW][kTileTok];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;

  // query heads first, then the K / V tile
  float qv[kQIters];
#pragma unroll
  for (int it = 0; it < kQIters; ++it) {
    int x = tid + it * 256;
    x = x < HPW * D ? x : HPW * D - 1;
    const int hh = x / D, e = x % D;
    const int hq = share_group ? hs * G + hh : hs;
    qv[it] = ld_f(q + (static_cast<int64_t>(bi) * Hq + hq) * D + e);
  }
  uint4 rk[kIters], rv[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int x = tid + it * 256;
    const int r = x / kVPR, cv = x % kVPR;
    const int rr = r < ntok ? r : ntok - 1;
    rk[it] = *reinterpret_cast<const uint4*>(kt + static_cast<int64_t>(rr) * D + cv * kVec);
    rv[it] = *reinterpret_cast<const uint4*>(vt + static_cast<int64_t>(rr) * D + cv * kVec);
  }
#pragma unroll
  for (int it = 0; it < kQIters; ++it) {
    const int x = tid + it * 256;
    if (x < HPW * D) s_q[x / D][x % D] = qv[it];
  }
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int x = tid + it * 256;
    const int r = x / kVPR, cv = x % kVPR;
    *reinterpret_cast<uint4*>(&s_k[r * kPadRow + cv * kVec]) = rk[it];
    *reinterpret_cast<uint4*>(&s_v[r * D + cv * kVec]) = rv[it];
  }
  __syncthreads();

  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  for (int h0 = 0; h0 < HPW; h0 += 4) {
    const int hh = h0 + wave;
    if (hh < HPW) {
      const int j = lane;
      float acc = 0.f;
#pragma unroll
      for (int cv = 0; cv < kVPR; ++cv) {
        float x[kVec];
        Elem<T>::unpack(*reinterpret_cast<const uint4*>(&s_k[j * kPadRow + cv * kVec]), x);
#pragma unroll
        for (int i = 0; i < kVec; ++i) acc = fmaf(x[i], s_q[hh][cv * kVec + i], acc);
      }
      const float z = j < ntok ? acc * scale + bias : -INFINITY;
      const float m = wave_max(z);
      const float p = j < ntok ? __expf(z - m) : 0.f;
      const float l = wave_sum(p);
      s_p[hh][j] = p;
      if (lane == 0) {
        if constexpr (kPublish)
          publish_f2(ws_ml + obase + hh, m, l);
        else
          ws_ml[obase + hh] = make_float2(m, l);
      }
    }
  }
  __syncthreads();
  for (int h0 = 0; h0 < HPW; h0 += 4) {
    const int hh = h0 + wave;
    if (hh < HPW) {
      // lane owns columns kCPL*lane .. +kCPL (adjacent, read together)
      float acc[kCPL];
#pragma unroll
      for (int c = 0; c < kCPL; ++c) acc[c] = 0.f;
#pragma unroll 16
      for (int j = 0; j < kTileTok; ++j) {
        const float pj = s_p[hh][j];                 // 0 beyond ntok
#pragma unroll
        for (int c = 0; c < kCPL; ++c) acc[c] = fmaf(pj, ld_f(&s_v[j * D + kCPL * lane + c]), acc[c]);
      }
      float* out = ws_acc + (obase + hh) * D + kCPL * lane;
      if constexpr (kPublish) {
        static_assert(kCPL == 1 || kCPL == 2, "columns per lane");
        if constexpr (kCPL == 2)
          publish_f2(out, acc[0], acc[1]);
        else
          publish_u32(out, __float_as_uint(acc[0]));
      } else {
#pragma unroll
        for (int c = 0; c < kCPL; ++c) out[c] = acc[c];
      }
    }
  }
}

// Split-K combine: one workgroup per (selection head, query head of its
// group).  All ntiles partial accumulators of that query head are staged in
// LDS with one round of independent loads, then each output element sums
// them with the softmax weights exp(m_t - M).

// Offset (elements) of the first of the rows [start, start + ntok) of
// (batch bi, kv head kvh) in the K / V cache, which never cross a block:
// contiguous [B, Hkv, L, d], or through the page table into a pool
// [npages, Hkv, b, d].  An unmapped page (id outside the pool) empties the
// tile (ntok = 0).
template <int D>
__device__ __forceinline__ int64_t kv_tile_offset(int bi, int kvh, int Hkv, int64_t L, int b, int64_t start,
                                                  int& ntok, const int32_t* __restrict__ table, int64_t tstride,
                                                  int64_t npages) {
  if (table == nullptr) return ((static_cast<int64_t>(bi) * Hkv + kvh) * L + start) * D;
  const int64_t blk = start / b;
  const int64_t pg = table[static_cast<int64_t>(bi) * tstride + blk];
  if (pg < 0 || pg >= npages) {
    ntok = 0;
    return 0;
  }
  return ((pg * Hkv + kvh) * b + (start - blk * b)) * D;
}

template <typename T, int D, int HPW>
__global__ __launch_bounds__(256) void decode_attn_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, int Hq, int Hkv, int Hsel,
    int share_group, int64_t L, int64_t pos, int b, int K, int tpu, float* __restrict__ ws_acc,
    float2* __restrict__ ws_ml, const int32_t* __restrict__ table, int64_t tstride, int64_t npages) {
  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int G = Hq / Hkv;
  const int kvh = share_group ? hs : hs / G;
  const int unit = blockIdx.x / tpu, sub = blockIdx.x % tpu;
  const int ntiles = (K + 1) * tpu;
  const int tile = blockIdx.x;

  int64_t start = 0;
  int ntok = 0;
  float bias = 0.f;
  const int64_t c0 = pos / b;
  if (unit < K) {
    const int32_t c = idx[static_cast<int64_t>(bh) * K + unit];
    if (c >= 0 && c < c0) {
      start = static_cast<int64_t>(c) * b + sub * kTileTok;
      ntok = b - sub * kTileTok < kTileTok ? b - sub * kTileTok : kTileTok;
      if (logg != nullptr) bias = logg[static_cast<int64_t>(bh) * K + unit];
    }
  } else {
    start = c0 * b + sub * kTileTok;
    const int64_t n = pos + 1 - start;
    const int cap = b - sub * kTileTok < kTileTok ? b - sub * kTileTok : kTileTok;
    ntok = n <= 0 ? 0 : (n < cap ? static_cast<int>(n) : cap);
  }

  const int64_t obase = (static_cast<int64_t>(bh) * ntiles + tile) * HPW;
  const int64_t off = ntok > 0 ? kv_tile_offset<D>(bi, kvh, Hkv, L, b, start, ntok, table, tstride, npages) : 0;
  if (ntok == 0) {
    for (int x = tid; x < HPW * D; x += 256) ws_acc[obase * D + x] = 0.f;
    if (tid < HPW) ws_ml[obase + tid] = make_float2(-INFINITY, 0.f);
  } else if constexpr (std::is_same<T, bf16_t>::value) {
    const int hq0 = share_group ? hs * G : hs;
    tile_partial_bf16<D, HPW, false>(q + (static_cast<int64_t>(bi) * Hq + hq0) * D, k + off, v + off, ntok, bias,
                                     ws_acc, ws_ml, obase);
  } else {
    tile_partial<T, D, HPW>(q, k + off, v + off, bi, hs, G, Hq, share_group, ntok, bias, ws_acc, ws_ml, obase);
  }
}

template <typename T, int D, int HPW>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ ws_acc,
                                                             const float2* __restrict__ ws_ml, int Hq,
                                                             int Hkv, int Hsel, int share_group,
                                                             int ntiles, T* __restrict__ o,
                                                             float* __restrict__ lse) {
  __shared__ __align__(16) float s_acc[kMaxTiles * D];
  __shared__ float2 s_ml[kMaxTiles];
  const int tid = threadIdx.x;
  const int hh = blockIdx.x, bh = blockIdx.y;
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int G = Hq / Hkv;
  const int64_t base = static_cast<int64_t>(bh) * ntiles * HPW;   // partial (tile t, head hh) at base + t*HPW + hh
  constexpr int kV4 = D / 4;
  const int n4 = ntiles * kV4;
#pragma unroll 8
  for (int x = tid; x < n4; x += 256) {
    const int t = x / kV4, c = x % kV4;
    reinterpret_cast<float4*>(s_acc)[x] = reinterpret_cast<const float4*>(ws_acc + (base + t * HPW + hh) * D)[c];
  }
  for (int t = tid; t < ntiles; t += 256) s_ml[t] = ws_ml[base + t * HPW + hh];
  __syncthreads();
  // softmax weights of the partials, once
  __shared__ float s_wt[kMaxTiles];
  __shared__ float s_M;
  if (tid < kWave) {
    float mloc = -INFINITY;
    for (int t = tid; t < ntiles; t += kWave) mloc = fmaxf(mloc, s_ml[t].x);
    const float M = wave_max(mloc);
    for (int t = tid; t < ntiles; t += kWave) {
      const float mt = s_ml[t].x;
      s_wt[t] = (M == -INFINITY || mt == -INFINITY) ? 0.f : __expf(mt - M);
    }
    if (tid == 0) s_M = M;
  }
  __syncthreads();
  if (tid >= D) return;
  const float M = s_M;
  float lsum = 0.f, acc = 0.f;
#pragma unroll 8
  for (int t = 0; t < ntiles; ++t) {
    const float w = s_wt[t];
    lsum = fmaf(s_ml[t].y, w, lsum);
    acc = fmaf(s_acc[t * D + tid], w, acc);
  }
  const int hq = share_group ? hs * G + hh : hs;
  const int64_t orow = static_cast<int64_t>(bi) * Hq + hq;   // one query row
  o[orow * D + tid] = Elem<T>::from_float(lsum > 0.f ? acc / lsum : 0.f);
  if (tid == 0 && lse != nullptr) lse[orow] = lsum > 0.f ? M + __logf(lsum) : -INFINITY;
}

// Decode of the two-branch head (one query row; local = NONE, window w,
// alpha): branch L over the selected units (tiles of 64 keys, each biased by
// its log gate when given), branch S over the window keys pos - w < j <= pos
// (tiles of 64 from the window's first key).  One workgroup per tile writes an
// online-softmax partial as the SAS decode does; the combine merges each
// branch on its own and mixes o = alpha o_L + (1 - alpha) o_S ("FreeSolo"
// review, two-branch head).  Units that are not candidates of the row (cells
// of the query block or later) are empty.
template <typename T, int D, int HPW>
__global__ __launch_bounds__(256) void decode_mix_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, int Hq, int Hkv, int Hsel,
    int share_group, int64_t L, int64_t pos, int b, int prefix_mode, int qblock, int K, int tpu, int window,
    int ntiles, float* __restrict__ ws_acc, float2* __restrict__ ws_ml) {
  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int G = Hq / Hkv;
  const int kvh = share_group ? hs : hs / G;
  const int tile = blockIdx.x;
  const int nsel = K * tpu;
  int64_t start = 0;
  int ntok = 0;
  float bias = 0.f;
  if (tile < nsel) {
    const int unit = tile / tpu, sub = tile % tpu;
    const int64_t ncand = prefix_mode == 0 ? pos / b : (static_cast<int64_t>(qblock) * (pos / qblock)) / b;
    const int32_t c = idx[static_cast<int64_t>(bh) * K + unit];
    if (c >= 0 && c < ncand) {
      start = static_cast<int64_t>(c) * b + sub * kTileTok;
      ntok = b - sub * kTileTok < kTileTok ? b - sub * kTileTok : kTileTok;
      if (logg != nullptr) bias = logg[static_cast<int64_t>(bh) * K + unit];
    }
  } else {
    const int64_t wlo = pos - window + 1 > 0 ? pos - window + 1 : 0;
    start = wlo + static_cast<int64_t>(tile - nsel) * kTileTok;
    const int64_t n = pos + 1 - start;
    ntok = n <= 0 ? 0 : (n < kTileTok ? static_cast<int>(n) : kTileTok);
  }
  const int64_t obase = (static_cast<int64_t>(bh) * ntiles + tile) * HPW;
  if (ntok == 0) {
    for (int x = tid; x < HPW * D; x += 256) ws_acc[obase * D + x] = 0.f;
    if (tid < HPW) ws_ml[obase + tid] = make_float2(-INFINITY, 0.f);
  } else {
    const int64_t off = ((static_cast<int64_t>(bi) * Hkv + kvh) * L + start) * D;
    tile_partial<T, D, HPW>(q, k + off, v + off, bi, hs, G, Hq, share_group, ntok, bias, ws_acc, ws_ml, obase);
  }
}

// Combine of the two branches: tiles [0, nsel) form branch L, the rest branch
// S; each is merged with its own max, then o = alpha o_L + (1 - alpha) o_S
// (o_L = 0 when branch L is empty); lse is branch L's.
template <typename T, int D, int HPW>
__global__ __launch_bounds__(256) void decode_mix_combine_kernel(const float* __restrict__ ws_acc,
                                                                 const float2* __restrict__ ws_ml, int Hq, int Hkv,
                                                                 int Hsel, int share_group, int nsel, int ntiles,
                                                                 const float* __restrict__ alpha, T* __restrict__ o,
                                                                 float* __restrict__ lse) {
  __shared__ __align__(16) float s_acc[kMaxTiles * D];
  __shared__ float2 s_ml[kMaxTiles];
  __shared__ float s_wt[kMaxTiles];
  __shared__ float s_M[2];
  const int tid = threadIdx.x;
  const int hh = blockIdx.x, bh = blockIdx.y;
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int G = Hq / Hkv;
  const int64_t base = static_cast<int64_t>(bh) * ntiles * HPW;
  constexpr int kV4 = D / 4;
  const int n4 = ntiles * kV4;
#pragma unroll 8
  for (int x = tid; x < n4; x += 256) {
    const int t = x / kV4, c = x % kV4;
    reinterpret_cast<float4*>(s_acc)[x] = reinterpret_cast<const float4*>(ws_acc + (base + t * HPW + hh) * D)[c];
  }
  for (int t = tid; t < ntiles; t += 256) s_ml[t] = ws_ml[base + t * HPW + hh];
  __syncthreads();
  if (tid < 2 * kWave) {
    // wave 0: branch L, wave 1: branch S
    const int br = tid / kWave, ln = tid % kWave;
    const int t0 = br == 0 ? 0 : nsel, t1 = br == 0 ? nsel : ntiles;
    float mloc = -INFINITY;
    for (int t = t0 + ln; t < t1; t += kWave) mloc = fmaxf(mloc, s_ml[t].x);
    const float M = wave_max(mloc);
    for (int t = t0 + ln; t < t1; t += kWave) {
      const float mt = s_ml[t].x;
      s_wt[t] = (M == -INFINITY || mt == -INFINITY) ? 0.f : __expf(mt - M);
    }
    if (ln == 0) s_M[br] = M;
  }
  __syncthreads();
  if (tid >= D) return;
  float lsum[2] = {0.f, 0.f}, acc[2] = {0.f, 0.f};
  for (int t = 0; t < ntiles; ++t) {
    const int br = t < nsel ? 0 : 1;
    const float w = s_wt[t];
    lsum[br] = fmaf(s_ml[t].y, w, lsum[br]);
    acc[br] = fmaf(s_acc[t * D + tid], w, acc[br]);
  }
  const int hq = share_group ? hs * G + hh : hs;
  const float a = alpha[hq];
  const float oL = lsum[0] > 0.f ? acc[0] / lsum[0] : 0.f;
  const float oS = lsum[1] > 0.f ? acc[1] / lsum[1] : 0.f;
  const int64_t orow = static_cast<int64_t>(bi) * Hq + hq;   // one query row
  o[orow * D + tid] = Elem<T>::from_float(a * oL + (1.f - a) * oS);
  if (tid == 0 && lse != nullptr) lse[orow] = lsum[0] > 0.f ? s_M[0] + __logf(lsum[0]) : -INFINITY;
}

// ======================================================== rows: forward
struct OnlineState {
  float m, l;
};

// Attend the keys [start, start + n) of one row (one wave), updating the
// running (m, l) and the lane's accumulator columns lane + 64 t.
template <typename T, int D>
__device__ __forceinline__ void attend_segment(const T* __restrict__ kbase, const T* __restrict__ vbase,
                                               const float* s_q, int64_t start, int64_t n,
                                               float bias, float scale, int lane, OnlineState& st,
                                               float (&acc)[D / kWave]) {
  constexpr int kVec = Elem<T>::kVec;
  for (int64_t off = 0; off < n; off += kWave) {
    const int64_t cnt = n - off < kWave ? n - off : kWave;
    const int64_t key = start + off + lane;
    float z = -INFINITY;
    if (lane < cnt) {
      const T* kr = kbase + key * D;
      float a = 0.f;
#pragma unroll
      for (int cv = 0; cv < D / kVec; ++cv) {
        float x[kVec];
        Elem<T>::unpack(*reinterpret_cast<const uint4*>(kr + cv * kVec), x);
#pragma unroll
        for (int i = 0; i < kVec; ++i) a = fmaf(x[i], s_q[cv * kVec + i], a);
      }
      z = a * scale + bias;
    }
    const float mc = wave_max(z);
    const float mn = fmaxf(st.m, mc);
    const float corr = __expf(st.m - mn);
    const float p = lane < cnt ? __expf(z - mn) : 0.f;
    st.l = st.l * corr + wave_sum(p);
    st.m = mn;
#pragma unroll
    for (int t = 0; t < D / kWave; ++t) acc[t] *= corr;
    for (int jj = 0; jj < cnt; ++jj) {
      const float pj = __shfl(p, jj, kWave);
      const T* vr = vbase + (start + off + jj) * D;
#pragma unroll
      for (int t = 0; t < D / kWave; ++t) acc[t] = fmaf(pj, ld_f(vr + lane + t * kWave), acc[t]);
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void rows_attn_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, const float* __restrict__ alpha,
    int Hq, int Hkv, int Hsel, int share_group, int nq, int64_t q_pos0, int64_t L, int b,
    int prefix_mode, int qblock, int K, int local, int window, T* __restrict__ o,
    float* __restrict__ lse) {
  __shared__ float s_q[4][D];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int row = blockIdx.x * 4 + wave;
  if (row >= nq) return;
  const int bh = blockIdx.y;
  const int bi = bh / Hq, h = bh % Hq;
  const int G = Hq / Hkv;
  const int kvh = h / G;
  const int hs = share_group ? kvh : h;
  const int64_t i = q_pos0 + row;
  const int64_t qrow = (static_cast<int64_t>(bi) * Hq + h) * nq + row;
  for (int e = lane; e < D; e += kWave) s_q[wave][e] = ld_f(q + qrow * D + e);
  wave_lds_sync();

  const T* kb = k + (static_cast<int64_t>(bi) * Hkv + kvh) * L * D;
  const T* vb = v + (static_cast<int64_t>(bi) * Hkv + kvh) * L * D;
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const int64_t ncand = num_candidates(i, b, prefix_mode, qblock);
  const int64_t so = ((static_cast<int64_t>(bi) * Hsel + hs) * nq + row) * K;

  OnlineState st{-INFINITY, 0.f};
  float acc[D / kWave];
#pragma unroll
  for (int t = 0; t < D / kWave; ++t) acc[t] = 0.f;
  if (local == 0) {
    const int64_t c0 = i / b;
    attend_segment<T, D>(kb, vb, s_q[wave], c0 * b, i - c0 * b + 1, 0.f, scale, lane, st, acc);
  }
  for (int t = 0; t < K; ++t) {
    const int32_t c = idx[so + t];
    if (c < 0 || c >= ncand) continue;
    const float bias = logg != nullptr ? logg[so + t] : 0.f;
    attend_segment<T, D>(kb, vb, s_q[wave], static_cast<int64_t>(c) * b, b, bias, scale, lane, st, acc);
  }
  const float invl = st.l > 0.f ? 1.f / st.l : 0.f;
  float out[D / kWave];
#pragma unroll
  for (int t = 0; t < D / kWave; ++t) out[t] = acc[t] * invl;
  if (lse != nullptr && lane == 0) lse[qrow] = st.l > 0.f ? st.m + __logf(st.l) : -INFINITY;

  if (window > 0 && alpha != nullptr) {
    OnlineState sw{-INFINITY, 0.f};
    float accw[D / kWave];
#pragma unroll
    for (int t = 0; t < D / kWave; ++t) accw[t] = 0.f;
    const int64_t j0 = i - window + 1 > 0 ? i - window + 1 : 0;
    attend_segment<T, D>(kb, vb, s_q[wave], j0, i - j0 + 1, 0.f, scale, lane, sw, accw);
    const float a = alpha[h];
    const float invw = sw.l > 0.f ? 1.f / sw.l : 0.f;
#pragma unroll
    for (int t = 0; t < D / kWave; ++t) out[t] = a * out[t] + (1.f - a) * (accw[t] * invw);
  }
#pragma unroll
  for (int t = 0; t < D / kWave; ++t) o[qrow * D + lane + t * kWave] = Elem<T>::from_float(out[t]);
}

// ======================================================== rows: backward
// D_i = do_i . o_i: D / kVec lanes per row, one 16-byte vector of o and of
// dout each, summed over the row's lanes.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                      int64_t rows, float* __restrict__ Dbuf) {
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kLPR = D / kVec;            // lanes per row
  constexpr int kRPB = 256 / kLPR;          // rows per workgroup
  const int tid = threadIdx.x;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kRPB + tid / kLPR;
  const int cg = tid % kLPR;
  float a = 0.f;
  if (r < rows) {
    float x[kVec], y[kVec];
    Elem<T>::unpack(*reinterpret_cast<const uint4*>(o + r * D + cg * kVec), x);
    Elem<T>::unpack(*reinterpret_cast<const uint4*>(dout + r * D + cg * kVec), y);
#pragma unroll
    for (int i = 0; i < kVec; ++i) a = fmaf(x[i], y[i], a);
  }
  a = group_sum<kLPR>(a);
  if (r < rows && cg == 0) Dbuf[r] = a;
}

// dq and the block sums of dS for one segment of keys (one wave)
template <typename T, int D>
__device__ __forceinline__ float dq_segment(const T* __restrict__ kbase, const T* __restrict__ vbase,
                                            const float* s_q, const float* s_do, int64_t start,
                                            int64_t n, float bias, float scale, float lse_i,
                                            float D_i, int lane, float (&dq)[D / kWave]) {
  constexpr int kVec = Elem<T>::kVec;
  float dsum = 0.f;
  for (int64_t off = 0; off < n; off += kWave) {
    const int64_t cnt = n - off < kWave ? n - off : kWave;
    const int64_t key = start + off + lane;
    float ds = 0.f;
    if (lane < cnt) {
      const T* kr = kbase + key * D;
      const T* vr = vbase + key * D;
      float a = 0.f, dp = 0.f;
#pragma unroll
      for (int cv = 0; cv < D / kVec; ++cv) {
        float x[kVec], y[kVec];
        Elem<T>::unpack(*reinterpret_cast<const uint4*>(kr + cv * kVec), x);
        Elem<T>::unpack(*reinterpret_cast<const uint4*>(vr + cv * kVec), y);
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
          a = fmaf(x[i], s_q[cv * kVec + i], a);
          dp = fmaf(y[i], s_do[cv * kVec + i], dp);
        }
      }
      const float p = __expf(a * scale + bias - lse_i);
      ds = p * (dp - D_i);
    }
    dsum += wave_sum(ds);
    for (int jj = 0; jj < cnt; ++jj) {
      const float dsj = __shfl(ds, jj, kWave);
      const T* kr = kbase + (start + off + jj) * D;
#pragma unroll
      for (int t = 0; t < D / kWave; ++t) dq[t] = fmaf(dsj, ld_f(kr + lane + t * kWave), dq[t]);
    }
  }
  return dsum;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dbuf,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, int Hq, int Hkv, int Hsel,
    int share_group, int nq, int64_t q_pos0, int64_t L, int b, int K, T* __restrict__ dq,
    float* __restrict__ dg) {
  __shared__ float s_q[4][D];
  __shared__ float s_do[4][D];
  __shared__ float s_dg[4][64];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int row = blockIdx.x * 4 + wave;
  if (row >= nq) return;
  const int bh = blockIdx.y;                 // b * Hsel + hs
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int G = Hq / Hkv;
  const int kvh = share_group ? hs : hs / G;
  const int nheads = share_group ? G : 1;
  const int64_t i = q_pos0 + row;
  const int64_t so = (static_cast<int64_t>(bh) * nq + row) * K;
  const T* kb = k + (static_cast<int64_t>(bi) * Hkv + kvh) * L * D;
  const T* vb = v + (static_cast<int64_t>(bi) * Hkv + kvh) * L * D;
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const int64_t ncand = i / b;
  const int64_t c0 = i / b;
  s_dg[wave][lane] = 0.f;

  for (int hh = 0; hh < nheads; ++hh) {
    const int h = share_group ? hs * G + hh : hs;
    const int64_t qrow = (static_cast<int64_t>(bi) * Hq + h) * nq + row;
    wave_lds_sync();
    for (int e = lane; e < D; e += kWave) {
      s_q[wave][e] = ld_f(q + qrow * D + e);
      s_do[wave][e] = ld_f(dout + qrow * D + e);
    }
    wave_lds_sync();
    const float lse_i = lse[qrow], D_i = Dbuf[qrow];
    float dqa[D / kWave];
#pragma unroll
    for (int t = 0; t < D / kWave; ++t) dqa[t] = 0.f;
    dq_segment<T, D>(kb, vb, s_q[wave], s_do[wave], c0 * b, i - c0 * b + 1, 0.f, scale, lse_i, D_i,
                     lane, dqa);
    for (int t = 0; t < K; ++t) {
      const int32_t c = idx[so + t];
      if (c < 0 || c >= ncand) continue;
      const float bias = logg != nullptr ? logg[so + t] : 0.f;
      const float sum = dq_segment<T, D>(kb, vb, s_q[wave], s_do[wave], static_cast<int64_t>(c) * b, b,
                                         bias, scale, lse_i, D_i, lane, dqa);
      if (lane == 0) s_dg[wave][t] += sum;
    }
#pragma unroll
    for (int t = 0; t < D / kWave; ++t)
      dq[qrow * D + lane + t * kWave] = Elem<T>::from_float(dqa[t] * scale);
  }
  wave_lds_sync();
  if (lane < K) {
    const int32_t c = idx[so + lane];
    float g = 0.f;
    if (c >= 0 && c < ncand) {
      const float lg = logg != nullptr ? logg[so + lane] : 0.f;
      g = s_dg[wave][lane] * __expf(-lg);
    }
    dg[so + lane] = g;
  }
}

// dk, dv of one key block: every (query head, row) that reads the block is
// gathered in row order (current-block rows first, then rows that selected
// the block, found by an ordered compaction) so the sums are deterministic.
// 256 threads: key j of the block = tid / (256/BS), columns split over the
// 256/BS lanes that share a key.
template <typename T, int D, int BS>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dbuf,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, int Hq, int Hkv, int Hsel,
    int share_group, int nq, int64_t q_pos0, int64_t L, int K, T* __restrict__ dk,
    T* __restrict__ dv) {
  constexpr int kParts = 256 / BS;           // lanes sharing one key
  constexpr int kCP = D / kParts;            // columns per lane
  static_assert(kCP >= 1 && kCP <= 32, "block size out of range for this kernel");
  __shared__ int s_row[256];
  __shared__ float s_bias[256];
  __shared__ int s_wcount[4];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int j = tid / kParts, part = tid % kParts;
  const int64_t c = blockIdx.x;
  const int bkv = blockIdx.y;
  const int bi = bkv / Hkv, kvh = bkv % Hkv;
  const int G = Hq / Hkv;
  const int64_t kpos = c * BS + j;
  const bool kvalid = kpos < L;
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const int64_t kvoff = ((static_cast<int64_t>(bi) * Hkv + kvh) * L + (kvalid ? kpos : 0)) * D + part * kCP;

  float kr[kCP], vr[kCP], dka[kCP], dva[kCP];
#pragma unroll
  for (int t = 0; t < kCP; ++t) {
    kr[t] = kvalid ? ld_f(k + kvoff + t) : 0.f;
    vr[t] = kvalid ? ld_f(v + kvoff + t) : 0.f;
    dka[t] = 0.f;
    dva[t] = 0.f;
  }

  auto process = [&](int h, int row, float bias, bool causal) {
    const int64_t qrow = (static_cast<int64_t>(bi) * Hq + h) * nq + row;
    const T* qp = q + qrow * D + part * kCP;
    const T* dp = dout + qrow * D + part * kCP;
    float a = 0.f, dpv = 0.f;
#pragma unroll
    for (int t = 0; t < kCP; ++t) {
      a = fmaf(ld_f(qp + t), kr[t], a);
      dpv = fmaf(ld_f(dp + t), vr[t], dpv);
    }
#pragma unroll
    for (int m = 1; m < kParts; m <<= 1) {
      a += __shfl_xor(a, m, kWave);
      dpv += __shfl_xor(dpv, m, kWave);
    }
    const int64_t ipos = q_pos0 + row;
    if (kvalid && (!causal || kpos <= ipos)) {
      const float p = __expf(a * scale + bias - lse[qrow]);
      const float ds = p * (dpv - Dbuf[qrow]) * scale;
#pragma unroll
      for (int t = 0; t < kCP; ++t) {
        dka[t] = fmaf(ds, ld_f(qp + t), dka[t]);
        dva[t] = fmaf(p, ld_f(dp + t), dva[t]);
      }
    }
  };

  for (int g = 0; g < G; ++g) {
    const int h = kvh * G + g;
    const int hs = share_group ? kvh : h;
    // (a) rows whose current block is c
    {
      int64_t r0 = c * BS - q_pos0, r1 = c * BS + BS - q_pos0;
      if (r0 < 0) r0 = 0;
      if (r1 > nq) r1 = nq;
      for (int64_t r = r0; r < r1; ++r) process(h, static_cast<int>(r), 0.f, true);
    }
    // (b) rows after block c that selected it
    int64_t rstart = (c + 1) * BS - q_pos0;
    if (rstart < 0) rstart = 0;
    for (int64_t r0 = rstart; r0 < nq; r0 += 256) {
      const int64_t r = r0 + tid;
      int slot = -1;
      if (r < nq) {
        const int32_t* ir = idx + ((static_cast<int64_t>(bi) * Hsel + hs) * nq + r) * K;
        for (int t = 0; t < K; ++t)
          if (ir[t] == static_cast<int32_t>(c)) { slot = t; break; }
      }
      const bool hit = slot >= 0;
      const uint64_t mask = __ballot(hit);
      const int before = __popcll(mask & ((1ull << lane) - 1ull));
      __syncthreads();
      if (lane == 0) s_wcount[wave] = __popcll(mask);
      __syncthreads();
      int base = 0;
      for (int w = 0; w < wave; ++w) base += s_wcount[w];
      const int total = s_wcount[0] + s_wcount[1] + s_wcount[2] + s_wcount[3];
      if (hit) {
        s_row[base + before] = static_cast<int>(r);
        s_bias[base + before] =
            logg != nullptr ? logg[((static_cast<int64_t>(bi) * Hsel + hs) * nq + r) * K + slot] : 0.f;
      }
      __syncthreads();
      for (int x = 0; x < total; ++x) process(h, s_row[x], s_bias[x], false);
    }
  }
  if (kvalid) {
#pragma unroll
    for (int t = 0; t < kCP; ++t) {
      dk[kvoff + t] = Elem<T>::from_float(dka[t]);
      dv[kvoff + t] = Elem<T>::from_float(dva[t]);
    }
  }
}

// ======================================================== launchers
static bool use_decode_attn(const AttnLaunch& p) {
  return p.nq == 1 && p.local == 0 && p.window == 0 && p.alpha == nullptr && p.b <= 128;
}

static int decode_tpu(const AttnLaunch& p) { return decode_step_tpu(p); }

static int heads_per_wg(const AttnLaunch& p) { return p.share_group ? p.Hq / p.Hkv : 1; }

// two-branch decode: selected-unit tiles, then the window's tiles
static int mix_tiles(const AttnLaunch& p) {
  return p.K * decode_tpu(p) + (p.window + kTileTok - 1) / kTileTok;
}

static bool use_decode_mix(const AttnLaunch& p) {
  return p.nq == 1 && p.local == 1 && p.window > 0 && p.alpha != nullptr && p.b <= 128 &&
         p.pages.table == nullptr && mix_tiles(p) <= kMaxTiles;
}

size_t attn_fwd_workspace_bytes(const AttnLaunch& p) {
  const bool mix = use_decode_mix(p);
  if (!use_decode_attn(p) && !mix) return attn_tile_fwd_supported(p) ? attn_tile_fwd_workspace_bytes(p) : 0;
  const size_t heads = static_cast<size_t>(p.B) * p.Hsel;
  const size_t ntiles = mix ? static_cast<size_t>(mix_tiles(p)) : static_cast<size_t>(p.K + 1) * decode_tpu(p);
  const size_t hpw = heads_per_wg(p);
  return align256(heads * ntiles * hpw * p.d * sizeof(float)) +
         align256(heads * ntiles * hpw * sizeof(float2));
}

size_t decode_step_workspace_bytes(const AttnLaunch& p) {
  return attn_fwd_workspace_bytes(p) + align256(static_cast<size_t>(p.B) * p.Hsel * sizeof(uint32_t));
}

size_t attn_bwd_workspace_bytes(const BwdLaunch& p) {
  const size_t dbuf = align256(static_cast<size_t>(p.a.B) * p.a.Hq * p.a.nq * sizeof(float));
  return attn_tile_bwd_supported(p) ? dbuf + attn_tile_bwd_bitmap_bytes(p) : dbuf;
}

template <typename T, int D, int HPW>
static hipError_t launch_decode_attn_h(const AttnLaunch& p, void* ws, hipStream_t st) {
  const int tpu = decode_tpu(p);
  const int ntiles = (p.K + 1) * tpu;
  const size_t heads = static_cast<size_t>(p.B) * p.Hsel;
  char* base = static_cast<char*>(ws);
  float* acc = reinterpret_cast<float*>(base);
  float2* ml = reinterpret_cast<float2*>(base + align256(heads * ntiles * HPW * p.d * sizeof(float)));
  hipError_t e = launch(false, decode_attn_partial_kernel<T, D, HPW>, dim3(ntiles, static_cast<unsigned>(heads)),
                        dim3(256), st, static_cast<const T*>(p.q), static_cast<const T*>(p.k),
                        static_cast<const T*>(p.v), p.idx, p.logg, p.Hq, p.Hkv, p.Hsel, p.share_group, p.L,
                        p.q_pos0, p.b, p.K, tpu, acc, ml, p.pages.table, p.pages.tstride, p.pages.npages);
  if (e != hipSuccess) return e;
  return launch(true, decode_combine_kernel<T, D, HPW>, dim3(HPW, static_cast<unsigned>(heads)), dim3(256), st,
                acc, ml, p.Hq, p.Hkv, p.Hsel, p.share_group, ntiles, static_cast<T*>(p.o), p.lse);
}

template <typename T, int D, int HPW>
static hipError_t launch_decode_mix_h(const AttnLaunch& p, void* ws, hipStream_t st) {
  const int tpu = decode_tpu(p);
  const int ntiles = mix_tiles(p);
  const size_t heads = static_cast<size_t>(p.B) * p.Hsel;
  char* base = static_cast<char*>(ws);
  float* acc = reinterpret_cast<float*>(base);
  float2* ml = reinterpret_cast<float2*>(base + align256(heads * ntiles * HPW * p.d * sizeof(float)));
  hipError_t e = launch(false, decode_mix_partial_kernel<T, D, HPW>, dim3(ntiles, static_cast<unsigned>(heads)),
                        dim3(256), st, static_cast<const T*>(p.q), static_cast<const T*>(p.k),
                        static_cast<const T*>(p.v), p.idx, p.logg, p.Hq, p.Hkv, p.Hsel, p.share_group, p.L,
                        p.q_pos0, p.b, p.prefix_mode, p.qblock, p.K, tpu, p.window, ntiles, acc, ml);
  if (e != hipSuccess) return e;
  return launch(true, decode_mix_combine_kernel<T, D, HPW>, dim3(HPW, static_cast<unsigned>(heads)), dim3(256),
                st, acc, ml, p.Hq, p.Hkv, p.Hsel, p.share_group, p.K * tpu, ntiles, p.alpha, static_cast<T*>(p.o),
                p.lse);
}

template <typename T, int D>
static hipError_t launch_decode_mix_t(const AttnLaunch& p, void* ws, hipStream_t st) {
  switch (heads_per_wg(p)) {
    case 1: return launch_decode_mix_h<T, D, 1>(p, ws, st);
    case 2: return launch_decode_mix_h<T, D, 2>(p, ws, st);
    case 4: return launch_decode_mix_h<T, D, 4>(p, ws, st);
    default: return launch_decode_mix_h<T, D, 8>(p, ws, st);
  }
}

template <typename T, int D>
static hipError_t launch_decode_attn_t(const AttnLaunch& p, void* ws, hipStream_t st) {
  switch (heads_per_wg(p)) {
    case 1: return launch_decode_attn_h<T, D, 1>(p, ws, st);
    case 2: return launch_decode_attn_h<T, D, 2>(p, ws, st);
    case 4: return launch_decode_attn_h<T, D, 4>(p, ws, st);
    default: return launch_decode_attn_h<T, D, 8>(p, ws, st);
  }
}

template <typename T, int D>
static hipError_t launch_rows_fwd_t(const AttnLaunch& p, hipStream_t st) {
  dim3 grid((p.nq + 3) / 4, static_cast<unsigned>(p.B * p.Hq));
  return launch(true, rows_attn_fwd_kernel<T, D>, grid, dim3(256), st, static_cast<const T*>(p.q),
                static_cast<const T*>(p.k), static_cast<const T*>(p.v), p.idx, p.logg, p.alpha, p.Hq,
                p.Hkv, p.Hsel, p.share_group, p.nq, p.q_pos0, p.L, p.b, p.prefix_mode, p.qblock, p.K,
                p.local, p.window, static_cast<T*>(p.o), p.lse);
}

hipError_t launch_attn_fwd(const AttnLaunch& p, void* ws, hipStream_t st) {
  if (use_decode_attn(p)) {
    if (p.dtype == 1) return p.d == 64 ? launch_decode_attn_t<bf16_t, 64>(p, ws, st) : launch_decode_attn_t<bf16_t, 128>(p, ws, st);
    return p.d == 64 ? launch_decode_attn_t<float, 64>(p, ws, st) : launch_decode_attn_t<float, 128>(p, ws, st);
  }
  if (use_decode_mix(p)) {
    if (p.dtype == 1) return p.d == 64 ? launch_decode_mix_t<bf16_t, 64>(p, ws, st) : launch_decode_mix_t<bf16_t, 128>(p, ws, st);
    return p.d == 64 ? launch_decode_mix_t<float, 64>(p, ws, st) : launch_decode_mix_t<float, 128>(p, ws, st);
  }
  if (attn_tile_fwd_supported(p)) return launch_attn_tile_fwd(p, ws, st);
  if (p.dtype == 1) return p.d == 64 ? launch_rows_fwd_t<bf16_t, 64>(p, st) : launch_rows_fwd_t<bf16_t, 128>(p, st);
  return p.d == 64 ? launch_rows_fwd_t<float, 64>(p, st) : launch_rows_fwd_t<float, 128>(p, st);
}

template <typename T, int D>
static hipError_t launch_bwd_t(const BwdLaunch& p, void* ws, hipStream_t st) {
  const AttnLaunch& a = p.a;
  float* Dbuf = static_cast<float*>(ws);
  const int64_t rows = static_cast<int64_t>(a.B) * a.Hq * a.nq;
  constexpr int kPreRows = 256 / (D / Elem<T>::kVec);
  hipError_t e = launch(false, bwd_pre_kernel<T, D>, dim3(static_cast<unsigned>((rows + kPreRows - 1) / kPreRows)),
                        dim3(256), st, static_cast<const T*>(p.o), static_cast<const T*>(p.dout), rows, Dbuf);
  if (e != hipSuccess) return e;
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (attn_tile_bwd_supported(p)) {
      uint32_t* bits = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) +
                                                   align256(static_cast<size_t>(rows) * sizeof(float)));
      return launch_attn_tile_bwd(p, Dbuf, bits, st);
    }
  }
  e = launch(false, bwd_dq_kernel<T, D>, dim3((a.nq + 3) / 4, static_cast<unsigned>(a.B * a.Hsel)), dim3(256),
             st, static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
             static_cast<const T*>(p.dout), p.lse, Dbuf, a.idx, a.logg, a.Hq, a.Hkv, a.Hsel, a.share_group,
             a.nq, a.q_pos0, a.L, a.b, a.K, static_cast<T*>(p.dq), p.dg);
  if (e != hipSuccess) return e;
  const int64_t nblk = (a.L + a.b - 1) / a.b;
  const dim3 grid(static_cast<unsigned>(nblk), static_cast<unsigned>(a.B * a.Hkv));
  auto kern = a.b == 16 ? bwd_dkdv_kernel<T, D, 16> : (a.b == 32 ? bwd_dkdv_kernel<T, D, 32>
                                                                  : bwd_dkdv_kernel<T, D, 64>);
  return launch(true, kern, grid, dim3(256), st, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                static_cast<const T*>(a.v), static_cast<const T*>(p.dout), p.lse, Dbuf, a.idx, a.logg,
                a.Hq, a.Hkv, a.Hsel, a.share_group, a.nq, a.q_pos0, a.L, a.K, static_cast<T*>(p.dk),
                static_cast<T*>(p.dv));
}

hipError_t launch_attn_bwd(const BwdLaunch& p, void* ws, hipStream_t st) {
  if (p.a.dtype == 1) return p.a.d == 64 ? launch_bwd_t<bf16_t, 64>(p, ws, st) : launch_bwd_t<bf16_t, 128>(p, ws, st);
  return p.a.d == 64 ? launch_bwd_t<float, 64>(p, ws, st) : launch_bwd_t<float, 128>(p, ws, st);
}

}  // namespace spa
