// decode_merge.h -- the two-level top-K merge of the decode path's chunk
// winners, shared by the merge kernel and the fused merge + attention kernel.
// Order: score desc, lower index first on ties ("SAS" review Alg. 1 ranks the
// blocks by score; the tie rule and ascending output are this library's);
// gate log g = s - LSE over every candidate ("SAS" review §4.2.2).
//
// Top-K by threshold: the k-th largest score T is found with a bitwise search
// over ballot counts (wave_kth_largest); the kept set is every score > T plus
// the lowest-index scores == T.  Candidates are laid out so that position
// order is index order, which makes the lower-index tie rule and the ascending
// output a single ordered compaction (ballot + mbcnt).
#pragma once

#include "spa_device.h"

namespace spa {

// Ordered compaction of one wave's NV x 64 positions (position i*64 + lane):
// keeps keys > t and the first `need_eq` keys == t; calls emit(slot, i) for
// every kept position.  Returns the number kept.
template <int NV, typename Emit>
__device__ __forceinline__ int wave_select_ordered(const uint32_t (&key)[NV], uint32_t t, int need_eq,
                                                   Emit&& emit) {
  int kept = 0, eq_seen = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint64_t eq = __ballot(key[i] == t && key[i] != 0u);
    const bool take = key[i] > t || (key[i] == t && key[i] != 0u && eq_seen + lanes_below(eq) < need_eq);
    const uint64_t tm = __ballot(take);
    if (take) emit(kept + lanes_below(tm), i);
    kept += __popcll(tm);
    eq_seen += __popcll(eq);
  }
  return kept;
}

// Level 1 of the merge, all four waves: wave w keeps the top-min(K, valid)
// records of its quarter of the chunks (records laid out chunk by chunk, each
// in index order) in index order in s_win[w K ..] (0 padded); lane 0 writes
// the wave's share of the (max, sum exp) partials to s_ml[w] and to s_lo[w]
// a lower bound of the overall K-th largest key (its own top-K threshold if
// it held K valid records, else 0).  NV = records per lane in a quarter.  The
// caller synchronises before level 2.
template <int NV>
__device__ __forceinline__ void merge_level1(const uint64_t* __restrict__ rec, const float2* __restrict__ mlp,
                                             int nchunks, int K, uint64_t* s_win, float2* s_ml, uint32_t* s_lo) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int c0 = (nchunks * wave) / 4, c1 = (nchunks * (wave + 1)) / 4;
  const int n = (c1 - c0) * K;
  uint64_t r[NV];
  uint32_t key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int pidx = i * kWave + lane;
    r[i] = pidx < n ? rec[static_cast<int64_t>(c0) * K + pidx] : 0ull;
  }
  float m = -INFINITY, l = 0.f;
  for (int ch = tid; ch < nchunks; ch += 256) {
    const float2 v = mlp[ch];
    ml_combine(m, l, v.x, v.y);
  }
  {
    float m2 = xor_lanes_f<32>(m), l2 = xor_lanes_f<32>(l); ml_combine(m, l, m2, l2);
    m2 = xor_lanes_f<16>(m); l2 = xor_lanes_f<16>(l); ml_combine(m, l, m2, l2);
    m2 = xor_lanes_f<8>(m); l2 = xor_lanes_f<8>(l); ml_combine(m, l, m2, l2);
    m2 = xor_lanes_f<4>(m); l2 = xor_lanes_f<4>(l); ml_combine(m, l, m2, l2);
    m2 = xor_lanes_f<2>(m); l2 = xor_lanes_f<2>(l); ml_combine(m, l, m2, l2);
    m2 = xor_lanes_f<1>(m); l2 = xor_lanes_f<1>(l); ml_combine(m, l, m2, l2);
  }
  if (lane == 0) s_ml[wave] = make_float2(m, l);
  int nvalid = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    key[i] = static_cast<uint32_t>(r[i] >> 32);
    nvalid += __popcll(__ballot(key[i] != 0u));
  }
  const int k1 = nvalid < K ? nvalid : K;
  const uint32_t t1 = wave_kth_largest<NV>(key, k1);
  int ngt1 = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) ngt1 += __popcll(__ballot(key[i] > t1));
  const int kept1 = wave_select_ordered<NV>(key, t1, k1 - ngt1, [&](int slot, int i) {
    s_win[wave * K + slot] = r[i];
  });
  for (int x = kept1 + lane; x < K; x += kWave) s_win[wave * K + x] = 0ull;
  if (lane == 0) s_lo[wave] = k1 == K ? t1 : 0u;
}

// Level 2 of the merge, one wave: the top-kk (kk = min(K, candidates)) of the
// 4 K level-1 survivors; calls emit(slot, block, log g) for slots 0 .. kept-1
// in ascending block order (log g = 0 with the gate off) and returns kept.
// NV2 x 64 >= 4 K.
template <int NV2, typename Emit>
__device__ __forceinline__ int merge_level2(const uint64_t* s_win, const float2* s_ml, const uint32_t* s_lo, int K,
                                            int kk, int gate, Emit&& emit) {
  const int lane = threadIdx.x % kWave;
  float mm = s_ml[0].x, ll = s_ml[0].y;
  for (int w = 1; w < 4; ++w) ml_combine(mm, ll, s_ml[w].x, s_ml[w].y);
  const float lse = mm + __logf(ll);
  uint64_t r2[NV2];
  uint32_t key2[NV2];
#pragma unroll
  for (int i = 0; i < NV2; ++i) {
    const int pidx = i * kWave + lane;
    r2[i] = pidx < 4 * K ? s_win[pidx] : 0ull;
    key2[i] = static_cast<uint32_t>(r2[i] >> 32);
  }
  // the K-th largest lies between the best level-1 threshold and the top key
  uint32_t lo = s_lo[0];
  for (int w = 1; w < 4; ++w) lo = s_lo[w] > lo ? s_lo[w] : lo;
  const uint32_t t = wave_kth_largest<NV2>(key2, kk, lo, wave_max_key<NV2>(key2));
  int ngt = 0;
#pragma unroll
  for (int i = 0; i < NV2; ++i) ngt += __popcll(__ballot(key2[i] > t));
  return wave_select_ordered<NV2>(key2, t, kk - ngt, [&](int slot, int i) {
    emit(slot, static_cast<int32_t>(static_cast<uint32_t>(r2[i])), gate ? from_orderable_f32(key2[i]) - lse : 0.f);
  });
}

}  // namespace spa
