// decode_step.hip -- the one-call decode step (one query row, bf16): top-K
// block selection with the softmax log gate, then exact attention over the
// current block and the selected blocks ("SAS" review §3 Eq. 3, Alg. 1,
// §4.1 Eq. 4, §4.2.2, §4.3 Eq. 9; "Monodratic" news page: guaranteed local
// block, exact softmax on the selected set), in two kernels:
//
//  1. decode_score_kernel (select.hip): every candidate block's score, each
//     chunk's (max, sum exp) and each 64-block group's largest score.
//  2. decode_step_kernel (here): one workgroup per (selection head, kept
//     tile).  The workgroups of selected slots each select the head's top-K
//     from the scores, attend to their tile (tile_partial_bf16) and publish
//     the split-K partial; the head's last workgroup to finish combines.
//
// Selection without a merge of chunk winners: the groups are disjoint, so the
// K-th largest of the 64-block group maxima is a lower bound of the K-th
// largest score (with fewer than 2 K groups, a bound from the threads' maxima
// takes its place).  Only the scores at or above it survive (about 1.2 K for
// unclustered scores); each of up to 256 survivors is ranked by counting the
// survivors with a larger 64-bit key (score, then lower index first); with
// more (scores clustered or tied near the bound) the whole workgroup searches
// the K-th key over every candidate.  Either way the result is the exact
// top-K_eff, stored ascending.
#include <type_traits>

#include "decode_tile.h"
#include "spa_device.h"
#include "spa_launch.h"

namespace spa {

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = shfl_xor_u64(v, off);
    v = o > v ? o : v;
  }
  return v;
}

// Block-wide k-th largest of the keys of candidates tid + 256 j (j < n):
// (hk[j] << 32 | ~candidate), 0 where hk[j] = 0, distinct otherwise; the
// answer lies in [lo, hi].  s_part is LDS scratch of 2 x 4 counts.
template <int NJ>
__device__ __forceinline__ uint64_t block_kth_largest_u64(const uint32_t (&hk)[NJ], int n, int k, uint64_t lo,
                                                          uint64_t hi, int* s_part) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const uint64_t diff = lo ^ hi;
  if (diff == 0ull) return lo;
  const int top = 63 - __builtin_clzll(diff);
  uint64_t t = lo & ~((top == 63 ? 0ull : (2ull << top)) - 1ull);
  int par = 0;
  for (int bit = top; bit >= 0; --bit) {
    const uint64_t cand = t | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint64_t key = hk[j] == 0u ? 0ull
                                       : ((static_cast<uint64_t>(hk[j]) << 32) |
                                          static_cast<uint64_t>(~static_cast<uint32_t>(tid + 256 * j)));
      if (j < n) cnt += __popcll(__ballot(key >= cand));
    }
    if (lane == 0) s_part[par * 4 + wave] = cnt;
    __syncthreads();
    const int tot = s_part[par * 4] + s_part[par * 4 + 1] + s_part[par * 4 + 2] + s_part[par * 4 + 3];
    par ^= 1;
    if (tot >= k) {
      t = cand;
      if (tot == k) break;
    }
  }
  return t;
}

// Appends to s_list the keys (score, then lower index first) of the
// candidates tid + 256 j of this thread's set bits j of m, their scores read
// from s_sc, at slots reserved with one LDS atomic on s_cnt per wave; slots
// at or past cap are dropped (the count still grows).  The lane prefix comes
// from the kBits bits of the per-lane counts (one ballot each); the loop runs
// as many times as the wave's fullest lane has bits.
template <int kBits, typename M>
__device__ __forceinline__ void wave_emit(M m, const float* s_sc, uint64_t* s_list, int* s_cnt, int cap) {
  const int tid = threadIdx.x, lane = tid % kWave;
  const int mine = sizeof(M) == 8 ? __popcll(static_cast<uint64_t>(m)) : __popc(static_cast<uint32_t>(m));
  int below = 0, total = 0;
#pragma unroll
  for (int bit = 0; bit < kBits; ++bit) {
    const uint64_t bl = __ballot((mine >> bit) & 1);
    below += lanes_below(bl) << bit;
    total += __popcll(bl) << bit;
  }
  if (total == 0) return;
  int base = 0;
  if (lane == 0) base = atomicAdd(s_cnt, total);
  int slot = __builtin_amdgcn_readfirstlane(base) + below;     // lane 0's (every lane is active)
  while (__ballot(m != 0) != 0ull) {
    if (m != 0) {
      const int j = sizeof(M) == 8 ? __builtin_ctzll(static_cast<uint64_t>(m)) : __builtin_ctz(static_cast<uint32_t>(m));
      m &= m - 1;
      const uint32_t c = static_cast<uint32_t>(tid + 256 * j);
      if (slot < cap)
        s_list[slot] = (static_cast<uint64_t>(orderable_f32(s_sc[c])) << 32) | static_cast<uint64_t>(~c);
      ++slot;
    }
  }
}

__device__ __forceinline__ int ascending_place(const int32_t* win, int kk, int32_t cw);

// What step_select leaves for its workgroup: the block of the workgroup's
// slot and its log gate, the slot's place in ascending block order, and the
// LDS state step_order reads.
struct StepPick {
  int32_t c;            // the slot's block, -1 for an empty slot
  float bias;           // its log gate (0 with the gate off)
  int at;               // its place among the K slots in ascending block order
  const int32_t* win;   // the winners by score rank (LDS), INT32_MAX from kk on
  const float* sc;      // every candidate's score (LDS)
  float lse;            // LSE over every candidate
  int kk;
};

// Exact top-kk of one selection head: scores [nch * 256] (-inf past the
// candidates; candidate x at x), the chunks' (max, sum exp) and the groups'
// maxima gmax [nch * 4].  Slot `unit` takes the winner of score rank unit
// (slots kk .. K - 1 are empty); its partial goes to the slot's place in
// ascending block order, the count of winners below it, so that the split-K
// partials lie in ascending block order whichever workgroup made them.  The
// order of every slot (the selection's output) is left to step_order, which
// only the workgroup that writes the output needs.
template <int NCH>
__device__ __forceinline__ void step_select(const float* __restrict__ scores, const float2* __restrict__ cml,
                                            const float* __restrict__ gmax, int nch, int64_t ncand, int K,
                                            int unit, StepPick& pick) {
  using mask_t = typename std::conditional<(NCH > 32), uint64_t, uint32_t>::type;
  constexpr int kBits = NCH >= 64 ? 7 : NCH >= 32 ? 6 : NCH >= 16 ? 5 : 3;   // bits of a lane's count
  constexpr int kSurvMax = 256;        // one survivor per thread in the ranking
  __shared__ float s_sc[NCH * 256];
  __shared__ __align__(16) uint64_t s_key[kSurvMax];
  __shared__ __align__(16) int32_t s_win[kStepMaxK];
  __shared__ uint32_t s_lo;
  __shared__ int s_cnt;
  __shared__ float s_lse;
  __shared__ int s_part[8];
  __shared__ uint64_t s_hi[4];
  __shared__ uint32_t s_tb[4];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int kk = static_cast<int>(ncand < K ? ncand : K);
  // the group maxima bound the kk-th score usefully only when there are
  // several times kk groups
  const bool group_bound = 4 * nch >= 2 * kk;

  // the group maxima and chunk sums first (wave 0 forms the bound and the
  // LSE while the scores are in flight), then candidates tid + 256 j; every
  // load is unconditional (clamped addresses, masked after) so that the waits
  // count exactly the loads a value needs
  float gv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gi = i * kWave + lane;
    gv[i] = gmax[gi < 4 * nch ? gi : 4 * nch - 1];
  }
  float2 cv = cml[lane < nch ? lane : nch - 1];
  float sv[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) sv[j] = scores[tid + 256 * (j < nch ? j : nch - 1)];
  if (tid == 0) s_cnt = 0;
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i * kWave + lane >= 4 * nch) gv[i] = -INFINITY;
    if (lane >= nch) cv = make_float2(-INFINITY, 0.f);
    // the LSE over every candidate, merged as decode_merge.h merges it (the
    // three empty waves of that merge leave (m, l) as it is)
    float m = -INFINITY, l = 0.f;
    ml_combine(m, l, cv.x, cv.y);
    {
      float m2 = xor_lanes_f<32>(m), l2 = xor_lanes_f<32>(l); ml_combine(m, l, m2, l2);
      m2 = xor_lanes_f<16>(m); l2 = xor_lanes_f<16>(l); ml_combine(m, l, m2, l2);
      m2 = xor_lanes_f<8>(m); l2 = xor_lanes_f<8>(l); ml_combine(m, l, m2, l2);
      m2 = xor_lanes_f<4>(m); l2 = xor_lanes_f<4>(l); ml_combine(m, l, m2, l2);
      m2 = xor_lanes_f<2>(m); l2 = xor_lanes_f<2>(l); ml_combine(m, l, m2, l2);
      m2 = xor_lanes_f<1>(m); l2 = xor_lanes_f<1>(l); ml_combine(m, l, m2, l2);
    }
    const float lse = m + __logf(l);
    // lower bound of the kk-th largest score: the kk-th largest of the
    // lanes' group maxima (each lane's largest of its groups: a subset of the
    // group maxima, so at least kk groups, hence kk scores, reach it), found
    // by sorting the 64 lane maxima; 0 (no bound) below kk such lanes
    if (group_bound) {
      float gl = gv[0];
#pragma unroll
      for (int i = 1; i < 4; ++i) gl = fmaxf(gl, gv[i]);
      const uint32_t gsorted = wave_sort_desc_u32(gl == -INFINITY ? 0u : orderable_f32(gl));
      const uint32_t lo = kk > 0 ? __shfl(gsorted, kk - 1, kWave) : 0u;
      if (lane == 0) s_lo = lo;
    }
    if (lane == 0) s_lse = lse;
  }
  // every score to LDS: the survivors' keys are formed from it
#pragma unroll
  for (int j = 0; j < NCH; ++j)
    if (j < nch) s_sc[256 * j + tid] = sv[j];
  const int64_t rem = ncand - tid;
  const int nv = rem <= 0 ? 0 : static_cast<int>((rem + 255) / 256 < nch ? (rem + 255) / 256 : nch);
  const mask_t valid = nv >= 8 * static_cast<int>(sizeof(mask_t)) ? ~mask_t(0) : ((mask_t(1) << nv) - 1);
  if (!group_bound) {
    // Few groups (short contexts): the threads' maxima instead.  Each wave's
    // ceil(kk / 4)-th largest thread maximum: every wave has that many
    // disjoint candidate sets at or above its figure, so the smallest of the
    // four figures is reached by kk scores.
    float tmx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
      if ((valid >> j) & 1) tmx = fmaxf(tmx, sv[j]);
    const uint32_t tsorted = wave_sort_desc_u32(tmx == -INFINITY ? 0u : orderable_f32(tmx));
    const uint32_t tb = kk > 0 ? __shfl(tsorted, (kk + 3) / 4 - 1, kWave) : 0u;
    if (lane == 0) s_tb[wave] = tb;
  }
  __syncthreads();
  uint32_t lo = s_lo;
  if (!group_bound) {
    lo = s_tb[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) lo = s_tb[w] < lo ? s_tb[w] : lo;
  }
  // survivors: candidates scoring at or above the bound (a float compare:
  // the same order as the keys, +0 and -0 alike), as one bit per slot j
  const float lof = lo == 0u ? -INFINITY : from_orderable_f32(lo);
  mask_t sm = 0;
#pragma unroll
  for (int j = 0; j < NCH; ++j) sm |= sv[j] >= lof ? (mask_t(1) << j) : mask_t(0);
  sm &= valid;
  wave_emit<kBits>(sm, s_sc, s_key, &s_cnt, kSurvMax);
  __syncthreads();
  int ns = s_cnt;
  if (ns > kSurvMax) {
    // many scores tie near the bound: search the kk-th key over every
    // candidate, then keep exactly the kk at or above it
    uint32_t hk[NCH];
    uint64_t kmax = 0ull;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      hk[j] = ((valid >> j) & 1) ? orderable_f32(sv[j]) : 0u;
      const uint64_t key = hk[j] == 0u ? 0ull
                                       : ((static_cast<uint64_t>(hk[j]) << 32) |
                                          static_cast<uint64_t>(~static_cast<uint32_t>(tid + 256 * j)));
      kmax = key > kmax ? key : kmax;
    }
    kmax = wave_max_u64(kmax);
    if (lane == 0) s_hi[wave] = kmax;
    __syncthreads();
    uint64_t hi = s_hi[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) hi = s_hi[w] > hi ? s_hi[w] : hi;
    const uint64_t kth = block_kth_largest_u64<NCH>(hk, nch, kk, static_cast<uint64_t>(lo) << 32, hi, s_part);
    mask_t km = 0;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const uint64_t key = (static_cast<uint64_t>(hk[j]) << 32) |
                           static_cast<uint64_t>(~static_cast<uint32_t>(tid + 256 * j));
      km |= (hk[j] != 0u && key >= kth) ? (mask_t(1) << j) : mask_t(0);
    }
    __syncthreads();
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    wave_emit<kBits>(km, s_sc, s_key, &s_cnt, kSurvMax);
    __syncthreads();
    ns = kk;
  }
  // rank each survivor on its key (score, then lower index first): ranks
  // below kk are the winners, kept at their rank.  Key 0 pads the list to a
  // multiple of 8 and INT32_MAX the winners to 64, so that each loop below
  // reads several entries per LDS load.
  const int ns8 = (ns + 7) & ~7;
  const uint64_t key = tid < ns ? s_key[tid] : 0ull;
  if (tid >= ns && tid < ns8) s_key[tid] = 0ull;
  if (tid >= kk && tid < kStepMaxK) s_win[tid] = INT32_MAX;
  __syncthreads();
  if (tid < ns) {
    int rank = 0;
    const ulonglong2* kp = reinterpret_cast<const ulonglong2*>(s_key);
#pragma unroll 4
    for (int i = 0; i < ns8 / 2; ++i) {
      const ulonglong2 x = kp[i];
      rank += (x.x > key ? 1 : 0) + (x.y > key ? 1 : 0);
    }
    if (rank < kk) s_win[rank] = static_cast<int32_t>(~static_cast<uint32_t>(key));
  }
  __syncthreads();
  pick.win = s_win;
  pick.sc = s_sc;
  pick.lse = s_lse;
  pick.kk = kk;
  pick.c = -1;
  pick.bias = 0.f;
  pick.at = unit;
  if (unit < kk) {
    pick.c = s_win[unit];
    pick.bias = s_sc[pick.c] - s_lse;
    pick.at = ascending_place(s_win, kk, pick.c);
  }
}

// A winner's place in ascending block order: the count of winners below it
// (winners are distinct blocks; the entries from kk on are INT32_MAX).
__device__ __forceinline__ int ascending_place(const int32_t* win, int kk, int32_t cw) {
  int at = 0;
  const int4* wp = reinterpret_cast<const int4*>(win);
#pragma unroll 4
  for (int i = 0; i < (kk + 3) / 4; ++i) {
    const int4 w = wp[i];
    at += (w.x < cw ? 1 : 0) + (w.y < cw ? 1 : 0) + (w.z < cw ? 1 : 0) + (w.w < cw ? 1 : 0);
  }
  return at;
}

// Every slot of the selection in ascending block order into s_idx / s_lg
// (log gates; 0 with the gate off), -1 / 0 in slots kk .. K - 1.
__device__ __forceinline__ void step_order(const StepPick& pk, int K, int gate, int32_t* s_idx, float* s_lg) {
  const int tid = threadIdx.x;
  if (tid < K) {
    if (tid < pk.kk) {
      const int32_t cw = pk.win[tid];
      const int at = ascending_place(pk.win, pk.kk, cw);
      s_idx[at] = cw;
      s_lg[at] = gate ? pk.sc[cw] - pk.lse : 0.f;
    } else {
      s_idx[tid] = -1;
      s_lg[tid] = 0.f;
    }
  }
  __syncthreads();
}

// One workgroup per (selection head, kept tile): tiles u tpu .. u tpu + tpu - 1
// of selected slot u < K, then those of the current block.
template <int D, int HPW, int NCH>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ scores, const float2* __restrict__ cml, const float* __restrict__ gmax, int nch,
    int64_t ncand, int gate, int32_t* __restrict__ idx, float* __restrict__ logg, int32_t* __restrict__ k_eff,
    int Hq, int Hkv, int Hsel, int share_group, int64_t L, int64_t pos, int b, int K, int tpu,
    float* __restrict__ ws_acc, float2* __restrict__ ws_ml, const int32_t* __restrict__ table, int64_t tstride,
    int64_t npages, uint32_t* __restrict__ ctr, bf16_t* __restrict__ o, float* __restrict__ lse,
    uint64_t* __restrict__ ws_u) {
  __shared__ int32_t s_idx[kStepMaxK];
  __shared__ float s_lg[kStepMaxK];
  __shared__ uint32_t s_last;
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
  StepPick pk{};
  int place = tile;   // where the tile's partial goes: slots in ascending block order, then the current block
  if (unit < K) {
    step_select<NCH>(scores + static_cast<int64_t>(bh) * nch * kDecodeChunk, cml + static_cast<int64_t>(bh) * nch,
                     gmax + static_cast<int64_t>(bh) * nch * 4, nch, ncand, K, unit, pk);
    place = pk.at * tpu + sub;
    const int32_t c = pk.c;
    if (c >= 0 && c < c0) {
      start = static_cast<int64_t>(c) * b + sub * kTileTok;
      ntok = b - sub * kTileTok < kTileTok ? b - sub * kTileTok : kTileTok;
      bias = gate ? pk.bias : 0.f;
    }
  } else {
    start = c0 * b + sub * kTileTok;
    const int64_t n = pos + 1 - start;
    const int cap = b - sub * kTileTok < kTileTok ? b - sub * kTileTok : kTileTok;
    ntok = n <= 0 ? 0 : (n < cap ? static_cast<int>(n) : cap);
  }

  const int64_t obase = (static_cast<int64_t>(bh) * ntiles + place) * HPW;
  int64_t off = 0;
  if (ntok > 0) {
    if (table == nullptr) {
      off = ((static_cast<int64_t>(bi) * Hkv + kvh) * L + start) * D;
    } else {
      // paged K / V: an unmapped page (id outside the pool) empties the tile
      const int64_t blk = start / b;
      const int64_t pg = table[static_cast<int64_t>(bi) * tstride + blk];
      if (pg < 0 || pg >= npages)
        ntok = 0;
      else
        off = ((pg * Hkv + kvh) * b + (start - blk * b)) * D;
    }
  }
  if (ntok == 0) {
    for (int x = tid; x < HPW * D; x += 256) publish_u32(ws_acc + obase * D + x, 0u);
    if (tid < HPW) publish_f2(ws_ml + obase + tid, -INFINITY, 0.f);
  } else {
    const int hq0 = share_group ? hs * G : hs;
    tile_partial_bf16<D, HPW, true>(q + (static_cast<int64_t>(bi) * Hq + hq0) * D, k + off, v + off, ntok, bias,
                                    ws_acc, ws_ml, obase);
  }

  // The head's last workgroup to finish merges the partials (split-K
  // combine): every partial is published before the arrival is counted.
  wait_published();
  __syncthreads();
  if (tid == 0) s_last = count_arrival(ctr + bh) == static_cast<uint32_t>(ntiles - 1) ? 1u : 0u;
  if (unit == 0 && sub == 0) {
    // the selection's output, off the tiles' path
    step_order(pk, K, gate, s_idx, s_lg);
    const int64_t o0 = static_cast<int64_t>(bh) * K;      // one query row
    for (int x = tid; x < K; x += 256) {
      idx[o0 + x] = s_idx[x];
      if (logg != nullptr) logg[o0 + x] = s_lg[x];
    }
    if (tid == 0 && k_eff != nullptr) k_eff[bh] = static_cast<int32_t>(ncand < K ? ncand : K);
  }
  __syncthreads();
  if (s_last == 0u) return;
  // every workgroup of the head (and the whole scorer) is done with u
  if (ws_u != nullptr && tid < D) ws_u[static_cast<int64_t>(bh) * D + tid] = 0ull;
  combine_partials<bf16_t, D, HPW>(ws_acc, ws_ml, bh, bi, hs, G, Hq, share_group, ntiles, o, lse);
}

template <int D, int HPW, int NCH>
static hipError_t launch_step_h(const SelectLaunch& s, const DecodeStepWs& w, const AttnLaunch& p, void* ws_att,
                                hipStream_t st) {
  const int tpu = decode_step_tpu(p);
  const int ntiles = (p.K + 1) * tpu;
  const size_t heads = static_cast<size_t>(p.B) * p.Hsel;
  char* base = static_cast<char*>(ws_att);
  float* acc = reinterpret_cast<float*>(base);
  float2* ml = reinterpret_cast<float2*>(base + align256(heads * ntiles * HPW * p.d * sizeof(float)));
  return launch(true, decode_step_kernel<D, HPW, NCH>, dim3(ntiles, static_cast<unsigned>(heads)), dim3(256), st,
                static_cast<const bf16_t*>(p.q), static_cast<const bf16_t*>(p.k), static_cast<const bf16_t*>(p.v),
                static_cast<const float*>(w.scores), static_cast<const float2*>(w.ml), static_cast<const float*>(w.t2),
                w.nch, s.max_cand, s.gate, s.idx, s.logg, s.k_eff, p.Hq, p.Hkv, p.Hsel, p.share_group, p.L,
                p.q_pos0, p.b, p.K, tpu, acc, ml, p.pages.table, p.pages.tstride, p.pages.npages, w.ctr,
                static_cast<bf16_t*>(p.o), p.lse, w.u);
}

template <int D, int HPW>
static hipError_t launch_step_n(const SelectLaunch& s, const DecodeStepWs& w, const AttnLaunch& p, void* ws_att,
                                hipStream_t st) {
  if (w.nch <= 4) return launch_step_h<D, HPW, 4>(s, w, p, ws_att, st);
  if (w.nch <= 16) return launch_step_h<D, HPW, 16>(s, w, p, ws_att, st);
  if (w.nch <= 32) return launch_step_h<D, HPW, 32>(s, w, p, ws_att, st);
  return launch_step_h<D, HPW, 64>(s, w, p, ws_att, st);
}

template <int D>
static hipError_t launch_step_d(const SelectLaunch& s, const DecodeStepWs& w, const AttnLaunch& p, void* ws_att,
                                hipStream_t st) {
  switch (p.share_group ? p.Hq / p.Hkv : 1) {
    case 1: return launch_step_n<D, 1>(s, w, p, ws_att, st);
    case 2: return launch_step_n<D, 2>(s, w, p, ws_att, st);
    case 4: return launch_step_n<D, 4>(s, w, p, ws_att, st);
    default: return launch_step_n<D, 8>(s, w, p, ws_att, st);
  }
}

// Scorer, then selection + attention + combine (bf16, decode_fusable
// selections only).  ws_sel holds scores, chunk sums and group bounds; ws_att
// the partials, then the arrival counters.
hipError_t launch_decode_fused_attn(const SelectLaunch& s, void* ws_sel, const AttnLaunch& a, void* ws_att,
                                    hipStream_t st) {
  const DecodeStepWs w = decode_step_ws(s, ws_sel, static_cast<char*>(ws_att) + attn_fwd_workspace_bytes(a));
  hipError_t e = launch_decode_step_scores(s, w, st);
  if (e != hipSuccess) return e;
  return a.d == 64 ? launch_step_d<64>(s, w, a, ws_att, st) : launch_step_d<128>(s, w, a, ws_att, st);
}

size_t decode_step_select_bytes(const SelectLaunch& p) { return decode_step_ws(p, nullptr, nullptr).sel_bytes; }

}  // namespace spa
