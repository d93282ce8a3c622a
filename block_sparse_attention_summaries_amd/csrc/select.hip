// select.hip -- selector scores, softmax log gate and deterministic top-K on
// gfx950.
//
// Score of candidate block c for a query row at position i (selection head hs):
//   s_c = q_hat . ktilde_c / sqrt(d)  [+ lambda a_c erf((i - p_c)/(2 sigma))]
// ("SAS" review §3 Eq. 3 and Alg. 1; "FreeSolo" review, "How it works").
// Gate: log g_c = s_c - LSE over every candidate ("SAS" review §4.2.2).
// Order: score desc, lower index first on ties; output ascending, -1 padded.
//
// Two paths:
//  * decode (one query row, current-block prefix, no erf term): the candidate
//    blocks of each selection head are split into chunks of 256; one
//    workgroup per chunk streams the bf16 summaries (16-byte loads, several
//    lanes per block) and keeps the chunk's (max, sum exp) and its top-K.  A
//    second small kernel (one workgroup per head) selects the top-K among the
//    chunk winners in two levels (4 waves, then one), finishes the LSE and
//    writes the ascending indices and log gates.  Both selections are threshold searches over ballot counts with
//    an ordered compaction (no sorting network).  The kernel boundary
//    publishes the chunk results; an in-kernel hand-off would need an
//    agent-scope release per workgroup, which on gfx950 writes back the L2.
//  * rows (any number of rows): one thread per query row, summaries staged in
//    LDS 64 candidates at a time and read as broadcasts, a sorted top-K held
//    in registers; the erf term is formed in fp64 so the ranking of scores
//    near ~10 is not decided by fp32 rounding.
#include <type_traits>

#include "decode_merge.h"
#include "spa_device.h"
#include "spa_launch.h"

namespace spa {

// ------------------------------------------------------------------ decode
// Top-K by threshold: the k-th largest score T is found with a bitwise
// search over ballot counts (wave_kth_largest); the kept set is every score
// > T plus the lowest-index scores == T.  Candidates are laid out so that
// position order is index order, which makes the lower-index tie rule and
// the ascending output a single ordered compaction (ballot + mbcnt).

// Per-selection-head query of the scores: u = W^T q_hat with the projection,
// q_hat without; q_hat is the mean of the G query heads of a shared
// selection (fp32, summed in head order), else the head's query.  Formed by
// the whole workgroup into s_uv[D] (synchronised on return).  The same
// arithmetic wherever it is formed: thread slices of kEPG rows of W, then the
// kEGroups slice sums added in order.
template <typename T, int D>
__device__ __forceinline__ void form_u(const T* __restrict__ q, const float* __restrict__ proj_w, int Hq, int Hkv,
                                       int Hsel, int share_group, int bh, float* s_uv) {
  constexpr int kQuads = D / 4;             // float4 column groups of W
  constexpr int kEGroups = 256 / kQuads;    // row groups (one per thread slice)
  constexpr int kEPG = D / kEGroups;        // rows of W per thread
  constexpr int kGMax = 8;
  __shared__ float s_q[D];
  __shared__ float s_u[kEGroups][D];
  const int tid = threadIdx.x;
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int G = Hq / Hkv;
  const bool proj = proj_w != nullptr;
  // query heads and this thread's slice of W (rows eg*kEPG .., columns 4jq ..)
  const int gq = share_group ? G : 1;
  const int hq0 = share_group ? hs * G : hs;
  const int eq = tid % D;
  float qv[kGMax];
#pragma unroll
  for (int g = 0; g < kGMax; ++g) {
    const int h = hq0 + (g < gq ? g : gq - 1);
    qv[g] = ld_f(q + (static_cast<int64_t>(bi) * Hq + h) * D + eq);
  }
  const int jq = tid % kQuads, eg = tid / kQuads;
  float4 wq[kEPG];
  if (proj) {
#pragma unroll
    for (int i = 0; i < kEPG; ++i)
      wq[i] = reinterpret_cast<const float4*>(proj_w + static_cast<int64_t>(eg * kEPG + i) * D)[jq];
  }
  if (tid < D) {
    float qsum = 0.f;
#pragma unroll
    for (int g = 0; g < kGMax; ++g)
      if (g < gq) qsum += qv[g];
    s_q[tid] = qsum / static_cast<float>(gq);
  }
  lds_barrier();
  if (proj) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kEPG; ++i) {
      const float qe = s_q[eg * kEPG + i];
      a.x = fmaf(wq[i].x, qe, a.x);
      a.y = fmaf(wq[i].y, qe, a.y);
      a.z = fmaf(wq[i].z, qe, a.z);
      a.w = fmaf(wq[i].w, qe, a.w);
    }
    reinterpret_cast<float4*>(s_u[eg])[jq] = a;
    lds_barrier();
    if (tid < D) {
      float u = 0.f;
#pragma unroll
      for (int g = 0; g < kEGroups; ++g) u += s_u[g][tid];
      s_uv[tid] = u;
    }
  } else if (tid < D) {
    s_uv[tid] = s_q[tid];
  }
  lds_barrier();
}

// Summary layout of the chunk scorer: a wave covers 64 candidate blocks,
// kLPB lanes per block reading 16-byte vectors (kVec elements), kRounds load
// rounds.
template <typename T, int D, bool F8>
struct ChunkLoads {
  static constexpr int kVec = F8 ? 16 : Elem<T>::kVec;   // summary elements per 16-byte load
  static constexpr int kElemBytes = F8 ? 1 : static_cast<int>(sizeof(T));
  static constexpr int kLPB = D / kVec;           // lanes per block row
  static constexpr int kBPR = kWave / kLPB;       // blocks per load round of a wave
  static constexpr int kRounds = kWave / kBPR;    // rounds to cover the wave's 64 blocks
  uint4 raw[kRounds];
  float bscale[F8 ? kRounds : 1];

  // Requests the chunk's summaries (unconditional: rows past the candidates
  // read the last candidate and are masked by the callers).
  __device__ __forceinline__ void issue(const void* __restrict__ kbar_v, const float* __restrict__ kscale,
                                        int Hkv, int Hsel, int share_group, int G, int64_t ccap, int64_t ncand,
                                        int chunk, int bh) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int bi = bh / Hsel, hs = bh % Hsel;
    const int kvh = share_group ? hs : hs / G;
    const int cg = lane % kLPB, bl = lane / kLPB;
    const int64_t wbase = static_cast<int64_t>(chunk) * kDecodeChunk + wave * kWave;
    const int64_t hrow = (static_cast<int64_t>(bi) * Hkv + kvh) * ccap;
    const char* kb = static_cast<const char*>(kbar_v) + hrow * D * kElemBytes;
    const int64_t clast = ncand > 0 ? ncand - 1 : 0;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int64_t c = wbase + r * kBPR + bl;
      const int64_t cc = c < clast ? c : clast;
      raw[r] = *reinterpret_cast<const uint4*>(kb + (cc * D + cg * kVec) * kElemBytes);
      if constexpr (F8) bscale[r] = kscale[hrow + cc];
    }
  }

  // Scores q.ktilde / sqrt(D) of the wave's blocks into s_score[wave * 64 ..],
  // u from s_uv.
  __device__ __forceinline__ void score(const float* s_uv, float* s_score) const {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int cg = lane % kLPB, bl = lane / kLPB;
    float uc[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) uc[i] = s_uv[cg * kVec + i];
    const float scale = 1.0f / sqrtf(static_cast<float>(D));
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      float x[kVec];
      if constexpr (F8)
        fp8_e4m3_unpack16(raw[r], x);
      else
        Elem<T>::unpack(raw[r], x);
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < kVec; ++i) p = fmaf(x[i], uc[i], p);
      p = group_sum<kLPB>(p);
      if constexpr (F8) p *= bscale[r];
      if (cg == 0) s_score[wave * kWave + r * kBPR + bl] = p * scale;
    }
  }
};

// Scores of one chunk of 256 candidate blocks of one selection head (block
// cbase + x in s_score[x]; blocks past the candidates get garbage, callers
// mask them): u first (the query heads and, with a projection, W), then the
// chunk's summaries.  Ends with the scores in LDS, not yet synchronised.
template <typename T, int D, bool F8>
__device__ __forceinline__ void chunk_scores(
    const T* __restrict__ q, const void* __restrict__ kbar_v, const float* __restrict__ kscale,
    const float* __restrict__ proj_w, int Hq, int Hkv, int Hsel, int share_group, int64_t ccap, int64_t ncand,
    int chunk, int bh, float* s_score) {
  __shared__ float s_uv[D];
  form_u<T, D>(q, proj_w, Hq, Hkv, Hsel, share_group, bh, s_uv);
  __builtin_amdgcn_sched_barrier(0);
  ChunkLoads<T, D, F8> ld;
  ld.issue(kbar_v, kscale, Hkv, Hsel, share_group, Hq / Hkv, ccap, ncand, chunk, bh);
  ld.score(s_uv, s_score);
}

// One workgroup per (chunk of 256 candidate blocks, selection head).  Output:
// the chunk's top-min(K, n) candidates in index order as 64-bit
// (orderable score << 32 | block index) records (0 pads), and its (max, sum exp).
template <typename T, int D, bool F8>
__global__ __launch_bounds__(256) void decode_chunk_kernel(
    const T* __restrict__ q, const void* __restrict__ kbar_v, const float* __restrict__ kscale,
    const float* __restrict__ proj_w, int Hq, int Hkv, int Hsel, int share_group, int64_t ccap, int64_t ncand,
    int K, uint64_t* __restrict__ ws_keys, float2* __restrict__ ws_ml, int nchunks) {
  __shared__ float s_score[kDecodeChunk];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int chunk = blockIdx.x;
  const int bh = blockIdx.y;               // b * Hsel + hs
  const int64_t cbase = static_cast<int64_t>(chunk) * kDecodeChunk;
  (void)tid;
  chunk_scores<T, D, F8>(q, kbar_v, kscale, proj_w, Hq, Hkv, Hsel, share_group, ccap, ncand, chunk, bh, s_score);
  __syncthreads();
  if (wave != 0) return;

  // 5. wave 0: chunk (max, sum exp) and top-min(K, n) in index order
  const int nvalid = static_cast<int>(ncand - cbase < kDecodeChunk ? ncand - cbase : kDecodeChunk);
  uint32_t key[4];
  float sc[4];
  float mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pidx = i * kWave + lane;
    sc[i] = s_score[pidx];
    const bool ok = pidx < nvalid;
    key[i] = ok ? orderable_f32(sc[i]) : 0u;
    if (ok) mloc = fmaxf(mloc, sc[i]);
  }
  const float m = wave_max(mloc);
  float lloc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i * kWave + lane < nvalid) lloc += __expf(sc[i] - m);
  const float l = m == -INFINITY ? 0.f : wave_sum(lloc);
  const int kk = nvalid < K ? (nvalid > 0 ? nvalid : 0) : K;
  const uint32_t t = wave_kth_largest<4>(key, kk);
  int ngt = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) ngt += __popcll(__ballot(key[i] > t));
  uint64_t* out = ws_keys + (static_cast<int64_t>(bh) * nchunks + chunk) * K;
  const int kept = wave_select_ordered<4>(key, t, kk - ngt, [&](int slot, int i) {
    out[slot] = (static_cast<uint64_t>(key[i]) << 32) | static_cast<uint32_t>(cbase + i * kWave + lane);
  });
  for (int x = kept + lane; x < K; x += kWave) out[x] = 0ull;
  if (lane == 0) ws_ml[static_cast<int64_t>(bh) * nchunks + chunk] = make_float2(m, l);
}

// The one-call decode step's scorer.  With a projection, workgroup x = 0 of
// each selection head forms u = W^T q_hat once and publishes each element as
// a 64-bit word with a ready mark beside its fp32 bits (agent-scope stores:
// the mark travels in the same single-copy-atomic store as the value, so no
// separate flag and no wait for the values' completion are needed); the
// scoring workgroups x = 1 .. nch request their chunk's summaries first and
// poll their elements of u until every one is marked (a bounded wait: past
// it they form u themselves, with the same arithmetic), so that 256
// workgroups do not all read W while the summaries stream in.  Where the
// words do not fit their block (ws_u null), and without a projection, every
// scoring workgroup forms u (q_hat) itself.  A scoring workgroup writes every
// score of its chunk of 256 candidate blocks (-inf past the candidates), the
// chunk's (max, sum exp) with the same arithmetic as decode_chunk_kernel, and
// the largest score of each 64-block group (-inf for a group without
// candidates): the K-th largest of these group maxima bounds the K-th largest
// score from below for the selection in the attention kernel.  It also clears
// the attention kernel's arrival counters (the kernel boundary publishes
// them); the attention kernel clears the marked words for the next call.
constexpr int kUFlagSpin = 4096;
constexpr uint64_t kUReady = 1ull << 32;   // ready mark beside each published element of u

template <typename T, int D, bool F8>
__global__ __launch_bounds__(256) void decode_score_kernel(
    const T* __restrict__ q, const void* __restrict__ kbar_v, const float* __restrict__ kscale,
    const float* __restrict__ proj_w, int Hq, int Hkv, int Hsel, int share_group, int64_t ccap, int64_t ncand,
    float* __restrict__ ws_scores, float2* __restrict__ ws_ml, float* __restrict__ ws_t2, int nchunks,
    uint32_t* __restrict__ zero_ctr, int nzero, uint64_t* __restrict__ ws_u) {
  __shared__ float s_score[kDecodeChunk];
  __shared__ float s_uv[D];
  __shared__ uint32_t s_miss;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int bh = blockIdx.y;               // b * Hsel + hs
  const bool proj = proj_w != nullptr;
  const bool handoff = proj && ws_u != nullptr;
  const int uw = handoff ? 1 : 0;
  if (handoff && blockIdx.x == 0) {
    // u of this selection head, for the head's scoring workgroups
    form_u<T, D>(q, proj_w, Hq, Hkv, Hsel, share_group, bh, s_uv);
    if (tid < D) publish_u64(ws_u + static_cast<int64_t>(bh) * D + tid, kUReady | __float_as_uint(s_uv[tid]));
    return;
  }
  const int chunk = blockIdx.x - uw;
  if (chunk == 0 && bh == 0)
    for (int x = tid; x < nzero; x += 256) zero_ctr[x] = 0u;
  const int64_t cbase = static_cast<int64_t>(chunk) * kDecodeChunk;
  ChunkLoads<T, D, F8> ld;
  ld.issue(kbar_v, kscale, Hkv, Hsel, share_group, Hq / Hkv, ccap, ncand, chunk, bh);
  if (handoff) {
    if (tid == 0) s_miss = 0u;
    __syncthreads();
    if (tid < D) {
      // each element of u carries its own ready mark: no separate flag to wait for
      uint64_t w = 0ull;
      for (int it = 0; it < kUFlagSpin; ++it) {
        w = acquire_u64(ws_u + static_cast<int64_t>(bh) * D + tid);
        if (__builtin_amdgcn_read_exec() == __builtin_amdgcn_ballot_w64((w & kUReady) != 0ull)) break;
        __builtin_amdgcn_s_sleep(2);
      }
      if ((w & kUReady) == 0ull) s_miss = 1u;
      s_uv[tid] = __uint_as_float(static_cast<uint32_t>(w));
    }
    __syncthreads();
    if (s_miss != 0u) form_u<T, D>(q, proj_w, Hq, Hkv, Hsel, share_group, bh, s_uv);
  } else {
    form_u<T, D>(q, proj_w, Hq, Hkv, Hsel, share_group, bh, s_uv);
  }
  ld.score(s_uv, s_score);
  __syncthreads();
  const int nvalid = static_cast<int>(ncand - cbase < kDecodeChunk ? ncand - cbase : kDecodeChunk);
  // every thread: one score (its 64-block group is its wave)
  const bool ok = tid < nvalid;
  const float sv = ok ? s_score[tid] : -INFINITY;
  ws_scores[(static_cast<int64_t>(bh) * nchunks + chunk) * kDecodeChunk + tid] = sv;
  const float gmax = wave_max(sv);
  if (lane == 0) ws_t2[(static_cast<int64_t>(bh) * nchunks + chunk) * 4 + wave] = gmax;
  if (wave != 0) return;
  // wave 0: the chunk's (max, sum exp), as decode_chunk_kernel forms it
  float sc[4];
  float mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pidx = i * kWave + lane;
    sc[i] = s_score[pidx];
    if (pidx < nvalid) mloc = fmaxf(mloc, sc[i]);
  }
  const float m = wave_max(mloc);
  float lloc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i * kWave + lane < nvalid) lloc += __expf(sc[i] - m);
  const float l = m == -INFINITY ? 0.f : wave_sum(lloc);
  if (lane == 0) ws_ml[static_cast<int64_t>(bh) * nchunks + chunk] = make_float2(m, l);
}

// One workgroup (4 waves) per selection head: the two-level merge of the
// chunk winners (decode_merge.h) writes the ascending indices and log gates.
template <int NV, int NV2>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const uint64_t* __restrict__ ws_keys, const float2* __restrict__ ws_ml, int nchunks, int K,
    int64_t ncand, int gate, int32_t* __restrict__ idx, float* __restrict__ logg,
    int32_t* __restrict__ k_eff) {
  __shared__ uint64_t s_win[4 * 64];
  __shared__ float2 s_ml[4];
  __shared__ uint32_t s_lo[4];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int bh = blockIdx.x;
  merge_level1<NV>(ws_keys + static_cast<int64_t>(bh) * nchunks * K, ws_ml + static_cast<int64_t>(bh) * nchunks,
                   nchunks, K, s_win, s_ml, s_lo);
  __syncthreads();
  if (wave != 0) return;
  const int64_t o = static_cast<int64_t>(bh) * K;          // one query row
  const int kk = static_cast<int>(ncand < K ? ncand : K);
  const int kept = merge_level2<NV2>(s_win, s_ml, s_lo, K, kk, gate, [&](int slot, int32_t c, float lg) {
    idx[o + slot] = c;
    if (logg != nullptr) logg[o + slot] = lg;
  });
  for (int x = kept + lane; x < K; x += kWave) {
    idx[o + x] = -1;
    if (logg != nullptr) logg[o + x] = 0.f;
  }
  if (lane == 0 && k_eff != nullptr) k_eff[bh] = kk;
}

// -------------------------------------------------------------------- rows
template <typename T, int D, int KMAX, bool kErf>
__global__ __launch_bounds__(256) void rows_select_kernel(
    const T* __restrict__ q, const T* __restrict__ kbar, const float* __restrict__ max_norm,
    const float* __restrict__ centre, const float* __restrict__ proj_w,
    const float* __restrict__ erf_lambda, const float* __restrict__ erf_sigma, int Hq, int Hkv,
    int Hsel, int nq, int64_t q_pos0, int64_t ccap, int b, int prefix_mode, int qblock,
    int share_group, int K, int gate, int32_t* __restrict__ idx, float* __restrict__ logg,
    int32_t* __restrict__ k_eff) {
  using S = typename std::conditional<kErf, double, float>::type;
  constexpr int kTile = 64;
  __shared__ float s_kb[kTile][D];
  __shared__ float s_a[kTile];
  __shared__ float s_p[kTile];

  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int G = Hq / Hkv;
  const int kvh = share_group ? hs : hs / G;
  const int row0 = blockIdx.x * 256;
  const int row = row0 + tid;
  const bool active = row < nq;
  const int last_row = (row0 + 255 < nq ? row0 + 255 : nq - 1);
  const int64_t pos = q_pos0 + (active ? row : last_row);
  const int64_t ncand = active ? num_candidates(pos, b, prefix_mode, qblock) : 0;
  const int64_t wg_cand = num_candidates(q_pos0 + last_row, b, prefix_mode, qblock);

  float qh[D];
#pragma unroll
  for (int e = 0; e < D; ++e) qh[e] = 0.f;
  if (active) {
    if (share_group) {
      for (int g = 0; g < G; ++g) {
        const T* qp = q + ((static_cast<int64_t>(bi) * Hq + hs * G + g) * nq + row) * D;
#pragma unroll
        for (int e = 0; e < D; ++e) qh[e] += ld_f(qp + e);
      }
#pragma unroll
      for (int e = 0; e < D; ++e) qh[e] = qh[e] / static_cast<float>(G);
    } else {
      const T* qp = q + ((static_cast<int64_t>(bi) * Hq + hs) * nq + row) * D;
#pragma unroll
      for (int e = 0; e < D; ++e) qh[e] = ld_f(qp + e);
    }
  }
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  double lam = 0.0, inv2sig = 0.0;
  if (kErf) {
    lam = static_cast<double>(erf_lambda[hs]);
    inv2sig = 1.0 / (2.0 * static_cast<double>(erf_sigma[hs]));
  }

  S ts[KMAX];
  int ti[KMAX];
#pragma unroll
  for (int t = 0; t < KMAX; ++t) {
    ts[t] = -INFINITY;
    ti[t] = 0x7FFFFFFF;
  }
  float m_run = -INFINITY, l_run = 0.f;

  const T* kb = kbar + (static_cast<int64_t>(bi) * Hkv + kvh) * ccap * D;
  for (int64_t c0 = 0; c0 < wg_cand; c0 += kTile) {
    const int nt = static_cast<int>(wg_cand - c0 < kTile ? wg_cand - c0 : kTile);
    __syncthreads();
    if (proj_w == nullptr) {
      for (int x = tid; x < nt * D; x += 256) {
        const int cc = x / D, e = x % D;
        s_kb[cc][e] = ld_f(kb + (c0 + cc) * D + e);
      }
    } else {
      // ktilde_c = W kbar_c, formed once per staged tile for all rows
      for (int x = tid; x < nt * D; x += 256) {
        const int cc = x / D, e = x % D;
        const T* kr = kb + (c0 + cc) * D;
        float acc = 0.f;
        for (int f = 0; f < D; ++f) acc = fmaf(proj_w[e * D + f], ld_f(kr + f), acc);
        s_kb[cc][e] = acc;
      }
    }
    if (kErf && tid < nt) {
      s_a[tid] = max_norm[(static_cast<int64_t>(bi) * Hkv + kvh) * ccap + c0 + tid];
      s_p[tid] = centre[c0 + tid];
    }
    __syncthreads();
    for (int cc = 0; cc < nt; ++cc) {
      const int64_t c = c0 + cc;
      if (c >= ncand) break;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(qh[e], s_kb[cc][e], dot);
      S sc;
      if (kErf) {
        const double x = (static_cast<double>(pos) - static_cast<double>(s_p[cc])) * inv2sig;
        const double ev = x >= 6.0 ? 1.0 : (x <= -6.0 ? -1.0 : erf(x));
        sc = static_cast<double>(dot * scale) + lam * static_cast<double>(s_a[cc]) * ev;
      } else {
        sc = dot * scale;
      }
      if (gate) {
        const float sf = static_cast<float>(sc);
        if (sf > m_run) {
          l_run = l_run * __expf(m_run - sf) + 1.f;
          m_run = sf;
        } else {
          l_run += __expf(sf - m_run);
        }
      }
      const int ci = static_cast<int>(c);
      if (sel_better(sc, ci, ts[KMAX - 1], ti[KMAX - 1])) topk_push(ts, ti, sc, ci);
    }
  }
  if (!active) return;

  const int keff = static_cast<int>(ncand < K ? ncand : K);
  // keep the first keff, order them by index (unused slots sort last)
#pragma unroll
  for (int t = 0; t < KMAX; ++t)
    if (t >= keff) ti[t] = 0x7FFFFFFF;
  sort_by_index(ts, ti);
  const float lse = m_run + __logf(l_run);
  const int64_t o = ((static_cast<int64_t>(bi) * Hsel + hs) * nq + row) * K;
#pragma unroll
  for (int t = 0; t < KMAX; ++t) {
    if (t < K) {
      const bool ok = t < keff;
      idx[o + t] = ok ? ti[t] : -1;
      if (logg != nullptr) logg[o + t] = (ok && gate) ? static_cast<float>(ts[t] - static_cast<S>(lse)) : 0.f;
    }
  }
  if (k_eff != nullptr) k_eff[(static_cast<int64_t>(bi) * Hsel + hs) * nq + row] = keff;
}

// ------------------------------------------------------------------ launch
// Records per lane each merge wave may hold (a quarter of the chunk winners;
// up to 4 x 64 x 64 records per head).
constexpr int kMergeMaxNV = 64;

static int merge_nv(const SelectLaunch& p) {
  const int64_t nch = decode_num_chunks(p.max_cand > 0 ? p.max_cand : 1);
  const int64_t quarter = ((nch + 3) / 4) * p.K;
  int nv = 1;
  while (static_cast<int64_t>(nv) * kWave < quarter) nv *= 2;
  return nv;
}

static bool use_decode_path(const SelectLaunch& p) {
  return p.nq == 1 && p.prefix_mode == 0 && p.erf_lambda == nullptr && merge_nv(p) <= kMergeMaxNV;
}

size_t select_workspace_bytes(const SelectLaunch& p) {
  if (!use_decode_path(p)) return rows_select_mfma_supported(p) ? rows_select_mfma_ws_bytes(p) : 0;
  return decode_select_ws(p, nullptr).bytes;
}

template <typename T, int D>
static hipError_t launch_chunks_t(const SelectLaunch& p, void* ws, hipStream_t st) {
  const DecodeSelectWs w = decode_select_ws(p, ws);
  auto kern = p.kbar_scale != nullptr ? decode_chunk_kernel<T, D, true> : decode_chunk_kernel<T, D, false>;
  return launch(false, kern, dim3(w.nch, static_cast<unsigned>(p.B * p.Hsel)), dim3(256), st,
                static_cast<const T*>(p.q), p.kbar, p.kbar_scale, p.proj_w, p.Hq, p.Hkv, p.Hsel, p.share_group,
                p.ccap, p.max_cand, p.K, w.keys, w.ml, w.nch);
}

bool decode_select_path(const SelectLaunch& p) { return use_decode_path(p); }

bool decode_fusable(const SelectLaunch& p) {
  return use_decode_path(p) && p.dtype == kDtypeBf16 && p.K <= kStepMaxK &&
         static_cast<int64_t>(p.B) * p.Hsel <= kStepMaxHeads &&
         decode_num_chunks(p.max_cand > 0 ? p.max_cand : 1) <= kStepMaxChunks;
}

template <typename T, int D>
static hipError_t launch_step_scores_t(const SelectLaunch& p, const DecodeStepWs& w, hipStream_t st) {
  auto kern = p.kbar_scale != nullptr ? decode_score_kernel<T, D, true> : decode_score_kernel<T, D, false>;
  const unsigned gx = static_cast<unsigned>(w.nch + (p.proj_w != nullptr && w.u != nullptr ? 1 : 0));
  return launch(false, kern, dim3(gx, static_cast<unsigned>(p.B * p.Hsel)), dim3(256), st,
                static_cast<const T*>(p.q), p.kbar, p.kbar_scale, p.proj_w, p.Hq, p.Hkv, p.Hsel, p.share_group,
                p.ccap, p.max_cand, w.scores, w.ml, w.t2, w.nch, w.ctr, static_cast<int>(p.B * p.Hsel), w.u);
}

hipError_t launch_decode_step_scores(const SelectLaunch& p, const DecodeStepWs& w, hipStream_t st) {
  return p.d == 64 ? launch_step_scores_t<bf16_t, 64>(p, w, st) : launch_step_scores_t<bf16_t, 128>(p, w, st);
}

int decode_merge_nv(const SelectLaunch& p) { return merge_nv(p); }

hipError_t launch_decode_chunks(const SelectLaunch& p, void* ws, hipStream_t st) {
  if (p.dtype == kDtypeBf16)
    return p.d == 64 ? launch_chunks_t<bf16_t, 64>(p, ws, st) : launch_chunks_t<bf16_t, 128>(p, ws, st);
  return p.d == 64 ? launch_chunks_t<float, 64>(p, ws, st) : launch_chunks_t<float, 128>(p, ws, st);
}

template <typename T, int D>
static hipError_t launch_decode_t(const SelectLaunch& p, void* ws, hipStream_t st) {
  const int64_t ncand = p.max_cand;
  const size_t heads = static_cast<size_t>(p.B) * p.Hsel;
  const DecodeSelectWs w = decode_select_ws(p, ws);
  const int nch = w.nch;
  uint64_t* keys = w.keys;
  float2* ml = w.ml;
  hipError_t e = launch_chunks_t<T, D>(p, ws, st);
  if (e != hipSuccess) return e;
  void (*merge)(const uint64_t*, const float2*, int, int, int64_t, int, int32_t*, float*, int32_t*);
  const bool small_k = p.K <= 32;
#define SPA_MERGE(NVV) (small_k ? decode_merge_kernel<NVV, 2> : decode_merge_kernel<NVV, 4>)
  switch (merge_nv(p)) {
    case 1: merge = SPA_MERGE(1); break;
    case 2: merge = SPA_MERGE(2); break;
    case 4: merge = SPA_MERGE(4); break;
    case 8: merge = SPA_MERGE(8); break;
    case 16: merge = SPA_MERGE(16); break;
    case 32: merge = SPA_MERGE(32); break;
    default: merge = SPA_MERGE(64); break;
  }
#undef SPA_MERGE
  return launch(true, merge, dim3(static_cast<unsigned>(heads)), dim3(256), st, keys, ml, nch, p.K, ncand,
                p.gate, p.idx, p.logg, p.k_eff);
}

template <typename T, int D, int KMAX>
static hipError_t launch_rows_k(const SelectLaunch& p, hipStream_t st) {
  dim3 grid((p.nq + 255) / 256, static_cast<unsigned>(p.B * p.Hsel));
  auto kern = p.erf_lambda != nullptr ? rows_select_kernel<T, D, KMAX, true>
                                       : rows_select_kernel<T, D, KMAX, false>;
  return launch(true, kern, grid, dim3(256), st, static_cast<const T*>(p.q),
                static_cast<const T*>(p.kbar), p.max_norm, p.centre, p.proj_w, p.erf_lambda,
                p.erf_sigma, p.Hq, p.Hkv, p.Hsel, p.nq, p.q_pos0, p.ccap, p.b, p.prefix_mode, p.qblock,
                p.share_group, p.K, p.gate, p.idx, p.logg, p.k_eff);
}

template <typename T, int D>
static hipError_t launch_rows_t(const SelectLaunch& p, hipStream_t st) {
  if (p.K <= 4) return launch_rows_k<T, D, 4>(p, st);
  if (p.K <= 8) return launch_rows_k<T, D, 8>(p, st);
  if (p.K <= 16) return launch_rows_k<T, D, 16>(p, st);
  if (p.K <= 32) return launch_rows_k<T, D, 32>(p, st);
  return launch_rows_k<T, D, 64>(p, st);
}

hipError_t launch_score_select(const SelectLaunch& p, void* ws, hipStream_t st) {
  if (use_decode_path(p)) {
    if (p.dtype == 1) return p.d == 64 ? launch_decode_t<bf16_t, 64>(p, ws, st) : launch_decode_t<bf16_t, 128>(p, ws, st);
    return p.d == 64 ? launch_decode_t<float, 64>(p, ws, st) : launch_decode_t<float, 128>(p, ws, st);
  }
  if (rows_select_mfma_supported(p)) return launch_rows_select_mfma(p, ws, st);
  if (p.dtype == 1) return p.d == 64 ? launch_rows_t<bf16_t, 64>(p, st) : launch_rows_t<bf16_t, 128>(p, st);
  return p.d == 64 ? launch_rows_t<float, 64>(p, st) : launch_rows_t<float, 128>(p, st);
}

}  // namespace spa
