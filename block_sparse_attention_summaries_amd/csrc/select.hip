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
//    lanes per block), keeps the chunk's online (max, sum exp) and its top-K
//    as packed 64-bit keys (wave bitonic sort + bitonic merges).  A second
//    kernel merges the chunk lists per head, finishes the LSE and writes the
//    ascending indices and log gates.
//  * rows (any number of rows): one thread per query row, summaries staged in
//    LDS 64 candidates at a time and read as broadcasts, a sorted top-K held
//    in registers; the erf term is formed in fp64 so the ranking of scores
//    near ~10 is not decided by fp32 rounding.
#include <type_traits>

#include "spa_device.h"
#include "spa_launch.h"

namespace spa {

// ------------------------------------------------------------------ decode
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_chunk_kernel(
    const T* __restrict__ q, const T* __restrict__ kbar, const float* __restrict__ proj_w,
    int Hq, int Hkv, int Hsel, int share_group, int64_t ccap, int64_t ncand, int K,
    uint64_t* __restrict__ ws_keys, float2* __restrict__ ws_ml, int nchunks) {
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kLPB = D / kVec;           // lanes per block row
  constexpr int kBPR = kWave / kLPB;       // blocks per load round of a wave
  constexpr int kRounds = kWave / kBPR;    // rounds to cover the wave's 64 blocks
  __shared__ float s_q[D];
  __shared__ float s_u[D];
  __shared__ float s_score[kDecodeChunk];
  __shared__ uint64_t s_keys[4][kWave];
  __shared__ float2 s_ml[4];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int chunk = blockIdx.x;
  const int bh = blockIdx.y;               // b * Hsel + hs
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int G = Hq / Hkv;
  const int kvh = share_group ? hs : hs / G;

  // q_hat (mean over the group's query heads when shared), then u = W^T q_hat
  if (tid < D) {
    float acc = 0.f;
    if (share_group) {
      for (int g = 0; g < G; ++g)
        acc += ld_f(q + (static_cast<int64_t>(bi) * Hq + hs * G + g) * D + tid);
      acc = acc / static_cast<float>(G);
    } else {
      acc = ld_f(q + (static_cast<int64_t>(bi) * Hq + hs) * D + tid);
    }
    s_q[tid] = acc;
  }
  __syncthreads();
  if (tid < D) {
    float u = s_q[tid];
    if (proj_w != nullptr) {
      u = 0.f;
      for (int e = 0; e < D; ++e) u = fmaf(proj_w[e * D + tid], s_q[e], u);
    }
    s_u[tid] = u;
  }
  __syncthreads();

  const int cg = lane % kLPB, bl = lane / kLPB;
  float uc[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i) uc[i] = s_u[cg * kVec + i];

  const int64_t wbase = static_cast<int64_t>(chunk) * kDecodeChunk + wave * kWave;
  const T* kb = kbar + (static_cast<int64_t>(bi) * Hkv + kvh) * ccap * D;
  uint4 raw[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    int64_t c = wbase + r * kBPR + bl;
    if (c < ncand)
      raw[r] = *reinterpret_cast<const uint4*>(kb + c * D + cg * kVec);
    else
      raw[r] = make_uint4(0, 0, 0, 0);
  }
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    float x[kVec];
    Elem<T>::unpack(raw[r], x);
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < kVec; ++i) p = fmaf(x[i], uc[i], p);
#pragma unroll
    for (int m = kLPB / 2; m > 0; m >>= 1) p += __shfl_xor(p, m, kWave);
    if (cg == 0) s_score[wave * kWave + r * kBPR + bl] = p * scale;
  }
  __syncthreads();

  const int64_t c = wbase + lane;
  const bool valid = c < ncand;
  const float s = s_score[wave * kWave + lane];
  uint64_t key = valid ? make_key(s, static_cast<int32_t>(c)) : 0ull;
  key = wave_sort_desc(key, lane);
  s_keys[wave][lane] = key;
  float m = wave_max(valid ? s : -INFINITY);
  float l = wave_sum(valid ? __expf(s - m) : 0.f);
  if (m == -INFINITY) l = 0.f;
  if (lane == 0) s_ml[wave] = make_float2(m, l);
  __syncthreads();

  if (wave == 0) {
    uint64_t top = s_keys[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) top = wave_merge_top_desc(top, s_keys[w][kWave - 1 - lane], lane);
    const int64_t o = static_cast<int64_t>(bh) * nchunks + chunk;
    if (lane < K) ws_keys[o * K + lane] = top;
    if (lane == 0) {
      float mm = s_ml[0].x, ll = s_ml[0].y;
      for (int w = 1; w < 4; ++w) ml_combine(mm, ll, s_ml[w].x, s_ml[w].y);
      ws_ml[o] = make_float2(mm, ll);
    }
  }
}

__global__ __launch_bounds__(256) void decode_merge_kernel(
    const uint64_t* __restrict__ ws_keys, const float2* __restrict__ ws_ml, int nchunks, int K,
    int64_t ncand, int gate, int nq, int row, int32_t* __restrict__ idx, float* __restrict__ logg,
    int32_t* __restrict__ k_eff) {
  __shared__ uint64_t s_top[4][kWave];
  __shared__ float2 s_ml[4];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int bh = blockIdx.x;
  const uint64_t* keys = ws_keys + static_cast<int64_t>(bh) * nchunks * K;

  uint64_t top = 0ull;
  for (int ch = wave; ch < nchunks; ch += 4) {
    const int r = kWave - 1 - lane;
    uint64_t brev = r < K ? keys[static_cast<int64_t>(ch) * K + r] : 0ull;
    top = wave_merge_top_desc(top, brev, lane);
  }
  s_top[wave][lane] = top;

  float m = -INFINITY, l = 0.f;
  for (int ch = tid; ch < nchunks; ch += 256) {
    float2 v = ws_ml[static_cast<int64_t>(bh) * nchunks + ch];
    ml_combine(m, l, v.x, v.y);
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    float m2 = __shfl_xor(m, off, kWave), l2 = __shfl_xor(l, off, kWave);
    ml_combine(m, l, m2, l2);
  }
  if (lane == 0) s_ml[wave] = make_float2(m, l);
  __syncthreads();
  if (wave != 0) return;

  top = s_top[0][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) top = wave_merge_top_desc(top, s_top[w][kWave - 1 - lane], lane);
  float mm = s_ml[0].x, ll = s_ml[0].y;
  for (int w = 1; w < 4; ++w) ml_combine(mm, ll, s_ml[w].x, s_ml[w].y);
  const float lse = mm + __logf(ll);

  const int keff = static_cast<int>(ncand < K ? ncand : K);
  // re-sort the kept keys by index ascending: key2 = (~index << 32) | score bits
  uint64_t key2 = 0ull;
  if (lane < keff && top != 0ull) {
    const uint32_t ci = static_cast<uint32_t>(key_index(top));
    key2 = (static_cast<uint64_t>(~ci) << 32) | __float_as_uint(key_score(top));
  }
  key2 = wave_sort_desc(key2, lane);
  const int64_t o = (static_cast<int64_t>(bh) * nq + row) * K;
  if (lane < K) {
    if (lane < keff) {
      const int32_t ci = static_cast<int32_t>(~static_cast<uint32_t>(key2 >> 32));
      const float sc = __uint_as_float(static_cast<uint32_t>(key2));
      idx[o + lane] = ci;
      if (logg != nullptr) logg[o + lane] = gate ? (sc - lse) : 0.f;
    } else {
      idx[o + lane] = -1;
      if (logg != nullptr) logg[o + lane] = 0.f;
    }
  }
  if (lane == 0 && k_eff != nullptr) k_eff[static_cast<int64_t>(bh) * nq + row] = keff;
}

// -------------------------------------------------------------------- rows
template <typename S>
__device__ __forceinline__ bool better(S s1, int i1, S s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

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
      if (better(sc, ci, ts[KMAX - 1], ti[KMAX - 1])) {
        ts[KMAX - 1] = sc;
        ti[KMAX - 1] = ci;
#pragma unroll
        for (int t = KMAX - 1; t > 0; --t) {
          if (better(ts[t], ti[t], ts[t - 1], ti[t - 1])) {
            S xs = ts[t]; ts[t] = ts[t - 1]; ts[t - 1] = xs;
            int xi = ti[t]; ti[t] = ti[t - 1]; ti[t - 1] = xi;
          }
        }
      }
    }
  }
  if (!active) return;

  const int keff = static_cast<int>(ncand < K ? ncand : K);
  // keep the first keff, order them by index (unused slots sort last)
#pragma unroll
  for (int t = 0; t < KMAX; ++t)
    if (t >= keff) ti[t] = 0x7FFFFFFF;
#pragma unroll
  for (int a = 0; a < KMAX; ++a) {
#pragma unroll
    for (int t = KMAX - 1; t > a; --t) {
      if (ti[t] < ti[t - 1]) {
        S xs = ts[t]; ts[t] = ts[t - 1]; ts[t - 1] = xs;
        int xi = ti[t]; ti[t] = ti[t - 1]; ti[t - 1] = xi;
      }
    }
  }
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
static bool use_decode_path(const SelectLaunch& p) {
  return p.nq == 1 && p.prefix_mode == 0 && p.erf_lambda == nullptr;
}

size_t select_workspace_bytes(const SelectLaunch& p) {
  if (!use_decode_path(p)) return 0;
  const int64_t nch = decode_num_chunks(p.max_cand > 0 ? p.max_cand : 1);
  const size_t heads = static_cast<size_t>(p.B) * p.Hsel;
  return align256(heads * nch * p.K * sizeof(uint64_t)) + align256(heads * nch * sizeof(float2));
}

template <typename T, int D>
static hipError_t launch_decode_t(const SelectLaunch& p, void* ws, hipStream_t st) {
  const int64_t ncand = p.max_cand;
  const int nch = static_cast<int>(decode_num_chunks(ncand > 0 ? ncand : 1));
  const size_t heads = static_cast<size_t>(p.B) * p.Hsel;
  uint64_t* keys = static_cast<uint64_t*>(ws);
  float2* ml = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                         align256(heads * nch * p.K * sizeof(uint64_t)));
  hipLaunchKernelGGL((decode_chunk_kernel<T, D>), dim3(nch, static_cast<unsigned>(heads)), dim3(256),
                     0, st, static_cast<const T*>(p.q), static_cast<const T*>(p.kbar), p.proj_w,
                     p.Hq, p.Hkv, p.Hsel, p.share_group, p.ccap, ncand, p.K, keys, ml, nch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(static_cast<unsigned>(heads)), dim3(256), 0, st,
                     keys, ml, nch, p.K, ncand, p.gate, 1, 0, p.idx, p.logg, p.k_eff);
  return hipGetLastError();
}

template <typename T, int D, int KMAX>
static hipError_t launch_rows_k(const SelectLaunch& p, hipStream_t st) {
  dim3 grid((p.nq + 255) / 256, static_cast<unsigned>(p.B * p.Hsel));
  if (p.erf_lambda != nullptr) {
    hipLaunchKernelGGL((rows_select_kernel<T, D, KMAX, true>), grid, dim3(256), 0, st,
                       static_cast<const T*>(p.q), static_cast<const T*>(p.kbar), p.max_norm,
                       p.centre, p.proj_w, p.erf_lambda, p.erf_sigma, p.Hq, p.Hkv, p.Hsel, p.nq,
                       p.q_pos0, p.ccap, p.b, p.prefix_mode, p.qblock, p.share_group, p.K, p.gate,
                       p.idx, p.logg, p.k_eff);
  } else {
    hipLaunchKernelGGL((rows_select_kernel<T, D, KMAX, false>), grid, dim3(256), 0, st,
                       static_cast<const T*>(p.q), static_cast<const T*>(p.kbar), p.max_norm,
                       p.centre, p.proj_w, p.erf_lambda, p.erf_sigma, p.Hq, p.Hkv, p.Hsel, p.nq,
                       p.q_pos0, p.ccap, p.b, p.prefix_mode, p.qblock, p.share_group, p.K, p.gate,
                       p.idx, p.logg, p.k_eff);
  }
  return hipGetLastError();
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
  if (p.dtype == 1) return p.d == 64 ? launch_rows_t<bf16_t, 64>(p, st) : launch_rows_t<bf16_t, 128>(p, st);
  return p.d == 64 ? launch_rows_t<float, 64>(p, st) : launch_rows_t<float, 128>(p, st);
}

}  // namespace spa
