// select_mfma.hip -- per-row selector scores, softmax log gate and top-K for
// many query rows (prefill / training) with bf16 MFMA (gfx950
// v_mfma_f32_32x32x16_bf16).  Same results as rows_select_kernel in
// select.hip: "SAS" review §3 Eq. 3 (score q.kbar/sqrt(d)), §4.2.2 (softmax
// log gate); "FreeSolo" review, "How it works" (cell score plus the erf
// position bias lambda_h a_c erf((i - p_c)/(2 sigma_h))).
//
// A workgroup of 4 waves covers 128 query rows (4 tiles of 32) of one
// selection head; each wave walks its own rows' candidates without workgroup
// barriers (the A operand rows come straight from memory, one tile ahead).
// Per tile of 32 candidates, S^T = Kbar Q^T (candidates x queries) gives each
// lane one query row and 16 candidates, so every lane keeps its row's running
// top list and gate (max, sum exp) in registers; the two half-waves of a row
// merge at the end.  The MFMA forms q.kbar from zero and one fma adds the
// bias; scores run in units of 1/scale until the walk ends.  The grid runs
// every head's longest rows first (row tiles from the last).
//
// Group selection scores with the mean query of the G heads, which is not a
// bf16 value: it is formed in fp32 and split into three bf16 terms
// (hi + mid + lo carries 27 significant bits), so three MFMA products give the
// fp32 dot product to within fp32 rounding.
//
// erf term: the bias reaches ~10, where fp32 cannot rank to 1e-6.  The scan
// ranks fp32 scores (the filter read from the head's table of row - cell b,
// erf_table_kernel, when the centres are the cell middles, else a
// branch-free erf approximation per score; a tile whose every (row, cell)
// pair lies where the filter is 1 skips it) in a list twice the budget long,
// admitting only scores within the largest possible band of the row's
// running K-th best (over both half-waves' lists).  At the end, list entries within twice a proven error bound of the
// fp32 K-th best are re-scored exactly (fp64 dot product and bias) and the
// exact top-K is taken from them; with the gate off, a row whose (K+1)-th
// entry lies below that band keeps its first K entries as they are, and
// otherwise re-scores only the entries not certainly inside.  If the list's
// last entry is itself within the band, a candidate may have been dropped,
// and the row is re-scored exactly in full.
#include "spa_device.h"
#include "spa_launch.h"

namespace spa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 sbf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float sfloatx16_t;

__device__ __forceinline__ sbf16x8_t sel_bf16x8(uint4 v) { return __builtin_bit_cast(sbf16x8_t, v); }

// erf for the fp32 filter: Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (|error| <= 1.5e-7 in exact arithmetic), branch
// free.  Evaluated in fp32 with the hardware reciprocal and exp2 (1 ulp each)
// its error stays below 1e-6 for every x.
__device__ __forceinline__ float erf_filter(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
  const float poly =
      fmaf(fmaf(fmaf(fmaf(1.061405429f, t, -1.453152027f), t, 1.421413741f), t, -0.284496736f), t,
           0.254829592f) * t;
  const float g = __builtin_amdgcn_exp2f(-(ax * ax) * 1.4426950408889634f);
  return copysignf(fmaf(-poly, g, 1.0f), x);
}

// First tile of the erf walk: the lane's list is empty, so its KL best of
// the tile's 16 scores come from a sorting network instead of 16 inserts.
// Each score becomes a key with its tile slot r in the low 4 mantissa bits
// (keys are distinct; a key is within 16 ulp, 2^-19 relative, of its score,
// which the error bounds below include); -inf (no candidate) becomes the
// finite -3.4e38 (the largest finite negative) first, so no key is a NaN.  Batcher's bitonic sort orders
// the two halves, the better of each mirrored pair of the halves forms a
// bitonic sequence holding the best 8 of 16, and a half-cleaner cascade sorts
// it; KL = 16 sorts all 16 with the full network.
__device__ __forceinline__ void key_ce(float& a, float& b) {
  const float hi = __builtin_fmaxf(a, b);
  b = __builtin_fminf(a, b);
  a = hi;
}

template <int N>
__device__ __forceinline__ void bitonic_sort_keys(float* k) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1)
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          if ((i & size) == 0)
            key_ce(k[i], k[j]);
          else
            key_ce(k[j], k[i]);
        }
      }
}

template <int KL>
__device__ __forceinline__ void first_tile_list(const float (&sv)[16], int c_lane, float (&ls)[KL], int (&li)[KL]) {
  static_assert(KL == 8 || KL == 16, "first-tile network: lists of 8 or 16");
  float k[16];
#pragma unroll
  for (int r = 0; r < 16; ++r)
    k[r] = __uint_as_float((__float_as_uint(__builtin_fmaxf(sv[r], -3.40282347e38f)) & ~15u) | static_cast<uint32_t>(r));
  if constexpr (KL == 16) {
    bitonic_sort_keys<16>(k);
  } else {
    bitonic_sort_keys<8>(k);
    bitonic_sort_keys<8>(k + 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) k[i] = __builtin_fmaxf(k[i], k[15 - i]);
#pragma unroll
    for (int stride = 4; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((i & stride) == 0) key_ce(k[i], k[i + stride]);
  }
#pragma unroll
  for (int t = 0; t < KL; ++t) {
    const uint32_t r = __float_as_uint(k[t]) & 15u;
    const bool ok = k[t] > -1e38f;
    ls[t] = ok ? k[t] : -INFINITY;
    li[t] = ok ? c_lane + static_cast<int>(((r & 12u) << 1) | (r & 3u)) : 0x7FFFFFFF;
  }
}

// Per-head tables of the FreeSolo filter erf((i - p_c)/(2 sigma_h)).  With
// the centres at the cell middles p_c = c b + (b - 1)/2 the argument is
// x_j = (j - (b - 1)/2)/(2 sigma) for the integer j = i - c b, so the filter
// is a function of j.  tab64 holds erf_exact(x_j) for j in [-neg, n64 - neg)
// (entry j + neg): the fp64 value the exact re-score uses, with x formed as
// it forms it.  tab32 holds the same values rounded to fp32 for the MFMA walk,
// laid out by residue: j = (q - qoff) b + res sits at res * qs + q, so the
// 16 candidates a lane scores in one tile (cells c0 + m, m in four runs of
// four) are four runs of neighbouring entries at fixed offsets from one base.
// From jsat on (x >= 4) every fp32 entry is 1 (1 - erf(4) < 2^-25).
constexpr int kTab32Cap = 8192;           // fp32 entries per head (32 KB of LDS in the scorer)
constexpr int kTab64Cap = 16384;          // fp64 entries per head
constexpr size_t kErfTabBytes = kTab32Cap * sizeof(float) + kTab64Cap * sizeof(double);

struct ErfTabGeom {
  int neg, qoff, qs, n64, jsat;
  bool ok32, ok64;
};

// The same arithmetic in the table kernel and the scorer.  j >= -neg covers
// every (row, cell) pair a tile walk forms (cells up to one tile past a row's
// candidates); tab32 reaches 32 b + 64 past jsat, the farthest pair of a tile
// that is not wholly past jsat; tab64 reaches x = 6, past which erf_exact is 1.
__device__ __forceinline__ ErfTabGeom erf_tab_geom(int b, float sigma) {
  ErfTabGeom g;
  const double hb = 0.5 * static_cast<double>(b - 1);
  const double x4 = hb + 8.0 * static_cast<double>(sigma);
  const double x6 = hb + 12.0 * static_cast<double>(sigma);
  g.neg = 40 * b + 64;
  g.qoff = (g.neg + b - 1) / b + 1;
  const bool fin4 = x4 < static_cast<double>(1 << 20), fin6 = x6 < static_cast<double>(1 << 20);
  g.jsat = fin4 ? static_cast<int>(ceil(x4)) : 0x7FFFFFFF;
  g.qs = fin4 ? (((g.jsat + 32 * b + 64) / b + g.qoff + 2) | 1) : 0;
  g.ok32 = fin4 && b * g.qs <= kTab32Cap;
  g.n64 = fin6 ? g.neg + static_cast<int>(ceil(x6)) + 2 : 0;
  g.ok64 = fin6 && g.n64 <= kTab64Cap;
  return g;
}

// One thread per j = e - neg, e in [0, kTab64Cap): grid (kTab64Cap / 256,
// Hsel).  A thread evaluates its filter value once and writes it to tab64
// (e < n64) and, rounded, to its tab32 entry (when j has one; the entries of
// tab32 below j = -neg are never read).  kTab64Cap - neg covers every j of
// tab32, since b qs <= kTab32Cap.
__global__ __launch_bounds__(256) void erf_table_kernel(const float* __restrict__ erf_sigma, int b,
                                                        float* __restrict__ tab32, double* __restrict__ tab64) {
  const int hs = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const ErfTabGeom g = erf_tab_geom(b, erf_sigma[hs]);
  const double hb = 0.5 * static_cast<double>(b - 1);
  const double inv2sig = 1.0 / (2.0 * static_cast<double>(erf_sigma[hs]));
  const int j = e - g.neg;
  const int q = (j >= 0 ? j / b : -((-j + b - 1) / b)) + g.qoff;   // floor(j / b) + qoff
  const int res = j - (q - g.qoff) * b;
  const bool in64 = g.ok64 && e < g.n64, in32 = g.ok32 && q >= 0 && q < g.qs;
  if (!in64 && !in32) return;
  const double v = erf_exact((static_cast<double>(j) - hb) * inv2sig);
  if (in64) tab64[static_cast<int64_t>(hs) * kTab64Cap + e] = v;
  if (in32) tab32[static_cast<int64_t>(hs) * kTab32Cap + res * g.qs + q] = static_cast<float>(v);
}

// NTERM = 1: one head's bf16 query; NTERM = 3: split group-mean query.
// List length: KMAX (no erf; fp32 ranking is final) or 2 KMAX (erf).
template <int D, int KMAX, int NTERM, bool kErf>
__global__ __launch_bounds__(256, (kErf && D == 64 && NTERM == 1 && KMAX == 4) ? 3 : 1) void rows_select_mfma_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kbar, const float* __restrict__ max_norm,
    const float* __restrict__ centre, const float* __restrict__ erf_lambda,
    const float* __restrict__ erf_sigma, int Hq, int Hkv, int Hsel, int nq, int64_t q_pos0,
    int64_t ccap, int b, int prefix_mode, int qblock, int share_group, int K, int gate,
    int32_t* __restrict__ idx, float* __restrict__ logg, int32_t* __restrict__ k_eff,
    const float* __restrict__ tab32, const double* __restrict__ tab64) {
  constexpr int kT = 32;                  // candidates per tile
  constexpr int kKS = D / 16;             // MFMA k-steps
  constexpr int KL = kErf ? 2 * KMAX : KMAX;
  static_assert(!kErf || KL <= 16, "list staging uses 16 LDS slots per lane");
  __shared__ __align__(16) float s_beta32[4][kT];   // per wave: lambda a_c of the tile's candidates
  __shared__ float s_p[4][kT];            // per wave: their centres (filter per score)
  __shared__ float s_sc[4][16][64];       // per wave: candidate slot r x lane
  __shared__ double s_x[4][64];           // per wave: half-row dot products
  __shared__ __align__(16) float s_erf[kErf ? kTab32Cap : 4];   // the head's tab32 (see erf_tab_geom)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  // x = (batch, selection head), y = row tile from the last: dispatch runs
  // every head's longest rows first, and a head's workgroups share an XCD
  const int rt = static_cast<int>(gridDim.y) - 1 - static_cast<int>(blockIdx.y);
  const int bh = blockIdx.x;
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int G = Hq / Hkv;
  const int kvh = share_group ? hs : hs / G;
  const int nh = share_group ? G : 1;
  const int h0 = share_group ? hs * G : hs;
  const int row = (rt * 4 + wave) * 32 + ql;
  const bool row_ok = row < nq;
  const int rowc = row_ok ? row : nq - 1;
  const int64_t pos = q_pos0 + rowc;
  const int64_t ncand = row_ok ? num_candidates(pos, b, prefix_mode, qblock) : 0;
  const int last_row = ((rt * 4 + 4) * 32 < nq ? (rt * 4 + 4) * 32 : nq) - 1;
  const int64_t wg_cand = num_candidates(q_pos0 + last_row, b, prefix_mode, qblock);
  // the wave walks the candidates of its own rows (its last row has the most)
  const int wave_last = ((rt * 4 + wave + 1) * 32 < nq ? (rt * 4 + wave + 1) * 32 : nq) - 1;
  const int64_t wave_cand = wave_last >= (rt * 4 + wave) * 32 ? num_candidates(q_pos0 + wave_last, b, prefix_mode, qblock) : 0;
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const __bf16* kb = kbar + (static_cast<int64_t>(bi) * Hkv + kvh) * ccap * D;
  const float* mn = max_norm + (static_cast<int64_t>(bi) * Hkv + kvh) * ccap;
  double lam = 0.0, inv2sig = 0.0;
  float lam32 = 0.f, inv2sig32 = 0.f;
  bool use_tab = false, use_t64 = false;
  ErfTabGeom tg{};
  int jsat = 0x7FFFFFFF;
  // this lane's query slices (k = 16 ks + 8 hl .. +7) as NTERM bf16 terms
  uint4 qt[NTERM][kKS];
  float qsq = 0.f;                        // squared norm of this lane's query half
  if constexpr (NTERM == 1) {
    const __bf16* qrow = q + ((static_cast<int64_t>(bi) * Hq + h0) * nq + rowc) * D;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      qt[0][ks] = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hl);
    }
  } else {
    float acc[kKS][8];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[ks][e] = 0.f;
    for (int g = 0; g < nh; ++g) {
      const __bf16* qrow = q + ((static_cast<int64_t>(bi) * Hq + h0 + g) * nq + rowc) * D;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        float f[8];
        Elem<bf16_t>::unpack(*reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hl), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[ks][e] += f[e];
      }
    }
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      uint32_t w[NTERM][4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[ks][e] / static_cast<float>(nh);
        qsq = fmaf(x, x, qsq);
#pragma unroll
        for (int t = 0; t < NTERM; ++t) {
          const uint16_t h = float_to_bf16_rne(x);
          x -= bf16_to_float(h);
          if (e & 1) {
            w[t][e >> 1] |= static_cast<uint32_t>(h) << 16;
          } else {
            w[t][e >> 1] = h;
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NTERM; ++t) qt[t][ks] = make_uint4(w[t][0], w[t][1], w[t][2], w[t][3]);
    }
  }
  // Each wave runs on its own (no workgroup barrier in the walk): the lane's
  // A operand (candidate c0 + ql, columns 16 ks + 8 hl .. +7) comes straight
  // from memory, one tile ahead; lanes 0..31 stage the tile's lambda a_c / scale
  // (and centres) in the wave's LDS slice.
  uint4 ka[kKS];
  float pre_a = 0.f, pre_p = 0.f;
#define SPA_FETCH_TILE(C0)                                                                    \
  do {                                                                                        \
    int64_t c = (C0) + ql;                                                                    \
    c = c < wave_cand ? c : wave_cand - 1;                                                    \
    _Pragma("unroll") for (int ks = 0; ks < kKS; ++ks)                                        \
      ka[ks] = *reinterpret_cast<const uint4*>(kb + c * D + 16 * ks + 8 * hl);                \
    if constexpr (kErf) {                                                                     \
      pre_a = mn[c];                                                                          \
      pre_p = centre[c];                                                                      \
    }                                                                                         \
  } while (0)

  if (wave_cand > 0) SPA_FETCH_TILE(0);

  // erf setup.  With the centres at the cell middles the filter is a function
  // of j = row - c b, read from the head's tables (erf_table_kernel); other
  // centres take the filter per score and erf_exact in the re-score.  Every
  // load here (the fp32 table, the wave's max norms, the workgroup's centres)
  // is issued before the first is waited for.
  float am = 0.f;                         // largest |a_c| over the wave's candidates
  if constexpr (kErf) {
    lam = static_cast<double>(erf_lambda[hs]);
    lam32 = erf_lambda[hs];
    inv2sig = 1.0 / (2.0 * static_cast<double>(erf_sigma[hs]));
    inv2sig32 = static_cast<float>(inv2sig);
    tg = erf_tab_geom(b, erf_sigma[hs]);
    constexpr int kTL = kTab32Cap / 4 / 256;      // 16-byte table loads per thread
    const int n4 = tg.ok32 ? (b * tg.qs + 3) / 4 : 0;
    const float4* src = reinterpret_cast<const float4*>(tab32 + static_cast<int64_t>(hs) * kTab32Cap);
    float4 tl[kTL];
#pragma unroll
    for (int u = 0; u < kTL; ++u) tl[u] = src[tid + 256 * u < n4 ? tid + 256 * u : 0];
    float av[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int64_t c = lane + 64 * t;
      av[t] = mn[c < wave_cand ? c : 0];
    }
    float cv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t c = tid + 256 * t;
      cv[t] = centre[c < wg_cand ? c : 0];
    }
    const float hb = static_cast<float>(b - 1) * 0.5f;
    int ok = 1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t c = tid + 256 * t;
      ok &= c >= wg_cand || cv[t] == static_cast<float>(c * b) + hb ? 1 : 0;
    }
    for (int64_t c = tid + 512; c < wg_cand; c += 256) ok &= centre[c] == static_cast<float>(c * b) + hb ? 1 : 0;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (lane + 64 * t < wave_cand) am = fmaxf(am, fabsf(av[t]));
    for (int64_t c = lane + 512; c < wave_cand; c += 64) am = fmaxf(am, fabsf(mn[c]));
    am = wave_max(am);
    ok &= static_cast<int64_t>(wg_cand) * b < (1 << 23) && q_pos0 + nq < (1 << 23) ? 1 : 0;
    // the table goes to LDS whether or not the centres allow it (it is read
    // only when they do); the barrier below publishes it
#pragma unroll
    for (int u = 0; u < kTL; ++u)
      if (tid + 256 * u < n4) reinterpret_cast<float4*>(s_erf)[tid + 256 * u] = tl[u];
    ok = __builtin_amdgcn_readfirstlane(__syncthreads_and(ok));
    use_tab = ok != 0 && tg.ok32;
    use_t64 = ok != 0 && tg.ok64;
    if (use_tab) jsat = tg.jsat;
  }
  if constexpr (kErf && NTERM == 1) {
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      float f[8];
      Elem<bf16_t>::unpack(qt[0][ks], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) qsq = fmaf(f[e], f[e], qsq);
    }
  }
  if constexpr (kErf) qsq += xor_lanes_f<32>(qsq);

  // The walk runs in units of 1/scale (the MFMA's own q.kbar, the bias
  // staged as lambda a_c / scale); list scores and the gate's max take the
  // scale once it ends.
  const float inv_scale = sqrtf(static_cast<float>(D));
  const float lam_s = lam32 * inv_scale;
  const float k2 = scale * 1.4426950408889634f;     // exp(x scale) = exp2(x k2)
  float ls[KL];                           // scores (1/scale units), best first
  int li[KL];
  float m_run = -INFINITY, l_run = 0.f;   // gate LSE over this lane's candidates

  // Tiles before ncand_min hold valid candidates for every row of the wave;
  // a tile whose candidates all lie jsat or more before the wave's first row
  // has erf = 1 for every score (its bias is the accumulator's initial value).
  const int64_t row0 = static_cast<int64_t>(rt * 4 + wave) * 32;
  const bool rows_all_ok = __ballot(!row_ok) == 0ull;
  const int64_t ncand_min = rows_all_ok ? num_candidates(q_pos0 + row0, b, prefix_mode, qblock) : 0;

#pragma unroll
  for (int t = 0; t < KL; ++t) {
    ls[t] = -INFINITY;
    li[t] = 0x7FFFFFFF;
  }
  // erf path: the list only has to hold every score within the final error
  // band of the row's K-th best (and flag a rescan when it may not).  The
  // band is at most twice err_max, the error bound below evaluated with
  // |score| <= |q| a_max / sqrt(d) + |lambda| a_max over the wave's largest
  // max norm a_max, so a score under the lane's current K-th best minus that
  // can be left out; 1/scale units, with 25 % to spare.
  float band = INFINITY;
  // relative error of the walk's bias lambda a_c erf / scale (taken 4x wider):
  // the fp32 products and roundings of lambda / scale and a_c, the table's
  // rounding to fp32 (2^-25), or the per-score filter's 1.2e-6
  const float bias_rel = use_tab ? 1.4e-6f : 6.2e-6f;
  // tab32 base of this lane's row: entry of candidate c0 + m is
  // t_base - c0 + 27 - (m - 4 hl); t_top keeps the 28 entries in the table
  const int t_base = use_tab ? static_cast<int>(pos % b) * tg.qs + static_cast<int>(pos / b) + tg.qoff - 4 * hl - 27 : 0;
  const int t_top = use_tab ? b * tg.qs - 28 : 0;
  if constexpr (kErf) {
    const float qn = sqrtf(qsq);
    const float sb = qn * am * scale + fabsf(lam32) * am;
    const float err_max = 5e-6f + 2.4e-6f * sb + bias_rel * fabsf(lam32) * am +
                          4.f * static_cast<float>(D * NTERM + 2) * 5.97e-8f * qn * am * scale;
    band = 2.5f * err_max * inv_scale;
  }
  {
    for (int64_t c0 = 0; c0 < wave_cand; c0 += kT) {
      if constexpr (kErf) {
        wave_lds_sync();                  // the previous tile's readers are done
        if (hl == 0) {
          s_beta32[wave][ql] = lam_s * pre_a;
          s_p[wave][ql] = pre_p;
        }
        wave_lds_sync();
      }
      // register r holds candidate c0 + 8 (r / 4) + 4 hl + (r % 4) of this
      // lane's row.  The MFMA forms q.kbar from zero; the bias lambda a_c /
      // scale (four 16-byte reads), times the filter erf unless the tile is
      // saturated, is added to it after, with one rounding.
      const bool sat = kErf && use_tab && q_pos0 + row0 - (c0 + kT - 1) * b >= jsat;
      sfloatx16_t st;
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
        for (int t = 0; t < NTERM; ++t)
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sel_bf16x8(ka[ks]), sel_bf16x8(qt[t][ks]), st, 0, 0, 0);
      }
      if (c0 + kT < wave_cand) SPA_FETCH_TILE(c0 + kT);
      float sv[16];
      if constexpr (kErf) {
        float bet[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 v4 = *reinterpret_cast<const float4*>(&s_beta32[wave][8 * q4 + 4 * hl]);
          bet[4 * q4] = v4.x;
          bet[4 * q4 + 1] = v4.y;
          bet[4 * q4 + 2] = v4.z;
          bet[4 * q4 + 3] = v4.w;
        }
        if (sat) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[r] = st[r] + bet[r];
        } else if (use_tab) {
          // tab32 entry of candidate m: t_base - c0 + 27 - (m - 4 hl)
          int tb = t_base - static_cast<int>(c0);
          tb = tb < 0 ? 0 : (tb > t_top ? t_top : tb);
          const float* te = s_erf + tb;
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[r] = fmaf(bet[r], te[27 - (8 * (r >> 2) + (r & 3))], st[r]);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float x32 =
                (static_cast<float>(pos) - s_p[wave][8 * (r >> 2) + 4 * hl + (r & 3)]) * inv2sig32;
            sv[r] = fmaf(bet[r], x32 < 4.0f ? erf_filter(x32) : 1.0f, st[r]);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = st[r];
      }
      if (c0 + kT > ncand_min) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (c0 + 8 * (r >> 2) + 4 * hl + (r & 3) >= ncand) sv[r] = -INFINITY;
      }
      if (gate) {
        float tm = m_run;
#pragma unroll
        for (int r = 0; r < 16; ++r) tm = fmaxf(tm, sv[r]);
        if (tm != -INFINITY) {
          float acc = l_run * __builtin_amdgcn_exp2f((m_run - tm) * k2);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc += __builtin_amdgcn_exp2f((sv[r] - tm) * k2);
          l_run = acc;
          m_run = tm;
        }
      }
      if constexpr (kErf) {
        if (c0 == 0) {
          first_tile_list<KL>(sv, 4 * hl, ls, li);
          continue;
        }
      }
      // admission against the tile-start list end: the wave enters the
      // insert only when one of its lanes holds a qualifying score
      float thr = ls[KL - 1];
      if constexpr (kErf) {
        // the row's running K-th best: the K-th of the union of this lane's
        // list and its partner half's (lane ^ 32).  The better of each
        // mirrored pair of the two sorted lists' first KMAX entries forms a
        // bitonic sequence holding the union's best KMAX; a half-cleaner
        // cascade sorts it.  A score below it minus the band cannot reach
        // the row's final top-K, whichever half holds it.
        float u[KMAX];
#pragma unroll
        for (int t = 0; t < KMAX; ++t) u[t] = __builtin_fmaxf(ls[t], xor_lanes_f<32>(ls[KMAX - 1 - t]));
#pragma unroll
        for (int stride = KMAX / 2; stride > 0; stride >>= 1)
#pragma unroll
          for (int t = 0; t < KMAX; ++t)
            if ((t & stride) == 0) key_ce(u[t], u[t + stride]);
        float lk = u[0];
#pragma unroll
        for (int t = 1; t < KMAX; ++t) lk = t == K - 1 ? u[t] : lk;
        thr = fmaxf(thr, lk - band);
      }
      float tmax = sv[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, sv[r]);
      if (__ballot(tmax > thr) == 0ull) continue;
      uint32_t mask = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s_sc[wave][r][lane] = sv[r];
        mask |= sv[r] > thr ? (1u << r) : 0u;
      }
      // within a lane candidates arrive in increasing index, so a tie keeps
      // the entry already held (the next admitted slot's LDS read is issued
      // before the current insert)
      if (mask != 0) {
        int r = __builtin_ctz(mask);
        mask &= mask - 1;
        float v = s_sc[wave][r][lane];
        while (true) {
          const bool more = mask != 0;
          const int rn = more ? __builtin_ctz(mask) : r;
          mask &= mask - 1;
          const float vn = s_sc[wave][rn][lane];
          if (v > thr && v > ls[KL - 1])
            topk_push_later(ls, li, v, static_cast<int>(c0) + 8 * (r >> 2) + 4 * hl + (r & 3));
          if (!more) break;
          r = rn;
          v = vn;
        }
      }
    }
  }
#undef SPA_FETCH_TILE
#pragma unroll
  for (int t = 0; t < KL; ++t) ls[t] *= scale;
  m_run *= scale;

  // merge the two half-waves of each row: the better of each entry and the
  // partner's mirrored entry forms a bitonic sequence holding the top KL of
  // both lists (Batcher's merge step); a half-cleaner cascade sorts it
  {
    float os[KL];
    int oi[KL];
#pragma unroll
    for (int t = 0; t < KL; ++t) {
      os[t] = xor_lanes_f<32>(ls[KL - 1 - t]);
      oi[t] = static_cast<int>(xor_lanes<32>(static_cast<uint32_t>(li[KL - 1 - t])));
    }
#pragma unroll
    for (int t = 0; t < KL; ++t) {
      if (sel_better(os[t], oi[t], ls[t], li[t])) {
        ls[t] = os[t];
        li[t] = oi[t];
      }
    }
    bitonic_clean_best_first(ls, li);
    const float m2 = xor_lanes_f<32>(m_run), l2 = xor_lanes_f<32>(l_run);
    ml_combine(m_run, l_run, m2, l2);
  }
  // both half-waves of a row hold the same merged list from here on
  if (!row_ok) return;
  const int keff = static_cast<int>(ncand < K ? ncand : K);
  const float lse = m_run + __logf(l_run);
  const int64_t o = ((static_cast<int64_t>(bi) * Hsel + hs) * nq + row) * K;

  if constexpr (!kErf) {
    if (hl != 0) return;
#pragma unroll
    for (int t = 0; t < KL; ++t)
      if (t >= keff) li[t] = 0x7FFFFFFF;
    sort_by_index(ls, li);  // unused slots (index 0x7FFFFFFF) sort last
#pragma unroll
    for (int t = 0; t < KL; ++t) {
      if (t < K) {
        const bool ok = t < keff;
        idx[o + t] = ok ? li[t] : -1;
        if (logg != nullptr) logg[o + t] = (ok && gate) ? ls[t] - lse : 0.f;
      }
    }
  } else {
    // Error bound of an fp32 score against the exact one, for any candidate of
    // this row: the MFMA's fp32 sum of d NTERM exact products from zero
    // (<= (d NTERM + 2) 2^-24 |q| |kbar_c| / sqrt(d), with |kbar_c| <= a_c);
    // the bias lambda a_c erf / scale (relative error <= 3.3e-7 with the
    // table: the roundings of sqrt(d), lambda / scale, its product with a_c,
    // the scale and the table's own 2^-25; the per-score filter adds its
    // 1.2e-6); the fma that adds it and the final scaling (<= 2 2^-24 |score|);
    // the first tile's keys (<= 15 2^-23 |score|, exact).  E takes the terms
    // other than the keys' 4x wider.
    const float amax = am;                 // every candidate this wave's rows scored
    float smax = 0.f;
#pragma unroll
    for (int t = 0; t < KL; ++t)
      if (li[t] != 0x7FFFFFFF) smax = fmaxf(smax, fabsf(ls[t]));
    const float err = 5e-6f + 2.4e-6f * smax + bias_rel * fabsf(lam32) * amax +
                      4.f * static_cast<float>(D * NTERM + 2) * 5.97e-8f * sqrtf(qsq) * amax * scale;
    const float kth32 = ncand >= K ? ls[K - 1] : -INFINITY;
    const float cut = kth32 - 2.f * err;
    // a dropped candidate scored at most ls[KL - 1]: if that is inside the band,
    // the list may be missing one of the exact top-K
    const bool rescan = ncand > KL && ls[KL - 1] >= cut;
    // gate off: only the set matters.  If the (K+1)-th listed score is below
    // the band, every candidate outside the first K scores exactly below every
    // one inside (|exact - fp32| <= err), so the first K are the exact top-K.
    const bool decided = !gate && (ncand <= K || ls[K] < cut);
    // gate off, not decided: an entry whose fp32 score passes the (K+1)-th
    // listed one (at least every fp32 score outside the first K) by more than
    // 2 err scores exactly above every candidate outside the first K, so it is
    // in the exact top-K; those entries (a prefix) keep their place and only
    // the rest of the qualifying prefix is scored exactly, for the other slots
    int m_sure = 0;
    if (!gate && !decided && !rescan) {
#pragma unroll
      for (int t = 0; t < KMAX; ++t) m_sure += (t < K && ls[t] > ls[K] + 2.f * err) ? 1 : 0;
    }
    // the qualifying entries are a prefix of the best-first list
    int* slot = reinterpret_cast<int*>(&s_sc[wave][0][0]);
    int n_ok = 0;
#pragma unroll
    for (int t = 0; t < KL; ++t) {
      slot[t * 64 + lane] = li[t];
      n_ok += (li[t] != 0x7FFFFFFF && ls[t] >= cut) ? 1 : 0;
    }

    // Exact score: the dot product of the bf16 query terms with kbar_c in fp64
    // (each half-wave takes its k-slices; the halves swap partial sums through
    // LDS and add them in the same order), plus the fp64 bias.  The next
    // candidate's loads are issued before the current one is scored.
    double es[KMAX];
    int ei[KMAX];
#pragma unroll
    for (int t = 0; t < KMAX; ++t) {
      es[t] = -INFINITY;
      ei[t] = 0x7FFFFFFF;
    }
    const double inv_sqrt_d = 1.0 / sqrt(static_cast<double>(D));
    const int64_t nsrc = decided ? 0 : (rescan ? ncand : n_ok - m_sure);
    uint4 kv[kKS];
    float cen = 0.f, anorm = 0.f;
    double t64v = 0.0;                      // tab64 entry of the candidate (when in the table)
    bool t64ok = false;
    int c = 0;
    const double* t64 = tab64 + static_cast<int64_t>(hs) * kTab64Cap;
#define SPA_LOAD_CAND(J)                                                                      \
  do {                                                                                        \
    c = rescan ? static_cast<int>(J) : slot[((J) + m_sure) * 64 + lane];                      \
    _Pragma("unroll") for (int ks = 0; ks < kKS; ++ks)                                        \
      kv[ks] = *reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(c) * D + 16 * ks + 8 * hl); \
    cen = centre[c];                                                                          \
    anorm = mn[c];                                                                            \
    const int64_t te = pos - static_cast<int64_t>(c) * b + tg.neg;                            \
    t64ok = use_t64 && te >= 0 && te < tg.n64;                                                \
    t64v = t64[t64ok ? te : 0];                                                               \
  } while (0)
    if (nsrc > 0) SPA_LOAD_CAND(0);
#pragma unroll 1
    for (int64_t j = 0; j < nsrc; ++j) {
      const int cj = c;
      double part = 0.0;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        float kf[8];
        Elem<bf16_t>::unpack(kv[ks], kf);
#pragma unroll
        for (int t = 0; t < NTERM; ++t) {
          // keep the query terms packed: without this the compiler hoists their
          // widening out of the loop and runs out of registers
          uint4 qp = qt[t][ks];
          asm volatile("" : "+v"(qp.x), "+v"(qp.y), "+v"(qp.z), "+v"(qp.w));
          float qf[8];
          Elem<bf16_t>::unpack(qp, qf);
          // bf16 x bf16 products are exact in fp32; the sum runs in fp64
#pragma unroll
          for (int e = 0; e < 8; ++e) part += static_cast<double>(qf[e] * kf[e]);
        }
      }
      const double x = (static_cast<double>(pos) - static_cast<double>(cen)) * inv2sig;
      const double beta = lam * static_cast<double>(anorm);
      const bool cj_t64 = t64ok;
      const double cj_erf = t64v;
      if (j + 1 < nsrc) SPA_LOAD_CAND(j + 1);
      s_x[wave][lane] = part;
      wave_lds_sync();
      const double other = s_x[wave][lane ^ 32];
      wave_lds_sync();
      const double dot = hl == 0 ? part + other : other + part;
      const double sc = dot * inv_sqrt_d + beta * (cj_t64 ? cj_erf : erf_exact(x));
      if (sel_better(sc, cj, es[KMAX - 1], ei[KMAX - 1])) topk_push(es, ei, sc, cj);
    }
#undef SPA_LOAD_CAND
    if (hl != 0) return;
    if (decided) {
#pragma unroll
      for (int t = 0; t < KMAX; ++t) {
        es[t] = t < K ? static_cast<double>(ls[t]) : -INFINITY;
        ei[t] = t < K ? li[t] : 0x7FFFFFFF;
      }
    } else if (m_sure > 0) {
      // the certain entries, then the best of the exactly scored ones
      double fe[KMAX];
      int fi[KMAX];
#pragma unroll
      for (int t = 0; t < KMAX; ++t) {
        double e = -INFINITY;
        int ix = 0x7FFFFFFF;
#pragma unroll
        for (int u = 0; u < KMAX; ++u) {
          if (u == t - m_sure) {
            e = es[u];
            ix = ei[u];
          }
        }
        fe[t] = t < m_sure ? static_cast<double>(ls[t]) : e;
        fi[t] = t < m_sure ? li[t] : ix;
      }
#pragma unroll
      for (int t = 0; t < KMAX; ++t) {
        es[t] = fe[t];
        ei[t] = fi[t];
      }
    }
#pragma unroll
    for (int t = 0; t < KMAX; ++t)
      if (t >= keff) ei[t] = 0x7FFFFFFF;
    sort_by_index(es, ei);
#pragma unroll
    for (int t = 0; t < KMAX; ++t) {
      if (t < K) {
        const bool ok = t < keff;
        idx[o + t] = ok ? ei[t] : -1;
        if (logg != nullptr) logg[o + t] = (ok && gate) ? static_cast<float>(es[t] - static_cast<double>(lse)) : 0.f;
      }
    }
  }
  if (k_eff != nullptr) k_eff[(static_cast<int64_t>(bi) * Hsel + hs) * nq + row] = keff;
}

bool rows_select_mfma_supported(const SelectLaunch& p) {
  const int kmax = p.erf_lambda != nullptr ? 8 : 32;
  return p.dtype == 1 && p.proj_w == nullptr && p.K <= kmax && (p.d == 64 || p.d == 128) &&
         (p.nq + 127) / 128 <= 65535;
}

// With the erf term: the per-head tables (tab32, then tab64) in the workspace.
size_t rows_select_mfma_ws_bytes(const SelectLaunch& p) {
  return p.erf_lambda != nullptr ? static_cast<size_t>(p.Hsel) * kErfTabBytes : 0;
}

template <int D, int KMAX, int NTERM, bool kErf>
static hipError_t launch_mfma_k(const SelectLaunch& p, void* ws, hipStream_t st) {
  float* tab32 = nullptr;
  double* tab64 = nullptr;
  if constexpr (kErf) {
    tab32 = static_cast<float*>(ws);
    tab64 = reinterpret_cast<double*>(static_cast<char*>(ws) + static_cast<size_t>(p.Hsel) * kTab32Cap * sizeof(float));
    const hipError_t e = launch(false, erf_table_kernel, dim3(kTab64Cap / 256, static_cast<unsigned>(p.Hsel)),
                                dim3(256), st, p.erf_sigma, p.b, tab32, tab64);
    if (e != hipSuccess) return e;
  }
  dim3 grid(static_cast<unsigned>(p.B * p.Hsel), (p.nq + 127) / 128);
  return launch(true, rows_select_mfma_kernel<D, KMAX, NTERM, kErf>, grid, dim3(256), st,
                static_cast<const __bf16*>(p.q), static_cast<const __bf16*>(p.kbar), p.max_norm, p.centre,
                p.erf_lambda, p.erf_sigma, p.Hq, p.Hkv, p.Hsel, p.nq, p.q_pos0, p.ccap, p.b, p.prefix_mode,
                p.qblock, p.share_group, p.K, p.gate, p.idx, p.logg, p.k_eff,
                static_cast<const float*>(tab32), static_cast<const double*>(tab64));
}

template <int D, int NTERM>
static hipError_t launch_mfma_n(const SelectLaunch& p, void* ws, hipStream_t st) {
  if (p.erf_lambda != nullptr) {
    if (p.K <= 4) return launch_mfma_k<D, 4, NTERM, true>(p, ws, st);
    return launch_mfma_k<D, 8, NTERM, true>(p, ws, st);
  }
  if (p.K <= 4) return launch_mfma_k<D, 4, NTERM, false>(p, ws, st);
  if (p.K <= 8) return launch_mfma_k<D, 8, NTERM, false>(p, ws, st);
  if (p.K <= 16) return launch_mfma_k<D, 16, NTERM, false>(p, ws, st);
  return launch_mfma_k<D, 32, NTERM, false>(p, ws, st);
}

template <int D>
static hipError_t launch_mfma_d(const SelectLaunch& p, void* ws, hipStream_t st) {
  const bool group_mean = p.share_group && p.Hq / p.Hkv > 1;
  return group_mean ? launch_mfma_n<D, 3>(p, ws, st) : launch_mfma_n<D, 1>(p, ws, st);
}

hipError_t launch_rows_select_mfma(const SelectLaunch& p, void* ws, hipStream_t st) {
  return p.d == 64 ? launch_mfma_d<64>(p, ws, st) : launch_mfma_d<128>(p, ws, st);
}

}  // namespace spa
