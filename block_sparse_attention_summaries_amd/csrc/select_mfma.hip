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
// merge at the end.
//
// Group selection scores with the mean query of the G heads, which is not a
// bf16 value: it is formed in fp32 and split into three bf16 terms
// (hi + mid + lo carries 27 significant bits), so three MFMA products give the
// fp32 dot product to within fp32 rounding.
//
// erf term: the bias reaches ~10, where fp32 cannot rank to 1e-6.  The scan
// ranks fp32 scores (a branch-free erf approximation, read from a per-
// workgroup table of row - cell b when the centres are the cell middles) in a
// list twice the budget long.  At the end, list entries within twice a proven
// error bound of the fp32 K-th best are re-scored exactly (fp64 dot product
// and bias) and the exact top-K is taken from them; with the gate off, a row
// whose (K+1)-th entry lies below that band keeps its first K entries as they
// are.  If the list's last entry is itself within the band, a candidate may
// have been dropped, and the row is re-scored exactly in full.
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

// NTERM = 1: one head's bf16 query; NTERM = 3: split group-mean query.
// List length: KMAX (no erf; fp32 ranking is final) or 2 KMAX (erf).
template <int D, int KMAX, int NTERM, bool kErf>
__global__ __launch_bounds__(256, (kErf && D == 64 && NTERM == 1 && KMAX == 4) ? 3 : 1) void rows_select_mfma_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kbar, const float* __restrict__ max_norm,
    const float* __restrict__ centre, const float* __restrict__ erf_lambda,
    const float* __restrict__ erf_sigma, int Hq, int Hkv, int Hsel, int nq, int64_t q_pos0,
    int64_t ccap, int b, int prefix_mode, int qblock, int share_group, int K, int gate,
    int32_t* __restrict__ idx, float* __restrict__ logg, int32_t* __restrict__ k_eff) {
  constexpr int kT = 32;                  // candidates per tile
  constexpr int kKS = D / 16;             // MFMA k-steps
  constexpr int KL = kErf ? 2 * KMAX : KMAX;
  constexpr int kErfTab = 6144;           // filter table entries (24 KB): x = 4 within it for sigma <= ~766
  static_assert(!kErf || KL <= 16, "list staging uses 16 LDS slots per lane");
  __shared__ __align__(16) float s_beta32[4][kT];   // per wave: lambda a_c of the tile's candidates
  __shared__ float s_p[4][kT];            // per wave: their centres (filter per score)
  __shared__ float s_sc[4][16][64];       // per wave: candidate slot r x lane
  __shared__ double s_x[4][64];           // per wave: half-row dot products
  __shared__ float s_erf[kErf ? kErfTab : 1];   // filter erf by row - cell b (see below)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  const int rt = static_cast<int>(gridDim.x) - 1 - static_cast<int>(blockIdx.x);  // long rows first
  const int bh = blockIdx.y;
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
  bool use_tab = false;
  if constexpr (kErf) {
    lam = static_cast<double>(erf_lambda[hs]);
    lam32 = erf_lambda[hs];
    inv2sig = 1.0 / (2.0 * static_cast<double>(erf_sigma[hs]));
    inv2sig32 = static_cast<float>(inv2sig);
    // With the centres c b + (b - 1) / 2 the filter's argument is
    // ((row - c b) - (b - 1) / 2) / (2 sigma), both differences exact in fp32:
    // the filter value is a function of j = row - c b, tabulated in LDS with
    // the same fp32 arithmetic (bit-identical scores).  j past the table holds
    // x >= 4, where the filter is 1.  Other centres, or a sigma whose x = 4
    // lies past the table, take the filter per score.
    const float hb = static_cast<float>(b - 1) * 0.5f;
    int ok = 1;
    for (int64_t c = tid; c < wg_cand; c += 256)
      ok &= centre[c] == static_cast<float>(c * b) + hb ? 1 : 0;
    ok &= (static_cast<float>(kErfTab - 1) - hb) * inv2sig32 >= 4.0f ? 1 : 0;
    ok &= static_cast<int64_t>(wg_cand) * b < (1 << 23) && q_pos0 + nq < (1 << 23) ? 1 : 0;
    use_tab = __builtin_amdgcn_readfirstlane(__syncthreads_and(ok)) != 0;
    if (use_tab) {
      for (int j = tid; j < kErfTab; j += 256) {
        const float x32 = (static_cast<float>(j) - hb) * inv2sig32;
        s_erf[j] = x32 < 4.0f ? erf_filter(x32) : 1.0f;
      }
    }
  }

  // this lane's query slices (k = 16 ks + 8 hl .. +7) as NTERM bf16 terms
  uint4 qt[NTERM][kKS];
  float qsq = 0.f;                        // squared norm of this lane's query half
  if constexpr (NTERM == 1) {
    const __bf16* qrow = q + ((static_cast<int64_t>(bi) * Hq + h0) * nq + rowc) * D;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      qt[0][ks] = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hl);
      if constexpr (kErf) {
        float f[8];
        Elem<bf16_t>::unpack(qt[0][ks], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) qsq = fmaf(f[e], f[e], qsq);
      }
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
  if constexpr (kErf) qsq += xor_lanes_f<32>(qsq);

  float ls[KL];                           // fp32 scores, best first
  int li[KL];
#pragma unroll
  for (int t = 0; t < KL; ++t) {
    ls[t] = -INFINITY;
    li[t] = 0x7FFFFFFF;
  }
  float m_run = -INFINITY, l_run = 0.f;   // gate LSE over this lane's candidates
  float amax_t = 0.f;                     // lanes 0..31: largest max norm staged

  // Each wave runs on its own (no workgroup barrier in the walk): the lane's
  // A operand (candidate c0 + ql, columns 16 ks + 8 hl .. +7) comes straight
  // from memory, one tile ahead; lanes 0..31 stage the tile's lambda a_c (and
  // centres) in the wave's LDS slice.
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

  for (int64_t c0 = 0; c0 < wave_cand; c0 += kT) {
    if constexpr (kErf) {
      wave_lds_sync();                    // the previous tile's readers are done
      if (hl == 0) {
        s_beta32[wave][ql] = lam32 * pre_a;
        s_p[wave][ql] = pre_p;
        amax_t = fmaxf(amax_t, fabsf(pre_a));
      }
      wave_lds_sync();
    }
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

    // register r holds candidate c0 + 8 (r / 4) + 4 hl + (r % 4) of this lane's
    // row.  Pass 1 (unrolled): scores, gate terms and the admission mask
    // against the tile-start list end; pass 2 walks the admitted slots only.
    float sv[16];
    uint32_t mask = 0;
    const float thr = ls[KL - 1];
    // erf bias terms of the lane's 16 candidates, their loads issued together:
    // m = 8 (r / 4) + 4 hl + (r % 4), so lambda a_c comes as four 16-byte reads
    float e32[16];
    float4 bet[4];
    if constexpr (kErf) {
      const int jb = static_cast<int>(pos - (c0 + 4 * hl) * b);   // j of candidate m = 4 hl
      if (use_tab) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = jb - (8 * (r >> 2) + (r & 3)) * b;
          e32[r] = s_erf[j < 0 ? 0 : (j < kErfTab ? j : kErfTab - 1)];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x32 = (static_cast<float>(pos) - s_p[wave][8 * (r >> 2) + 4 * hl + (r & 3)]) * inv2sig32;
          e32[r] = x32 < 4.0f ? erf_filter(x32) : 1.0f;
        }
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) bet[q4] = *reinterpret_cast<const float4*>(&s_beta32[wave][8 * q4 + 4 * hl]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * hl + (r & 3);
      float s = st[r] * scale;
      if constexpr (kErf) {
        const float4 bq = bet[r >> 2];
        const float bm = (r & 3) == 0 ? bq.x : (r & 3) == 1 ? bq.y : (r & 3) == 2 ? bq.z : bq.w;
        s = fmaf(bm, e32[r], s);
      }
      s_sc[wave][r][lane] = s;
      const bool valid = c0 + m < ncand;
      sv[r] = valid ? s : -INFINITY;
      mask |= (valid && s > thr) ? (1u << r) : 0u;
    }
    if (gate) {
      float tm = m_run;
#pragma unroll
      for (int r = 0; r < 16; ++r) tm = fmaxf(tm, sv[r]);
      if (tm != -INFINITY) {
        float acc = l_run * __expf(m_run - tm);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc += __expf(sv[r] - tm);
        l_run = acc;
        m_run = tm;
      }
    }
    // within a lane candidates arrive in increasing index, so a tie keeps the
    // entry already held
    // (the next admitted slot's LDS read is issued before the current insert)
    if (mask != 0) {
      int r = __builtin_ctz(mask);
      mask &= mask - 1;
      float v = s_sc[wave][r][lane];
      while (true) {
        const bool more = mask != 0;
        const int rn = more ? __builtin_ctz(mask) : r;
        mask &= mask - 1;
        const float vn = s_sc[wave][rn][lane];
        if (v > ls[KL - 1]) topk_push_later(ls, li, v, static_cast<int>(c0) + 8 * (r >> 2) + 4 * hl + (r & 3));
        if (!more) break;
        r = rn;
        v = vn;
      }
    }
  }
#undef SPA_FETCH_TILE

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
    // this row: the filter erf and its fp32 argument (<= 1.2e-6 |lambda a_c|),
    // the final fma and operand roundings (<= 1.2e-7 |score|), and the MFMA's
    // fp32 accumulation of d NTERM products (<= (d NTERM + 2) 2^-24 |q|
    // |kbar_c| / sqrt(d), with |kbar_c| <= a_c).  E takes each term at least
    // 4x wider.
    const float amax = wave_max(amax_t);   // every candidate this wave's rows scored
    float smax = 0.f;
#pragma unroll
    for (int t = 0; t < KL; ++t)
      if (li[t] != 0x7FFFFFFF) smax = fmaxf(smax, fabsf(ls[t]));
    const float err = 5e-6f * (1.f + smax + fabsf(lam32) * amax) +
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
    const int64_t nsrc = decided ? 0 : (rescan ? ncand : n_ok);
    uint4 kv[kKS];
    float cen = 0.f, anorm = 0.f;
    int c = 0;
#define SPA_LOAD_CAND(J)                                                                      \
  do {                                                                                        \
    c = rescan ? static_cast<int>(J) : slot[(J) * 64 + lane];                                 \
    _Pragma("unroll") for (int ks = 0; ks < kKS; ++ks)                                        \
      kv[ks] = *reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(c) * D + 16 * ks + 8 * hl); \
    cen = centre[c];                                                                          \
    anorm = mn[c];                                                                            \
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
      if (j + 1 < nsrc) SPA_LOAD_CAND(j + 1);
      s_x[wave][lane] = part;
      wave_lds_sync();
      const double other = s_x[wave][lane ^ 32];
      wave_lds_sync();
      const double dot = hl == 0 ? part + other : other + part;
      const double sc = dot * inv_sqrt_d + beta * erf_exact(x);
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
  return p.dtype == 1 && p.proj_w == nullptr && p.K <= kmax && (p.d == 64 || p.d == 128);
}

template <int D, int KMAX, int NTERM, bool kErf>
static hipError_t launch_mfma_k(const SelectLaunch& p, hipStream_t st) {
  dim3 grid((p.nq + 127) / 128, static_cast<unsigned>(p.B * p.Hsel));
  return launch(true, rows_select_mfma_kernel<D, KMAX, NTERM, kErf>, grid, dim3(256), st,
                static_cast<const __bf16*>(p.q), static_cast<const __bf16*>(p.kbar), p.max_norm, p.centre,
                p.erf_lambda, p.erf_sigma, p.Hq, p.Hkv, p.Hsel, p.nq, p.q_pos0, p.ccap, p.b, p.prefix_mode,
                p.qblock, p.share_group, p.K, p.gate, p.idx, p.logg, p.k_eff);
}

template <int D, int NTERM>
static hipError_t launch_mfma_n(const SelectLaunch& p, hipStream_t st) {
  if (p.erf_lambda != nullptr) {
    if (p.K <= 4) return launch_mfma_k<D, 4, NTERM, true>(p, st);
    return launch_mfma_k<D, 8, NTERM, true>(p, st);
  }
  if (p.K <= 4) return launch_mfma_k<D, 4, NTERM, false>(p, st);
  if (p.K <= 8) return launch_mfma_k<D, 8, NTERM, false>(p, st);
  if (p.K <= 16) return launch_mfma_k<D, 16, NTERM, false>(p, st);
  return launch_mfma_k<D, 32, NTERM, false>(p, st);
}

template <int D>
static hipError_t launch_mfma_d(const SelectLaunch& p, hipStream_t st) {
  const bool group_mean = p.share_group && p.Hq / p.Hkv > 1;
  return group_mean ? launch_mfma_n<D, 3>(p, st) : launch_mfma_n<D, 1>(p, st);
}

hipError_t launch_rows_select_mfma(const SelectLaunch& p, hipStream_t st) {
  return p.d == 64 ? launch_mfma_d<64>(p, st) : launch_mfma_d<128>(p, st);
}

}  // namespace spa
