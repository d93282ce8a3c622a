// retain.hip -- FS-L fixed-state retention and the per-query selection inside
// the kept set, on gfx950 ("FreeSolo" review, the two variants: before any
// query arrives each head keeps only its W most recent cells and its P cells
// of largest max key norm; each query then takes its top K inside that set).
//
// Kept set of a (batch, kv head) with ncand prefix cells: the W most recent
// cells plus the P older cells of largest max_norm, lower index first on
// equal norms; ascending, -1 padded to W + P.
//   retain_cells_kernel   one 1024-thread workgroup per (batch, kv head): the
//                         P-th largest older norm by a bitwise threshold
//                         search (workgroup ballot counts), then the older
//                         cells above it and the first equal ones in cell
//                         order by an ordered compaction, then the recent
//                         cells.
//   select_subset_kernel  one workgroup per (batch, selection head, query
//                         row), a list slot per thread: fp64 scores of the
//                         listed cells that are candidates of the row
//                         (q_hat . kbar / sqrt(d), plus the erf position
//                         bias), the gate over those cells, and the top K by
//                         a threshold search over the scores' orderable bits
//                         (higher score, then lower cell); the kept slots are
//                         written in list order, which is ascending cell order.
#include "spa_device.h"
#include "spa_launch.h"

namespace spa {

constexpr int kSubsetMaxCap = 256;  // listed cells per head: one per thread

// One 1024-thread workgroup per (batch, kv head).  The older cells' norms
// sit in registers 16384 at a time (cell s0 + j * 1024 + tid in key[j]); t is
// the kr-th largest (kr = min(P, older cells)); every older cell above t is
// kept, and the first kr - #(above t) cells equal to t in cell order; both
// rank and position come from per-(chunk, wave) ballot counts and a prefix
// over them, so the kept cells come out in cell order.
__global__ __launch_bounds__(kWgThreads) void retain_cells_kernel(const float* __restrict__ max_norm, int64_t ccap,
                                                                 int64_t ncand, int W, int P,
                                                                 int32_t* __restrict__ cells,
                                                                 int32_t* __restrict__ count) {
  constexpr int kRegs = 16;
  constexpr int64_t kSpan = static_cast<int64_t>(kWgThreads) * kRegs;
  constexpr int kEnt = kRegs * kWgWaves;       // (chunk, wave) entries per span: 4 per lane of wave 0
  static_assert(kEnt == 4 * kWave, "four entries per lane");
  __shared__ int s_part[2 * kWgWaves];
  __shared__ uint32_t s_lohi[2 * kWgWaves];
  __shared__ int s_cnt[kEnt];
  __shared__ int64_t s_base[kEnt];
  __shared__ int64_t s_tot;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t head = blockIdx.x;
  const float* a = max_norm + head * ccap;
  const int cap = W + P;
  const int64_t n_old = ncand > W ? ncand - W : 0;
  const int kr = static_cast<int>(n_old < P ? n_old : P);
  int32_t* out = cells + head * cap;

  // wave 0: exclusive prefix of the span's kEnt counts (entry e = chunk e / 16,
  // wave e % 16, i.e. cell order) on top of `run`; the total into s_tot
  auto scan_entries = [&](int64_t run) {
    if (wave == 0) {
      int v[4];
      int sum = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = s_cnt[lane * 4 + r];
        sum += v[r];
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int up = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += up;
      }
      int64_t pre = run + incl - sum;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s_base[lane * 4 + r] = pre;
        pre += v[r];
      }
      if (lane == kWave - 1) s_tot = incl;
    }
    __syncthreads();
  };

  int64_t kept = 0;
  if (kr > 0) {
    uint32_t key[kRegs];                       // 0 marks a slot past the older cells
#pragma unroll
    for (int j = 0; j < kRegs; ++j) {          // clamped, so the loads issue together
      const int64_t c = j * kWgThreads + tid;
      const uint32_t kv = orderable_f32(a[c < n_old ? c : n_old - 1]);
      key[j] = c < n_old ? kv : 0u;
    }
    const uint32_t t = wg_kth_largest_f32<kRegs>(key, a, n_old, kr, s_part, s_lohi);
    // cells above t
    int gt = 0;
#pragma unroll
    for (int j = 0; j < kRegs; ++j) gt += __popcll(__ballot(key[j] > t));
    for (int64_t c0 = kSpan; c0 < n_old; c0 += kWgThreads) {
      const int64_t c = c0 + tid;
      gt += __popcll(__ballot(c < n_old && orderable_f32(a[c < n_old ? c : n_old - 1]) > t));
    }
    if (lane == 0) s_part[wave] = gt;
    __syncthreads();
    int ngt = 0;
#pragma unroll
    for (int w = 0; w < kWgWaves; ++w) ngt += s_part[w];
    const int need_eq = kr - ngt;              // cells equal to t still to keep, lowest first
    int64_t eq_run = 0;
    for (int64_t s0 = 0; s0 < n_old; s0 += kSpan) {
      if (s0 > 0) {
#pragma unroll
        for (int j = 0; j < kRegs; ++j) {
          const int64_t c = s0 + j * kWgThreads + tid;
          const uint32_t kv = orderable_f32(a[c < n_old ? c : n_old - 1]);
          key[j] = c < n_old ? kv : 0u;
        }
      }
      // ranks among the cells equal to t
#pragma unroll
      for (int j = 0; j < kRegs; ++j) {
        const int ce = __popcll(__ballot(key[j] == t));
        if (lane == 0) s_cnt[j * kWgWaves + wave] = ce;
      }
      __syncthreads();
      scan_entries(eq_run);
      bool keep[kRegs];
#pragma unroll
      for (int j = 0; j < kRegs; ++j) {
        const uint64_t me = __ballot(key[j] == t);
        const int64_t rank = s_base[j * kWgWaves + wave] + lanes_below(me);
        keep[j] = key[j] > t || (key[j] == t && rank < need_eq);
      }
      eq_run += s_tot;
      __syncthreads();                         // ranks read before the counts are rewritten
      // positions of the kept cells
#pragma unroll
      for (int j = 0; j < kRegs; ++j) {
        const int ck = __popcll(__ballot(keep[j]));
        if (lane == 0) s_cnt[j * kWgWaves + wave] = ck;
      }
      __syncthreads();
      scan_entries(kept);
#pragma unroll
      for (int j = 0; j < kRegs; ++j) {
        const uint64_t mk = __ballot(keep[j]);
        if (keep[j]) out[s_base[j * kWgWaves + wave] + lanes_below(mk)] = static_cast<int32_t>(s0 + j * kWgThreads + tid);
      }
      kept += s_tot;
      __syncthreads();                         // bases read before the next span rewrites them
    }
  }
  // the W recent cells, then padding
  const int64_t nrec = ncand - n_old;
  for (int64_t x = tid; x < nrec; x += kWgThreads) out[kept + x] = static_cast<int32_t>(n_old + x);
  for (int64_t x = kept + nrec + tid; x < cap; x += kWgThreads) out[x] = -1;
  if (tid == 0) count[head] = static_cast<int32_t>(kept + nrec);
}

// ---------------------------------------------------------------- select
// One workgroup per (batch, selection head, query row); thread j scores list
// slot j (all loads issued from clamped addresses before the arithmetic).
template <typename T, int D>
__global__ __launch_bounds__(256) void select_subset_kernel(
    const T* __restrict__ q, const T* __restrict__ kbar, const float* __restrict__ max_norm,
    const float* __restrict__ centre, int Hq, int Hkv, int Hsel, int share_group, int nq, int64_t q_pos0,
    int64_t ccap, int b, int prefix_mode, int qblock, const float* __restrict__ erf_lambda,
    const float* __restrict__ erf_sigma, const int32_t* __restrict__ cells, const int32_t* __restrict__ count,
    int cap, int K, int gate, int32_t* __restrict__ idx, float* __restrict__ logg, int32_t* __restrict__ k_eff) {
  static_assert(kSubsetMaxCap == 4 * kWave, "one list slot per thread");
  constexpr int kVec = Elem<T>::kVec;
  __shared__ double s_q[D];
  __shared__ double s_sc[kSubsetMaxCap];
  __shared__ int32_t s_cid[kSubsetMaxCap];
  __shared__ double s_red[2][4];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int bh = blockIdx.y;
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int G = Hq / Hkv;
  const int kvh = share_group ? hs : hs / G;
  const int row = blockIdx.x;
  const int64_t pos = q_pos0 + row;
  const int64_t ncand = prefix_mode == 0 ? pos / b : (static_cast<int64_t>(qblock) * (pos / qblock)) / b;
  const int64_t hb = static_cast<int64_t>(bi) * Hkv + kvh;

  // this slot's cell and its summary row (slot 0's cell stands in for empty slots)
  const int nl = count[hb];
  const int32_t* lst = cells + hb * cap;
  const int j = tid;
  const int c = j < nl && j < cap ? lst[j] : -1;
  const bool ok = c >= 0 && c < ncand;
  const int64_t cc = ok ? c : 0;
  uint4 raw[D / kVec];
  const uint4* kr = reinterpret_cast<const uint4*>(kbar + (hb * ccap + cc) * D);
#pragma unroll
  for (int v = 0; v < D / kVec; ++v) raw[v] = kr[v];
  const bool erf_on = erf_lambda != nullptr;
  const double ac = erf_on ? static_cast<double>(max_norm[hb * ccap + cc]) : 0.0;
  const double pc = erf_on ? static_cast<double>(centre[cc]) : 0.0;

  // q_hat in fp64 (mean of the group's heads, summed in head order)
  if (wave == 0) {
    const int gq = share_group ? G : 1;
    const int h0 = share_group ? hs * G : hs;
    for (int e = lane; e < D; e += kWave) {
      double sq = 0.0;
      for (int g = 0; g < gq; ++g)
        sq += static_cast<double>(ld_f(q + ((static_cast<int64_t>(bi) * Hq + h0 + g) * nq + row) * D + e));
      s_q[e] = sq / static_cast<double>(gq);
    }
  }
  __syncthreads();

  const double inv_sqrt_d = 1.0 / sqrt(static_cast<double>(D));
  double sv = -INFINITY;
  if (ok) {
    double dot = 0.0;
#pragma unroll
    for (int v = 0; v < D / kVec; ++v) {
      float x[kVec];
      Elem<T>::unpack(raw[v], x);
#pragma unroll
      for (int t = 0; t < kVec; ++t) dot = fma(static_cast<double>(x[t]), s_q[v * kVec + t], dot);
    }
    sv = dot * inv_sqrt_d;
    if (erf_on) {
      const double lam = static_cast<double>(erf_lambda[hs]);
      const double sig = static_cast<double>(erf_sigma[hs]);
      sv += lam * ac * erf((static_cast<double>(pos) - pc) / (2.0 * sig));
    }
  }
  s_sc[j] = sv;
  s_cid[j] = ok ? c : -1;

  // gate: LSE over the listed candidates (wave maxima and sums, then over the waves)
  double m = sv;
  for (int off = 32; off >= 1; off >>= 1) {
    const double o = __shfl_xor(m, off);
    m = o > m ? o : m;
  }
  if (lane == 0) s_red[0][wave] = m;
  __syncthreads();
  m = s_red[0][0];
#pragma unroll
  for (int w = 1; w < 4; ++w) m = s_red[0][w] > m ? s_red[0][w] : m;
  double l = ok ? exp(sv - m) : 0.0;
  for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
  if (lane == 0) s_red[1][wave] = l;
  __syncthreads();
  if (wave != 0) return;
  l = s_red[1][0] + s_red[1][1] + s_red[1][2] + s_red[1][3];

  // top K (higher score, then lower list slot = lower cell), kept in list order
  double sc[4];
  bool okv[4], taken[4];
  int32_t cid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cid[i] = s_cid[i * kWave + lane];
    okv[i] = cid[i] >= 0;
    sc[i] = s_sc[i * kWave + lane];
  }
  const int kk = wave_top_f64x4(sc, okv, K, taken);
  const double lse = kk > 0 ? m + log(l) : 0.0;
  const int64_t o = (static_cast<int64_t>(bh) * nq + row) * K;
  int kept = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t tm = __ballot(taken[i]);
    if (taken[i]) {
      const int slot = kept + lanes_below(tm);
      idx[o + slot] = cid[i];
      if (logg != nullptr) logg[o + slot] = gate ? static_cast<float>(sc[i] - lse) : 0.f;
    }
    kept += __popcll(tm);
  }
  for (int x = kept + lane; x < K; x += kWave) {
    idx[o + x] = -1;
    if (logg != nullptr) logg[o + x] = 0.f;
  }
  if (lane == 0 && k_eff != nullptr) k_eff[static_cast<int64_t>(bh) * nq + row] = kk;
}

hipError_t launch_retain_cells(const float* max_norm, int B, int Hkv, int64_t ccap, int64_t ncand, int W, int P,
                               int32_t* cells, int32_t* count, hipStream_t st) {
  return launch(true, retain_cells_kernel, dim3(static_cast<unsigned>(B * Hkv)), dim3(kWgThreads), st, max_norm, ccap,
                ncand, W, P, cells, count);
}

template <typename T, int D>
static hipError_t launch_subset_t(const SelectLaunch& p, const int32_t* cells, const int32_t* count, int cap,
                                  hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.nq), static_cast<unsigned>(p.B * p.Hsel));
  return launch(true, select_subset_kernel<T, D>, grid, dim3(256), st, static_cast<const T*>(p.q),
                static_cast<const T*>(p.kbar), p.max_norm, p.centre, p.Hq, p.Hkv, p.Hsel, p.share_group, p.nq,
                p.q_pos0, p.ccap, p.b, p.prefix_mode, p.qblock, p.erf_lambda, p.erf_sigma, cells, count, cap, p.K,
                p.gate, p.idx, p.logg, p.k_eff);
}

hipError_t launch_score_select_subset(const SelectLaunch& p, const int32_t* cells, const int32_t* count, int cap,
                                      hipStream_t st) {
  if (p.dtype == kDtypeBf16)
    return p.d == 64 ? launch_subset_t<bf16_t, 64>(p, cells, count, cap, st)
                     : launch_subset_t<bf16_t, 128>(p, cells, count, cap, st);
  return p.d == 64 ? launch_subset_t<float, 64>(p, cells, count, cap, st)
                   : launch_subset_t<float, 128>(p, cells, count, cap, st);
}

}  // namespace spa
