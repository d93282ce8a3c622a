// forest.hip -- FS-B hierarchical selection on gfx950 ("FreeSolo" review, the
// two variants: no cell is dropped; each head builds a forest over the whole
// prefix and one over the cells at or above the median max key norm; nodes
// hold a mean key, a radius, a max norm and a min position; a beam of width
// W_b = 16 descends them, the node score U bounding the cell scores below;
// the reached cells are re-ranked by logsumexp over their token keys and the
// top K are read).
//
// Forest over m member cells (ascending): fanout 16; node j of level 1 groups
// members [16 j, 16 j + 16), node j of level l groups nodes [16 j, 16 j + 16)
// of level l - 1; levels are added until one has at most 16 nodes.  Node
// fields (fp32, nearest): mu = (sum of the cells' mean keys, summed child by
// child in fp64) / cells, r = max ||kbar_c - mu|| over the cells below, a = max
// max-norm, p = min centre.
//   U_v = q_hat . mu / sqrt(d) + ||q_hat|| r / sqrt(d) + lambda a erf((i - p) / (2 sigma)).
//
//   forest_build_kernel   one workgroup per (batch, kv head, forest): the
//                         median by a radix select (four 8-bit passes over an
//                         LDS histogram), the members by an ordered compaction,
//                         then the levels bottom-up (fp64 sums in the
//                         workspace) and the radii (a thread per level-1 node,
//                         a wave per node above).
//   forest_select_kernel  one wave per (batch, selection head, query row):
//                         per forest, the beam (up to 256 children scored in
//                         fp64, the 16 best kept by repeated arg-max, lower id
//                         first on ties), then the union of the reached cells
//                         re-ranked by the logsumexp of their token scores.
#include "spa_device.h"
#include "spa_launch.h"

namespace spa {

constexpr int kFan = 16;       // fanout
constexpr int kBeam = 16;      // beam width per level
constexpr int kMaxLev = 8;     // levels of a forest (16^8 cells)

struct ForestShape {
  int nl;
  int64_t n[kMaxLev], off[kMaxLev];
};

__host__ __device__ inline ForestShape forest_shape(int64_t m) {
  ForestShape s{};
  int64_t cur = m, off = 0;
  while (cur > kFan && s.nl < kMaxLev) {
    cur = (cur + kFan - 1) / kFan;
    s.n[s.nl] = cur;
    s.off[s.nl] = off;
    off += cur;
    ++s.nl;
  }
  return s;
}

// the shape written straight into (LDS) arrays, without a private copy
__device__ inline void forest_shape_into(int64_t m, ForestShape* out) {
  int64_t cur = m, off = 0;
  int nl = 0;
  while (cur > kFan && nl < kMaxLev) {
    cur = (cur + kFan - 1) / kFan;
    out->n[nl] = cur;
    out->off[nl] = off;
    off += cur;
    ++nl;
  }
  out->nl = nl;
}

int64_t forest_nodes(int64_t m) {
  const ForestShape s = forest_shape(m);
  return s.nl ? s.off[s.nl - 1] + s.n[s.nl - 1] : 0;
}

// ---------------------------------------------------------------- build
template <typename T, int D>
__global__ __launch_bounds__(256) void forest_build_kernel(
    const T* __restrict__ kbar, const float* __restrict__ max_norm, const float* __restrict__ centre, int64_t ccap,
    int64_t n, int64_t NN, int32_t* __restrict__ members, int32_t* __restrict__ nmem, float* __restrict__ mu,
    float* __restrict__ rad, float* __restrict__ amax, float* __restrict__ pmin, double* __restrict__ sums) {
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_cnt[256];
  __shared__ uint32_t s_sel[2];
  __shared__ ForestShape s_sh;                 // in LDS: its arrays are indexed by loop variables
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t head = blockIdx.x;
  const int f = blockIdx.y;
  const float* a = max_norm + head * ccap;
  const T* kb = kbar + head * ccap * D;
  int32_t* mem = members + (head * 2 + f) * n;
  const int64_t fb = (head * 2 + f) * NN;
  double* sm = sums + fb * D;

  // 1. median: the ceil(n/2)-th largest max norm (exact, by an 8-bit radix select)
  uint32_t thr = 0u;
  if (f == 1 && n > 0) {
    uint32_t prefix = 0u, mask = 0u;
    uint32_t kr = static_cast<uint32_t>((n + 1) / 2);
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      s_hist[tid] = 0u;
      __syncthreads();
      for (int64_t c = tid; c < n; c += 256) {
        const uint32_t key = orderable_f32(a[c]);
        if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t rem = kr;
        int dg = 255;
        for (; dg > 0; --dg) {
          if (s_hist[dg] >= rem) break;
          rem -= s_hist[dg];
        }
        s_sel[0] = static_cast<uint32_t>(dg);
        s_sel[1] = rem;
      }
      __syncthreads();
      prefix |= s_sel[0] << shift;
      mask |= 255u << shift;
      kr = s_sel[1];
      __syncthreads();
    }
    thr = prefix;
  }
  // 2. members in cell order (ordered compaction: a contiguous range per thread)
  const int64_t per = (n + 255) / 256;
  const int64_t c0 = tid * per, c1 = c0 + per < n ? c0 + per : n;
  uint32_t cnt = 0;
  for (int64_t c = c0; c < c1; ++c) cnt += (f == 0 || orderable_f32(a[c]) >= thr) ? 1u : 0u;
  s_cnt[tid] = cnt;
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0;
    for (int t = 0; t < 256; ++t) {
      const uint32_t v = s_cnt[t];
      s_cnt[t] = run;
      run += v;
    }
    s_sel[0] = run;
  }
  __syncthreads();
  const int64_t m = s_sel[0];
  {
    int64_t w = s_cnt[tid];
    for (int64_t c = c0; c < c1; ++c)
      if (f == 0 || orderable_f32(a[c]) >= thr) mem[w++] = static_cast<int32_t>(c);
  }
  for (int64_t x = m + tid; x < n; x += 256) mem[x] = -1;
  if (tid == 0) {
    nmem[head * 2 + f] = static_cast<int32_t>(m);
    forest_shape_into(m, &s_sh);
  }
  __syncthreads();

  // 3. node sums, means, max norms and min positions, level by level
  const ForestShape& sh = s_sh;
  for (int l = 0; l < sh.nl; ++l) {
    const int64_t nn = sh.n[l], off = sh.off[l];
    const int64_t nchild = l == 0 ? m : sh.n[l - 1];
    int64_t span = kFan;
    for (int x = 0; x < l; ++x) span *= kFan;
    for (int64_t x = tid; x < nn * D; x += 256) {
      const int64_t j = x / D;
      const int e = static_cast<int>(x % D);
      double s = 0.0;
      for (int64_t y = j * kFan; y < (j + 1) * kFan && y < nchild; ++y)
        s += l == 0 ? static_cast<double>(ld_f(kb + static_cast<int64_t>(mem[y]) * D + e))
                    : sm[(sh.off[l - 1] + y) * D + e];
      sm[(off + j) * D + e] = s;
      const int64_t cells = (j + 1) * span <= m ? span : m - j * span;
      mu[(fb + off + j) * D + e] = static_cast<float>(s / static_cast<double>(cells));
    }
    for (int64_t j = tid; j < nn; j += 256) {
      float am = 0.f, pm = INFINITY;
      for (int64_t y = j * kFan; y < (j + 1) * kFan && y < nchild; ++y) {
        const float av = l == 0 ? a[mem[y]] : amax[fb + sh.off[l - 1] + y];
        const float pv = l == 0 ? centre[mem[y]] : pmin[fb + sh.off[l - 1] + y];
        am = av > am ? av : am;
        pm = pv < pm ? pv : pm;
      }
      amax[fb + off + j] = am;
      pmin[fb + off + j] = pm;
    }
    __syncthreads();
  }
  // 4. radii: max distance of the cells below to the node's (fp32) mean
  for (int l = 0; l < sh.nl; ++l) {
    const int64_t nn = sh.n[l], off = sh.off[l];
    int64_t span = kFan;
    for (int x = 0; x < l; ++x) span *= kFan;
    if (l == 0) {
      for (int64_t j = tid; j < nn; j += 256) {
        const float* mv = mu + (fb + off + j) * D;
        double best = 0.0;
        for (int64_t y = j * kFan; y < (j + 1) * kFan && y < m; ++y) {
          const T* kr = kb + static_cast<int64_t>(mem[y]) * D;
          double ss = 0.0;
          for (int e = 0; e < D; ++e) {
            const double df = static_cast<double>(ld_f(kr + e)) - static_cast<double>(mv[e]);
            ss += df * df;
          }
          best = ss > best ? ss : best;
        }
        rad[fb + off + j] = static_cast<float>(sqrt(best));
      }
    } else {
      for (int64_t j = wave; j < nn; j += 4) {
        const float* mv = mu + (fb + off + j) * D;
        double best = 0.0;
        const int64_t y1 = (j + 1) * span < m ? (j + 1) * span : m;
        for (int64_t y = j * span + lane; y < y1; y += kWave) {
          const T* kr = kb + static_cast<int64_t>(mem[y]) * D;
          double ss = 0.0;
          for (int e = 0; e < D; ++e) {
            const double df = static_cast<double>(ld_f(kr + e)) - static_cast<double>(mv[e]);
            ss += df * df;
          }
          best = ss > best ? ss : best;
        }
        for (int o = 32; o >= 1; o >>= 1) {
          const double ob = __shfl_xor(best, o);
          best = ob > best ? ob : best;
        }
        if (lane == 0) rad[fb + off + j] = static_cast<float>(sqrt(best));
      }
    }
  }
  // 5. slots past this forest's nodes (the high-norm forest is smaller)
  const int64_t used = sh.nl ? sh.off[sh.nl - 1] + sh.n[sh.nl - 1] : 0;
  for (int64_t x = used * D + tid; x < NN * D; x += 256) mu[fb * D + x] = 0.f;
  for (int64_t x = used + tid; x < NN; x += 256) {
    rad[fb + x] = 0.f;
    amax[fb + x] = 0.f;
    pmin[fb + x] = 0.f;
  }
}

// ---------------------------------------------------------------- select
// Top-16 of the wave's 4 x 64 (score, slot) pairs (slot = i * 64 + lane, ok
// marks the valid ones) by repeated arg-max, higher score then lower slot;
// sets taken[] for the kept pairs and returns how many were kept.
__device__ __forceinline__ int fs_top16(const double (&sc)[4], const bool (&ok)[4], int want, bool (&taken)[4]) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int i = 0; i < 4; ++i) taken[i] = false;
  int nv = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) nv += __popcll(__ballot(ok[i]));
  const int kk = nv < want ? nv : want;
  for (int t = 0; t < kk; ++t) {
    double bv = -INFINITY;
    int bj = 1 << 30;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = i * kWave + lane;
      if (ok[i] && !taken[i] && (sc[i] > bv || (sc[i] == bv && j < bj))) {
        bv = sc[i];
        bj = j;
      }
    }
    for (int o = 32; o >= 1; o >>= 1) {
      const double ov = __shfl_xor(bv, o);
      const int oj = __shfl_xor(bj, o);
      if (ov > bv || (ov == bv && oj < bj)) {
        bv = ov;
        bj = oj;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i * kWave + lane == bj) taken[i] = true;
  }
  return kk;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void forest_select_kernel(
    const T* __restrict__ q, const T* __restrict__ kbar, const float* __restrict__ max_norm,
    const float* __restrict__ centre, const T* __restrict__ kcache, int64_t L, int Hq, int Hkv, int Hsel,
    int share_group, int nq, int64_t q_pos0, int64_t ccap, int b, const float* __restrict__ erf_lambda,
    const float* __restrict__ erf_sigma, const int32_t* __restrict__ members, const int32_t* __restrict__ nmem,
    const float* __restrict__ mu, const float* __restrict__ rad, const float* __restrict__ amax,
    const float* __restrict__ pmin, int64_t n, int64_t NN, int K, int32_t* __restrict__ idx,
    int32_t* __restrict__ k_eff) {
  __shared__ double s_q[4][D];
  __shared__ int64_t s_front[4][kBeam];
  __shared__ int32_t s_reach[4][2 * kBeam];
  __shared__ double s_lse[4][2 * kBeam];
  __shared__ ForestShape s_sh[4];              // in LDS: its arrays are indexed by loop variables
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int bh = blockIdx.y;
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int G = Hq / Hkv;
  const int kvh = share_group ? hs : hs / G;
  const int row = blockIdx.x * 4 + wave;
  if (row >= nq) return;                       // whole wave leaves; no workgroup barrier below
  const int64_t head = static_cast<int64_t>(bi) * Hkv + kvh;
  const double pos = static_cast<double>(q_pos0 + row);
  const double isd = 1.0 / sqrt(static_cast<double>(D));
  const bool erf_on = erf_lambda != nullptr;
  const double lam = erf_on ? static_cast<double>(erf_lambda[hs]) : 0.0;
  const double sig = erf_on ? static_cast<double>(erf_sigma[hs]) : 1.0;

  // q_hat (fp64) and its norm
  const int gq = share_group ? G : 1;
  const int h0 = share_group ? hs * G : hs;
  double qq = 0.0;
  for (int e = lane; e < D; e += kWave) {
    double s = 0.0;
    for (int g = 0; g < gq; ++g)
      s += static_cast<double>(ld_f(q + ((static_cast<int64_t>(bi) * Hq + h0 + g) * nq + row) * D + e));
    s /= static_cast<double>(gq);
    s_q[wave][e] = s;
    qq += s * s;
  }
  for (int o = 32; o >= 1; o >>= 1) qq += __shfl_xor(qq, o);
  const double qn = sqrt(qq);
  wave_lds_sync();

  int nreach = 0;
  for (int f = 0; f < 2; ++f) {
    const int64_t m = nmem[head * 2 + f];
    const int32_t* mem = members + (head * 2 + f) * n;
    const int64_t fb = (head * 2 + f) * NN;
    if (lane == 0) forest_shape_into(m, &s_sh[wave]);
    wave_lds_sync();
    const ForestShape& sh = s_sh[wave];
    int nf = static_cast<int>(sh.nl ? sh.n[sh.nl - 1] : m);
    if (lane < nf) s_front[wave][lane] = lane;
    wave_lds_sync();
    int lev = sh.nl;
    bool first = true;
    for (;;) {
      // candidates: the frontier itself for a forest of cells only, else its children
      const bool own = first && sh.nl == 0;
      const int child_lev = own ? 0 : lev - 1;
      const int64_t nchild = child_lev == 0 ? m : sh.n[child_lev - 1];
      double sc[4];
      bool ok[4];
      int64_t id[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = i * kWave + lane;
        int64_t cid = -1;
        if (own) {
          cid = x < nf ? s_front[wave][x] : -1;
        } else if (x / kFan < nf) {
          const int64_t ch = s_front[wave][x / kFan] * kFan + (x % kFan);
          cid = ch < nchild ? ch : -1;
        }
        ok[i] = cid >= 0;
        id[i] = cid;
        double s = -INFINITY;
        if (ok[i]) {
          double dot = 0.0;
          if (child_lev == 0) {
            const int64_t c = mem[cid];
            const T* kr = kbar + (head * ccap + c) * D;
            for (int e = 0; e < D; ++e) dot = fma(s_q[wave][e], static_cast<double>(ld_f(kr + e)), dot);
            s = dot * isd;
            if (erf_on)
              s += lam * static_cast<double>(max_norm[head * ccap + c]) *
                   erf((pos - static_cast<double>(centre[c])) / (2.0 * sig));
          } else {
            const int64_t node = fb + sh.off[child_lev - 1] + cid;
            const float* mv = mu + node * D;
            for (int e = 0; e < D; ++e) dot = fma(s_q[wave][e], static_cast<double>(mv[e]), dot);
            s = dot * isd + qn * static_cast<double>(rad[node]) * isd;
            if (erf_on)
              s += lam * static_cast<double>(amax[node]) * erf((pos - static_cast<double>(pmin[node])) / (2.0 * sig));
          }
        }
        sc[i] = s;
      }
      bool taken[4];
      fs_top16(sc, ok, kBeam, taken);
      wave_lds_sync();
      // new frontier in candidate (ascending id) order
      int kept = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint64_t tm = __ballot(taken[i]);
        if (taken[i]) s_front[wave][kept + lanes_below(tm)] = id[i];
        kept += __popcll(tm);
      }
      wave_lds_sync();
      nf = kept;
      first = false;
      if (child_lev == 0) break;
      lev = child_lev;
    }
    // reached cells of this forest, skipping those the first forest reached
    const int base = nreach;
    bool add = false;
    int32_t cell = -1;
    if (lane < nf) {
      cell = mem[s_front[wave][lane]];
      add = true;
      for (int y = 0; y < base; ++y)
        if (s_reach[wave][y] == cell) add = false;
    }
    const uint64_t am = __ballot(add);
    if (add) s_reach[wave][base + lanes_below(am)] = cell;
    nreach = base + __popcll(am);
    wave_lds_sync();
  }

  // re-rank: logsumexp of each reached cell's token scores; the cells in
  // ascending order first (ties then go to the lower cell)
  int32_t my = lane < nreach ? s_reach[wave][lane] : 0x7fffffff;
  int rank = 0;
  for (int y = 0; y < nreach; ++y) rank += s_reach[wave][y] < my ? 1 : 0;
  wave_lds_sync();
  if (lane < nreach) s_reach[wave][rank] = my;
  wave_lds_sync();
  const int per = kWave / b;                   // cells per pass (b <= 64)
  const int grp = lane / b, tok = lane % b;
  for (int c0 = 0; c0 < nreach; c0 += per) {
    const int x = c0 + grp;
    double z = -INFINITY;
    if (x < nreach) {
      const int64_t c = s_reach[wave][x];
      const T* kr = kcache + (head * L + c * b + tok) * D;
      double dot = 0.0;
      for (int e = 0; e < D; ++e) dot = fma(s_q[wave][e], static_cast<double>(ld_f(kr + e)), dot);
      z = dot * isd;
    }
    double mx = z;
    for (int o = b / 2; o >= 1; o >>= 1) {
      const double ov = __shfl_xor(mx, o);
      mx = ov > mx ? ov : mx;
    }
    double sexp = x < nreach ? exp(z - mx) : 0.0;
    for (int o = b / 2; o >= 1; o >>= 1) sexp += __shfl_xor(sexp, o);
    if (x < nreach && tok == 0) s_lse[wave][x] = mx + log(sexp);
  }
  wave_lds_sync();
  double sc[4];
  bool ok[4], taken[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int x = i * kWave + lane;
    ok[i] = x < nreach;
    sc[i] = ok[i] ? s_lse[wave][x] : -INFINITY;
  }
  const int kk = fs_top16(sc, ok, K, taken);
  const int64_t o = (static_cast<int64_t>(bh) * nq + row) * K;
  int kept = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t tm = __ballot(taken[i]);
    if (taken[i]) idx[o + kept + lanes_below(tm)] = s_reach[wave][i * kWave + lane];
    kept += __popcll(tm);
  }
  for (int x = kept + lane; x < K; x += kWave) idx[o + x] = -1;
  if (lane == 0 && k_eff != nullptr) k_eff[static_cast<int64_t>(bh) * nq + row] = kk;
}

// ---------------------------------------------------------------- launch
size_t forest_workspace_bytes(int B, int Hkv, int d, int64_t n) {
  return align256(static_cast<size_t>(B) * Hkv * 2 * static_cast<size_t>(forest_nodes(n)) * d * sizeof(double));
}

template <typename T, int D>
static hipError_t launch_build_t(const ForestLaunch& p, hipStream_t st) {
  return launch(true, forest_build_kernel<T, D>, dim3(static_cast<unsigned>(p.B * p.Hkv), 2), dim3(256), st,
                static_cast<const T*>(p.kbar), p.max_norm, p.centre, p.ccap, p.n, forest_nodes(p.n), p.members,
                p.nmem, p.mu, p.rad, p.amax, p.pmin, static_cast<double*>(p.ws));
}

hipError_t launch_forest_build(const ForestLaunch& p, hipStream_t st) {
  if (p.dtype == kDtypeBf16) return p.d == 64 ? launch_build_t<bf16_t, 64>(p, st) : launch_build_t<bf16_t, 128>(p, st);
  return p.d == 64 ? launch_build_t<float, 64>(p, st) : launch_build_t<float, 128>(p, st);
}

template <typename T, int D>
static hipError_t launch_fsel_t(const SelectLaunch& s, const ForestLaunch& p, const void* k, int64_t L,
                                hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((s.nq + 3) / 4), static_cast<unsigned>(s.B * s.Hsel));
  return launch(true, forest_select_kernel<T, D>, grid, dim3(256), st, static_cast<const T*>(s.q),
                static_cast<const T*>(s.kbar), s.max_norm, s.centre, static_cast<const T*>(k), L, s.Hq, s.Hkv, s.Hsel,
                s.share_group, s.nq, s.q_pos0, s.ccap, s.b, s.erf_lambda, s.erf_sigma,
                static_cast<const int32_t*>(p.members), static_cast<const int32_t*>(p.nmem),
                static_cast<const float*>(p.mu), static_cast<const float*>(p.rad), static_cast<const float*>(p.amax),
                static_cast<const float*>(p.pmin), p.n, forest_nodes(p.n), s.K, s.idx, s.k_eff);
}

hipError_t launch_forest_select(const SelectLaunch& s, const ForestLaunch& p, const void* k, int64_t L,
                                hipStream_t st) {
  if (s.dtype == kDtypeBf16)
    return s.d == 64 ? launch_fsel_t<bf16_t, 64>(s, p, k, L, st) : launch_fsel_t<bf16_t, 128>(s, p, k, L, st);
  return s.d == 64 ? launch_fsel_t<float, 64>(s, p, k, L, st) : launch_fsel_t<float, 128>(s, p, k, L, st);
}

}  // namespace spa
