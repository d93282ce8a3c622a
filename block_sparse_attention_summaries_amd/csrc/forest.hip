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
//   build                 forest_members_kernel, one workgroup per (batch, kv
//                         head, forest): the median by a bitwise threshold
//                         search (workgroup counts), the members by an
//                         ordered compaction of ballot masks;
//                         forest_level1_kernel and forest_level_kernel (one
//                         launch per level above, a wave per node): fp64
//                         sums in the workspace, child by child;
//                         forest_radius_kernel: one thread per cell against
//                         every node above it (maxima reduced per node, then
//                         an integer atomic max of the fp64 squared distance).
//   forest_select_kernel  one 1024-thread workgroup per (batch, selection
//                         head, query row), a half per forest: the beam (up
//                         to 256 children scored in fp64, two lanes each;
//                         the 16 best kept by a threshold search over the
//                         scores' orderable bits, lower id first on ties),
//                         then the union
//                         of the reached cells re-ranked by the logsumexp of
//                         their token scores (32 lanes per cell).
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
// Members of both forests, one 1024-thread workgroup per (batch, kv head,
// forest).  The high-norm forest's threshold is the ceil(n/2)-th largest max
// norm, found by a bitwise search over the norms' orderable bits below the
// common prefix of the smallest and largest (ballot counts summed over the
// workgroup, stopping once exactly that many are at or above the candidate);
// its members are then written in cell order from per-wave ballot masks
// (chunks of 1024 cells, a prefix over chunks and waves).  Cells are held in
// registers 16384 at a time.
constexpr int kMemThreads = kWgThreads;
constexpr int kMemWaves = kWgWaves;

__global__ __launch_bounds__(kMemThreads) void forest_members_kernel(
    const float* __restrict__ max_norm, int64_t ccap, int64_t n, int64_t NN, int d, int32_t* __restrict__ members,
    int32_t* __restrict__ nmem, float* __restrict__ mu, float* __restrict__ rad, float* __restrict__ amax,
    float* __restrict__ pmin, unsigned long long* __restrict__ rbits) {
  constexpr int kRegs = 16;                    // cells per thread in registers
  constexpr int64_t kSpan = static_cast<int64_t>(kMemThreads) * kRegs;
  __shared__ int s_cnt[kRegs][kMemWaves];
  __shared__ int64_t s_wbase[kRegs][kMemWaves];
  __shared__ uint32_t s_lohi[2][kMemWaves];
  __shared__ int s_part[2][kMemWaves];
  __shared__ int64_t s_tot;
  __shared__ ForestShape s_sh;                 // in LDS: its arrays are indexed by loop variables
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t head = blockIdx.x;
  const int f = blockIdx.y;
  const float* a = max_norm + head * ccap;
  int32_t* mem = members + (head * 2 + f) * n;
  const int64_t fb = (head * 2 + f) * NN;

  int64_t m = n;
  if (f == 0) {
    for (int64_t c = tid; c < n; c += kMemThreads) mem[c] = static_cast<int32_t>(c);
  } else {
    uint32_t key[kRegs];                       // 0 marks a slot past the prefix (below every norm's key)
    // keys of cells [s0, s0 + kSpan): cell s0 + j * 1024 + tid in key[j]
    auto load_span = [&](int64_t s0) {
      if (s0 + kSpan <= n) {                   // unclamped, so the loads issue together
        float raw[kRegs];
#pragma unroll
        for (int j = 0; j < kRegs; ++j) raw[j] = a[s0 + j * kMemThreads + tid];
#pragma unroll
        for (int j = 0; j < kRegs; ++j) key[j] = orderable_f32(raw[j]);
      } else {
#pragma unroll
        for (int j = 0; j < kRegs; ++j) {
          const int64_t c = s0 + j * kMemThreads + tid;
          const uint32_t kv = orderable_f32(a[c < n ? c : n - 1]);
          key[j] = c < n ? kv : 0u;
        }
      }
    };
    load_span(0);
    // 1. threshold: the largest t with at least ceil(n/2) norms at or above it
    const uint32_t t = wg_kth_largest_f32<kRegs>(key, a, n, static_cast<int>((n + 1) / 2), &s_part[0][0],
                                                 &s_lohi[0][0]);
    // 2. members in cell order
    int64_t base = 0;
    for (int64_t s0 = 0; s0 < n; s0 += kSpan) {
      if (s0 > 0) load_span(s0);
#pragma unroll
      for (int j = 0; j < kRegs; ++j) {
        const int cj = __popcll(__ballot(key[j] >= t));
        if (lane == 0) s_cnt[j][wave] = cj;
      }
      __syncthreads();
      if (wave == 0) {                         // entries (chunk j, wave w) in cell order, four per lane
        int v[4];
        int run = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = lane * 4 + r;
          v[r] = s_cnt[e / kMemWaves][e % kMemWaves];
          run += v[r];
        }
        int incl = run;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int up = __shfl_up(incl, o, kWave);
          if (lane >= o) incl += up;
        }
        int64_t pre = base + incl - run;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = lane * 4 + r;
          s_wbase[e / kMemWaves][e % kMemWaves] = pre;
          pre += v[r];
        }
        if (lane == kWave - 1) s_tot = incl;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kRegs; ++j) {
        const uint64_t mk = __ballot(key[j] >= t);
        const int64_t wb = s_wbase[j][wave];
        if (key[j] >= t) mem[wb + lanes_below(mk)] = static_cast<int32_t>(s0 + j * kMemThreads + tid);
      }
      base += s_tot;
      __syncthreads();                         // counts and bases are rewritten next span
    }
    m = base;
  }
  for (int64_t x = m + tid; x < n; x += kMemThreads) mem[x] = -1;
  if (tid == 0) {
    nmem[head * 2 + f] = static_cast<int32_t>(m);
    forest_shape_into(m, &s_sh);
  }
  __syncthreads();

  // node fields come from forest_level1_kernel and forest_level_kernel, radii
  // from forest_radius_kernel: clear their fp64 maxima here
  const ForestShape& sh = s_sh;
  for (int64_t x = tid; x < NN; x += kMemThreads) rbits[fb + x] = 0ull;
  // slots past this forest's nodes (the high-norm forest is smaller)
  const int64_t used = sh.nl ? sh.off[sh.nl - 1] + sh.n[sh.nl - 1] : 0;
  for (int64_t x = used * d + tid; x < NN * d; x += kMemThreads) mu[fb * d + x] = 0.f;
  for (int64_t x = used + tid; x < NN; x += kMemThreads) {
    rad[fb + x] = 0.f;
    amax[fb + x] = 0.f;
    pmin[fb + x] = 0.f;
  }
}

// Level 1: one wave per node, lanes over the columns: the 16 members' mean
// keys summed in member order (fp64), the mean, and the max norm / min centre.
template <typename T, int D>
__global__ __launch_bounds__(256) void forest_level1_kernel(const T* __restrict__ kbar,
                                                            const float* __restrict__ max_norm,
                                                            const float* __restrict__ centre, int64_t ccap, int64_t n,
                                                            int64_t NN, const int32_t* __restrict__ members,
                                                            const int32_t* __restrict__ nmem, float* __restrict__ mu,
                                                            float* __restrict__ amax, float* __restrict__ pmin,
                                                            double* __restrict__ sums) {
  constexpr int kCols = D / kWave;             // columns per lane
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int64_t head = blockIdx.y;
  const int f = blockIdx.z;
  const int64_t m = nmem[head * 2 + f];
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 4 + wave;   // level-1 node
  if (m <= kFan || j * kFan >= m) return;      // whole wave leaves
  const int64_t fb = (head * 2 + f) * NN;
  const int32_t* mem = members + (head * 2 + f) * n;
  const int cnt = static_cast<int>(m - j * kFan < kFan ? m - j * kFan : kFan);
  int32_t cell[kFan];
#pragma unroll
  for (int t = 0; t < kFan; ++t) cell[t] = mem[j * kFan + (t < cnt ? t : cnt - 1)];
  double sacc[kCols];
#pragma unroll
  for (int u = 0; u < kCols; ++u) sacc[u] = 0.0;
  float vals[kFan][kCols];
#pragma unroll
  for (int t = 0; t < kFan; ++t)
#pragma unroll
    for (int u = 0; u < kCols; ++u) vals[t][u] = ld_f(kbar + (head * ccap + cell[t]) * D + u * kWave + lane);
#pragma unroll
  for (int t = 0; t < kFan; ++t)
#pragma unroll
    for (int u = 0; u < kCols; ++u)
      if (t < cnt) sacc[u] += static_cast<double>(vals[t][u]);
#pragma unroll
  for (int u = 0; u < kCols; ++u) {
    const int e = u * kWave + lane;
    sums[(fb + j) * D + e] = sacc[u];
    mu[(fb + j) * D + e] = static_cast<float>(sacc[u] / static_cast<double>(cnt));
  }
  // max norm and min centre of the members (lanes 0..15 one member each)
  float am = 0.f, pm = INFINITY;
  if (lane < cnt) {
    const int32_t c = mem[j * kFan + lane];
    am = max_norm[head * ccap + c];
    pm = centre[c];
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) {
    const float oa = __shfl_xor(am, o), op = __shfl_xor(pm, o);
    am = oa > am ? oa : am;
    pm = op < pm ? op : pm;
  }
  if (lane == 0) {
    amax[fb + j] = am;
    pmin[fb + j] = pm;
  }
}

// Level l + 1 (l >= 1), one launch per level: a wave per node, lanes over
// the columns, the 16 children's fp64 sums loaded together and added in order.
template <int D>
__global__ __launch_bounds__(256) void forest_level_kernel(int l, int64_t NN, const int32_t* __restrict__ nmem,
                                                           float* __restrict__ mu, float* __restrict__ amax,
                                                           float* __restrict__ pmin, double* __restrict__ sums) {
  constexpr int kCols = D / kWave;
  __shared__ ForestShape s_sh;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t head = blockIdx.y;
  const int f = blockIdx.z;
  const int64_t m = nmem[head * 2 + f];
  if (tid == 0) forest_shape_into(m, &s_sh);
  __syncthreads();
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (l >= s_sh.nl || j >= s_sh.n[l]) return;  // whole wave leaves
  const int64_t fb = (head * 2 + f) * NN;
  const int64_t off = s_sh.off[l], poff = s_sh.off[l - 1], nprev = s_sh.n[l - 1];
  int64_t span = kFan;
  for (int x = 0; x < l; ++x) span *= kFan;     // cells under a node of this level
  const int cnt = static_cast<int>(nprev - j * kFan < kFan ? nprev - j * kFan : kFan);
  double v[kFan][kCols];
#pragma unroll
  for (int t = 0; t < kFan; ++t) {
    const int64_t y = j * kFan + (t < cnt ? t : cnt - 1);
#pragma unroll
    for (int u = 0; u < kCols; ++u) v[t][u] = sums[(fb + poff + y) * D + u * kWave + lane];
  }
  double sacc[kCols];
#pragma unroll
  for (int u = 0; u < kCols; ++u) sacc[u] = 0.0;
#pragma unroll
  for (int t = 0; t < kFan; ++t)
#pragma unroll
    for (int u = 0; u < kCols; ++u)
      if (t < cnt) sacc[u] += v[t][u];
  const int64_t cells = (j + 1) * span <= m ? span : m - j * span;
#pragma unroll
  for (int u = 0; u < kCols; ++u) {
    const int e = u * kWave + lane;
    sums[(fb + off + j) * D + e] = sacc[u];
    mu[(fb + off + j) * D + e] = static_cast<float>(sacc[u] / static_cast<double>(cells));
  }
  float am = 0.f, pm = INFINITY;
  if (lane < cnt) {
    am = amax[fb + poff + j * kFan + lane];
    pm = pmin[fb + poff + j * kFan + lane];
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) {
    const float oa = __shfl_xor(am, o), op = __shfl_xor(pm, o);
    am = oa > am ? oa : am;
    pm = op < pm ? op : pm;
  }
  if (lane == 0) {
    amax[fb + off + j] = am;
    pmin[fb + off + j] = pm;
  }
}

// Radii: one thread per member cell computes its fp64 squared distance to the
// mean of every node above it and folds it into that node's maximum (the bit
// patterns of non-negative doubles order as unsigned integers, so an integer
// atomic max is exact and order-independent).
template <typename T, int D>
__global__ __launch_bounds__(256) void forest_radius_kernel(const T* __restrict__ kbar, int64_t ccap, int64_t n,
                                                            int64_t NN, const int32_t* __restrict__ members,
                                                            const int32_t* __restrict__ nmem,
                                                            const float* __restrict__ mu,
                                                            unsigned long long* __restrict__ rbits) {
  constexpr int kVec = Elem<T>::kVec;
  __shared__ ForestShape s_sh;
  __shared__ double s_red[4];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t head = blockIdx.y;
  const int f = blockIdx.z;
  const int64_t m = nmem[head * 2 + f];
  if (tid == 0) forest_shape_into(m, &s_sh);
  __syncthreads();
  const int64_t x0 = static_cast<int64_t>(blockIdx.x) * 256;
  if (x0 >= m || s_sh.nl == 0) return;         // whole workgroup leaves
  const int64_t x = x0 + tid;
  const bool in = x < m;                       // threads past the members take part with 0
  const int64_t fb = (head * 2 + f) * NN;
  float kv[D];
  {
    const int64_t c = members[(head * 2 + f) * n + (in ? x : m - 1)];
    const T* kr = kbar + (head * ccap + c) * D;
#pragma unroll
    for (int v = 0; v < D / kVec; ++v) {
      float t[kVec];
      Elem<T>::unpack(*reinterpret_cast<const uint4*>(kr + v * kVec), t);
#pragma unroll
      for (int u = 0; u < kVec; ++u) kv[v * kVec + u] = t[u];
    }
  }
  int64_t span = kFan;
  for (int l = 0; l < s_sh.nl; ++l, span *= kFan) {
    const int64_t node = fb + s_sh.off[l] + (in ? x : m - 1) / span;
    const float4* mv = reinterpret_cast<const float4*>(mu + node * D);
    double ss = 0.0;
#pragma unroll
    for (int v = 0; v < D / 4; ++v) {
      const float4 w = mv[v];
      double df = static_cast<double>(kv[4 * v]) - static_cast<double>(w.x);
      ss += df * df;
      df = static_cast<double>(kv[4 * v + 1]) - static_cast<double>(w.y);
      ss += df * df;
      df = static_cast<double>(kv[4 * v + 2]) - static_cast<double>(w.z);
      ss += df * df;
      df = static_cast<double>(kv[4 * v + 3]) - static_cast<double>(w.w);
      ss += df * df;
    }
    if (!in) ss = 0.0;
    if (span == kFan) {
      // a level-1 node is 16 consecutive lanes
#pragma unroll
      for (int o = kFan / 2; o >= 1; o >>= 1) {
        const double os = __shfl_xor(ss, o);
        ss = os > ss ? os : ss;
      }
      if (in && (x % kFan) == 0) atomicMax(&rbits[node], static_cast<unsigned long long>(__double_as_longlong(ss)));
    } else {
      // nodes above span whole workgroups (256 members each)
#pragma unroll
      for (int o = kWave / 2; o >= 1; o >>= 1) {
        const double os = __shfl_xor(ss, o);
        ss = os > ss ? os : ss;
      }
      if (lane == 0) s_red[wave] = ss;
      __syncthreads();
      if (tid == 0) {
        double bm = s_red[0];
        for (int w = 1; w < 4; ++w) bm = s_red[w] > bm ? s_red[w] : bm;
        atomicMax(&rbits[fb + s_sh.off[l] + x0 / span], static_cast<unsigned long long>(__double_as_longlong(bm)));
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(256) void forest_radius_final_kernel(const unsigned long long* __restrict__ rbits,
                                                                  int64_t total, float* __restrict__ rad) {
  const int64_t x = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (x < total) rad[x] = static_cast<float>(sqrt(__longlong_as_double(static_cast<long long>(rbits[x]))));
}

// ---------------------------------------------------------------- select
// One 1024-thread workgroup per (batch, selection head, query row); each
// half runs one forest's beam search.  A level's up to 256 candidates take
// two lanes each (half of the columns apiece, the halves added in a fixed
// order), so every load of the level is in flight at once; the forest's
// first wave keeps the best 16 (a threshold search over the scores'
// orderable bits, lower id first on ties).  The reached cells are re-ranked
// with 32 lanes per cell (tokens g, g + 32, ...), and the final top K is
// found by counting, for each cell, the cells that beat it.
constexpr int kSelThreads = 1024;

template <typename T, int D>
__global__ __launch_bounds__(kSelThreads) void forest_select_kernel(
    const T* __restrict__ q, const T* __restrict__ kbar, const float* __restrict__ max_norm,
    const float* __restrict__ centre, const T* __restrict__ kcache, int64_t L, int Hq, int Hkv, int Hsel,
    int share_group, int nq, int64_t q_pos0, int64_t ccap, int b, const float* __restrict__ erf_lambda,
    const float* __restrict__ erf_sigma, const int32_t* __restrict__ members, const int32_t* __restrict__ nmem,
    const float* __restrict__ mu, const float* __restrict__ rad, const float* __restrict__ amax,
    const float* __restrict__ pmin, int64_t n, int64_t NN, int K, int32_t* __restrict__ idx,
    int32_t* __restrict__ k_eff) {
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kHalf = D / 2;                 // columns per lane of a candidate
  __shared__ double s_q[D];
  __shared__ double s_qn;
  __shared__ int64_t s_front[2][kBeam];
  __shared__ int s_nf[2];
  __shared__ double s_sc[2][256];
  __shared__ int64_t s_cid[2][256];
  __shared__ int32_t s_reach[2 * kBeam];
  __shared__ int s_nreach;
  __shared__ double s_lse[2 * kBeam];
  __shared__ ForestShape s_sh[2];              // in LDS: its arrays are indexed by loop variables
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int bh = blockIdx.y;
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int G = Hq / Hkv;
  const int kvh = share_group ? hs : hs / G;
  const int row = blockIdx.x;
  const int64_t head = static_cast<int64_t>(bi) * Hkv + kvh;
  const double pos = static_cast<double>(q_pos0 + row);
  const double isd = 1.0 / sqrt(static_cast<double>(D));
  const bool erf_on = erf_lambda != nullptr;
  const double lam = erf_on ? static_cast<double>(erf_lambda[hs]) : 0.0;
  const double sig = erf_on ? static_cast<double>(erf_sigma[hs]) : 1.0;

  // q_hat (fp64) and its norm
  if (wave == 0) {
    const int gq = share_group ? G : 1;
    const int h0 = share_group ? hs * G : hs;
    double qq = 0.0;
    for (int e = lane; e < D; e += kWave) {
      double sq = 0.0;
      for (int g = 0; g < gq; ++g)
        sq += static_cast<double>(ld_f(q + ((static_cast<int64_t>(bi) * Hq + h0 + g) * nq + row) * D + e));
      sq /= static_cast<double>(gq);
      s_q[e] = sq;
      qq += sq * sq;
    }
    for (int o = 32; o >= 1; o >>= 1) qq += __shfl_xor(qq, o);
    if (lane == 0) s_qn = sqrt(qq);
  }

  // threads [512 f, 512 f + 512) run forest f: candidate x = ht / 2, column
  // half hf = ht % 2
  const int f = tid / 512, ht = tid % 512, x = ht >> 1, hf = ht & 1, fw = ht / kWave;
  const int64_t m = nmem[head * 2 + f];
  const int32_t* mem = members + (head * 2 + f) * n;
  const int64_t fb = (head * 2 + f) * NN;
  if (ht == 0) {
    forest_shape_into(m, &s_sh[f]);
    s_nf[f] = static_cast<int>(s_sh[f].nl ? s_sh[f].n[s_sh[f].nl - 1] : m);
  }
  __syncthreads();
  const double qn = s_qn;
  const ForestShape& sh = s_sh[f];
  if (ht < s_nf[f]) s_front[f][ht] = ht;
  // rounds: one per level below the top, one for a forest of cells only; the
  // whole-prefix forest has the most
  const int rounds = s_sh[0].nl ? s_sh[0].nl : 1;
  const int my_rounds = sh.nl ? sh.nl : 1;
  for (int r = 0; r < rounds; ++r) {
    __syncthreads();                           // frontier written
    const bool active = r < my_rounds;
    const int nf = s_nf[f];
    const bool own = sh.nl == 0;               // a forest of cells only: score the frontier itself
    const int child_lev = (own || !active) ? 0 : sh.nl - 1 - r;
    const int64_t nchild = child_lev == 0 ? m : sh.n[child_lev - 1];
    int64_t cid = -1;                          // candidate x (ascending id with x)
    if (!active) {
    } else if (own) {
      cid = x < nf ? s_front[f][x] : -1;
    } else if (x / kFan < nf) {
      const int64_t ch = s_front[f][x / kFan] * kFan + (x % kFan);
      cid = ch < nchild ? ch : -1;
    }
    // this lane's half of the candidate's dot product, loads issued first
    // from clamped (valid) addresses
    double part = 0.0, extra = 0.0, ew = 0.0, ex = 0.0;   // extra: the radius and erf terms
    if (child_lev == 0) {
      const int64_t c = mem[cid >= 0 ? cid : 0];
      uint4 raw[kHalf / kVec];
      const uint4* kr = reinterpret_cast<const uint4*>(kbar + (head * ccap + c) * D + hf * kHalf);
#pragma unroll
      for (int v = 0; v < kHalf / kVec; ++v) raw[v] = kr[v];
      const float an = max_norm[head * ccap + c], pc = centre[c];
      double pc4[4] = {0.0, 0.0, 0.0, 0.0};    // four independent chains
#pragma unroll
      for (int v = 0; v < kHalf / kVec; ++v) {
        float t[kVec];
        Elem<T>::unpack(raw[v], t);
#pragma unroll
        for (int u = 0; u < kVec; ++u)
          pc4[u & 3] = fma(s_q[hf * kHalf + v * kVec + u], static_cast<double>(t[u]), pc4[u & 3]);
      }
      part = (pc4[0] + pc4[1]) + (pc4[2] + pc4[3]);
      ew = lam * static_cast<double>(an);
      ex = (pos - static_cast<double>(pc)) / (2.0 * sig);
    } else {
      const int64_t node = fb + sh.off[child_lev - 1] + (cid >= 0 ? cid : 0);
      float4 w[kHalf / 4];
      const float4* mv = reinterpret_cast<const float4*>(mu + node * D + hf * kHalf);
#pragma unroll
      for (int v = 0; v < kHalf / 4; ++v) w[v] = mv[v];
      const float rn = rad[node], an = amax[node], pn = pmin[node];
      double pn4[4] = {0.0, 0.0, 0.0, 0.0};    // four independent chains
#pragma unroll
      for (int v = 0; v < kHalf / 4; ++v) {
        const int e = hf * kHalf + 4 * v;
        pn4[0] = fma(s_q[e], static_cast<double>(w[v].x), pn4[0]);
        pn4[1] = fma(s_q[e + 1], static_cast<double>(w[v].y), pn4[1]);
        pn4[2] = fma(s_q[e + 2], static_cast<double>(w[v].z), pn4[2]);
        pn4[3] = fma(s_q[e + 3], static_cast<double>(w[v].w), pn4[3]);
      }
      part = (pn4[0] + pn4[1]) + (pn4[2] + pn4[3]);
      extra = qn * static_cast<double>(rn) * isd;
      ew = lam * static_cast<double>(an);
      ex = (pos - static_cast<double>(pn)) / (2.0 * sig);
    }
    if (erf_on && hf == 0) extra += ew * erf_exact(ex);
    const double other = __shfl_xor(part, 1);
    const double odd_extra = __shfl_xor(extra, 1);
    const double dot = hf == 0 ? part + other : other + part;
    const double sv = dot * isd + (hf == 0 ? extra : odd_extra);
    if (hf == 0) {
      s_sc[f][x] = sv;
      s_cid[f][x] = cid;
    }
    __syncthreads();                           // scores written, frontier read
    if (active && fw == 0) {
      // the forest's first wave keeps the best 16 (score, then lower id)
      double sc[4];
      bool ok[4], taken[4];
      int64_t id[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        id[i] = s_cid[f][i * kWave + lane];
        ok[i] = id[i] >= 0;
        sc[i] = s_sc[f][i * kWave + lane];
      }
      wave_top_f64x4(sc, ok, kBeam, taken);
      // new frontier in candidate (ascending id) order
      int kept = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint64_t tm = __ballot(taken[i]);
        if (taken[i]) s_front[f][kept + lanes_below(tm)] = id[i];
        kept += __popcll(tm);
      }
      if (lane == 0) s_nf[f] = kept;
    }
  }
  __syncthreads();                             // last frontiers written
  if (wave == 0) {
    // reached cells: the whole-prefix forest's, then the other's not yet there
    const int nf0 = s_nf[0], nf1 = s_nf[1];
    if (lane < nf0) s_reach[lane] = members[(head * 2) * n + s_front[0][lane]];
    wave_lds_sync();
    const int32_t cell1 = members[(head * 2 + 1) * n + s_front[1][lane < nf1 ? lane : 0]];
    bool add = lane < nf1;
    for (int y = 0; y < nf0; ++y) add = add && s_reach[y] != cell1;
    const uint64_t am = __ballot(add);
    if (add) s_reach[nf0 + lanes_below(am)] = cell1;
    const int nreach = nf0 + __popcll(am);
    wave_lds_sync();
    // ascending cell order (ties in the re-rank then go to the lower cell)
    const int32_t my = lane < nreach ? s_reach[lane] : 0x7fffffff;
    int rank = 0;
    for (int y = 0; y < nreach; ++y) rank += s_reach[y] < my ? 1 : 0;
    wave_lds_sync();
    if (lane < nreach) s_reach[rank] = my;
    if (lane == 0) s_nreach = nreach;
  }
  __syncthreads();

  // re-rank: logsumexp of each reached cell's token scores, 32 lanes per cell
  // (tokens g, g + 32, ...), the max and the sum over the cell's lanes
  const int nreach = s_nreach;
  {
    const int cs = tid / 32, g = tid % 32;
    const int64_t c = s_reach[cs < nreach ? cs : nreach - 1];
    const T* kc = kcache + (head * L + c * b) * D;
    constexpr int kMaxTok = 128 / 32;
    double z[kMaxTok];
#pragma unroll
    for (int k = 0; k < kMaxTok; ++k) {
      z[k] = -INFINITY;
      // q_hat is read from LDS per token: held in registers it would take D
      // doubles per lane
      asm volatile("" ::: "memory");
      if (32 * k < b) {
        const int tok = g + 32 * k;
        const uint4* kr = reinterpret_cast<const uint4*>(kc + static_cast<int64_t>(tok < b ? tok : b - 1) * D);
        uint4 raw[D / kVec];
#pragma unroll
        for (int v = 0; v < D / kVec; ++v) raw[v] = kr[v];
        double d4[4] = {0.0, 0.0, 0.0, 0.0};  // four independent chains
#pragma unroll
        for (int v = 0; v < D / kVec; ++v) {
          float t[kVec];
          Elem<T>::unpack(raw[v], t);
#pragma unroll
          for (int u = 0; u < kVec; ++u) d4[u & 3] = fma(s_q[v * kVec + u], static_cast<double>(t[u]), d4[u & 3]);
        }
        if (tok < b) z[k] = ((d4[0] + d4[1]) + (d4[2] + d4[3])) * isd;
      }
    }
    double mx = z[0];
#pragma unroll
    for (int k = 1; k < kMaxTok; ++k) mx = z[k] > mx ? z[k] : mx;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
      const double ov = __shfl_xor(mx, o);
      mx = ov > mx ? ov : mx;
    }
    double sexp = 0.0;
#pragma unroll
    for (int k = 0; k < kMaxTok; ++k)
      if (z[k] != -INFINITY) sexp += exp(z[k] - mx);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) sexp += __shfl_xor(sexp, o);
    if (cs < nreach && g == 0) s_lse[cs] = mx + log(sexp);
  }
  __syncthreads();
  if (wave != 0) return;
  // top K of the reached cells (higher logsumexp, then lower cell), written
  // in ascending cell order
  const bool okc = lane < nreach;
  const double mine = okc ? s_lse[lane] : -INFINITY;
  int beat = 0;
  for (int y = 0; y < nreach; ++y) {
    const double o = s_lse[y];
    beat += (o > mine || (o == mine && y < lane)) ? 1 : 0;
  }
  const int kk = nreach < K ? nreach : K;
  const bool take = okc && beat < K;
  const int64_t o = (static_cast<int64_t>(bh) * nq + row) * K;
  const uint64_t tm = __ballot(take);
  if (take) idx[o + lanes_below(tm)] = s_reach[lane];
  for (int xx = kk + lane; xx < K; xx += kWave) idx[o + xx] = -1;
  if (lane == 0 && k_eff != nullptr) k_eff[static_cast<int64_t>(bh) * nq + row] = kk;
}

// ---------------------------------------------------------------- launch
// fp64 node sums, then the radii's fp64 squared maxima (as bits)
size_t forest_workspace_bytes(int B, int Hkv, int d, int64_t n) {
  const size_t nodes = static_cast<size_t>(B) * Hkv * 2 * static_cast<size_t>(forest_nodes(n));
  return align256(nodes * d * sizeof(double)) + align256(nodes * sizeof(unsigned long long));
}

template <typename T, int D>
static hipError_t launch_build_t(const ForestLaunch& p, hipStream_t st) {
  const int64_t NN = forest_nodes(p.n);
  const size_t nodes = static_cast<size_t>(p.B) * p.Hkv * 2 * static_cast<size_t>(NN);
  double* sums = static_cast<double*>(p.ws);
  unsigned long long* rbits =
      reinterpret_cast<unsigned long long*>(static_cast<char*>(p.ws) + align256(nodes * p.d * sizeof(double)));
  const unsigned heads = static_cast<unsigned>(p.B * p.Hkv);
  hipError_t e = launch(false, forest_members_kernel, dim3(heads, 2), dim3(kMemThreads), st, p.max_norm, p.ccap, p.n, NN,
                        p.d, p.members, p.nmem, p.mu, p.rad, p.amax, p.pmin, rbits);
  if (e != hipSuccess || NN == 0) return e;
  const ForestShape sh = forest_shape(p.n);    // the whole-prefix forest has the most levels
  e = launch(false, forest_level1_kernel<T, D>, dim3(static_cast<unsigned>((sh.n[0] + 3) / 4), heads, 2), dim3(256),
             st, static_cast<const T*>(p.kbar), p.max_norm, p.centre, p.ccap, p.n, NN,
             static_cast<const int32_t*>(p.members), static_cast<const int32_t*>(p.nmem), p.mu, p.amax, p.pmin, sums);
  if (e != hipSuccess) return e;
  for (int l = 1; l < sh.nl; ++l) {
    e = launch(false, forest_level_kernel<D>, dim3(static_cast<unsigned>((sh.n[l] + 3) / 4), heads, 2), dim3(256),
               st, l, NN, static_cast<const int32_t*>(p.nmem), p.mu, p.amax, p.pmin, sums);
    if (e != hipSuccess) return e;
  }
  e = launch(false, forest_radius_kernel<T, D>,
             dim3(static_cast<unsigned>((p.n + 255) / 256), static_cast<unsigned>(p.B * p.Hkv), 2), dim3(256), st,
             static_cast<const T*>(p.kbar), p.ccap, p.n, NN, static_cast<const int32_t*>(p.members),
             static_cast<const int32_t*>(p.nmem), static_cast<const float*>(p.mu), rbits);
  if (e != hipSuccess) return e;
  const int64_t total = static_cast<int64_t>(nodes);
  return launch(true, forest_radius_final_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), st,
                static_cast<const unsigned long long*>(rbits), total, p.rad);
}

hipError_t launch_forest_build(const ForestLaunch& p, hipStream_t st) {
  if (p.dtype == kDtypeBf16) return p.d == 64 ? launch_build_t<bf16_t, 64>(p, st) : launch_build_t<bf16_t, 128>(p, st);
  return p.d == 64 ? launch_build_t<float, 64>(p, st) : launch_build_t<float, 128>(p, st);
}

template <typename T, int D>
static hipError_t launch_fsel_t(const SelectLaunch& s, const ForestLaunch& p, const void* k, int64_t L,
                                hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(s.nq), static_cast<unsigned>(s.B * s.Hsel));
  return launch(true, forest_select_kernel<T, D>, grid, dim3(kSelThreads), st, static_cast<const T*>(s.q),
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
