// select_bwd.hip -- selector-side backward (bf16, gfx950 MFMA): the gate
// gradient dg carried back through log g = s - LSE(s) into the query, the
// block summaries, the learned projection and the keys ("SAS" review, "How it
// works", step 5: the loss reaches the selector through g; §4.2.2 softmax
// gate; §4.3 Eq. 9; §3 mean-key summaries).  With p = softmax(s) over a
// row's candidates (so g_m = p_m) and its selection S fixed:
//   ds_c = p_c ([c in S] dg_c - sum_{m in S} p_m dg_m),
//   dq_hat = sum_c ds_c ktilde_c / sqrt(d)   (each head of a shared selection
//            receives dq_hat / G),
//   dktilde_c = sum_rows ds_c q_hat / sqrt(d),
// with ktilde = kbar, or W kbar under the projection.  The projection is
// moved to the query side, where it is exact on the bf16 summaries: with
// u = W^T q_hat the scores are u . kbar / sqrt(d), dkbar_c = W^T dktilde_c =
// sum_rows ds_c u / sqrt(d), and with r = sum_c ds_c kbar_c / sqrt(d) per row,
// dq_hat = W r and dW = sum_rows q_hat r^T.  Optionally dk_j += dkbar_c / b
// for every token of block c (the summary is the block mean).
// Scores are recomputed from q_hat (or u) rounded to bf16 (a gradient needs
// ~1e-3, not the ranking accuracy of the forward selection).
//
// Launches:
//   rows        4 waves x 32 rows of one selection head; pass 1 over the
//               candidate tiles gives each row's LSE and sum_S p dg (saved to
//               the workspace), pass 2 accumulates dq_hat^T (or r^T) +=
//               Kbar^T dS^T;
//   candidates  one 32-candidate tile per workgroup; the four waves take the
//               later rows 32 at a time, S = Q_hat Kbar^T puts one candidate
//               per lane, dKbar += dS^T Q_hat, and the waves' sums are added in
//               wave order;
//   projection  U = Q_hat W before, dQ = R W^T and dW = Q_hat^T R (partial
//               sums per row chunk, added in chunk order) after;
//   mean        dk += dkbar / b over the tokens of each summarised block.
#include "spa_device.h"
#include "spa_launch.h"

namespace spa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 sbbf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float sbfloatx16_t;

constexpr int kST = 32;               // candidates / rows per tile
constexpr float kSLog2e = 1.4426950408889634f;

__device__ __forceinline__ sbbf16x8_t sb_bf16x8(uint4 v) { return __builtin_bit_cast(sbbf16x8_t, v); }
// tile element held by register r of half-wave h when A rows are fed permuted
__device__ __forceinline__ int sb_elem(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }
__device__ __forceinline__ int sb_perm(int m) {
  const int a = m >> 3, h = (m >> 2) & 1, c = m & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + c;
}
__device__ __forceinline__ uint4 sb_pack8(const float* x) {
  sbbf16x8_t v;
#pragma unroll
  for (int t = 0; t < 8; ++t) v[t] = static_cast<__bf16>(x[t]);
  return __builtin_bit_cast(uint4, v);
}
// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): two MFMA operands that
// carry x to about 16 significant bits
__device__ __forceinline__ void sb_split8(const float* x, uint4& hi, uint4& lo) {
  sbbf16x8_t h, l;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    h[t] = static_cast<__bf16>(x[t]);
    l[t] = static_cast<__bf16>(x[t] - static_cast<float>(h[t]));
  }
  hi = __builtin_bit_cast(uint4, h);
  lo = __builtin_bit_cast(uint4, l);
}
__device__ __forceinline__ void sb_store_t8(uint16_t* dst, int pitch, uint4 w) {
  dst[0 * pitch] = static_cast<uint16_t>(w.x);
  dst[1 * pitch] = static_cast<uint16_t>(w.x >> 16);
  dst[2 * pitch] = static_cast<uint16_t>(w.y);
  dst[3 * pitch] = static_cast<uint16_t>(w.y >> 16);
  dst[4 * pitch] = static_cast<uint16_t>(w.z);
  dst[5 * pitch] = static_cast<uint16_t>(w.z >> 16);
  dst[6 * pitch] = static_cast<uint16_t>(w.w);
  dst[7 * pitch] = static_cast<uint16_t>(w.w >> 16);
}

// dg of one row's selected candidates in [c0, c0 + 32) into its dg table row
// (already zeroed); the two half-waves take alternate slots, 8 slots per
// lane at a time with every load issued before the first is used.
__device__ __forceinline__ void sb_fill_dg(float* __restrict__ trow, const int32_t* __restrict__ sel,
                                           const float* __restrict__ dgr, int K, int hl, int c0, int ncand) {
  for (int t0 = hl; t0 < K; t0 += 16) {
    int cc[8];
    float dd[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + 2 * u;
      const int tc = t < K ? t : K - 1;
      cc[u] = sel[tc];
      dd[u] = dgr[tc];
      if (t >= K) cc[u] = -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (cc[u] >= c0 && cc[u] < c0 + 32 && cc[u] < ncand) trow[cc[u] - c0] = dd[u];
  }
}

// q_hat of one row as 8 bf16 (columns 8 j .. 8 j + 7): the mean of nh heads
// (summed in head order in fp32), rounded to nearest even.
__device__ __forceinline__ uint4 qhat8(const __bf16* __restrict__ q0, int64_t head_stride, int nh, int j) {
  float a[8];
  Elem<bf16_t>::unpack(*reinterpret_cast<const uint4*>(q0 + 8 * j), a);
  for (int g = 1; g < nh; ++g) {
    float f[8];
    Elem<bf16_t>::unpack(*reinterpret_cast<const uint4*>(q0 + g * head_stride + 8 * j), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] += f[e];
  }
  if (nh > 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = a[e] / static_cast<float>(nh);
  }
  return sb_pack8(a);
}

}  // namespace

// ---------------------------------------------------------------- rows
template <int D>
struct SbRowSmem {
  static constexpr int kKPitch = D + 8;
  static constexpr int kTPitch = kST + 8;
  __bf16 k[kST * kKPitch];                 // Kbar tile, row-major
  __bf16 kt[D * kTPitch];                  // Kbar tile, transposed
  float dgt[4][32][kST + 4];               // per wave: dg of (row, candidate), 0 if not selected
};

template <int D>
__global__ __launch_bounds__(256, 2) void select_bwd_rows_kernel(
    const __bf16* __restrict__ q, int qHeads, int nh_in, const __bf16* __restrict__ kbar, int Hkv, int Hsel,
    int G, int share_group, int nq, int64_t q_pos0, int64_t ccap, int b, int K, const int32_t* __restrict__ idx,
    const float* __restrict__ dg, float* __restrict__ out, int outHeads, int nh_out, float2* __restrict__ ws_row) {
  __shared__ SbRowSmem<D> sm;
  constexpr int kKS = D / 16;
  constexpr int kDB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  // dispatch order w runs the heads fastest and the row tiles from the last
  // (the longest: a row's candidates grow with it) to the first
  const uint32_t wid = blockIdx.y * gridDim.x + blockIdx.x;
  const int bh = static_cast<int>(wid % gridDim.y);
  const int rtile = static_cast<int>(gridDim.x - 1 - wid / gridDim.y);
  const int bi = bh / Hsel, hs = bh % Hsel;
  const int kvh = share_group ? hs : hs / G;
  // query source rows: q_hat = mean of heads hs * nh_in .. + nh_in - 1 of q
  const int h0 = hs * nh_in;
  const int row = (rtile * 4 + wave) * 32 + ql;
  const bool row_ok = row < nq;
  const int rowc = row_ok ? row : nq - 1;
  const int64_t pos = q_pos0 + rowc;
  const int lb = __builtin_ctz(b);          // b is a power of two
  const int ncand = row_ok ? static_cast<int>(pos >> lb) : 0;
  const int row_end = (rtile * 4 + 4) * 32;
  const int last_row = (row_end < nq ? row_end : nq) - 1;
  const int wg_cand = static_cast<int>((q_pos0 + last_row) >> lb);
  const __bf16* kb = kbar + (static_cast<int64_t>(bi) * Hkv + kvh) * ccap * D;
  const int64_t so = ((static_cast<int64_t>(bi) * Hsel + hs) * nq + rowc) * K;
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const float scale2 = scale * kSLog2e;

  // B operand q_hat^T (lane: row, k-slice 16 ks + 8 hl .. +7)
  uint4 qreg[kKS];
  {
    const __bf16* q0 = q + ((static_cast<int64_t>(bi) * qHeads + h0) * nq + rowc) * D;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qreg[ks] = qhat8(q0, static_cast<int64_t>(nq) * D, nh_in, 2 * ks + hl);
  }
  // staging: 16-byte vectors x and x + 256 of the tile (key x % 32, columns 8 (x / 32) ..)
  constexpr int kLd = kST * D / 8 / 256;
  static_assert(kLd == 1 || kLd == 2, "one or two vectors per thread");
  auto stage = [&](int c0) {
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      const int x = tid + 256 * i;
      const int kr = x % kST, cv = x / kST;
      int c = c0 + kr;
      c = c < wg_cand ? c : wg_cand - 1;
      const uint4 w = *reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(c) * D + cv * 8);
      *reinterpret_cast<uint4*>(&sm.k[kr * SbRowSmem<D>::kKPitch + cv * 8]) = w;
      sb_store_t8(reinterpret_cast<uint16_t*>(sm.kt) + cv * 8 * SbRowSmem<D>::kTPitch + kr,
                  SbRowSmem<D>::kTPitch, w);
    }
  };
  // dg of this row's selected candidates in [c0, c0 + 32), 0 elsewhere
  auto fill_dgt = [&](int c0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sm.dgt[wave][ql][16 * hl + e] = 0.f;
    wave_lds_sync();
    if (row_ok) sb_fill_dg(sm.dgt[wave][ql], idx + so, dg + so, K, hl, c0, ncand);
    wave_lds_sync();
  };
  // S^T = Kbar_perm q_hat^T: register r holds candidate c0 + sb_elem(r, hl)
  auto scores = [&](sbfloatx16_t& st) {
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.f;
    const __bf16* krow = &sm.k[sb_perm(ql) * SbRowSmem<D>::kKPitch];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const uint4 a = *reinterpret_cast<const uint4*>(krow + 16 * ks + 8 * hl);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sb_bf16x8(a), sb_bf16x8(qreg[ks]), st, 0, 0, 0);
    }
  };

  // ---- pass 1: LSE and T = sum_S exp(s - m) dg (log2 domain, online)
  float m2 = -INFINITY, l = 0.f, T = 0.f;
  for (int c0 = 0; c0 < wg_cand; c0 += kST) {
    __syncthreads();
    stage(c0);
    fill_dgt(c0);
    __syncthreads();
    sbfloatx16_t st;
    scores(st);
    float z[16], dgv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = sb_elem(r, hl);
      z[r] = c0 + m < ncand ? st[r] * scale2 : -INFINITY;
      dgv[r] = sm.dgt[wave][ql][m];
    }
    float tm = m2;
#pragma unroll
    for (int r = 0; r < 16; ++r) tm = fmaxf(tm, z[r]);
    if (tm != -INFINITY) {
      const float corr = __builtin_amdgcn_exp2f(m2 - tm);
      float ls = 0.f, ts = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(z[r] - tm);
        ls += p;
        ts = fmaf(p, dgv[r], ts);
      }
      l = l * corr + ls;
      T = T * corr + ts;
      m2 = tm;
    }
  }
  {
    // merge the two half-waves of each row
    const float mo = xor_lanes_f<32>(m2), lo = xor_lanes_f<32>(l), to = xor_lanes_f<32>(T);
    const float mm = fmaxf(m2, mo);
    if (mm != -INFINITY) {
      const float a = __builtin_amdgcn_exp2f(m2 - mm), bb = __builtin_amdgcn_exp2f(mo - mm);
      l = l * a + lo * bb;
      T = T * a + to * bb;
      m2 = mm;
    }
  }
  const float lse2 = l > 0.f ? m2 + __log2f(l) : 0.f;
  const float sig = l > 0.f ? T / l : 0.f;                   // sum_S p_m dg_m
  if (row_ok && hl == 0) ws_row[(static_cast<int64_t>(bi) * Hsel + hs) * nq + row] = make_float2(lse2, sig);

  // ---- pass 2: dq_hat^T += Kbar^T dS^T
  sbfloatx16_t acc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  for (int c0 = 0; c0 < wg_cand; c0 += kST) {
    __syncthreads();
    stage(c0);
    fill_dgt(c0);
    __syncthreads();
    sbfloatx16_t st;
    scores(st);
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = sb_elem(r, hl);
      const float p = c0 + m < ncand ? __builtin_amdgcn_exp2f(st[r] * scale2 - lse2) : 0.f;
      ds[r] = p * (sm.dgt[wave][ql][m] - sig);
    }
    // ds sums to zero over a row's candidates, so dq_hat only sees how the
    // summaries differ; rounding ds to one bf16 would leak the summaries'
    // common part, hence the hi + lo split
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      uint4 pbh, pbl;
      sb_split8(&ds[8 * s2], pbh, pbl);
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const uint4 a = *reinterpret_cast<const uint4*>(
            &sm.kt[(32 * db + ql) * SbRowSmem<D>::kTPitch + 16 * s2 + 8 * hl]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sb_bf16x8(a), sb_bf16x8(pbh), acc[db], 0, 0, 0);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sb_bf16x8(a), sb_bf16x8(pbl), acc[db], 0, 0, 0);
      }
    }
  }
  if (!row_ok) return;
  // dq_hat^T register r of block db holds d = 32 db + 8 (r / 4) + 4 hl + (r % 4)
  // written to heads hs * nh_out .. + nh_out - 1 of out, each / nh_out
  const float f = scale / static_cast<float>(nh_out);
  for (int g = 0; g < nh_out; ++g) {
    float* orow = out + ((static_cast<int64_t>(bi) * outHeads + hs * nh_out + g) * nq + row) * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
        *reinterpret_cast<float4*>(orow + 32 * db + 8 * a4 + 4 * hl) =
            make_float4(acc[db][4 * a4] * f, acc[db][4 * a4 + 1] * f, acc[db][4 * a4 + 2] * f,
                        acc[db][4 * a4 + 3] * f);
  }
}

// ---------------------------------------------------------------- candidates
template <int D>
struct SbCandSmem {
  static constexpr int kTPitch = kST + 8;
  __bf16 qt[4][D * kTPitch];               // per wave: q_hat^T of its row tile
  float dgt[4][32][kST + 4];               // per wave: dg of (row, candidate)
  float2 rs[4][32];                        // per wave: (lse2, sum_S p dg) per row
  float red[kST * D];                      // cross-wave sum
};

template <int D>
__global__ __launch_bounds__(256) void select_bwd_cands_kernel(
    const __bf16* __restrict__ q, int qHeads, int nh_in, const __bf16* __restrict__ kbar, int Hkv, int Hsel,
    int G, int share_group, int nq, int64_t q_pos0, int64_t ccap, int b, int K, const int32_t* __restrict__ idx,
    const float* __restrict__ dg, const float2* __restrict__ ws_row, float* __restrict__ dkbar) {
  // blockIdx.z of gridDim.z takes an equal share of the row tiles; with
  // several shares each writes its own copy of dkbar (summed later in order)
  __shared__ SbCandSmem<D> sm;
  constexpr int kKS = D / 16;
  constexpr int kDB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  const int c0 = blockIdx.x * kST;                 // this candidate tile
  const int bkv = blockIdx.y;
  const int bi = bkv / Hkv, kvh = bkv % Hkv;
  const int nsel = share_group ? 1 : G;            // selection heads reading this kv head
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const float scale2 = scale * kSLog2e;
  const __bf16* kb = kbar + (static_cast<int64_t>(bi) * Hkv + kvh) * ccap * D;
  const int myc = c0 + ql;                         // this lane's candidate
  const int lb = __builtin_ctz(b);                 // b is a power of two
  // B operand Kbar^T: lane = candidate, k-slice 16 ks + 8 hl .. +7
  uint4 kreg[kKS];
  {
    const int cc = myc < ccap ? myc : static_cast<int>(ccap) - 1;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      kreg[ks] = *reinterpret_cast<const uint4*>(kb + static_cast<int64_t>(cc) * D + 16 * ks + 8 * hl);
  }
  sbfloatx16_t acc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  uint16_t* tw = reinterpret_cast<uint16_t*>(sm.qt[wave]);
  // rows that have candidate c0 as a candidate: pos >= (c0 + 1) b
  int64_t r0 = (c0 + 1) * static_cast<int64_t>(b) - q_pos0;
  r0 = r0 < 0 ? 0 : r0;
  const int ntile_all = r0 < nq ? static_cast<int>((nq - r0 + 31) / 32) : 0;
  const int share = (ntile_all + gridDim.z - 1) / gridDim.z;
  const int rt_begin = share * blockIdx.z;
  const int ntile = rt_begin + share < ntile_all ? rt_begin + share : ntile_all;
  dkbar += static_cast<int64_t>(blockIdx.z) * gridDim.y * ccap * D;
  for (int sh = 0; sh < nsel; ++sh) {
    const int hs = share_group ? kvh : kvh * G + sh;
    const int h0 = hs * nh_in;
    for (int rt = rt_begin + wave; rt < ntile; rt += 4) {
      const int e0 = static_cast<int>(r0) + rt * 32;
      // A operand: q_hat rows pi(ql) (rows past nq are zero), loads issued
      // first; also q_hat^T into LDS below
      const int ea = e0 + sb_perm(ql);
      uint4 qa[kKS];
      {
        const bool aok = ea < nq;
        const __bf16* q0 = q + ((static_cast<int64_t>(bi) * qHeads + h0) * nq + (aok ? ea : nq - 1)) * D;
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
          qa[ks] = qhat8(q0, static_cast<int64_t>(nq) * D, nh_in, 2 * ks + hl);
          if (!aok) qa[ks] = make_uint4(0, 0, 0, 0);
        }
      }
      // per-row scalars and the dg table of this row tile (lane ql = tile row)
      const int er = e0 + ql;
      const bool rok = er < nq;
      const int64_t sr = ((static_cast<int64_t>(bi) * Hsel + hs) * nq + (rok ? er : nq - 1));
      const float2 rsv_own = ws_row[sr];
      if (hl == 0) sm.rs[wave][ql] = rok ? rsv_own : make_float2(0.f, 0.f);
#pragma unroll
      for (int e = 0; e < 16; ++e) sm.dgt[wave][ql][16 * hl + e] = 0.f;
      wave_lds_sync();
      if (rok)
        sb_fill_dg(sm.dgt[wave][ql], idx + sr * K, dg + sr * K, K, hl, c0,
                   static_cast<int>((q_pos0 + er) >> lb));
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        sb_store_t8(tw + (16 * ks + 8 * hl) * SbCandSmem<D>::kTPitch + sb_perm(ql), SbCandSmem<D>::kTPitch, qa[ks]);
      wave_lds_sync();
      // S = q_hat Kbar^T: lane = candidate, register r = tile row sb_elem(r, hl)
      sbfloatx16_t s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sb_bf16x8(qa[ks]), sb_bf16x8(kreg[ks]), s, 0, 0, 0);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = sb_elem(r, hl);
        const int er2 = e0 + m;
        const bool cand = er2 < nq && myc < ((q_pos0 + er2) >> lb);
        const float2 rsv = sm.rs[wave][m];
        const float p = cand ? __builtin_amdgcn_exp2f(s[r] * scale2 - rsv.x) : 0.f;
        ds[r] = p * (sm.dgt[wave][m][ql] - rsv.y);
      }
      // dKbar += dS^T q_hat: B = q_hat (lane: d = 32 db + ql, k-slice rows 16 s2 + 8 hl .. +7)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint4 pa = sb_pack8(&ds[8 * s2]);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const uint4 bt = *reinterpret_cast<const uint4*>(tw + (32 * db + ql) * SbCandSmem<D>::kTPitch + 16 * s2 + 8 * hl);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sb_bf16x8(pa), sb_bf16x8(bt), acc[db], 0, 0, 0);
        }
      }
      wave_lds_sync();
    }
  }
  // waves' sums in wave order; register r of block db holds candidate
  // 8 (r / 4) + 4 hl + (r % 4), column d = 32 db + ql
  __syncthreads();
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 8 * (r >> 2) + 4 * hl + (r & 3);
          float* p = &sm.red[c * D + 32 * db + ql];
          *p = (w == 0) ? acc[db][r] : *p + acc[db][r];
        }
    }
    __syncthreads();
  }
  for (int x = tid; x < kST * D; x += 256) {
    const int c = x / D, e = x % D;
    if (c0 + c < ccap) dkbar[((static_cast<int64_t>(bi) * Hkv + kvh) * ccap + c0 + c) * D + e] = sm.red[x] * scale;
  }
}

// ---------------------------------------------------------------- shared inputs
// q_hat of every (batch, selection head, row) as bf16 [B, Hsel, nq, d]: the
// mean of the nh heads hs * nh .. of q, as the row kernels would form it.
template <int D>
__global__ __launch_bounds__(256) void qhat_kernel(const __bf16* __restrict__ q, int Hq, int nh, int Hsel, int nq,
                                                   int64_t nvec, __bf16* __restrict__ qh) {
  constexpr int kV = D / 8;
  const int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (v >= nvec) return;
  const int64_t n = v / kV;
  const int j = static_cast<int>(v % kV);
  const int64_t row = n % nq, bh = n / nq;
  const int64_t hs = bh % Hsel, bi = bh / Hsel;
  const __bf16* q0 = q + ((bi * Hq + hs * nh) * nq + row) * D;
  *reinterpret_cast<uint4*>(qh + n * D + 8 * j) = qhat8(q0, static_cast<int64_t>(nq) * D, nh, j);
}

// out[x] = sum over shares s of part[s][x], in share order
__global__ __launch_bounds__(256) void sum_shares_kernel(const float4* __restrict__ part, int nshare, int64_t n4,
                                                         float4* __restrict__ out) {
  const int64_t x = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (x >= n4) return;
  float4 a = part[x];
  for (int s = 1; s < nshare; ++s) {
    const float4 v = part[s * n4 + x];
    a.x += v.x;
    a.y += v.y;
    a.z += v.z;
    a.w += v.w;
  }
  out[x] = a;
}

// ---------------------------------------------------------------- projection
// Row-times-matrix for the projection, rows n = (batch, selection head,
// row), out[n][j] = sum_k x[n][k] M[k][j]:
//   kDQ = false: x = q_hat (mean of the nh heads hs * nh .. of q, fp32),
//                M = W, written as bf16 U [B, Hsel, nq, d];
//   kDQ = true:  x = r (fp32), M = W^T, written / nh to the nh query heads.
// A workgroup takes 64 rows; k runs in chunks of 32 staged in LDS (x
// transposed, M row-major); each thread accumulates 4 rows x d/16 columns.
template <int D, bool kDQ>
__global__ __launch_bounds__(256) void proj_rows_kernel(const __bf16* __restrict__ q, int Hq, int nh,
                                                        const float* __restrict__ r, const float* __restrict__ W,
                                                        int Hsel, int nq, int64_t nrows, __bf16* __restrict__ uout,
                                                        float* __restrict__ dq) {
  constexpr int kRows = 64, kKC = 32, kCW = D / 16;
  __shared__ __align__(16) float ms[kKC][D + 4];
  __shared__ __align__(16) float xs[kKC][kRows + 4];
  const int tid = threadIdx.x;
  const int tcol = tid % 16, trow = tid / 16;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kRows;
  float acc[4][kCW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < kCW; ++c) acc[i][c] = 0.f;
  // this thread's staging slot: row sr, 8 consecutive k from 8 * sk
  const int sr = tid / 4, sk = tid % 4;
  const int64_t sn = n0 + sr;
  const bool s_ok = sn < nrows;
  const int64_t snc = s_ok ? sn : nrows - 1;
  for (int k0 = 0; k0 < D; k0 += kKC) {
    __syncthreads();
    for (int x = tid; x < kKC * D; x += 256) {
      if (kDQ) {
        const int jj = x / kKC, kk = x % kKC;         // W[jj][k0 + kk] read along its row
        ms[kk][jj] = W[jj * D + k0 + kk];
      } else {
        const int kk = x / D, jj = x % D;
        ms[kk][jj] = W[(k0 + kk) * D + jj];
      }
    }
    float xv[8];
    if (kDQ) {
      const float4* src = reinterpret_cast<const float4*>(r + snc * D + k0 + 8 * sk);
      const float4 a = src[0], b2 = src[1];
      xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
      xv[4] = b2.x; xv[5] = b2.y; xv[6] = b2.z; xv[7] = b2.w;
    } else {
      const int64_t row = snc % nq, bh = snc / nq;
      const int64_t hs = bh % Hsel, bi = bh / Hsel;
      const __bf16* q0 = q + ((bi * Hq + hs * nh) * nq + row) * D + k0 + 8 * sk;
      Elem<bf16_t>::unpack(*reinterpret_cast<const uint4*>(q0), xv);
      for (int g = 1; g < nh; ++g) {
        float f[8];
        Elem<bf16_t>::unpack(*reinterpret_cast<const uint4*>(q0 + static_cast<int64_t>(g) * nq * D), f);
#pragma unroll
        for (int t = 0; t < 8; ++t) xv[t] += f[t];
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) xv[t] = xv[t] / static_cast<float>(nh);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) xs[8 * sk + t][sr] = s_ok ? xv[t] : 0.f;
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < kKC; ++kk) {
      const float4 xr = *reinterpret_cast<const float4*>(&xs[kk][4 * trow]);
      float m[kCW];
#pragma unroll
      for (int c = 0; c < kCW; c += 4) {
        const float4 mv = *reinterpret_cast<const float4*>(&ms[kk][kCW * tcol + c]);
        m[c] = mv.x; m[c + 1] = mv.y; m[c + 2] = mv.z; m[c + 3] = mv.w;
      }
#pragma unroll
      for (int c = 0; c < kCW; ++c) {
        acc[0][c] = fmaf(xr.x, m[c], acc[0][c]);
        acc[1][c] = fmaf(xr.y, m[c], acc[1][c]);
        acc[2][c] = fmaf(xr.z, m[c], acc[2][c]);
        acc[3][c] = fmaf(xr.w, m[c], acc[3][c]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = n0 + 4 * trow + i;
    if (n >= nrows) continue;
    if (kDQ) {
      const int64_t row = n % nq, bh = n / nq;
      const int64_t hs = bh % Hsel, bi = bh / Hsel;
      const float inv = 1.0f / static_cast<float>(nh);
      for (int g = 0; g < nh; ++g) {
        float* o = dq + ((bi * Hq + hs * nh + g) * nq + row) * D + kCW * tcol;
#pragma unroll
        for (int c = 0; c < kCW; c += 4)
          *reinterpret_cast<float4*>(o + c) =
              make_float4(acc[i][c] * inv, acc[i][c + 1] * inv, acc[i][c + 2] * inv, acc[i][c + 3] * inv);
      }
    } else {
      __bf16* o = uout + n * D + kCW * tcol;
#pragma unroll
      for (int c = 0; c < kCW; c += 4) {
        __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v;
        v[0] = static_cast<__bf16>(acc[i][c]);
        v[1] = static_cast<__bf16>(acc[i][c + 1]);
        v[2] = static_cast<__bf16>(acc[i][c + 2]);
        v[3] = static_cast<__bf16>(acc[i][c + 3]);
        *reinterpret_cast<uint2*>(o + c) = __builtin_bit_cast(uint2, v);
      }
    }
  }
}

// dW partial sums: part[chunk][e][f] = sum over the chunk's rows of
// q_hat_n[e] r_n[f]; rows are staged 32 at a time, each thread owns a
// (d/16) x (d/16) block of dW.
template <int D>
__global__ __launch_bounds__(256) void proj_dw_partial_kernel(const __bf16* __restrict__ q, int Hq, int nh,
                                                              const float* __restrict__ r, int Hsel, int nq,
                                                              int64_t nrows, int64_t rows_per_chunk,
                                                              float* __restrict__ part) {
  constexpr int kTB = D / 16;
  constexpr int kNR = 32;
  constexpr int kQV = kNR * D / 8 / 256;         // 8-element q vectors per thread and stage
  constexpr int kRV = kNR * D / 4 / 256;         // float4 r vectors per thread and stage
  __shared__ __align__(16) float qs[kNR][D + 4];
  __shared__ __align__(16) float rs[kNR][D + 4];
  const int tid = threadIdx.x;
  const int e0 = kTB * (tid / 16), f0 = kTB * (tid % 16);
  float acc[kTB][kTB];
#pragma unroll
  for (int x = 0; x < kTB; ++x)
#pragma unroll
    for (int y = 0; y < kTB; ++y) acc[x][y] = 0.f;
  const int64_t n_begin = static_cast<int64_t>(blockIdx.x) * rows_per_chunk;
  const int64_t n_end = n_begin + rows_per_chunk < nrows ? n_begin + rows_per_chunk : nrows;
  for (int64_t nb = n_begin; nb < n_end; nb += kNR) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kQV; ++i) {
      const int x = tid + 256 * i;
      const int rr = x / (D / 8), j8 = x % (D / 8);
      const int64_t n = nb + rr;
      float v[8];
      if (n < n_end) {
        const int64_t row = n % nq, bh = n / nq;
        const int64_t hs = bh % Hsel, bi = bh / Hsel;
        const __bf16* q0 = q + ((bi * Hq + hs * nh) * nq + row) * D + 8 * j8;
        Elem<bf16_t>::unpack(*reinterpret_cast<const uint4*>(q0), v);
        for (int g = 1; g < nh; ++g) {
          float f[8];
          Elem<bf16_t>::unpack(*reinterpret_cast<const uint4*>(q0 + static_cast<int64_t>(g) * nq * D), f);
#pragma unroll
          for (int t = 0; t < 8; ++t) v[t] += f[t];
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = v[t] / static_cast<float>(nh);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = 0.f;
      }
      *reinterpret_cast<float4*>(&qs[rr][8 * j8]) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(&qs[rr][8 * j8 + 4]) = make_float4(v[4], v[5], v[6], v[7]);
    }
#pragma unroll
    for (int i = 0; i < kRV; ++i) {
      const int x = tid + 256 * i;
      const int rr = x / (D / 4), j4 = x % (D / 4);
      const int64_t n = nb + rr;
      const float4 v = n < n_end ? *reinterpret_cast<const float4*>(r + n * D + 4 * j4) : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(&rs[rr][4 * j4]) = v;
    }
    __syncthreads();
#pragma unroll 2
    for (int rr = 0; rr < kNR; ++rr) {
      float a[kTB], bv[kTB];
#pragma unroll
      for (int t = 0; t < kTB; t += 4) {
        const float4 av = *reinterpret_cast<const float4*>(&qs[rr][e0 + t]);
        const float4 bw = *reinterpret_cast<const float4*>(&rs[rr][f0 + t]);
        a[t] = av.x; a[t + 1] = av.y; a[t + 2] = av.z; a[t + 3] = av.w;
        bv[t] = bw.x; bv[t + 1] = bw.y; bv[t + 2] = bw.z; bv[t + 3] = bw.w;
      }
#pragma unroll
      for (int x = 0; x < kTB; ++x)
#pragma unroll
        for (int y = 0; y < kTB; ++y) acc[x][y] = fmaf(a[x], bv[y], acc[x][y]);
    }
  }
  float* dst = part + static_cast<int64_t>(blockIdx.x) * D * D;
#pragma unroll
  for (int x = 0; x < kTB; ++x)
#pragma unroll
    for (int y = 0; y < kTB; y += 4)
      *reinterpret_cast<float4*>(dst + (e0 + x) * D + f0 + y) =
          make_float4(acc[x][y], acc[x][y + 1], acc[x][y + 2], acc[x][y + 3]);
}

// dW = sum of the chunk partials in chunk order
__global__ __launch_bounds__(256) void proj_dw_sum_kernel(const float* __restrict__ part, int nchunk, int dd,
                                                          float* __restrict__ dw) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= dd) return;
  // loads of 16 chunks issued together, added in chunk order
  float s = 0.f;
  int c = 0;
  for (; c + 16 <= nchunk; c += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = part[static_cast<int64_t>(c + u) * dd + x];
#pragma unroll
    for (int u = 0; u < 16; ++u) s += v[u];
  }
  for (; c < nchunk; ++c) s += part[static_cast<int64_t>(c) * dd + x];
  dw[x] = s;
}

// ---------------------------------------------------------------- mean
// dk_j += dkbar_c / b for every token j of block c < ccap of one (batch, kv
// head); 8 elements per thread, rounded to bf16 (nearest even) after the add.
template <int D>
__global__ __launch_bounds__(256) void summary_mean_bwd_kernel(const float* __restrict__ dkbar,
                                                               __bf16* __restrict__ dk, int64_t ccap, int64_t L,
                                                               int lb, float inv_b) {
  constexpr int kV = D / 8;                     // 8-element vectors per token
  const int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (v >= (ccap << lb) * kV) return;
  const int64_t head = blockIdx.y;
  const int64_t t = v / kV;
  const int e8 = static_cast<int>(v % kV);
  const int64_t c = t >> lb;
  uint4* dst = reinterpret_cast<uint4*>(dk + (head * L + t) * D + 8 * e8);
  const float4* src = reinterpret_cast<const float4*>(dkbar + (head * ccap + c) * D + 8 * e8);
  const float4 a = src[0], bq = src[1];
  float x[8];
  Elem<bf16_t>::unpack(*dst, x);
  x[0] = fmaf(a.x, inv_b, x[0]);
  x[1] = fmaf(a.y, inv_b, x[1]);
  x[2] = fmaf(a.z, inv_b, x[2]);
  x[3] = fmaf(a.w, inv_b, x[3]);
  x[4] = fmaf(bq.x, inv_b, x[4]);
  x[5] = fmaf(bq.y, inv_b, x[5]);
  x[6] = fmaf(bq.z, inv_b, x[6]);
  x[7] = fmaf(bq.w, inv_b, x[7]);
  *dst = sb_pack8(x);
}

// ---------------------------------------------------------------- launch
namespace {
struct SbWs {
  size_t row, qh, dkp, u, r, part, total;
  int64_t nrows, rows_per_chunk;
  int nchunk, nshare;
};
// row shares of the candidate kernel: enough workgroups to cover the chip
// about four times, each share at least 8 row tiles
int cand_shares(const SelectLaunch& p) {
  const int64_t wgs = ((p.ccap + kST - 1) / kST) * p.B * p.Hkv;
  int64_t s = (1024 + wgs - 1) / wgs;
  const int64_t by_rows = (p.nq / 32 + 7) / 8;
  s = s < by_rows ? s : by_rows;
  s = s < 16 ? s : 16;
  return s < 1 ? 1 : static_cast<int>(s);
}
SbWs select_bwd_ws(const SelectLaunch& p) {
  SbWs w{};
  w.nrows = static_cast<int64_t>(p.B) * p.Hsel * p.nq;
  w.row = 0;
  size_t off = align256(static_cast<size_t>(w.nrows) * sizeof(float2));
  w.nshare = cand_shares(p);
  if (p.proj_w == nullptr && p.share_group && p.Hq > p.Hkv) {
    w.qh = off;                                  // q_hat once, shared by both kernels
    off += align256(static_cast<size_t>(w.nrows) * p.d * 2);
  }
  if (w.nshare > 1) {
    w.dkp = off;
    off += align256(static_cast<size_t>(w.nshare) * p.B * p.Hkv * p.ccap * p.d * 4);
  }
  if (p.proj_w != nullptr) {
    const int64_t per = (w.nrows + 511) / 512;
    w.rows_per_chunk = per < 256 ? 256 : (per + 31) / 32 * 32;
    w.nchunk = static_cast<int>((w.nrows + w.rows_per_chunk - 1) / w.rows_per_chunk);
    w.u = off;
    off += align256(static_cast<size_t>(w.nrows) * p.d * 2);
    w.r = off;
    off += align256(static_cast<size_t>(w.nrows) * p.d * 4);
    w.part = off;
    off += align256(static_cast<size_t>(w.nchunk) * p.d * p.d * 4);
  }
  w.total = off;
  return w;
}
}  // namespace

size_t select_bwd_workspace_bytes(const SelectLaunch& p) { return select_bwd_ws(p).total; }

template <int D>
static hipError_t launch_select_bwd_d(const SelectLaunch& p, const SelectGrads& g, void* ws, hipStream_t st) {
  const SbWs w = select_bwd_ws(p);
  char* base = static_cast<char*>(ws);
  float2* ws_row = reinterpret_cast<float2*>(base + w.row);
  const int G = p.Hq / p.Hkv;
  const int nh = p.share_group ? G : 1;
  const auto* q = static_cast<const __bf16*>(p.q);
  const auto* kbar = static_cast<const __bf16*>(p.kbar);
  const dim3 rows_grid((p.nq + 127) / 128, static_cast<unsigned>(p.B * p.Hsel));
  const int ntile = static_cast<int>((p.ccap + kST - 1) / kST);
  // candidate tiles cover every summary slot (slots that are no row's
  // candidate get zero gradient); row shares write partial copies
  const dim3 cand_grid(ntile, static_cast<unsigned>(p.B * p.Hkv), static_cast<unsigned>(w.nshare));
  float* dkbar_c = w.nshare > 1 ? reinterpret_cast<float*>(base + w.dkp) : g.dkbar;
  const int64_t dkbar_n4 = static_cast<int64_t>(p.B) * p.Hkv * p.ccap * D / 4;
  const dim3 sum_grid(static_cast<unsigned>((dkbar_n4 + 255) / 256));
  hipError_t e;
  if (p.proj_w == nullptr) {
    // query source: q itself (one head per selection) or q_hat formed once
    const __bf16* qs = q;
    int qs_heads = p.Hq, qs_nh = nh;
    if (nh > 1) {
      __bf16* qh = reinterpret_cast<__bf16*>(base + w.qh);
      const int64_t nvec = w.nrows * (D / 8);
      e = launch(false, qhat_kernel<D>, dim3(static_cast<unsigned>((nvec + 255) / 256)), dim3(256), st, q, p.Hq,
                 nh, p.Hsel, p.nq, nvec, qh);
      if (e != hipSuccess) return e;
      qs = qh;
      qs_heads = p.Hsel;
      qs_nh = 1;
    }
    e = launch(false, select_bwd_rows_kernel<D>, rows_grid, dim3(256), st, qs, qs_heads, qs_nh, kbar, p.Hkv,
               p.Hsel, G, p.share_group, p.nq, p.q_pos0, p.ccap, p.b, p.K, p.idx, g.dg, g.dq, p.Hq, nh, ws_row);
    if (e != hipSuccess) return e;
    e = launch(false, select_bwd_cands_kernel<D>, cand_grid, dim3(256), st, qs, qs_heads, qs_nh, kbar, p.Hkv,
               p.Hsel, G, p.share_group, p.nq, p.q_pos0, p.ccap, p.b, p.K, p.idx, g.dg, ws_row, dkbar_c);
    if (e != hipSuccess) return e;
    if (w.nshare > 1)
      e = launch(false, sum_shares_kernel, sum_grid, dim3(256), st, reinterpret_cast<const float4*>(dkbar_c),
                 w.nshare, dkbar_n4, reinterpret_cast<float4*>(g.dkbar));
  } else {
    __bf16* u = reinterpret_cast<__bf16*>(base + w.u);
    float* r = reinterpret_cast<float*>(base + w.r);
    float* part = reinterpret_cast<float*>(base + w.part);
    const dim3 proj_grid(static_cast<unsigned>((w.nrows + 63) / 64));
    e = launch(false, proj_rows_kernel<D, false>, proj_grid, dim3(256), st, q, p.Hq, nh,
               static_cast<const float*>(nullptr), p.proj_w, p.Hsel, p.nq, w.nrows, u, static_cast<float*>(nullptr));
    if (e != hipSuccess) return e;
    // rows and candidates on u = W^T q_hat (one source head per selection head)
    e = launch(false, select_bwd_rows_kernel<D>, rows_grid, dim3(256), st, static_cast<const __bf16*>(u), p.Hsel,
               1, kbar, p.Hkv, p.Hsel, G, p.share_group, p.nq, p.q_pos0, p.ccap, p.b, p.K, p.idx, g.dg, r, p.Hsel,
               1, ws_row);
    if (e != hipSuccess) return e;
    e = launch(false, select_bwd_cands_kernel<D>, cand_grid, dim3(256), st, static_cast<const __bf16*>(u), p.Hsel,
               1, kbar, p.Hkv, p.Hsel, G, p.share_group, p.nq, p.q_pos0, p.ccap, p.b, p.K, p.idx, g.dg, ws_row,
               dkbar_c);
    if (e != hipSuccess) return e;
    if (w.nshare > 1) {
      e = launch(false, sum_shares_kernel, sum_grid, dim3(256), st, reinterpret_cast<const float4*>(dkbar_c),
                 w.nshare, dkbar_n4, reinterpret_cast<float4*>(g.dkbar));
      if (e != hipSuccess) return e;
    }
    e = launch(false, proj_rows_kernel<D, true>, proj_grid, dim3(256), st, q, p.Hq, nh,
               static_cast<const float*>(r), p.proj_w, p.Hsel, p.nq, w.nrows, static_cast<__bf16*>(nullptr), g.dq);
    if (e != hipSuccess) return e;
    e = launch(false, proj_dw_partial_kernel<D>, dim3(w.nchunk), dim3(256), st, q, p.Hq, nh,
               static_cast<const float*>(r), p.Hsel, p.nq, w.nrows, w.rows_per_chunk, part);
    if (e != hipSuccess) return e;
    e = launch(g.dk == nullptr, proj_dw_sum_kernel, dim3((D * D + 255) / 256), dim3(256), st,
               static_cast<const float*>(part), w.nchunk, D * D, g.dproj_w);
  }
  if (e != hipSuccess || g.dk == nullptr) return e;
  const int64_t nvec = (p.ccap * p.b) * (D / 8);
  return launch(true, summary_mean_bwd_kernel<D>, dim3(static_cast<unsigned>((nvec + 255) / 256),
                                                       static_cast<unsigned>(p.B * p.Hkv)),
                dim3(256), st, static_cast<const float*>(g.dkbar), static_cast<__bf16*>(g.dk), p.ccap, g.L,
                __builtin_ctz(p.b), 1.0f / static_cast<float>(p.b));
}

hipError_t launch_select_bwd(const SelectLaunch& p, const SelectGrads& g, void* ws, hipStream_t st) {
  return p.d == 64 ? launch_select_bwd_d<64>(p, g, ws, st) : launch_select_bwd_d<128>(p, g, ws, st);
}

}  // namespace spa
