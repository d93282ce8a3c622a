// attn_bwd_mfma.hip -- MFMA (bf16, gfx950 v_mfma_f32_32x32x16_bf16) backward of
// the block-sparse attention in the SAS mode (current block + K selected
// blocks with log gates).  Same results as the VALU kernels in attn.hip
// ("SAS" review §4.1 Eq. 4, §4.2.2 Eq. 5): with p_ij recomputed from lse,
//   D_i = do_i . o_i,  dS_ij = p_ij (do_i . v_j - D_i),
//   dq_i = sum_j dS_ij k_j / sqrt(d),  dk_j = sum_i dS_ij q_i / sqrt(d),
//   dv_j = sum_i p_ij do_i,  dg_im = sum_{j in B_m} dS_ij / g_im.
//
// Three launches after the D_i pass:
//   mark     one bit per (selection head, block, row) for "row selected block"
//            (a bitmap, so the dk / dv pass can list a block's rows in order),
//            built per 256-row slice in LDS and written whole
//            (launch_mark_rows, shared with the routed-cell forward);
//   dq / dg  like the forward tile kernel: a workgroup holds 32-row tiles of
//            the heads sharing a selection, walks the ascending union of their
//            key tiles, S^T = K Q^T and dP^T = V dO^T put one row per lane,
//            dQ^T += K^T dS^T accumulates in MFMA registers, and per-slot sums
//            of dS land in LDS (summed over the heads at the end, in order);
//   dk / dv  one workgroup per 32-key tile: the rows that read it (its block's
//            own rows, causally, then the rows that selected the block, in row
//            order) are taken 32 at a time; S = Q K^T and dP = dO V^T put one
//            key per lane, dV += P^T dO and dK += dS^T Q accumulate in MFMA
//            registers, and the four waves' sums are added in a fixed order.
#include <type_traits>

#include "spa_device.h"
#include "spa_launch.h"

namespace spa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bbf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float bfloatx16_t;

constexpr int kBT = 32;               // keys (or rows) per tile
constexpr int kBMaxKeyTiles = 2048;   // L <= 65536
constexpr int kBMaxSelK = 32;
constexpr float kBLog2e = 1.4426950408889634f;

__device__ __forceinline__ bbf16x8_t b_as_bf16x8(uint4 v) { return __builtin_bit_cast(bbf16x8_t, v); }

// Register r of half-wave h of a 32x32 MFMA result holds output row
// 8 (r / 4) + 4 h + (r % 4).  Feeding A row pi(m) instead of m (pi below)
// makes register r hold tile element 16 (r / 8) + 8 h + (r % 8), so the 8
// registers 8s .. 8s+7 of a lane are exactly the k-slice 16s + 8h .. +7 that
// lane supplies as an A or B operand of the next product.
__device__ __forceinline__ int b_tile_elem(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }
__device__ __forceinline__ int b_perm(int m) {
  const int a = m >> 3, h = (m >> 2) & 1, c = m & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + c;
}

__device__ __forceinline__ uint4 pack_bf16x8(const float* x) {
  bbf16x8_t v;
#pragma unroll
  for (int t = 0; t < 8; ++t) v[t] = static_cast<__bf16>(x[t]);
  return __builtin_bit_cast(uint4, v);
}

// 8 bf16 of a 16-byte vector, written as 2-byte LDS stores with stride `pitch`
// (a transposed copy).
__device__ __forceinline__ void store_transposed8(uint16_t* dst, int pitch, uint4 w) {
  dst[0 * pitch] = static_cast<uint16_t>(w.x);
  dst[1 * pitch] = static_cast<uint16_t>(w.x >> 16);
  dst[2 * pitch] = static_cast<uint16_t>(w.y);
  dst[3 * pitch] = static_cast<uint16_t>(w.y >> 16);
  dst[4 * pitch] = static_cast<uint16_t>(w.z);
  dst[5 * pitch] = static_cast<uint16_t>(w.z >> 16);
  dst[6 * pitch] = static_cast<uint16_t>(w.w);
  dst[7 * pitch] = static_cast<uint16_t>(w.w >> 16);
}

}  // namespace

// The mark bitmap: bits[((b Hsel + hs) nblk + c) nw + row / 32] bit row % 32
// = row selected c (launch_mark_rows).
// ---------------------------------------------------------------- dq / dg
template <int D>
struct DqSmem {
  static constexpr int kKPitch = D + 8;      // K / V rows (bf16)
  static constexpr int kTPitch = kBT + 8;    // K^T rows (bf16)
  __bf16 k[kBT * kKPitch];
  __bf16 v[kBT * kKPitch];
  __bf16 kt[D * kTPitch];
};

template <int D>
__global__ __launch_bounds__(256, 2) void attn_tile_dq_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dbuf,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, int Hq, int Hkv, int Hsel,
    int share_group, int nq, int64_t q_pos0, int64_t L, int b, int K, __bf16* __restrict__ dq,
    float* __restrict__ dg, int NH, int NT) {
  __shared__ DqSmem<D> sm;
  __shared__ uint32_t s_bits[kBMaxKeyTiles / 32];
  __shared__ uint16_t s_list[kBMaxKeyTiles];
  __shared__ int s_count;
  __shared__ int32_t s_idx[4][32][kBMaxSelK / 2 + 1];   // packed pairs of int16 units
  __shared__ float s_lg[4][32][kBMaxSelK];
  __shared__ float s_dg[4][32][kBMaxSelK];

  constexpr int kKS = D / 16;
  constexpr int kDB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  const int G = Hq / Hkv;
  const int hgroups = G / NH;
  const uint2 bxy = xcd_block_xy_last_first();             // XCD-aware, longest row tiles first
  const int bz = static_cast<int>(bxy.y);
  const int bi = bz / (Hkv * hgroups);
  const int kvh = (bz / hgroups) % Hkv;
  const int hg = bz % hgroups;
  const int hw = wave % NH;
  const int h = kvh * G + hg * NH + hw;                    // this wave's query head
  const int hs = share_group ? kvh : h;
  const int tile = static_cast<int>(bxy.x) * NT + wave / NH;   // this wave's 32-row tile
  const int row = tile * 32 + ql;
  const bool row_ok = row < nq;
  const int rowc = row_ok ? row : nq - 1;
  const int pos32 = static_cast<int>(q_pos0 + rowc);
  const int lb = __builtin_ctz(b);         // b is a power of two
  const int c_cur = pos32 >> lb;
  const int c_end = (c_cur + 1) * b;
  const int nkt = static_cast<int>((L + kBT - 1) / kBT);
  const int nwords = (nkt + 31) / 32;

  // ---- per-row selection tables (this wave's rows), unit = -1 when unused
  const int64_t so = ((static_cast<int64_t>(bi) * Hsel + hs) * nq + rowc) * K;
  for (int t = hl; t < K; t += 2) {
    const int32_t c = idx[so + t];
    const bool ok = row_ok && c >= 0 && c < c_cur;
    reinterpret_cast<int16_t*>(s_idx[wave][ql])[t] = static_cast<int16_t>(ok ? c : -1);
    s_lg[wave][ql][t] = (ok && logg != nullptr) ? logg[so + t] : 0.f;
    s_dg[wave][ql][t] = 0.f;
  }
  for (int x = tid; x < kBMaxKeyTiles / 32; x += 256) s_bits[x] = 0u;
  __syncthreads();
  {
    const int64_t wg_row0 = static_cast<int64_t>(bxy.x) * NT * 32;
    const int64_t wg_row1 = (wg_row0 + NT * 32 < nq ? wg_row0 + NT * 32 : nq) - 1;
    const int64_t p0 = q_pos0 + wg_row0, p1 = q_pos0 + wg_row1;
    for (int64_t t = (p0 / b) * b / kBT + tid; t <= p1 / kBT; t += 256) atomicOr(&s_bits[t >> 5], 1u << (t & 31));
  }
  for (int t = hl; t < K; t += 2) {
    const int c = reinterpret_cast<int16_t*>(s_idx[wave][ql])[t];
    if (c >= 0) {
      for (int kt = c * b / kBT; kt <= (c * b + b - 1) / kBT; ++kt) atomicOr(&s_bits[kt >> 5], 1u << (kt & 31));
    }
  }
  __syncthreads();
  if (wave == 0) {
    int base = 0;
    for (int w0 = 0; w0 < nwords; w0 += 64) {
      const int wi = w0 + lane;
      const uint32_t bits = wi < nwords ? s_bits[wi] : 0u;
      const int cnt = __popc(bits);
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int up = __shfl_up(incl, off, 64);
        if (lane >= off) incl += up;
      }
      int wpos = base + incl - cnt;
      uint32_t bb = bits;
      while (bb) {
        const int bit = __ffs(bb) - 1;
        bb &= bb - 1;
        s_list[wpos++] = static_cast<uint16_t>(wi * 32 + bit);
      }
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) s_count = base;
  }
  __syncthreads();

  // ---- B operands: Q^T and dO^T (lane: row, k-slice 16 ks + 8 hl .. +7)
  uint4 qreg[kKS], doreg[kKS];
  const int64_t qrow = (static_cast<int64_t>(bi) * Hq + h) * nq + rowc;
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    qreg[ks] = *reinterpret_cast<const uint4*>(q + qrow * D + 16 * ks + 8 * hl);
    doreg[ks] = *reinterpret_cast<const uint4*>(dout + qrow * D + 16 * ks + 8 * hl);
  }
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const float scale2 = kBLog2e * scale;
  const float lse2 = lse[qrow] * kBLog2e;
  const float Drow = Dbuf[qrow];
  const int64_t kvbase = (static_cast<int64_t>(bi) * Hkv + kvh) * L * D;

  bfloatx16_t acc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  int cur = 0;                             // cursor into this row's units; the unit
  int nu;                                  // there (past the end: INT_MAX) and its
  float nlg;                               // log2 gate are kept in registers
  {
    const int16_t* urow = reinterpret_cast<const int16_t*>(s_idx[wave][ql]);
    nu = K > 0 ? urow[0] : 0x7FFFFFFF;
    nlg = K > 0 ? s_lg[wave][ql][0] * kBLog2e : 0.f;
  }

  // staging: 16-byte vectors x and x + 256 of the K and V tiles per thread
  constexpr int kLd = kBT * D / 8 / 256;
  static_assert(kLd == 1 || kLd == 2, "one or two vectors per thread per tile");
  uint4 kld0, vld0, kld1 = make_uint4(0, 0, 0, 0), vld1 = make_uint4(0, 0, 0, 0);
  const int ntl = s_count;
  // thread x moves key x % 32, columns 8 (x / 32) .. +7 (and x + 256): each
  // transposed 2-byte LDS store of a wave then covers 32 consecutive keys
#define SPA_DQ_ISSUE(IT)                                                                    \
  do {                                                                                      \
    const int64_t kb0 = static_cast<int64_t>(s_list[IT]) * kBT;                             \
    int64_t key = kb0 + tid % kBT;                                                          \
    key = key < L ? key : L - 1;                                                            \
    kld0 = *reinterpret_cast<const uint4*>(k + kvbase + key * D + (tid / kBT) * 8);         \
    vld0 = *reinterpret_cast<const uint4*>(v + kvbase + key * D + (tid / kBT) * 8);         \
    if constexpr (kLd == 2) {                                                               \
      kld1 = *reinterpret_cast<const uint4*>(k + kvbase + key * D + (tid / kBT + 8) * 8);   \
      vld1 = *reinterpret_cast<const uint4*>(v + kvbase + key * D + (tid / kBT + 8) * 8);   \
    }                                                                                       \
  } while (0)
#define SPA_DQ_STAGE_ONE(KW, VW, X)                                                         \
  do {                                                                                      \
    const int kr = (X) % kBT, cv = (X) / kBT;                                               \
    *reinterpret_cast<uint4*>(&sm.k[kr * DqSmem<D>::kKPitch + cv * 8]) = KW;               \
    *reinterpret_cast<uint4*>(&sm.v[kr * DqSmem<D>::kKPitch + cv * 8]) = VW;               \
    store_transposed8(reinterpret_cast<uint16_t*>(sm.kt) + cv * 8 * DqSmem<D>::kTPitch + kr, \
                      DqSmem<D>::kTPitch, KW);                                              \
  } while (0)
#define SPA_DQ_STAGE()                                                                      \
  do {                                                                                      \
    SPA_DQ_STAGE_ONE(kld0, vld0, tid);                                                      \
    if constexpr (kLd == 2) SPA_DQ_STAGE_ONE(kld1, vld1, tid + 256);                        \
  } while (0)
  if (ntl > 0) {
    SPA_DQ_ISSUE(0);
    SPA_DQ_STAGE();
  }
  __syncthreads();
  int ks0n = ntl > 0 ? static_cast<int>(s_list[0]) * kBT : 0;
  for (int it = 0; it < ntl; ++it) {
    if (it + 1 < ntl) SPA_DQ_ISSUE(it + 1);
    const int ks0 = ks0n;                     // list entry read one tile ahead
    if (it + 1 < ntl) ks0n = static_cast<int>(s_list[it + 1]) * kBT;
    // bias (log2 domain) and gate slot of the two 16-key halves this lane holds
    float bias[2];
    int slot[2];
    {
      const int16_t* ur = reinterpret_cast<const int16_t*>(s_idx[wave][ql]);
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        const int uv = (ks0 + 16 * part + 8 * hl) >> lb;
        float bv = -INFINITY;
        int sl = -1;
        if (uv == c_cur) {
          bv = 0.f;
        } else {
          while (nu < uv) {   // advance past smaller units (unused slots hold -1)
            ++cur;
            nu = cur < K ? ur[cur] : 0x7FFFFFFF;
            nlg = cur < K ? s_lg[wave][ql][cur] * kBLog2e : 0.f;
          }
          if (nu == uv) {
            bv = nlg;
            sl = cur;
          }
        }
        bias[part] = row_ok ? bv : -INFINITY;
        slot[part] = row_ok ? sl : -1;
      }
    }
    const bool need = bias[0] != -INFINITY || bias[1] != -INFINITY;
    if (__ballot(need) != 0) {
      bfloatx16_t st, dpt;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[r] = 0.f;
        dpt[r] = 0.f;
      }
      const __bf16* krow = &sm.k[b_perm(ql) * DqSmem<D>::kKPitch];
      const __bf16* vrow = &sm.v[b_perm(ql) * DqSmem<D>::kKPitch];
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(krow + 16 * ks + 8 * hl);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b_as_bf16x8(a), b_as_bf16x8(qreg[ks]), st, 0, 0, 0);
        const uint4 av = *reinterpret_cast<const uint4*>(vrow + 16 * ks + 8 * hl);
        dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b_as_bf16x8(av), b_as_bf16x8(doreg[ks]), dpt, 0, 0, 0);
      }
      const bool causal = ks0 + kBT - 1 > pos32 && ks0 < c_end;
      float ds[16];
      float dsum[2] = {0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float z = fmaf(st[r], scale2, bias[r >> 3] - lse2);
        if (causal) {
          const int key = ks0 + b_tile_elem(r, hl);
          z = (key > pos32 && key < c_end) ? -INFINITY : z;
        }
        const float p = __builtin_amdgcn_exp2f(z);
        ds[r] = p * (dpt[r] - Drow);
        dsum[r >> 3] += ds[r];
      }
      // gate gradient: sum of dS over each unit's keys of the tile
      if (__ballot(slot[0] >= 0 || slot[1] >= 0) != 0) {
        dsum[0] += xor_lanes_f<32>(dsum[0]);
        dsum[1] += xor_lanes_f<32>(dsum[1]);
        if (hl == 0) {
          if (slot[0] >= 0 && slot[0] == slot[1]) {
            s_dg[wave][ql][slot[0]] += dsum[0] + dsum[1];
          } else {
            if (slot[0] >= 0) s_dg[wave][ql][slot[0]] += dsum[0];
            if (slot[1] >= 0) s_dg[wave][ql][slot[1]] += dsum[1];
          }
        }
      }
      // dQ^T += K^T dS^T: B = dS^T (keys 16 s2 + 8 hl + t of this lane's row)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint4 pb = pack_bf16x8(&ds[8 * s2]);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const uint4 a = *reinterpret_cast<const uint4*>(
              &sm.kt[(32 * db + ql) * DqSmem<D>::kTPitch + 16 * s2 + 8 * hl]);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b_as_bf16x8(a), b_as_bf16x8(pb), acc[db], 0, 0, 0);
        }
      }
    }
    lds_barrier();                          // every wave is done with the tile
    if (it + 1 < ntl) SPA_DQ_STAGE();
    lds_barrier();
  }
#undef SPA_DQ_ISSUE
#undef SPA_DQ_STAGE_ONE
#undef SPA_DQ_STAGE
  if (row_ok) {
    // dQ^T register r of block db holds d = 32 db + 8 (r / 4) + 4 hl + (r % 4)
    __bf16* orow = dq + qrow * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 w4;
#pragma unroll
        for (int c = 0; c < 4; ++c) w4[c] = static_cast<__bf16>(acc[db][4 * a4 + c] * scale);
        *reinterpret_cast<decltype(w4)*>(orow + 32 * db + 8 * a4 + 4 * hl) = w4;
      }
  }
  // dg: the heads of the selection in this workgroup, summed in head order
  __syncthreads();
  if (hw != 0 || !row_ok) return;
  for (int t = hl; t < K; t += 2) {
    float sum = 0.f;
    const bool ok = reinterpret_cast<int16_t*>(s_idx[wave][ql])[t] >= 0;
    if (share_group) {
      for (int x = 0; x < NH; ++x) sum += s_dg[wave + x][ql][t];
    } else {
      sum = s_dg[wave][ql][t];
    }
    dg[so + t] = ok ? sum * __expf(-s_lg[wave][ql][t]) : 0.f;
  }
}

// ---------------------------------------------------------------- dk / dv
template <int D>
struct DkvSmem {
  static constexpr int kKPitch = D + 8;      // K / V tile rows (bf16)
  static constexpr int kTPitch = kBT + 8;    // per-wave transposed Q / dO rows (bf16)
  static constexpr int kSeg = 2048;          // rows of the bitmap listed per pass
  __bf16 k[kBT * kKPitch];
  __bf16 v[kBT * kKPitch];
  union {
    __bf16 t[4][D * kTPitch];                // per wave: dO^T or Q^T of the row tile
    float red[2][kBT * D];                   // final cross-wave sums (dk, dv)
  } u;
  int rows[kSeg + 64];
  float bias[kSeg + 64];                     // natural log gate (0 on the block's own rows)
  float4 rs[4][32];                          // per wave, per tile row: lse2, D, bias2, pos
  int nrows;
  int wcount[64];
};

template <int D>
__global__ __launch_bounds__(256, 2) void attn_tile_dkdv_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dbuf,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, const uint32_t* __restrict__ bits,
    int Hq, int Hkv, int Hsel, int nq, int64_t q_pos0, int64_t L, int b, int K, int64_t nblk, int nw,
    __bf16* __restrict__ dk, __bf16* __restrict__ dv) {
  __shared__ DkvSmem<D> sm;
  constexpr int kKS = D / 16;
  constexpr int kDB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  const uint2 bxy = xcd_block_xy();                 // XCD-aware order: a head's key tiles share an L2
  const int kt = static_cast<int>(bxy.x);            // key tile
  const int bkv = static_cast<int>(bxy.y);
  const int bi = bkv / Hkv, kvh = bkv % Hkv;
  const int G = Hq / Hkv;
  const int g = wave % G, stride0 = wave / G, nstride = 4 / G;
  const int h = kvh * G + g;                         // this wave's query head
  const int hs = kvh;                                // the selection head (shared, or G = 1)
  const int key0 = kt * kBT;
  const int c = key0 / b;                            // the block of the tile
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const float scale2 = kBLog2e * scale;
  const int64_t kvbase = (static_cast<int64_t>(bi) * Hkv + kvh) * L * D;

  // K and V tile, row-major (rows past L are clamped copies; their results are dropped)
  for (int x = tid; x < kBT * D / 8; x += 256) {
    const int kr = x / (D / 8), cv = x % (D / 8);
    int64_t key = key0 + kr;
    key = key < L ? key : L - 1;
    *reinterpret_cast<uint4*>(&sm.k[kr * DkvSmem<D>::kKPitch + cv * 8]) =
        *reinterpret_cast<const uint4*>(k + kvbase + key * D + cv * 8);
    *reinterpret_cast<uint4*>(&sm.v[kr * DkvSmem<D>::kKPitch + cv * 8]) =
        *reinterpret_cast<const uint4*>(v + kvbase + key * D + cv * 8);
  }
  __syncthreads();
  // B operands K^T, V^T: lane = key ql, k-slice 16 ks + 8 hl .. +7, read from
  // the LDS tile per row tile (held in registers they would take 64 VGPRs and
  // leave room for one wave per SIMD at d = 128)
  const __bf16* krow_l = &sm.k[ql * DkvSmem<D>::kKPitch + 8 * hl];
  const __bf16* vrow_l = &sm.v[ql * DkvSmem<D>::kKPitch + 8 * hl];
  const int mykey = key0 + ql;

  bfloatx16_t dka[kDB], dva[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dka[db][r] = 0.f;
      dva[db][r] = 0.f;
    }

  // rows of the block's own span that can see a key of the tile (causal), then
  // the rows that selected the block, listed from the bitmap in row order
  const int64_t own_lo = key0 > c * static_cast<int64_t>(b) ? key0 : c * static_cast<int64_t>(b);
  int64_t r_lo = own_lo - q_pos0, r_hi = (c + 1) * static_cast<int64_t>(b) - 1 - q_pos0;
  r_lo = r_lo < 0 ? 0 : r_lo;
  r_hi = r_hi > nq - 1 ? nq - 1 : r_hi;
  const int n_own = r_hi >= r_lo ? static_cast<int>(r_hi - r_lo + 1) : 0;
  const uint32_t* brow = bits + ((static_cast<int64_t>(bi) * Hsel + hs) * nblk + c) * nw;
  const int64_t sel_first = (c + 1) * static_cast<int64_t>(b) - q_pos0;   // first row that can select c

  for (int seg0 = 0; seg0 < nq || seg0 == 0; seg0 += DkvSmem<D>::kSeg) {
    // ---- list this pass's rows
    __syncthreads();
    int base = 0;
    if (seg0 == 0) {
      for (int x = tid; x < n_own; x += 256) {
        sm.rows[x] = static_cast<int>(r_lo) + x;
        sm.bias[x] = 0.f;
      }
      base = n_own;
    }
    {
      // 64 words (2048 rows) per pass: one word per thread of wave 0
      int cnt = 0;
      uint32_t w = 0u;
      const int wi = seg0 / 32 + lane;
      if (wave == 0) {
        w = (wi < nw && static_cast<int64_t>(wi) * 32 + 31 >= sel_first) ? brow[wi] : 0u;
        cnt = __popc(w);
        int incl = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int up = __shfl_up(incl, off, 64);
          if (lane >= off) incl += up;
        }
        int wpos = base + incl - cnt;
        while (w) {
          const int bit = __ffs(w) - 1;
          w &= w - 1;
          sm.rows[wpos] = wi * 32 + bit;
          sm.bias[wpos] = 1.f;     // marker: look the gate up below
          ++wpos;
        }
        if (lane == 63) sm.nrows = base + incl;
      }
    }
    __syncthreads();
    const int n = sm.nrows;
    // gate of each selecting row for block c: the row's entries are loaded
    // eight at a time, then the slot holding c gives the log gate
    for (int x = tid; x < n; x += 256) {
      if (x < base) continue;
      const int r = sm.rows[x];
      float lg = 0.f;
      if (logg != nullptr) {
        const int64_t so = ((static_cast<int64_t>(bi) * Hsel + hs) * nq + r) * K;
        int slot = -1;
        for (int t0 = 0; t0 < K && slot < 0; t0 += 8) {
          int32_t iv[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) iv[t] = idx[so + (t0 + t < K ? t0 + t : 0)];
#pragma unroll
          for (int t = 7; t >= 0; --t)
            if (t0 + t < K && iv[t] == c) slot = t0 + t;
        }
        if (slot >= 0) lg = logg[so + slot];
      }
      sm.bias[x] = lg;
    }
    __syncthreads();

    // ---- row tiles of this pass
    const int ntile = (n + 31) / 32;
    uint16_t* tw = reinterpret_cast<uint16_t*>(sm.u.t[wave]);
    for (int rt = stride0; rt < ntile; rt += nstride) {
      const int e0 = rt * 32;
      // per-row scalars of this wave's head
      if (hl == 0) {
        const int e = e0 + ql;
        float4 rsv = make_float4(0.f, 0.f, -INFINITY, 0.f);
        if (e < n) {
          const int r = sm.rows[e];
          const int64_t qr = (static_cast<int64_t>(bi) * Hq + h) * nq + r;
          rsv.x = lse[qr] * kBLog2e;
          rsv.y = Dbuf[qr];
          rsv.z = (e < base && seg0 == 0) ? 0.f : sm.bias[e] * kBLog2e;
          // own-span rows are causal: store the row position, else "no limit"
          rsv.w = __int_as_float((e < base && seg0 == 0) ? static_cast<int>(q_pos0 + r) : 0x7FFFFFFF);
        }
        sm.rs[wave][ql] = rsv;
      }
      // A operands: rows pi(ql) of Q and dO (rows beyond the list are zero)
      const int ea = e0 + b_perm(ql);
      uint4 qa[kKS], da[kKS];
      if (ea < n) {
        const int64_t qr = (static_cast<int64_t>(bi) * Hq + h) * nq + sm.rows[ea];
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
          qa[ks] = *reinterpret_cast<const uint4*>(q + qr * D + 16 * ks + 8 * hl);
          da[ks] = *reinterpret_cast<const uint4*>(dout + qr * D + 16 * ks + 8 * hl);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
          qa[ks] = make_uint4(0, 0, 0, 0);
          da[ks] = make_uint4(0, 0, 0, 0);
        }
      }
      // S = Q K^T, dP = dO V^T (lane = key; register r = tile row b_tile_elem(r, hl))
      bfloatx16_t s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const uint4 kb = *reinterpret_cast<const uint4*>(krow_l + 16 * ks);
        const uint4 vb = *reinterpret_cast<const uint4*>(vrow_l + 16 * ks);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b_as_bf16x8(qa[ks]), b_as_bf16x8(kb), s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b_as_bf16x8(da[ks]), b_as_bf16x8(vb), dp, 0, 0, 0);
      }
      wave_lds_sync();
      float pr[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float4 rsv = sm.rs[wave][b_tile_elem(r, hl)];
        float z = fmaf(s[r], scale2, rsv.z - rsv.x);
        z = mykey > __float_as_int(rsv.w) ? -INFINITY : z;
        const float p = __builtin_amdgcn_exp2f(z);
        pr[r] = p;
        ds[r] = p * (dp[r] - rsv.y);
      }
      // dV += P^T dO: B = dO (lane: d = 32 db + ql, k-slice rows 16 s2 + 8 hl .. +7)
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        store_transposed8(tw + (16 * ks + 8 * hl) * DkvSmem<D>::kTPitch + b_perm(ql), DkvSmem<D>::kTPitch, da[ks]);
      wave_lds_sync();
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint4 pa = pack_bf16x8(&pr[8 * s2]);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const uint4 bt = *reinterpret_cast<const uint4*>(tw + (32 * db + ql) * DkvSmem<D>::kTPitch + 16 * s2 + 8 * hl);
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b_as_bf16x8(pa), b_as_bf16x8(bt), dva[db], 0, 0, 0);
        }
      }
      wave_lds_sync();
      // dK += dS^T Q
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        store_transposed8(tw + (16 * ks + 8 * hl) * DkvSmem<D>::kTPitch + b_perm(ql), DkvSmem<D>::kTPitch, qa[ks]);
      wave_lds_sync();
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint4 pa = pack_bf16x8(&ds[8 * s2]);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const uint4 bt = *reinterpret_cast<const uint4*>(tw + (32 * db + ql) * DkvSmem<D>::kTPitch + 16 * s2 + 8 * hl);
          dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b_as_bf16x8(pa), b_as_bf16x8(bt), dka[db], 0, 0, 0);
        }
      }
      wave_lds_sync();
    }
    if (seg0 + DkvSmem<D>::kSeg >= nq) break;
  }

  // ---- the four waves' sums, added in wave order; register r of block db
  // holds key 8 (r / 4) + 4 hl + (r % 4), column d = 32 db + ql
  __syncthreads();
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 8 * (r >> 2) + 4 * hl + (r & 3);
          const int d = 32 * db + ql;
          float* pk = &sm.u.red[0][key * D + d];
          float* pv = &sm.u.red[1][key * D + d];
          if (w == 0) {
            *pk = dka[db][r];
            *pv = dva[db][r];
          } else {
            *pk += dka[db][r];
            *pv += dva[db][r];
          }
        }
    }
    __syncthreads();
  }
  for (int x = tid; x < kBT * D / 4; x += 256) {
    const int key = x / (D / 4), d4 = (x % (D / 4)) * 4;
    if (key0 + key >= L) continue;
    const float4 a = *reinterpret_cast<const float4*>(&sm.u.red[0][key * D + d4]);
    const float4 bv = *reinterpret_cast<const float4*>(&sm.u.red[1][key * D + d4]);
    __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 wk, wv;
    wk[0] = static_cast<__bf16>(a.x * scale);
    wk[1] = static_cast<__bf16>(a.y * scale);
    wk[2] = static_cast<__bf16>(a.z * scale);
    wk[3] = static_cast<__bf16>(a.w * scale);
    wv[0] = static_cast<__bf16>(bv.x);
    wv[1] = static_cast<__bf16>(bv.y);
    wv[2] = static_cast<__bf16>(bv.z);
    wv[3] = static_cast<__bf16>(bv.w);
    const int64_t off = kvbase + static_cast<int64_t>(key0 + key) * D + d4;
    *reinterpret_cast<decltype(wk)*>(dk + off) = wk;
    *reinterpret_cast<decltype(wv)*>(dv + off) = wv;
  }
}

// ---------------------------------------------------------------- launch
bool attn_tile_bwd_supported(const BwdLaunch& p) {
  const AttnLaunch& a = p.a;
  const int G = a.Hq / a.Hkv;
  const bool groups_ok = (a.share_group && (G == 1 || G == 2 || G == 4)) || G == 1;
  return a.dtype == 1 && (a.d == 64 || a.d == 128) && (a.b == 32 || a.b == 64) && a.K <= kBMaxSelK &&
         (a.L + kBT - 1) / kBT <= kBMaxKeyTiles && groups_ok;
}

size_t attn_tile_bwd_bitmap_bytes(const BwdLaunch& p) {
  const AttnLaunch& a = p.a;
  const int64_t nblk = (a.L + a.b - 1) / a.b;
  const int64_t nw = (a.nq + 31) / 32;
  return align256(static_cast<size_t>(a.B) * a.Hsel * nblk * nw * sizeof(uint32_t));
}

template <int D>
static hipError_t launch_tile_bwd_d(const BwdLaunch& p, const float* Dbuf, uint32_t* bits, hipStream_t st) {
  const AttnLaunch& a = p.a;
  const int64_t nblk = (a.L + a.b - 1) / a.b;
  const int nw = (a.nq + 31) / 32;
  const int64_t heads = static_cast<int64_t>(a.B) * a.Hsel;
  // the readers of every block: the SAS candidate rule (blocks before the
  // row's own), every bitmap word written (no clearing pass)
  hipError_t e = launch_mark_rows(a.idx, a.nq, a.q_pos0, a.b, 0, 1, a.K, nblk, nw, heads, bits, st);
  if (e != hipSuccess) return e;
  const int G = a.Hq / a.Hkv;
  const int NH = G < 4 ? G : 4;
  const int NT = 4 / NH;
  const int ntiles = (a.nq + 31) / 32;
  e = launch(false, attn_tile_dq_kernel<D>, dim3((ntiles + NT - 1) / NT, static_cast<unsigned>(a.B * a.Hkv * (G / NH))),
             dim3(256), st, static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
             static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(p.dout), p.lse, Dbuf, a.idx, a.logg,
             a.Hq, a.Hkv, a.Hsel, a.share_group, a.nq, a.q_pos0, a.L, a.b, a.K, static_cast<__bf16*>(p.dq), p.dg,
             NH, NT);
  if (e != hipSuccess) return e;
  const int nkt = static_cast<int>((a.L + kBT - 1) / kBT);
  return launch(true, attn_tile_dkdv_kernel<D>, dim3(nkt, static_cast<unsigned>(a.B * a.Hkv)), dim3(256), st,
                static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v),
                static_cast<const __bf16*>(p.dout), p.lse, Dbuf, a.idx, a.logg, bits, a.Hq, a.Hkv, a.Hsel, a.nq,
                a.q_pos0, a.L, a.b, a.K, nblk, nw, static_cast<__bf16*>(p.dk), static_cast<__bf16*>(p.dv));
}

hipError_t launch_attn_tile_bwd(const BwdLaunch& p, const float* Dbuf, uint32_t* bits, hipStream_t st) {
  return p.a.d == 64 ? launch_tile_bwd_d<64>(p, Dbuf, bits, st) : launch_tile_bwd_d<128>(p, Dbuf, bits, st);
}

}  // namespace spa
