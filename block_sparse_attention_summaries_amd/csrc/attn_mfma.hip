// attn_mfma.hip -- MFMA (bf16, gfx950 v_mfma_f32_32x32x16_bf16) forward of
// the exact softmax attention over kept keys, for many query rows at once
// (prefill / training).  Same semantics as the per-row kernel in attn.hip:
//   branch L: current block (causal, bias 0) + selected units with their log
//             gate ("SAS" review §4.1 Eq. 4, §4.3 Eq. 9);
//   branch S: window i - w < j <= i, mixed o = alpha o_L + (1 - alpha) o_S
//             ("FreeSolo" review, "How it works").
//
// Work decomposition.  A workgroup of 4 waves covers 32-row query tiles of
// up to 4 query heads of one kv head (heads of a group share the K / V
// tiles).  It first builds, in LDS, the ascending list of 32-key tiles that
// any of its rows reads (current blocks, selected units, window band), then
// streams those tiles through LDS (double buffered): K row-major, V
// transposed.  Each wave computes S^T = K Q^T (keys x queries) so that one
// lane owns one query row: the softmax max / sum are in-lane plus one
// exchange between the two half-waves.  K rows are fed to the MFMA in a
// permuted order so that the probabilities a lane holds are exactly the
// B operand of O^T += V^T P^T for keys 16s + 8h .. +7 (h = half-wave), whose
// A operand is then one 16-byte read of the transposed V tile.  Per-row
// masks / biases come from a cursor walk over the row's ascending selection.
//
// Window mode with routed cells of 32 or 64 keys: branch L is computed
// cell-major instead (the cells a row tile's rows select are ~10x the 4 a row
// reads): the rows that selected each cell are listed, 32 at a time, and one
// wave per such unit writes each row's softmax partial over the cell; the
// tile kernel then walks the window band alone and merges a row's partials
// into o_L before the mix (kMode 2; see the routed-cells section below).
#include <type_traits>

#include "spa_device.h"
#include "spa_launch.h"

namespace spa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16_t;

constexpr int kKT = 32;               // keys per tile
constexpr int kMaxKeyTiles = 2048;    // key tiles per sequence (L <= 65536)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// key (within a 32-key tile) held in S^T register r by half-wave h: the
// MFMA A row m = 8a + 4h + c (r = 4a + c) is fed K row pi(m) with
// pi(8a + 4h + c) = 16 floor(a/2) + 8h + 4 (a mod 2) + c.
__device__ __forceinline__ int tile_key(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }
__device__ __forceinline__ int perm_row(int m) {
  const int a = m >> 3, h = (m >> 2) & 1, c = m & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + c;
}

template <int D>
struct TileSmem {
  static constexpr int kKPitch = D + 8;      // bf16 elements per K row in LDS
  static constexpr int kVPitch = kKT + 8;    // bf16 elements per V^T row in LDS
  __bf16 k[2][kKT * kKPitch];
  __bf16 vt[2][D * kVPitch];
};

// Selection data of one (wave) query tile: per row the ascending units and
// their log gates, read with a cursor as key tiles ascend.
constexpr int kMaxSelK = 32;
// Online softmax of the tile walk: largest exponent (log2) a probability may
// take above the reference max before the reference moves.
constexpr float kLazyMax = 8.0f;

// ------------------------------------------------- routed cells, cell-major
// Mix mode (routed cells + window) computes branch L per cell instead of per
// row tile: a row tile's union of selected cells is ~10x the 4 a row reads,
// while a cell's selecting rows fill whole 32-row tiles.  fwd_mark_kernel
// sets one bit per (selection head, cell, row) for "the row selected the
// cell"; the count and fill kernels turn the bitmap into units of 32
// selecting rows of one cell (row order); attn_cell_partial_kernel takes one
// unit per wave (attn_unit_partial_kernel one unit per workgroup, a wave per
// query head, when a group has four heads) and writes for each (row, slot of
// the cell in the row's selection) the softmax of the row over the cell's
// keys: o normalised (bf16) and (max, sum) in the log2 domain.  The tile kernel then runs the window
// branch only and merges a row's partials into o_L before the mix.

// One workgroup per (selection head, 256 rows = 8 bitmap words): the slice
// [cell][8 words] is built in LDS (atomics stay on chip) and written whole, so
// every word of the bitmap is written and no clearing pass is needed.
constexpr int kMarkWords = 8;
__global__ __launch_bounds__(256) void fwd_mark_kernel(const int32_t* __restrict__ idx, int nq, int64_t q_pos0, int b,
                                                       int prefix_mode, int qblock, int K, int64_t nblk, int nw,
                                                       uint32_t* __restrict__ bits) {
  __shared__ uint32_t s_w[kMaxKeyTiles * kMarkWords];   // nblk <= kMaxKeyTiles (cells of >= 32 keys)
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.y;
  const int w0 = blockIdx.x * kMarkWords;
  for (int x = tid; x < nblk * kMarkWords; x += 256) s_w[x] = 0u;
  __syncthreads();
  const int row = w0 * 32 + tid;
  if (row < nq) {
    const int64_t ncand = num_candidates(q_pos0 + row, b, prefix_mode, qblock);
    const int32_t* ir = idx + (bh * nq + row) * K;
    for (int t = 0; t < K; ++t) {
      const int32_t c = ir[t];
      if (c >= 0 && c < ncand && c < nblk) atomicOr(&s_w[c * kMarkWords + (tid >> 5)], 1u << (tid & 31));
    }
  }
  __syncthreads();
  for (int x = tid; x < nblk * kMarkWords; x += 256) {
    const int c = x / kMarkWords, j = x % kMarkWords;
    if (w0 + j < nw) bits[(bh * nblk + c) * nw + w0 + j] = s_w[x];
  }
}

// The bitmap of every (selection head, unit, row) for the candidate rule
// prefix_mode: the routed-cell pipeline here, and the backward's readers of a
// block (nblk <= kMaxKeyTiles).  Writes every word.
hipError_t launch_mark_rows(const int32_t* idx, int nq, int64_t q_pos0, int b, int prefix_mode, int qblock, int K,
                            int64_t nblk, int nw, int64_t heads, uint32_t* bits, hipStream_t st) {
  if (nblk > kMaxKeyTiles) return hipErrorInvalidValue;
  return launch(false, fwd_mark_kernel,
                dim3(static_cast<unsigned>((nw + kMarkWords - 1) / kMarkWords), static_cast<unsigned>(heads)),
                dim3(256), st, idx, nq, q_pos0, b, prefix_mode, qblock, K, nblk, nw, bits);
}

// Work units: a cell's selecting rows in tiles of 32 (row order), one unit
// per wave.  Each selection head has a region of `cap` unit slots (at most
// ncell + nq K / 32 units); its cells' units follow in cell order.
// cell_count_kernel: one wave per entry (head * ncell + cell) counts its rows;
// cell_fill_kernel: one wave per entry finds its first unit by summing the
// unit counts of the head's earlier cells, lists the rows, 32 per unit (the
// last unit padded with -1), writes the units' (entry, tile), and the head's
// last cell writes the head's unit count.
constexpr int kCellUnit = 32;
constexpr int kFillChunk = 8;                    // bitmap words per lane loaded together

__global__ __launch_bounds__(256) void cell_count_kernel(const uint32_t* __restrict__ bits, int64_t nblk, int nw,
                                                         int64_t ncell, int64_t heads, int32_t* __restrict__ cnt) {
  const int lane = threadIdx.x % kWave;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;   // head * ncell + cell
  if (e >= heads * ncell) return;                // whole wave leaves
  const int64_t bh = e / ncell, c = e % ncell;
  const uint32_t* brow = bits + (bh * nblk + c) * nw;
  int n = 0;
  for (int w = lane; w < nw; w += kWave) n += __popc(brow[w]);
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) n += __shfl_xor(n, o);
  if (lane == 0) cnt[e] = n;
}

__global__ __launch_bounds__(256) void cell_fill_kernel(const uint32_t* __restrict__ bits,
                                                        const int32_t* __restrict__ cnt, int64_t nblk, int nw,
                                                        int64_t ncell, int64_t nent, int64_t cap,
                                                        int2* __restrict__ units, int32_t* __restrict__ rows,
                                                        int32_t* __restrict__ nunits) {
  const int lane = threadIdx.x % kWave;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (e >= nent) return;                         // whole wave leaves
  const int64_t bh = e / ncell, c = e % ncell;
  const uint32_t* brow = bits + (bh * nblk + c) * nw;
  const int n = cnt[e];
  // units of the head's earlier cells
  int before = 0;
  for (int64_t x = lane; x < c; x += kWave) before += (cnt[bh * ncell + x] + kCellUnit - 1) / kCellUnit;
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) before += __shfl_xor(before, o);
  const int64_t u0 = bh * cap + before;
  const int m = (n + kCellUnit - 1) / kCellUnit;
  if (c == ncell - 1 && lane == 0) nunits[bh] = before + m;
  int32_t* rw = rows + static_cast<int64_t>(u0) * kCellUnit;
  for (int x = n + lane; x < m * kCellUnit; x += kWave) rw[x] = -1;
  for (int j = lane; j < m; j += kWave) units[u0 + j] = make_int2(static_cast<int>(e), j);
  // word w = x * 64 + lane: a run of consecutive rows spreads over the lanes
  int base = 0;
  for (int x0 = 0; x0 * kWave < nw; x0 += kFillChunk) {
    uint32_t wd[kFillChunk];
#pragma unroll
    for (int x = 0; x < kFillChunk; ++x) {
      const int w = (x0 + x) * kWave + lane;
      const uint32_t ld = brow[w < nw ? w : nw - 1];   // unconditional (clamped): the loads issue together
      wd[x] = w < nw ? ld : 0u;
    }
#pragma unroll
    for (int x = 0; x < kFillChunk; ++x) {
      const int pc = __popc(wd[x]);
      int incl = pc;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int up = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += up;
      }
      int rank = base + incl - pc;
      const int row0 = ((x0 + x) * kWave + lane) * 32;
      uint32_t mm = wd[x];
      while (mm != 0u) {
        rw[rank++] = row0 + __ffs(mm) - 1;
        mm &= mm - 1;
      }
      base += __shfl(incl, kWave - 1);
    }
  }
}

// One unit per wave (four independent waves per workgroup): 32 rows that
// selected one cell of NT key tiles.  The lane's K operand rows come straight
// from memory; V^T goes through the wave's own LDS slice.  For each query head
// of the group the rows' softmax over the cell's keys is written per
// (row, slot of the cell in the row's selection).
template <int D, int NT>
__global__ __launch_bounds__(256) void attn_cell_partial_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, const int2* __restrict__ units,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ nunits, int64_t cap, int64_t nheads, int64_t ncell,
    int Hq, int Hkv, int Hsel,
    int nq, int64_t L, int K, __bf16* __restrict__ cell_o, float2* __restrict__ cell_ml) {
  constexpr int kVPitch = kKT + 8;
  constexpr int kKS = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kLd = NT * kKT * (D / 8) / kWave;  // 16-byte vectors of V per lane
  constexpr int b = NT * kKT;                       // keys of a cell
  __shared__ __bf16 s_vt[4][NT][D * kVPitch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  const int64_t u = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (u >= nheads * cap || u % cap >= nunits[u / cap]) return;   // whole wave leaves; no workgroup barrier below
  const int2 unit = units[u];
  const int r0 = rows[u * kCellUnit + ql];       // -1 past the cell's last row
  const int64_t e = unit.x;
  const int64_t bkv = e / ncell;                 // Hsel == Hkv here: the selection head is the kv head
  const int c = static_cast<int>(e % ncell);
  const int bi = static_cast<int>(bkv / Hkv), kvh = static_cast<int>(bkv % Hkv);
  const int G = Hq / Hkv;                        // the group's query heads share the selection
  const int64_t kvbase = (static_cast<int64_t>(bi) * Hkv + kvh) * L * D;
  // loads issued together: the K operand (key perm_row(ql) of each tile) and the V rows
  uint4 ka[NT][kKS];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int64_t key = static_cast<int64_t>(c) * b + t * kKT + perm_row(ql);
    key = key < L ? key : L - 1;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) ka[t][ks] = *reinterpret_cast<const uint4*>(k + kvbase + key * D + 16 * ks + 8 * hl);
  }
  uint4 vv[kLd];
#pragma unroll
  for (int i = 0; i < kLd; ++i) {
    const int x = lane + kWave * i;
    int64_t key = static_cast<int64_t>(c) * b + x / (D / 8);
    key = key < L ? key : L - 1;
    vv[i] = *reinterpret_cast<const uint4*>(v + kvbase + key * D + (x % (D / 8)) * 8);
  }
  const bool ok = r0 >= 0;
  const int r = ok ? r0 : __shfl(r0, 0);         // a unit holds at least one row
  // the cell's slot (first match) and gate in the row's selection
  const int64_t so = ((static_cast<int64_t>(bi) * Hsel + kvh) * nq + r) * K;
  int slot = -1;
  float lg = 0.f;
#pragma unroll 4
  for (int t = 0; t < K; ++t) {
    const int32_t it = idx[so + t];
    const float lt = logg != nullptr ? logg[so + t] : 0.f;
    if (slot < 0 && it == c) {
      slot = t;
      lg = lt;
    }
  }
  slot = slot < 0 ? 0 : slot;                    // the bitmap marks only rows that selected the cell
  const float bias = lg * kLog2e;
  // V^T of the cell's key tiles into the wave's slice
#pragma unroll
  for (int i = 0; i < kLd; ++i) {
    const int x = lane + kWave * i;
    const int kr = x / (D / 8), cv = x % (D / 8);
    const uint4 vw = vv[i];
    uint16_t* vt = reinterpret_cast<uint16_t*>(s_vt[wave][kr / kKT]) + (cv * 8) * kVPitch + kr % kKT;
    vt[0 * kVPitch] = static_cast<uint16_t>(vw.x);
    vt[1 * kVPitch] = static_cast<uint16_t>(vw.x >> 16);
    vt[2 * kVPitch] = static_cast<uint16_t>(vw.y);
    vt[3 * kVPitch] = static_cast<uint16_t>(vw.y >> 16);
    vt[4 * kVPitch] = static_cast<uint16_t>(vw.z);
    vt[5 * kVPitch] = static_cast<uint16_t>(vw.z >> 16);
    vt[6 * kVPitch] = static_cast<uint16_t>(vw.w);
    vt[7 * kVPitch] = static_cast<uint16_t>(vw.w >> 16);
  }
  wave_lds_sync();
  const float scale2 = kLog2e / sqrtf(static_cast<float>(D));
  for (int g = 0; g < G; ++g) {
    const int h = kvh * G + g;
    uint4 qreg[kKS];
    const __bf16* qrow = q + ((static_cast<int64_t>(bi) * Hq + h) * nq + r) * D;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qreg[ks] = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hl);
    floatx16_t acc[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[db][x] = 0.f;
    float m2 = -INFINITY, lsum = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // S^T = K Q^T: this lane's row, keys tile_key(x, hl) of the tile
      floatx16_t st;
#pragma unroll
      for (int x = 0; x < 16; ++x) st[x] = 0.f;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[t][ks]), as_bf16x8(qreg[ks]), st, 0, 0, 0);
      float z[16];
      float mt = -INFINITY;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        z[x] = fmaf(st[x], scale2, bias);
        mt = fmaxf(mt, z[x]);
      }
      mt = fmaxf(mt, xor_lanes_f<32>(mt));
      const float mnew = fmaxf(m2, mt);
      const float msub = mnew == -INFINITY ? 0.f : mnew;
      const float corr = __builtin_amdgcn_exp2f(m2 - msub);
      float p[16], ps = 0.f;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        p[x] = __builtin_amdgcn_exp2f(z[x] - msub);
        ps += p[x];
      }
      ps += xor_lanes_f<32>(ps);
      lsum = lsum * corr + ps;
      m2 = mnew;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[db][x] *= corr;
      // O^T += V^T P^T
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8_t pb;
#pragma unroll
        for (int x = 0; x < 8; ++x) pb[x] = static_cast<__bf16>(p[8 * s2 + x]);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const uint4 a = *reinterpret_cast<const uint4*>(&s_vt[wave][t][(32 * db + ql) * kVPitch + 16 * s2 + 8 * hl]);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), pb, acc[db], 0, 0, 0);
        }
      }
    }
    if (ok) {
      const int64_t pr = ((static_cast<int64_t>(bi) * Hq + h) * nq + r) * K + slot;
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      // O^T register x of block db holds d = 32 db + 8 (x / 4) + 4 hl + (x % 4)
      __bf16* orow = cell_o + pr * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 w4;
#pragma unroll
          for (int x = 0; x < 4; ++x) w4[x] = static_cast<__bf16>(acc[db][4 * a4 + x] * inv);
          *reinterpret_cast<decltype(w4)*>(orow + 32 * db + 8 * a4 + 4 * hl) = w4;
        }
      if (hl == 0) cell_ml[pr] = make_float2(m2, lsum);
    }
  }
}

// One unit per workgroup when the group has four query heads: wave g takes
// head g of the group.  The unit's rows and their slots are looked up once
// and the cell's K rows and V^T staged once in LDS for the four waves
// (attn_cell_partial_kernel stages them per wave, for four units).  Per head
// the arithmetic is that of attn_cell_partial_kernel.
template <int D, int NT>
__global__ __launch_bounds__(256, 2) void attn_unit_partial_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, const int2* __restrict__ units,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ nunits, int64_t cap, int64_t nheads, int64_t ncell,
    int Hq, int Hkv, int Hsel, int nq, int64_t L, int K, __bf16* __restrict__ cell_o, float2* __restrict__ cell_ml) {
  constexpr int kKPitch = D + 8;                    // K rows (bf16)
  constexpr int kVPitch = kKT + 8;                  // V^T rows: the keys of one tile
  constexpr int kKS = D / 16;
  constexpr int kDB = D / 32;
  constexpr int b = NT * kKT;                       // keys of a cell
  __shared__ __align__(16) __bf16 s_k[b * kKPitch];
  __shared__ __align__(16) __bf16 s_vt[NT][D * kVPitch];
  __shared__ int s_row[32];
  __shared__ int s_slot[32];
  __shared__ float s_bias[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  const int64_t u = blockIdx.x;
  if (u >= nheads * cap || u % cap >= nunits[u / cap]) return;   // the whole workgroup leaves
  const int2 unit = units[u];
  const int64_t e = unit.x;
  const int64_t bkv = e / ncell;                 // Hsel == Hkv: the selection head is the kv head
  const int c = static_cast<int>(e % ncell);
  const int bi = static_cast<int>(bkv / Hkv), kvh = static_cast<int>(bkv % Hkv);
  const int G = Hq / Hkv;
  const int64_t kvbase = (static_cast<int64_t>(bi) * Hkv + kvh) * L * D;
  // the cell's K rows and V^T (V staged transposed, one tile of keys per slice)
  for (int x = tid; x < b * (D / 8); x += 256) {
    const int kr = x / (D / 8), cv = x % (D / 8);
    int64_t key = static_cast<int64_t>(c) * b + kr;
    key = key < L ? key : L - 1;
    *reinterpret_cast<uint4*>(&s_k[kr * kKPitch + cv * 8]) =
        *reinterpret_cast<const uint4*>(k + kvbase + key * D + cv * 8);
    const uint4 vw = *reinterpret_cast<const uint4*>(v + kvbase + key * D + cv * 8);
    uint16_t* vt = reinterpret_cast<uint16_t*>(s_vt[kr / kKT]) + (cv * 8) * kVPitch + kr % kKT;
    vt[0 * kVPitch] = static_cast<uint16_t>(vw.x);
    vt[1 * kVPitch] = static_cast<uint16_t>(vw.x >> 16);
    vt[2 * kVPitch] = static_cast<uint16_t>(vw.y);
    vt[3 * kVPitch] = static_cast<uint16_t>(vw.y >> 16);
    vt[4 * kVPitch] = static_cast<uint16_t>(vw.z);
    vt[5 * kVPitch] = static_cast<uint16_t>(vw.z >> 16);
    vt[6 * kVPitch] = static_cast<uint16_t>(vw.w);
    vt[7 * kVPitch] = static_cast<uint16_t>(vw.w >> 16);
  }
  // the unit's rows, the cell's slot (first match) and gate in each row's selection
  if (tid < 32) {
    const int r0 = rows[u * kCellUnit + tid];    // -1 past the cell's last row
    const int rfirst = rows[u * kCellUnit];      // a unit holds at least one row
    const int r = r0 >= 0 ? r0 : rfirst;
    const int64_t so = ((static_cast<int64_t>(bi) * Hsel + kvh) * nq + r) * K;
    int slot = -1;
    float lg = 0.f;
    for (int t = 0; t < K; ++t) {
      const int32_t it = idx[so + t];
      const float lt = logg != nullptr ? logg[so + t] : 0.f;
      if (slot < 0 && it == c) {
        slot = t;
        lg = lt;
      }
    }
    s_row[tid] = r0 >= 0 ? r : -1 - r;           // -1 - r: a padding lane reads row r, writes nothing
    s_slot[tid] = slot < 0 ? 0 : slot;
    s_bias[tid] = lg * kLog2e;
  }
  __syncthreads();
  const int rs = s_row[ql];
  const bool ok = rs >= 0;
  const int r = ok ? rs : -1 - rs;
  const int slot = s_slot[ql];
  const float bias = s_bias[ql];
  const float scale2 = kLog2e / sqrtf(static_cast<float>(D));
  const int h = kvh * G + wave;
  uint4 qreg[kKS];
  const __bf16* qrow = q + ((static_cast<int64_t>(bi) * Hq + h) * nq + r) * D;
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) qreg[ks] = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hl);
  floatx16_t acc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[db][x] = 0.f;
  float m2 = -INFINITY, lsum = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    // S^T = K Q^T: this lane's row, keys tile_key(x, hl) of the tile
    floatx16_t st;
#pragma unroll
    for (int x = 0; x < 16; ++x) st[x] = 0.f;
    const __bf16* krow = &s_k[(t * kKT + perm_row(ql)) * kKPitch + 8 * hl];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(krow + 16 * ks)),
                                                   as_bf16x8(qreg[ks]), st, 0, 0, 0);
    float z[16];
    float mt = -INFINITY;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      z[x] = fmaf(st[x], scale2, bias);
      mt = fmaxf(mt, z[x]);
    }
    mt = fmaxf(mt, xor_lanes_f<32>(mt));
    const float mnew = fmaxf(m2, mt);
    const float msub = mnew == -INFINITY ? 0.f : mnew;
    const float corr = __builtin_amdgcn_exp2f(m2 - msub);
    float p[16], ps = 0.f;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      p[x] = __builtin_amdgcn_exp2f(z[x] - msub);
      ps += p[x];
    }
    ps += xor_lanes_f<32>(ps);
    lsum = lsum * corr + ps;
    m2 = mnew;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[db][x] *= corr;
    // O^T += V^T P^T
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8_t pb;
#pragma unroll
      for (int x = 0; x < 8; ++x) pb[x] = static_cast<__bf16>(p[8 * s2 + x]);
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const uint4 a = *reinterpret_cast<const uint4*>(&s_vt[t][(32 * db + ql) * kVPitch + 16 * s2 + 8 * hl]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), pb, acc[db], 0, 0, 0);
      }
    }
  }
  if (ok) {
    const int64_t pr = ((static_cast<int64_t>(bi) * Hq + h) * nq + r) * K + slot;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    // O^T register x of block db holds d = 32 db + 8 (x / 4) + 4 hl + (x % 4)
    __bf16* orow = cell_o + pr * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 w4;
#pragma unroll
        for (int x = 0; x < 4; ++x) w4[x] = static_cast<__bf16>(acc[db][4 * a4 + x] * inv);
        *reinterpret_cast<decltype(w4)*>(orow + 32 * db + 8 * a4 + 4 * hl) = w4;
      }
    if (hl == 0) cell_ml[pr] = make_float2(m2, lsum);
  }
}

// kMode 0: selected blocks (SAS); 1: routed cells walked per row tile + window;
// 2: window walk only, branch L merged from attn_cell_partial_kernel's
// per-(row, slot) partials (cell_o / cell_ml); 3: SAS with the selected
// blocks computed block-major (the same partials): the walk covers the rows'
// current blocks only, and the row's partials join its softmax.
template <int D, int kMode, int NW>
__global__ __launch_bounds__(256, 2) void attn_tile_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ logg, const float* __restrict__ alpha,
    int Hq, int Hkv, int Hsel, int share_group, int nq, int64_t q_pos0, int64_t L, int b,
    int prefix_mode, int qblock, int K, int local, int window, __bf16* __restrict__ o,
    float* __restrict__ lse, int NH, int NT, const __bf16* __restrict__ cell_o,
    const float2* __restrict__ cell_ml) {
  constexpr bool kMix = kMode == 1 || kMode == 2;
  constexpr bool kCells = kMode == 2;
  constexpr bool kSasCells = kMode == 3;
  constexpr bool kUnitsApart = kCells || kSasCells;     // selected units come as partials
  __shared__ TileSmem<D> sm;
  __shared__ uint32_t s_bits[2][kMaxKeyTiles / 32];
  __shared__ uint16_t s_list[2][kMaxKeyTiles];
  __shared__ int s_count[2];
  // per wave (NW of them: with two, a workgroup fits four times in LDS)
  __shared__ int32_t s_idx[NW][32][kMaxSelK / 2 + 1];   // packed pairs of int16 units
  __shared__ float s_lg[NW][32][kMaxSelK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;              // half-wave, query lane
  const int G = Hq / Hkv;
  const int hgroups = G / NH;
  // XCD-aware order (a head's consecutive row tiles on one XCD share its L2):
  // the selected-block mode, where every tile of a head reads from the same
  // keys, and the window walk with the cells apart, where consecutive tiles'
  // windows overlap; the per-tile cell walk keeps the dispatch order
  // (measured faster there).  The selected-block walk's tiles grow with the
  // row (the union of the rows' selections), so it takes them last first.
  const uint2 bxy = kMode == 1 ? make_uint2(blockIdx.x, blockIdx.y)
                               : (kMode == 0 ? xcd_block_xy_last_first() : xcd_block_xy());
  const int bz = static_cast<int>(bxy.y);
  const int bi = bz / (Hkv * hgroups);
  const int kvh = (bz / hgroups) % Hkv;
  const int hg = bz % hgroups;
  const int h = kvh * G + hg * NH + (wave % NH);          // this wave's query head
  const int hs = share_group ? kvh : h;
  const int tile = static_cast<int>(bxy.x) * NT + wave / NH;   // this wave's 32-row tile
  const int row = tile * 32 + ql;
  const bool row_ok = row < nq;
  const int rowc = row_ok ? row : nq - 1;
  const int64_t pos = q_pos0 + rowc;
  const int64_t ncand = num_candidates(pos, b, prefix_mode, qblock);
  const int nkt = static_cast<int>((L + kKT - 1) / kKT);
  const int nwords = (nkt + 31) / 32;
  constexpr bool mix = kMix;

  // ---- per-row selection tables (this wave's rows), unit = -1 when unused
  const int64_t so = ((static_cast<int64_t>(bi) * Hsel + hs) * nq + rowc) * K;
  for (int t = hl; t < K; t += 2) {
    const int32_t c = idx[so + t];
    const bool ok = row_ok && c >= 0 && c < ncand;
    reinterpret_cast<int16_t*>(s_idx[wave][ql])[t] = static_cast<int16_t>(ok ? c : -1);
    s_lg[wave][ql][t] = (ok && logg != nullptr) ? logg[so + t] : 0.f;
  }
  // ---- key-tile lists: list 0 = branch L, list 1 = window branch
  constexpr int kThreads = 64 * NW;      // NW waves of 64
  for (int x = tid; x < 2 * (kMaxKeyTiles / 32); x += kThreads) (&s_bits[0][0])[x] = 0u;
  __syncthreads();
  // row range of the workgroup (positions)
  const int64_t wg_row0 = static_cast<int64_t>(bxy.x) * NT * 32;
  const int64_t wg_row1 = (wg_row0 + NT * 32 < nq ? wg_row0 + NT * 32 : nq) - 1;
  const int64_t p0 = q_pos0 + wg_row0, p1 = q_pos0 + wg_row1;
  if (local == 0) {
    // current blocks of the rows: keys [floor(p0/b) b, p1]
    const int64_t k0 = (p0 / b) * b;
    for (int64_t t = k0 / kKT + tid; t <= p1 / kKT; t += kThreads)
      atomicOr(&s_bits[0][t >> 5], 1u << (t & 31));
  }
  if (mix) {
    const int64_t k0 = p0 - window + 1 > 0 ? p0 - window + 1 : 0;
    for (int64_t t = k0 / kKT + tid; t <= p1 / kKT; t += kThreads)
      atomicOr(&s_bits[1][t >> 5], 1u << (t & 31));
  }
  for (int t = hl; t < K && !kUnitsApart; t += 2) {
    const int c = reinterpret_cast<int16_t*>(s_idx[wave][ql])[t];
    if (c >= 0) {
      const int64_t a0 = static_cast<int64_t>(c) * b, a1 = a0 + b - 1;
      for (int64_t kt = a0 / kKT; kt <= a1 / kKT; ++kt) atomicOr(&s_bits[0][kt >> 5], 1u << (kt & 31));
    }
  }
  __syncthreads();
  // compaction into ascending lists (wave 0: list 0, wave 1: list 1)
  // list li is built by wave li (NW >= 2), or both by wave 0 (NW == 1)
  for (int li = wave; li < 2; li += NW) {
    int base = 0;
    for (int w0 = 0; w0 < nwords; w0 += 64) {
      const int wi = w0 + lane;
      const uint32_t bits = wi < nwords ? s_bits[li][wi] : 0u;
      const int cnt = __popc(bits);
      // inclusive scan of cnt over the wave
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
        s_list[li][wpos++] = static_cast<uint16_t>(wi * 32 + bit);
      }
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) s_count[li] = base;
  }
  __syncthreads();

  // ---- Q^T operand (B of S^T = K Q^T): lane holds Q[row][16 ks + 8 hl .. +8]
  constexpr int kKS = D / 16;
  uint4 qreg[kKS];
  const __bf16* qrow = q + ((static_cast<int64_t>(bi) * Hq + h) * nq + rowc) * D;
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) qreg[ks] = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hl);

  const float scale2 = kLog2e / sqrtf(static_cast<float>(D));
  const int64_t kvbase = (static_cast<int64_t>(bi) * Hkv + kvh) * L * D;
  constexpr int kDB = D / 32;
  float out[kMix ? kDB * 16 : 1];
  float lse_L = -INFINITY;

  for (int branch = kCells ? 1 : 0; branch < (mix ? 2 : 1); ++branch) {
    const int ntl = s_count[branch];
    const uint16_t* list = s_list[branch];
    floatx16_t acc[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float m2 = -INFINITY, lsum = 0.f;     // running max (log2 domain), sum
    int cur = 0;                           // cursor into this row's units, whose
    int nu;                                // unit (past the end: INT_MAX) and
    float nlg;                             // log2 gate are kept in registers
    {
      const int16_t* urow = reinterpret_cast<const int16_t*>(s_idx[wave][ql]);
      nu = K > 0 ? urow[0] : 0x7FFFFFFF;
      nlg = K > 0 ? s_lg[wave][ql][0] * kLog2e : 0.f;
    }
    const int pos32 = static_cast<int>(pos);
    const int lb = __builtin_ctz(b);       // b is a power of two
    const int c_cur = pos32 >> lb;         // current unit of the row
    const int c_end = (c_cur + 1) * b;     // first key after it

    // staging: 2 x 16 B of K and of V per thread per tile (D = 128), 1 (D = 64).
    // Loads run kP - 1 tiles ahead of the tile being computed, in a ring of kP
    // register slots (the loop is unrolled kP times so every slot index is a
    // constant); LDS holds two tiles (computed / being staged).
    constexpr int kLd = kKT * D / 8 / kThreads;
    constexpr int kP = kLd == 1 ? 4 : 2;   // ring depth within the register budget
    // ring slots s = 0..3: K vectors s##k0, s##k1 and V vectors s##v0, s##v1
    uint4 sl0k0, sl0k1, sl0v0, sl0v1, sl1k0, sl1k1, sl1v0, sl1v1;
    uint4 sl2k0, sl2k1, sl2v0, sl2v1, sl3k0, sl3k1, sl3v0, sl3v1;
    static_assert(kLd == 1 || kLd == 2, "one or two 16-byte vectors per thread per tile");
    // vector i of a tile: thread tid moves key row (tid + kThreads i) / (D / 8), column group tid % (D / 8)
    // K: thread x takes key row x / (D / 8), columns 8 (x % (D / 8)) .. +7 (rows
    // contiguous in LDS).  V: key x % 32, columns 8 (x / 32) .. +7, so that each
    // transposed 2-byte LDS write of a wave covers 32 consecutive keys of a
    // V^T row and the other half-wave lands 8 rows (a half bank cycle) away.
#define SPA_ISSUE_ONE(R, IT, I)                                                               \
  do {                                                                                       \
    const int x = tid + (I) * kThreads;                                                      \
    const int64_t kb0 = static_cast<int64_t>(list[IT]) * kKT;                                \
    int64_t key = kb0 + x / (D / 8), vkey = kb0 + x % kKT;                                   \
    key = key < L ? key : L - 1;                                                             \
    vkey = vkey < L ? vkey : L - 1;                                                          \
    R##k##I = *reinterpret_cast<const uint4*>(k + kvbase + key * D + (x % (D / 8)) * 8);      \
    R##v##I = *reinterpret_cast<const uint4*>(v + kvbase + vkey * D + (x / kKT) * 8);         \
  } while (0)
#define SPA_ISSUE(R, IT)                                                                     \
  do {                                                                                       \
    SPA_ISSUE_ONE(R, IT, 0);                                                                 \
    if constexpr (kLd == 2) SPA_ISSUE_ONE(R, IT, 1);                                         \
  } while (0)
#define SPA_STAGE_ONE(R, BUF, I)                                                             \
  do {                                                                                       \
    const int x = tid + (I) * kThreads;                                                      \
    const int kr = x / (D / 8), cv = x % (D / 8);                                            \
    *reinterpret_cast<uint4*>(&sm.k[BUF][kr * TileSmem<D>::kKPitch + cv * 8]) = R##k##I;     \
    const uint4 vw = R##v##I;                                                                 \
    uint16_t* vt = reinterpret_cast<uint16_t*>(sm.vt[BUF]) + (x / kKT) * 8 * TileSmem<D>::kVPitch + x % kKT; \
    vt[0 * TileSmem<D>::kVPitch] = static_cast<uint16_t>(vw.x);                              \
    vt[1 * TileSmem<D>::kVPitch] = static_cast<uint16_t>(vw.x >> 16);                        \
    vt[2 * TileSmem<D>::kVPitch] = static_cast<uint16_t>(vw.y);                              \
    vt[3 * TileSmem<D>::kVPitch] = static_cast<uint16_t>(vw.y >> 16);                        \
    vt[4 * TileSmem<D>::kVPitch] = static_cast<uint16_t>(vw.z);                              \
    vt[5 * TileSmem<D>::kVPitch] = static_cast<uint16_t>(vw.z >> 16);                        \
    vt[6 * TileSmem<D>::kVPitch] = static_cast<uint16_t>(vw.w);                              \
    vt[7 * TileSmem<D>::kVPitch] = static_cast<uint16_t>(vw.w >> 16);                        \
  } while (0)
#define SPA_STAGE(R, BUF)                                                                    \
  do {                                                                                       \
    SPA_STAGE_ONE(R, BUF, 0);                                                                \
    if constexpr (kLd == 2) SPA_STAGE_ONE(R, BUF, 1);                                        \
  } while (0)
    if (ntl > 0) SPA_ISSUE(sl0, 0);
    if constexpr (kP == 4) {
      if (ntl > 1) SPA_ISSUE(sl1, 1);
      if (ntl > 2) SPA_ISSUE(sl2, 2);
    }
    if (ntl > 0) SPA_STAGE(sl0, 0);
    __syncthreads();
    // one tile of the ring: tile it0 + u lives in slot u; the step issues the
    // loads of tile it0 + u + kP - 1 into slot ri and stages slot rn (tile it0 + u + 1)
    int it0 = 0;
    int ks0n = ntl > 0 ? static_cast<int>(list[0]) * kKT : 0;
#define SPA_TILE_STEP(u, ri, rn)\
  do {                                                                                                   \
      const int it = it0 + u;                                                                            \
      if (it < ntl) {                                                                                    \
      const int buf = u & 1;               /* it0 is a multiple of kP (even) */                          \
      if (it + kP - 1 < ntl) SPA_ISSUE(ri, it + kP - 1);                                                 \
      const int ks0 = ks0n;   /* list entry read one tile ahead */                                       \
      if (it + 1 < ntl) ks0n = static_cast<int>(list[it + 1]) * kKT;                                     \
      /* Which of this wave's rows read the tile, with what bias (log2 domain). */                       \
      /* A tile that none of them reads is skipped (the workgroup's list is the */                       \
      /* union over all its waves). */                                                                   \
      float bias_lo = 0.f, bias_hi = 0.f;                                                                \
      bool need, masked = false;                                                                         \
      if (branch == 0) {                                                                                 \
        const int u_lo = (ks0 + 8 * hl) >> lb, u_hi = (ks0 + 16 + 8 * hl) >> lb;                         \
        const int16_t* ur = reinterpret_cast<const int16_t*>(s_idx[wave][ql]);                           \
        const int uu[2] = {u_lo, u_hi};                                                                  \
        float bb[2];                                                                                     \
_Pragma("unroll")                                                                                        \
        for (int part = 0; part < 2; ++part) {                                                           \
          const int uv = uu[part];                                                                       \
          float bv = -INFINITY;                                                                          \
          if (local == 0 && uv == c_cur) {                                                               \
            bv = 0.f;   /* causal mask applied per key below */                                          \
          } else if (kSasCells) {                                                                        \
            /* another row's current block: this row's selected blocks come as partials */              \
          } else {                                                                                       \
            while (nu < uv) {   /* advance past smaller units (unused slots hold -1) */                  \
              ++cur; nu = cur < K ? ur[cur] : 0x7FFFFFFF; nlg = cur < K ? s_lg[wave][ql][cur] * kLog2e : 0.f; }\
            if (nu == uv) bv = nlg;                                                                            \
          }                                                                                              \
          bb[part] = bv;                                                                                 \
        }                                                                                                \
        bias_lo = row_ok ? bb[0] : -INFINITY;                                                            \
        bias_hi = row_ok ? bb[1] : -INFINITY;                                                            \
        need = bias_lo != -INFINITY || bias_hi != -INFINITY;                                             \
        masked = local == 0 && (u_lo == c_cur || u_hi == c_cur) && ks0 + kKT - 1 > pos32;                \
      } else {                                                                                           \
        need = row_ok && ks0 <= pos32 && ks0 + kKT - 1 > pos32 - window;                                 \
        masked = !(ks0 + kKT - 1 <= pos32 && ks0 > pos32 - window);                                      \
        bias_lo = bias_hi = row_ok ? 0.f : -INFINITY;                                                    \
      }                                                                                                  \
      if (__ballot(need) != 0) {                                                                         \
        /* S^T = K Q^T for this wave's 32 rows */                                                        \
        floatx16_t st;                                                                                   \
_Pragma("unroll")                                                                                        \
        for (int r = 0; r < 16; ++r) st[r] = 0.f;                                                        \
        const __bf16* krow = &sm.k[buf][perm_row(ql) * TileSmem<D>::kKPitch];                            \
_Pragma("unroll")                                                                                        \
        for (int ks = 0; ks < kKS; ++ks) {                                                               \
          const uint4 a = *reinterpret_cast<const uint4*>(krow + 16 * ks + 8 * hl);                      \
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qreg[ks]), st, 0, 0, 0);  \
        }                                                                                                \
        float z[16];                                                                                     \
_Pragma("unroll")                                                                                        \
        for (int r = 0; r < 16; ++r) z[r] = fmaf(st[r], scale2, r < 8 ? bias_lo : bias_hi);              \
        if (__ballot(masked) != 0) {                                                                     \
          /* branch L: keys of the current unit after the row; branch S: keys */                         \
          /* outside (pos - window, pos] */                                                              \
          if (branch == 0) {                                                                             \
_Pragma("unroll")                                                                                        \
            for (int r = 0; r < 16; ++r) {                                                               \
              const int key = ks0 + tile_key(r, hl);                                                     \
              z[r] = (key > pos32 && key < c_end) ? -INFINITY : z[r];                                    \
            }                                                                                            \
          } else {                                                                                       \
            const int wlo = pos32 - window + 1;                                                          \
_Pragma("unroll")                                                                                        \
            for (int r = 0; r < 16; ++r) {                                                               \
              const int key = ks0 + tile_key(r, hl);                                                     \
              z[r] = (key > pos32 || key < wlo) ? -INFINITY : z[r];                                      \
            }                                                                                            \
          }                                                                                              \
        }                                                                                                \
        /* online softmax for this lane's row (two half-waves hold its 32 keys) */                       \
        float mt = z[0];                                                                                 \
_Pragma("unroll")                                                                                        \
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, z[r]);                                               \
        mt = fmaxf(mt, xor_lanes_f<32>(mt));                                                             \
        /* the reference max moves only when the tile's max passes it by more */                       \
        /* than kLazyMax (log2 domain): p <= 2^kLazyMax, and most tiles skip */                          \
        /* the accumulator rescale (corr = 1) */                                                         \
        const float mnew = mt > m2 + kLazyMax ? mt : m2;                                                 \
        /* hardware exp2 (exp2(-inf) = 0); a row with no key yet keeps zeros */                          \
        const float msub = mnew == -INFINITY ? 0.f : mnew;                                               \
        const float corr = __builtin_amdgcn_exp2f(m2 - msub);                                            \
        float p[16], ps = 0.f;                                                                           \
_Pragma("unroll")                                                                                        \
        for (int r = 0; r < 16; ++r) {                                                                   \
          p[r] = __builtin_amdgcn_exp2f(z[r] - msub);                                                    \
          ps += p[r];                                                                                    \
        }                                                                                                \
        ps += xor_lanes_f<32>(ps);                                                                       \
        lsum = lsum * corr + ps;                                                                         \
        m2 = mnew;                                                                                       \
        if (__ballot(corr != 1.f) != 0) {                                                                \
_Pragma("unroll")                                                                                        \
          for (int db = 0; db < kDB; ++db)                                                               \
_Pragma("unroll")                                                                                        \
            for (int r = 0; r < 16; ++r) acc[db][r] *= corr;                                             \
        }                                                                                                \
        /* O^T += V^T P^T: B = P^T (keys 16s + 8hl + t of this lane's row) */                            \
_Pragma("unroll")                                                                                        \
        for (int s2 = 0; s2 < 2; ++s2) {                                                                 \
          bf16x8_t pb;                                                                                   \
_Pragma("unroll")                                                                                        \
          for (int t = 0; t < 8; ++t) pb[t] = static_cast<__bf16>(p[8 * s2 + t]);                        \
_Pragma("unroll")                                                                                        \
          for (int db = 0; db < kDB; ++db) {                                                             \
            const uint4 a = *reinterpret_cast<const uint4*>(                                             \
                &sm.vt[buf][(32 * db + ql) * TileSmem<D>::kVPitch + 16 * s2 + 8 * hl]);                  \
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), pb, acc[db], 0, 0, 0);       \
          }                                                                                              \
        }                                                                                                \
      }                                                                                                  \
      /* next tile into the other buffer (last read two iterations ago); the */                          \
      /* barrier orders LDS only, so later tiles' loads stay in flight */                                \
      if (it + 1 < ntl) SPA_STAGE(rn, buf ^ 1);                                                          \
      lds_barrier();                                                                                     \
      }                                                                                                  \
  } while (0)
    for (it0 = 0; it0 < ntl; it0 += kP) {
      if constexpr (kP == 4) {
        SPA_TILE_STEP(0, sl3, sl1);
        SPA_TILE_STEP(1, sl0, sl2);
        SPA_TILE_STEP(2, sl1, sl3);
        SPA_TILE_STEP(3, sl2, sl0);
      } else {
        SPA_TILE_STEP(0, sl1, sl1);
        SPA_TILE_STEP(1, sl0, sl0);
      }
    }
#undef SPA_TILE_STEP
#undef SPA_ISSUE
#undef SPA_ISSUE_ONE
#undef SPA_STAGE
#undef SPA_STAGE_ONE
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    if (branch == 0) lse_L = lsum > 0.f ? (m2 + __log2f(lsum)) / kLog2e : -INFINITY;
    if constexpr (kCells) {
      // o = alpha o_L + (1 - alpha) o_S, o_L from the row's cell partials (each
      // selected cell once: the first slot holding it)
      const int16_t* ur = reinterpret_cast<const int16_t*>(s_idx[wave][ql]);
      const int64_t pr0 = ((static_cast<int64_t>(bi) * Hq + h) * nq + rowc) * K;
      float M = -INFINITY;
      for (int t = 0; t < K; ++t) {
        const int ct = ur[t];
        bool first = ct >= 0;
        for (int u = 0; u < t; ++u) first = first && ur[u] != ct;
        if (first) M = fmaxf(M, cell_ml[pr0 + t].x);
      }
      const float msub = M == -INFINITY ? 0.f : M;
      float ol[kDB * 16];
#pragma unroll
      for (int x = 0; x < kDB * 16; ++x) ol[x] = 0.f;
      float wsum = 0.f;
      for (int t = 0; t < K; ++t) {
        const int ct = ur[t];
        bool first = ct >= 0;
        for (int u = 0; u < t; ++u) first = first && ur[u] != ct;
        if (!first) continue;
        const float2 ml = cell_ml[pr0 + t];
        const float wt = ml.y * __builtin_amdgcn_exp2f(ml.x - msub);
        wsum += wt;
        const __bf16* orow = cell_o + (pr0 + t) * D;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const auto w4 = *reinterpret_cast<const __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16*>(
                orow + 32 * db + 8 * a4 + 4 * hl);
#pragma unroll
            for (int x = 0; x < 4; ++x) ol[db * 16 + 4 * a4 + x] = fmaf(wt, static_cast<float>(w4[x]), ol[db * 16 + 4 * a4 + x]);
          }
      }
      const float winv = wsum > 0.f ? 1.f / wsum : 0.f;
      lse_L = wsum > 0.f ? (M + __log2f(wsum)) / kLog2e : -INFINITY;
      const float a = alpha[h];
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = a * (ol[db * 16 + r] * winv) + (1.f - a) * (acc[db][r] * inv);
    } else if constexpr (kSasCells) {
      // one softmax over the current block (this walk: acc and lsum relative
      // to m2) and the row's selected blocks (partials: o normalised, (max,
      // sum) in the log2 domain), each selected block once (its first slot)
      const int16_t* ur = reinterpret_cast<const int16_t*>(s_idx[wave][ql]);
      const int64_t pr0 = ((static_cast<int64_t>(bi) * Hq + h) * nq + rowc) * K;
      float M = m2;
      for (int t = 0; t < K; ++t) {
        const int ct = ur[t];
        bool first = ct >= 0;
        for (int u = 0; u < t; ++u) first = first && ur[u] != ct;
        if (first) M = fmaxf(M, cell_ml[pr0 + t].x);
      }
      const float msub = M == -INFINITY ? 0.f : M;
      const float cw = __builtin_amdgcn_exp2f(m2 - msub);
      float den = lsum * cw;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= cw;
      for (int t = 0; t < K; ++t) {
        const int ct = ur[t];
        bool first = ct >= 0;
        for (int u = 0; u < t; ++u) first = first && ur[u] != ct;
        if (!first) continue;
        const float2 ml = cell_ml[pr0 + t];
        const float wt = ml.y * __builtin_amdgcn_exp2f(ml.x - msub);
        den += wt;
        const __bf16* orow = cell_o + (pr0 + t) * D;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const auto w4 = *reinterpret_cast<const __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16*>(
                orow + 32 * db + 8 * a4 + 4 * hl);
#pragma unroll
            for (int x = 0; x < 4; ++x) acc[db][4 * a4 + x] = fmaf(wt, static_cast<float>(w4[x]), acc[db][4 * a4 + x]);
          }
      }
      const float dinv = den > 0.f ? 1.f / den : 0.f;
      lse_L = den > 0.f ? (M + __log2f(den)) / kLog2e : -INFINITY;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= dinv;
    } else if constexpr (kMix) {
      if (branch == 0) {
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) out[db * 16 + r] = acc[db][r] * inv;
      } else {
        const float a = alpha[h];
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] = a * out[db * 16 + r] + (1.f - a) * (acc[db][r] * inv);
      }
    } else {
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= inv;
    }
    if (branch + 1 == (mix ? 2 : 1) && row_ok) {
      // O^T register r of block db holds d = 32 db + 8 (r / 4) + 4 hl + (r % 4)
      __bf16* orow = o + ((static_cast<int64_t>(bi) * Hq + h) * nq + row) * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 w4;
#pragma unroll
          for (int c = 0; c < 4; ++c) w4[c] = static_cast<__bf16>(acc[db][4 * a4 + c]);
          *reinterpret_cast<decltype(w4)*>(orow + 32 * db + 8 * a4 + 4 * hl) = w4;
        }
    }
  }
  if (!row_ok) return;
  if (lse != nullptr && hl == 0) lse[(static_cast<int64_t>(bi) * Hq + h) * nq + row] = lse_L;
}

bool attn_tile_fwd_supported(const AttnLaunch& p) {
  return p.dtype == 1 && p.nq > 1 && p.K <= kMaxSelK && p.b >= 16 &&
         (p.L + kKT - 1) / kKT <= kMaxKeyTiles && (p.d == 64 || p.d == 128);
}

// The cell-major branch L: mix mode, cells of one or two key tiles, a
// selection shared by the kv head's query heads (or one query head per kv
// head), and partials (K per row and query head) of at most 16 GiB; otherwise
// the tile kernel walks each row tile's cells itself.
constexpr size_t kMaxCellPartialBytes = static_cast<size_t>(16) << 30;
static bool cell_partials_fit(const AttnLaunch& p) {
  const int G = p.Hq / p.Hkv;
  const size_t parts = static_cast<size_t>(p.B) * p.Hq * p.nq * p.K;
  return (p.b == 32 || p.b == 64) && G <= 4 && (p.share_group || G == 1) && p.K >= 1 &&
         parts * (p.d * sizeof(__bf16) + sizeof(float2)) <= kMaxCellPartialBytes;
}
static bool use_cell_path(const AttnLaunch& p) {
  return p.window > 0 && p.alpha != nullptr && cell_partials_fit(p);
}
// SAS with the selected blocks block-major (the current block walked per row
// tile, the selected blocks as per-(row, slot) partials) where the masked-tile
// walk would waste the most: a 32-row tile walks the union of its rows'
// selected blocks (at most the prefix, at most 32 K blocks) plus the current
// one, while a row keeps K + 1.  Measured at 32 query / 8 kv heads, d = 128,
// b = 64, K = 16 (forward ms, masked tiles vs block-major with the per-wave
// partial kernel): 4 x 8K (union / kept 3.8) 3.7 vs 5.4; 1 x 32K (15.1) 10.2
// vs 5.8; 1 x 64K (30.1) 27.3 vs 12.0 (5.1 and 10.6 with the per-workgroup
// one).  The partials (K d bf16 per row and query head, written and read
// back) and the per-slot q reads are what the block-major form pays.
constexpr double kSasBlockMajorWaste = 7.0;   // the measured break-even, interpolated
static double sas_masked_waste(const AttnLaunch& p) {
  const double pmid = static_cast<double>(num_candidates(p.q_pos0 + p.nq / 2, p.b, p.prefix_mode, p.qblock));
  const double uni = pmid < 32.0 * p.K ? pmid : 32.0 * p.K;
  const double kept = pmid < p.K ? pmid : p.K;
  return (uni + 1.0) / (kept + 1.0);
}
static bool use_sas_cell_path(const AttnLaunch& p) {
  return !(p.window > 0 && p.alpha != nullptr) && p.local == 0 && cell_partials_fit(p) &&
         sas_masked_waste(p) >= kSasBlockMajorWaste;
}

struct CellWs {
  uint32_t* bits;      // [B Hsel, nblk, nw] row-selected-cell bitmap
  int32_t* cnt;        // [B Hsel ncell] selecting rows per cell
  int2* units;         // [B Hsel, cap] (head * ncell + cell, tile of 32 rows)
  int32_t* rows;       // [B Hsel, cap, 32] the units' rows, -1 past a cell's last row
  int32_t* nunits;     // [B Hsel] units of each head
  __bf16* o;           // [B, Hq, nq, K, d] per-(row, slot) normalised o of the cell
  float2* ml;          // [B, Hq, nq, K] (max, sum), log2 domain
  int64_t nblk, ncell, cap, max_units;
  int nw;
  size_t bytes;
};

static CellWs cell_ws(const AttnLaunch& p, void* ws) {
  CellWs w{};
  w.nblk = (p.L + p.b - 1) / p.b;
  w.nw = (p.nq + 31) / 32;
  w.ncell = num_candidates(p.q_pos0 + p.nq - 1, p.b, p.prefix_mode, p.qblock);
  const int64_t heads = static_cast<int64_t>(p.B) * p.Hsel;
  const int64_t nent = heads * (w.ncell > 0 ? w.ncell : 1);
  // units of a head: one partial tile per cell at most, plus one per 32 (row, cell) marks
  w.cap = (w.ncell > 0 ? w.ncell : 1) + (static_cast<int64_t>(p.nq) * p.K + kCellUnit - 1) / kCellUnit;
  w.max_units = heads * w.cap;
  const size_t parts = static_cast<size_t>(p.B) * p.Hq * p.nq * p.K;
  constexpr int kParts = 7;
  const size_t sz[kParts] = {static_cast<size_t>(heads) * w.nblk * w.nw * sizeof(uint32_t),
                             static_cast<size_t>(nent) * sizeof(int32_t),
                             static_cast<size_t>(w.max_units) * sizeof(int2),
                             static_cast<size_t>(w.max_units) * kCellUnit * sizeof(int32_t),
                             static_cast<size_t>(heads) * sizeof(int32_t),
                             parts * p.d * sizeof(__bf16),
                             parts * sizeof(float2)};
  char* base = static_cast<char*>(ws);
  size_t off[kParts];
  size_t total = 0;
  for (int x = 0; x < kParts; ++x) {
    off[x] = total;
    total += align256(sz[x]);
  }
  w.bits = reinterpret_cast<uint32_t*>(base + off[0]);
  w.cnt = reinterpret_cast<int32_t*>(base + off[1]);
  w.units = reinterpret_cast<int2*>(base + off[2]);
  w.rows = reinterpret_cast<int32_t*>(base + off[3]);
  w.nunits = reinterpret_cast<int32_t*>(base + off[4]);
  w.o = reinterpret_cast<__bf16*>(base + off[5]);
  w.ml = reinterpret_cast<float2*>(base + off[6]);
  w.bytes = total;
  return w;
}

size_t attn_tile_fwd_workspace_bytes(const AttnLaunch& p) {
  return (use_cell_path(p) || use_sas_cell_path(p)) ? cell_ws(p, nullptr).bytes : 0;
}

// The cell-major branch L: mark, count and fill build the units, then
// attn_cell_partial_kernel writes the per-(row, slot) partials into the workspace.
template <int D>
static hipError_t launch_cell_partials(const AttnLaunch& p, void* ws, hipStream_t st, const __bf16** cell_o,
                                       const float2** cell_ml) {
  const CellWs w = cell_ws(p, ws);
  const int64_t heads = static_cast<int64_t>(p.B) * p.Hsel;
  hipError_t e = launch_mark_rows(p.idx, p.nq, p.q_pos0, p.b, p.prefix_mode, p.qblock, p.K, w.nblk, w.nw, heads,
                                  w.bits, st);
  if (e != hipSuccess) return e;
  // cells that are candidates of some row: those before the last row's query block
  const int64_t ncell = num_candidates(p.q_pos0 + p.nq - 1, p.b, p.prefix_mode, p.qblock);
  if (ncell > 0) {
    const int64_t nent = heads * ncell;
    const unsigned wave_grid = static_cast<unsigned>((nent + 3) / 4);   // one wave per entry
    e = launch(false, cell_count_kernel, dim3(wave_grid), dim3(256), st, static_cast<const uint32_t*>(w.bits), w.nblk,
               w.nw, ncell, heads, w.cnt);
    if (e != hipSuccess) return e;
    e = launch(false, cell_fill_kernel, dim3(wave_grid), dim3(256), st, static_cast<const uint32_t*>(w.bits),
               static_cast<const int32_t*>(w.cnt), w.nblk, w.nw, ncell, nent, w.cap, w.units, w.rows, w.nunits);
    if (e != hipSuccess) return e;
    if (p.Hq / p.Hkv == 4) {                      // one unit per workgroup, one head per wave
      const dim3 wgrid(static_cast<unsigned>(w.max_units));
      e = p.b == 32 ? launch(false, attn_unit_partial_kernel<D, 1>, wgrid, dim3(256), st,
                             static_cast<const __bf16*>(p.q), static_cast<const __bf16*>(p.k),
                             static_cast<const __bf16*>(p.v), p.idx, p.logg, static_cast<const int2*>(w.units),
                             static_cast<const int32_t*>(w.rows), static_cast<const int32_t*>(w.nunits), w.cap,
                             heads, ncell, p.Hq, p.Hkv, p.Hsel, p.nq, p.L, p.K, w.o, w.ml)
                    : launch(false, attn_unit_partial_kernel<D, 2>, wgrid, dim3(256), st,
                             static_cast<const __bf16*>(p.q), static_cast<const __bf16*>(p.k),
                             static_cast<const __bf16*>(p.v), p.idx, p.logg, static_cast<const int2*>(w.units),
                             static_cast<const int32_t*>(w.rows), static_cast<const int32_t*>(w.nunits), w.cap,
                             heads, ncell, p.Hq, p.Hkv, p.Hsel, p.nq, p.L, p.K, w.o, w.ml);
      if (e != hipSuccess) return e;
      *cell_o = w.o;
      *cell_ml = w.ml;
      return hipSuccess;
    }
    const dim3 ugrid(static_cast<unsigned>((w.max_units + 3) / 4));     // one unit per wave
    const auto* q = static_cast<const __bf16*>(p.q);
    const auto* kk = static_cast<const __bf16*>(p.k);
    const auto* vv = static_cast<const __bf16*>(p.v);
    const auto* un = static_cast<const int2*>(w.units);
    const auto* rw = static_cast<const int32_t*>(w.rows);
    const auto* nu = static_cast<const int32_t*>(w.nunits);
    e = p.b == 32 ? launch(false, attn_cell_partial_kernel<D, 1>, ugrid, dim3(256), st, q, kk, vv, p.idx, p.logg, un,
                           rw, nu, w.cap, heads, ncell, p.Hq, p.Hkv, p.Hsel, p.nq, p.L, p.K, w.o, w.ml)
                  : launch(false, attn_cell_partial_kernel<D, 2>, ugrid, dim3(256), st, q, kk, vv, p.idx, p.logg, un,
                           rw, nu, w.cap, heads, ncell, p.Hq, p.Hkv, p.Hsel, p.nq, p.L, p.K, w.o, w.ml);
    if (e != hipSuccess) return e;
  }
  *cell_o = w.o;
  *cell_ml = w.ml;
  return hipSuccess;
}

template <int D, int kMode, int NW>
static hipError_t launch_tile_fwd_k(const AttnLaunch& p, int NH, int NT, const __bf16* cell_o, const float2* cell_ml,
                                    hipStream_t st) {
  const int G = p.Hq / p.Hkv;
  const int ntiles = (p.nq + 31) / 32;
  dim3 grid((ntiles + NT - 1) / NT, static_cast<unsigned>(p.B * p.Hkv * (G / NH)));
  return launch(true, attn_tile_fwd_kernel<D, kMode, NW>, grid, dim3(64 * NW), st, static_cast<const __bf16*>(p.q),
                static_cast<const __bf16*>(p.k), static_cast<const __bf16*>(p.v), p.idx, p.logg, p.alpha,
                p.Hq, p.Hkv, p.Hsel, p.share_group, p.nq, p.q_pos0, p.L, p.b, p.prefix_mode, p.qblock,
                p.K, p.local, p.window, static_cast<__bf16*>(p.o), p.lse, NH, NT, cell_o, cell_ml);
}

// Heads of a group share K / V tiles: up to 4 of them in a workgroup, one wave
// each.  In the selected-block modes a single head (d = 64) takes two row tiles
// per workgroup: the workgroup walks the union of its rows' key tiles, so fewer
// rows per union mean fewer tiles a wave waits through without needing them.
// With the cells computed apart, the walk is the window alone (contiguous), and
// a single head takes four row tiles: each staged key tile serves four waves.
hipError_t launch_attn_tile_fwd(const AttnLaunch& p, void* ws, hipStream_t st) {
  const int G = p.Hq / p.Hkv;
  const int NH = G < 4 ? G : 4;
  const int NT = 4 / NH;
  const bool mix = p.window > 0 && p.alpha != nullptr;
  if (mix && use_cell_path(p)) {
    const __bf16* cell_o = nullptr;
    const float2* cell_ml = nullptr;
    const hipError_t e = p.d == 64 ? launch_cell_partials<64>(p, ws, st, &cell_o, &cell_ml)
                                   : launch_cell_partials<128>(p, ws, st, &cell_o, &cell_ml);
    if (e != hipSuccess) return e;
    if (p.d == 64) return launch_tile_fwd_k<64, 2, 4>(p, NH, NT, cell_o, cell_ml, st);
    return launch_tile_fwd_k<128, 2, 4>(p, NH, NT, cell_o, cell_ml, st);
  }
  if (!mix && use_sas_cell_path(p)) {
    const __bf16* cell_o = nullptr;
    const float2* cell_ml = nullptr;
    const hipError_t e = p.d == 64 ? launch_cell_partials<64>(p, ws, st, &cell_o, &cell_ml)
                                   : launch_cell_partials<128>(p, ws, st, &cell_o, &cell_ml);
    if (e != hipSuccess) return e;
    if (p.d == 64) return launch_tile_fwd_k<64, 3, 4>(p, NH, NT, cell_o, cell_ml, st);
    return launch_tile_fwd_k<128, 3, 4>(p, NH, NT, cell_o, cell_ml, st);
  }
  if (G == 1 && p.d == 64) {
    return mix ? launch_tile_fwd_k<64, 1, 2>(p, 1, 2, nullptr, nullptr, st)
               : launch_tile_fwd_k<64, 0, 2>(p, 1, 2, nullptr, nullptr, st);
  }
  if (p.d == 64)
    return mix ? launch_tile_fwd_k<64, 1, 4>(p, NH, NT, nullptr, nullptr, st)
               : launch_tile_fwd_k<64, 0, 4>(p, NH, NT, nullptr, nullptr, st);
  return mix ? launch_tile_fwd_k<128, 1, 4>(p, NH, NT, nullptr, nullptr, st)
             : launch_tile_fwd_k<128, 0, 4>(p, NH, NT, nullptr, nullptr, st);
}

}  // namespace spa
