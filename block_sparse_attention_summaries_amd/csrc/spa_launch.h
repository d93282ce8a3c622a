// spa_launch.h -- internal launch descriptors passed from the C-ABI layer
// (api.hip) to the kernel translation units.  Arguments are already
// validated when these are filled in.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spa {

// Candidate blocks of a query row at absolute position pos: blocks before the
// row's own block (prefix_mode 0) or cells before its query block (mode 1).
__host__ __device__ inline int64_t num_candidates(int64_t pos, int b, int prefix_mode, int qblock) {
  return prefix_mode == 0 ? pos / b : (static_cast<int64_t>(qblock) * (pos / qblock)) / b;
}

// Paged K / V: the cache pointers are page pools [npages, Hkv, b, d] and
// logical block c of batch bi lives in page table[bi * tstride + c].  A null
// table means the contiguous [B, Hkv, L, d] layout.
struct KvPages {
  const int32_t* table = nullptr;
  int64_t tstride = 0;
  int64_t npages = 0;
};

struct SummaryLaunch {
  const void* k;
  int dtype, B, Hkv;
  int64_t L;
  int d, b;
  int64_t first_block, num_blocks, ccap;
  void* kbar;
  float* max_norm;
  float* centre;
  KvPages pages{};
};

struct SelectLaunch {
  const void* q;
  int dtype, B, Hq, Hkv, nq, d;
  int64_t q_pos0;
  const void* kbar;
  const float* max_norm;
  const float* centre;
  int64_t ccap;
  int b, prefix_mode, qblock, share_group;
  const float* proj_w;
  const float* erf_lambda;
  const float* erf_sigma;
  int K, gate;
  int32_t* idx;
  float* logg;
  int32_t* k_eff;
  int Hsel;
  int64_t max_cand;   // candidates of the last row (the largest count)
  const float* kbar_scale;   // non-NULL: kbar holds fp8 (E4M3) codes, one scale per block
};

struct SelectGrads {
  const float* dg;
  float* dq;
  float* dkbar;
  float* dproj_w;
  void* dk;          // may be NULL
  int64_t L;
};

// FS-B forests of every (batch, kv head): members [B, Hkv, 2, n], nmem
// [B, Hkv, 2], node fields [B, Hkv, 2, NN(, d)], NN = forest_nodes(n).
struct ForestLaunch {
  const void* kbar;
  int dtype, B, Hkv, d;
  int64_t ccap, n;
  const float* max_norm;
  const float* centre;
  int32_t* members;
  int32_t* nmem;
  float* mu;
  float* rad;
  float* amax;
  float* pmin;
  void* ws;
};

struct AttnLaunch {
  const void* q;
  const void* k;
  const void* v;
  int dtype, B, Hq, Hkv, nq, d;
  int64_t L, q_pos0;
  int b, prefix_mode, qblock;
  const int32_t* idx;
  const float* logg;
  int K, share_group, local, window;
  const float* alpha;
  void* o;
  float* lse;
  int Hsel;
  KvPages pages{};
};

struct BwdLaunch {
  AttnLaunch a;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dg;
};

// Optional per-call profiling events (see spa_profile_next_call): the i-th
// kernel launched by the next entry-point call records events[2i] when it
// begins and events[2i+1] when it ends (dispatch timestamps).  Thread-local.
struct ProfileEvents {
  hipEvent_t* events;   // 2 * count handles, or nullptr
  int count;            // kernels to bracket
  int next;             // launches made so far in this call
};
ProfileEvents& profile_events();

// Launch `kernel` on `st`.  Arguments are converted to the kernel's parameter
// types.  (`last` marks the final kernel of an entry-point call.)
template <typename... KArgs, typename... Args>
hipError_t launch(bool last, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                  Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  (void)last;
  ProfileEvents& pe = profile_events();
  hipEvent_t s = nullptr, e = nullptr;
  if (pe.events != nullptr && pe.next < pe.count) {
    s = pe.events[2 * pe.next];
    e = pe.events[2 * pe.next + 1];
  }
  ++pe.next;
  hipExtLaunchKernelGGL(kernel, grid, block, 0, st, s, e, 0, static_cast<KArgs>(args)...);
  return hipGetLastError();
}

// Decode selection: chunked scoring + per-chunk top-K, then a merge.
constexpr int kDecodeChunk = 256;  // candidate blocks per scoring workgroup

inline int64_t decode_num_chunks(int64_t max_cand) {
  return (max_cand + kDecodeChunk - 1) / kDecodeChunk;
}

// Workspace layout helpers (bytes, 256-aligned sections).
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Decode-path selection workspace: per (selection head, chunk) the chunk's
// top-K records, then its (max, sum exp).
struct DecodeSelectWs {
  uint64_t* keys;
  float2* ml;
  int nch;
  size_t bytes;
};
inline DecodeSelectWs decode_select_ws(const SelectLaunch& p, void* ws) {
  const int64_t nch = decode_num_chunks(p.max_cand > 0 ? p.max_cand : 1);
  const size_t heads = static_cast<size_t>(p.B) * p.Hsel;
  const size_t kbytes = align256(heads * nch * p.K * sizeof(uint64_t));
  char* base = static_cast<char*>(ws);
  return DecodeSelectWs{reinterpret_cast<uint64_t*>(base), reinterpret_cast<float2*>(base + kbytes),
                        static_cast<int>(nch), kbytes + align256(heads * nch * sizeof(float2))};
}

// The one-call decode step (bf16): a scorer kernel writes every candidate's
// score, each chunk's (max, sum exp) and each 64-block group's largest score;
// the attention kernel selects from them, attends and combines.  Workspace:
// the u block [kStepFlagBytes] at offset 0, then scores [heads, nch * 256]
// fp32, ml [heads, nch] float2, group maxima t2 [heads, nch * 4] fp32, then
// the split-K partials and one arrival counter per selection head
// (decode_step_workspace_bytes).  The u block holds u = W^T q_hat as
// [heads, d] 64-bit words (fp32 bits, ready mark in bit 32) when heads * d
// fits (kStepUWords); it reads zero between calls (the attention kernel
// clears the words the scorer set).  Its place and size do not depend on
// the problem's shape, so stale words can never read as ready.
constexpr int kStepMaxChunks = 64;   // candidates per row <= 16384
constexpr int kStepMaxK = 64;
constexpr int kStepMaxHeads = 4096;  // batch x selection heads
constexpr size_t kStepFlagBytes = 16384;                       // 256-aligned
constexpr int64_t kStepUWords = kStepFlagBytes / sizeof(uint64_t);
struct DecodeStepWs {
  float* scores;
  float2* ml;
  float* t2;
  uint64_t* u;   // null when heads * d > kStepUWords: every scorer forms u itself
  uint32_t* ctr;
  int nch;
  size_t sel_bytes;   // bytes of the u block, scores, ml and t2
};
inline DecodeStepWs decode_step_ws(const SelectLaunch& p, void* ws_sel, void* ctr) {
  const int64_t nch = decode_num_chunks(p.max_cand > 0 ? p.max_cand : 1);
  const size_t heads = static_cast<size_t>(p.B) * p.Hsel;
  const size_t fb = kStepFlagBytes;
  const size_t sb = align256(heads * nch * 256 * sizeof(float));
  const size_t mb = align256(heads * nch * sizeof(float2));
  const size_t tb = align256(heads * nch * 4 * sizeof(float));
  char* base = static_cast<char*>(ws_sel);
  const bool u_fits = static_cast<int64_t>(heads) * p.d <= kStepUWords;
  return DecodeStepWs{reinterpret_cast<float*>(base + fb), reinterpret_cast<float2*>(base + fb + sb),
                      reinterpret_cast<float*>(base + fb + sb + mb),
                      u_fits ? reinterpret_cast<uint64_t*>(base) : nullptr, static_cast<uint32_t*>(ctr),
                      static_cast<int>(nch), fb + sb + mb + tb};
}
hipError_t launch_decode_step_scores(const SelectLaunch& p, const DecodeStepWs& w, hipStream_t st);
size_t decode_step_select_bytes(const SelectLaunch& p);

// 64-key tiles per kept block of the decode attention (blocks of b <= 64 keys
// are one tile).
inline int decode_step_tpu(const AttnLaunch& p) { return p.b > 64 ? p.b / 64 : 1; }

// Element type codes of the launch structs (the C ABI's spa_dtype values).
constexpr int kDtypeF32 = 0, kDtypeBf16 = 1;



size_t select_workspace_bytes(const SelectLaunch& p);
size_t select_bwd_workspace_bytes(const SelectLaunch& p);
size_t attn_fwd_workspace_bytes(const AttnLaunch& p);
// attention part of the one-call decode step's workspace: the split-K
// partials (as attn_fwd) plus one arrival counter per selection head
size_t decode_step_workspace_bytes(const AttnLaunch& p);
size_t attn_bwd_workspace_bytes(const BwdLaunch& p);

hipError_t launch_block_summaries(const SummaryLaunch& p, hipStream_t st);
// fp8 summaries: codes [B, Hkv, ccap, d] uint8 and scales [B, Hkv, ccap] of
// blocks [first, first + num) from kbar (dtype); and the fp32 rebuild.
hipError_t launch_quantize_fp8(const void* kbar, int dtype, int B, int Hkv, int64_t ccap, int d, int64_t first,
                               int64_t num, uint8_t* codes, float* scales, hipStream_t st);
hipError_t launch_dequantize_fp8(const uint8_t* codes, const float* scales, int64_t rows, int d, float* out,
                                 hipStream_t st);
hipError_t launch_score_select(const SelectLaunch& p, void* ws, hipStream_t st);
hipError_t launch_select_bwd(const SelectLaunch& p, const SelectGrads& g, void* ws, hipStream_t st);
hipError_t launch_retain_cells(const float* max_norm, int B, int Hkv, int64_t ccap, int64_t ncand, int W, int P,
                               int32_t* cells, int32_t* count, hipStream_t st);
hipError_t launch_score_select_subset(const SelectLaunch& p, const int32_t* cells, const int32_t* count, int cap,
                                      hipStream_t st);
int64_t forest_nodes(int64_t m);
size_t forest_workspace_bytes(int B, int Hkv, int d, int64_t n);
hipError_t launch_forest_build(const ForestLaunch& p, hipStream_t st);
hipError_t launch_forest_select(const SelectLaunch& s, const ForestLaunch& p, const void* k, int64_t L,
                                hipStream_t st);
// the one-row chunk scorer + merge handles this selection (the path that reads fp8 summaries)
bool decode_select_path(const SelectLaunch& p);
bool decode_fusable(const SelectLaunch& p);
int decode_merge_nv(const SelectLaunch& p);
hipError_t launch_decode_chunks(const SelectLaunch& p, void* ws, hipStream_t st);
hipError_t launch_decode_fused_attn(const SelectLaunch& s, void* ws_sel, const AttnLaunch& a, void* ws_att,
                                    hipStream_t st);
bool rows_select_mfma_supported(const SelectLaunch& p);
hipError_t launch_rows_select_mfma(const SelectLaunch& p, void* ws, hipStream_t st);
size_t rows_select_mfma_ws_bytes(const SelectLaunch& p);
hipError_t launch_attn_fwd(const AttnLaunch& p, void* ws, hipStream_t st);
bool attn_tile_fwd_supported(const AttnLaunch& p);
hipError_t launch_attn_tile_fwd(const AttnLaunch& p, void* ws, hipStream_t st);
// workspace of the tile forward (the cell-major branch L of the mix mode; 0 otherwise)
size_t attn_tile_fwd_workspace_bytes(const AttnLaunch& p);
hipError_t launch_attn_bwd(const BwdLaunch& p, void* ws, hipStream_t st);
bool attn_tile_bwd_supported(const BwdLaunch& p);
size_t attn_tile_bwd_bitmap_bytes(const BwdLaunch& p);
hipError_t launch_attn_tile_bwd(const BwdLaunch& p, const float* Dbuf, uint32_t* bits, hipStream_t st);
hipError_t launch_zero_fill(void* ptr, size_t bytes, hipStream_t st);
// Bitmap [heads, nblk, nw] of "row selected unit c" (bit row % 32 of word
// row / 32), every word written; nblk <= 2048.
hipError_t launch_mark_rows(const int32_t* idx, int nq, int64_t q_pos0, int b, int prefix_mode, int qblock, int K,
                            int64_t nblk, int nw, int64_t heads, uint32_t* bits, hipStream_t st);

// probe.hip: dependent-load chain over next[0 .. mask] (one lane), final
// index to out[0].
hipError_t launch_load_chase(const uint32_t* next, uint32_t mask, int steps, uint32_t start, uint32_t* out,
                             hipStream_t st);

}  // namespace spa
