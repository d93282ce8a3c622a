// api.hip -- the extern "C" entry points of libsparse_attn (declared in
// include/sparse_attn.h): argument validation, status codes, workspace
// sizing and kernel dispatch on the caller's stream.  Nothing here allocates,
// frees, synchronises or reads device memory.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "spa_launch.h"
#include "../../include/sparse_attn.h"

// Device memory of sparse_decode_step_noalloc: the chunk winners and split-K
// partials that sparse_decode_step keeps in the caller's workspace.  Every
// GPU the library runs on holds its own copy until the process ends.  In host
// code this name is not a device address: the kernels get the address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[SPA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;
thread_local spa::ProfileEvents g_profile = {nullptr, 0, 0};

spa_status fail(spa_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

spa_status ok() {
  g_last_error.clear();
  return SPA_OK;
}

// A profiling request applies to one call only, launched or not.
struct ProfileScope {
  ~ProfileScope() { g_profile = spa::ProfileEvents{nullptr, 0, 0}; }
};

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define SPA_REQUIRE(cond, code, ...) \
  do {                               \
    if (!(cond)) return fail((code), __VA_ARGS__); \
  } while (0)

spa_status check_heads(int B, int Hq, int Hkv, int d, int dtype) {
  SPA_REQUIRE(dtype == SPA_DTYPE_F32 || dtype == SPA_DTYPE_BF16, SPA_ERR_UNSUPPORTED,
              "dtype %d not supported (0 = fp32, 1 = bf16)", dtype);
  SPA_REQUIRE(d == 64 || d == 128, SPA_ERR_UNSUPPORTED, "head dim d = %d not supported (64 or 128)", d);
  SPA_REQUIRE(B >= 1 && Hq >= 1 && Hkv >= 1, SPA_ERR_INVALID_ARG, "B, Hq, Hkv must be >= 1");
  SPA_REQUIRE(Hq % Hkv == 0, SPA_ERR_INVALID_ARG, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
  SPA_REQUIRE(Hq / Hkv <= 8 && pow2(Hq / Hkv), SPA_ERR_UNSUPPORTED,
              "group size G = %d not supported (1, 2, 4 or 8)", Hq / Hkv);
  SPA_REQUIRE(static_cast<int64_t>(B) * Hq <= 65535, SPA_ERR_UNSUPPORTED, "B * Hq = %lld exceeds 65535",
              static_cast<long long>(B) * Hq);
  return SPA_OK;
}

spa_status check_select(const spa_select_args* a, spa::SelectLaunch* p) {
  SPA_REQUIRE(a != nullptr, SPA_ERR_INVALID_ARG, "args is NULL");
  spa_status st = check_heads(a->B, a->Hq, a->Hkv, a->d, a->dtype);
  if (st != SPA_OK) return st;
  SPA_REQUIRE(a->q && a->kbar && a->idx, SPA_ERR_INVALID_ARG, "q, kbar and idx must be non-NULL");
  SPA_REQUIRE(aligned16(a->q) && aligned16(a->kbar), SPA_ERR_INVALID_ARG, "q and kbar must be 16-byte aligned");
  SPA_REQUIRE(a->nq >= 1 && a->q_pos0 >= 0, SPA_ERR_INVALID_ARG, "nq must be >= 1 and q_pos0 >= 0");
  SPA_REQUIRE(pow2(a->b) && a->b >= 16 && a->b <= 128, SPA_ERR_UNSUPPORTED,
              "block size b = %d not supported (power of two in [16, 128])", a->b);
  SPA_REQUIRE(a->K >= 1 && a->K <= 64, SPA_ERR_UNSUPPORTED, "K = %d not supported (1..64)", a->K);
  SPA_REQUIRE(a->gate == SPA_GATE_NONE || a->gate == SPA_GATE_SOFTMAX_LOG, SPA_ERR_INVALID_ARG,
              "gate = %d invalid", a->gate);
  SPA_REQUIRE(a->gate == SPA_GATE_NONE || a->logg != nullptr, SPA_ERR_INVALID_ARG,
              "logg must be non-NULL when the gate is on");
  SPA_REQUIRE(a->prefix_mode == SPA_PREFIX_CURRENT_BLOCK || a->prefix_mode == SPA_PREFIX_QUERY_BLOCK,
              SPA_ERR_INVALID_ARG, "prefix_mode = %d invalid", a->prefix_mode);
  if (a->prefix_mode == SPA_PREFIX_QUERY_BLOCK)
    SPA_REQUIRE(a->qblock >= a->b && a->qblock % a->b == 0, SPA_ERR_INVALID_ARG,
                "qblock = %d must be a positive multiple of b = %d", a->qblock, a->b);
  SPA_REQUIRE((a->erf_lambda == nullptr) == (a->erf_sigma == nullptr), SPA_ERR_INVALID_ARG,
              "erf_lambda and erf_sigma must both be given or both be NULL");
  if (a->erf_lambda != nullptr)
    SPA_REQUIRE(a->max_norm != nullptr && a->centre != nullptr, SPA_ERR_INVALID_ARG,
                "the erf term needs max_norm and centre");
  SPA_REQUIRE(a->ccap >= 1, SPA_ERR_INVALID_ARG, "ccap must be >= 1");
  const int Hsel = a->share_group ? a->Hkv : a->Hq;
  const int64_t last = a->q_pos0 + a->nq - 1;
  const int64_t max_cand = spa::num_candidates(last, a->b, a->prefix_mode,
                                               a->prefix_mode == SPA_PREFIX_QUERY_BLOCK ? a->qblock : 1);
  SPA_REQUIRE(max_cand <= a->ccap, SPA_ERR_INVALID_ARG,
              "kbar holds %lld blocks but the last row has %lld candidates",
              static_cast<long long>(a->ccap), static_cast<long long>(max_cand));
  SPA_REQUIRE(static_cast<int64_t>(a->B) * Hsel <= 65535, SPA_ERR_UNSUPPORTED, "B * Hsel exceeds 65535");
  SPA_REQUIRE(max_cand < (static_cast<int64_t>(1) << 31), SPA_ERR_UNSUPPORTED, "too many candidates");
  *p = spa::SelectLaunch{a->q, a->dtype, a->B, a->Hq, a->Hkv, a->nq, a->d, a->q_pos0, a->kbar,
                         a->max_norm, a->centre, a->ccap, a->b, a->prefix_mode,
                         a->prefix_mode == SPA_PREFIX_QUERY_BLOCK ? a->qblock : 1, a->share_group ? 1 : 0,
                         a->proj_w, a->erf_lambda, a->erf_sigma, a->K, a->gate, a->idx, a->logg,
                         a->k_eff, Hsel, max_cand, a->kbar_scale};
  if (a->kbar_scale != nullptr)
    SPA_REQUIRE(spa::decode_select_path(*p), SPA_ERR_UNSUPPORTED,
                "fp8 summaries (kbar_scale) are read by the one-row decode scorer only: nq = 1, "
                "CURRENT_BLOCK candidates, no erf term");
  return SPA_OK;
}

spa_status check_attn(const spa_attn_args* a, spa::AttnLaunch* p) {
  SPA_REQUIRE(a != nullptr, SPA_ERR_INVALID_ARG, "args is NULL");
  spa_status st = check_heads(a->B, a->Hq, a->Hkv, a->d, a->dtype);
  if (st != SPA_OK) return st;
  SPA_REQUIRE(a->q && a->k && a->v && a->o && a->idx, SPA_ERR_INVALID_ARG,
              "q, k, v, o and idx must be non-NULL");
  SPA_REQUIRE(aligned16(a->q) && aligned16(a->k) && aligned16(a->v), SPA_ERR_INVALID_ARG,
              "q, k and v must be 16-byte aligned");
  SPA_REQUIRE(a->nq >= 1 && a->q_pos0 >= 0 && a->L >= 1 && a->q_pos0 + a->nq <= a->L,
              SPA_ERR_INVALID_ARG, "need nq >= 1, q_pos0 >= 0 and q_pos0 + nq <= L");
  SPA_REQUIRE(pow2(a->b) && a->b >= 16 && a->b <= 128, SPA_ERR_UNSUPPORTED,
              "block size b = %d not supported (power of two in [16, 128])", a->b);
  SPA_REQUIRE(a->K >= 1 && a->K <= 64, SPA_ERR_UNSUPPORTED, "K = %d not supported (1..64)", a->K);
  SPA_REQUIRE(a->prefix_mode == SPA_PREFIX_CURRENT_BLOCK || a->prefix_mode == SPA_PREFIX_QUERY_BLOCK,
              SPA_ERR_INVALID_ARG, "prefix_mode = %d invalid", a->prefix_mode);
  if (a->prefix_mode == SPA_PREFIX_QUERY_BLOCK)
    SPA_REQUIRE(a->qblock >= a->b && a->qblock % a->b == 0, SPA_ERR_INVALID_ARG,
                "qblock = %d must be a positive multiple of b = %d", a->qblock, a->b);
  const bool sas = a->local == SPA_LOCAL_CURRENT_BLOCK && a->window == 0 && a->alpha == nullptr;
  const bool mix = a->local == SPA_LOCAL_NONE && a->window > 0 && a->alpha != nullptr;
  SPA_REQUIRE(sas || mix, SPA_ERR_UNSUPPORTED,
              "supported modes: (local=CURRENT_BLOCK, window=0, alpha=NULL) or "
              "(local=NONE, window>0, alpha!=NULL)");
  SPA_REQUIRE(a->L < (static_cast<int64_t>(1) << 31), SPA_ERR_UNSUPPORTED, "L must be < 2^31");
  const int Hsel = a->share_group ? a->Hkv : a->Hq;
  *p = spa::AttnLaunch{a->q, a->k, a->v, a->dtype, a->B, a->Hq, a->Hkv, a->nq, a->d, a->L, a->q_pos0,
                       a->b, a->prefix_mode, a->prefix_mode == SPA_PREFIX_QUERY_BLOCK ? a->qblock : 1,
                       a->idx, a->logg, a->K, a->share_group ? 1 : 0, a->local, a->window, a->alpha,
                       a->o, a->lse, Hsel};
  return SPA_OK;
}

spa_status check_bwd(const spa_attn_args* a, const void* o, const void* dout, const float* lse, void* dq, void* dk,
              void* dv, float* dg, spa::BwdLaunch* p) {
  spa::AttnLaunch al;
  spa_status st = check_attn(a, &al);
  if (st != SPA_OK) return st;
  SPA_REQUIRE(a->local == SPA_LOCAL_CURRENT_BLOCK && a->window == 0 && a->alpha == nullptr,
              SPA_ERR_UNSUPPORTED, "the backward supports the current-block + selected-blocks mode only");
  SPA_REQUIRE(a->prefix_mode == SPA_PREFIX_CURRENT_BLOCK, SPA_ERR_UNSUPPORTED,
              "the backward supports prefix_mode = CURRENT_BLOCK only");
  SPA_REQUIRE(a->b <= 64, SPA_ERR_UNSUPPORTED, "the backward supports b <= 64");
  SPA_REQUIRE(o && dout && lse && dq && dk && dv && dg, SPA_ERR_INVALID_ARG,
              "o, dout, lse, dq, dk, dv and dg must be non-NULL");
  SPA_REQUIRE(aligned16(o) && aligned16(dout) && aligned16(dq) && aligned16(dk) && aligned16(dv),
              SPA_ERR_INVALID_ARG, "o, dout, dq, dk and dv must be 16-byte aligned");
  *p = spa::BwdLaunch{al, o, dout, lse, dq, dk, dv, dg};
  return SPA_OK;
}

spa_status check_select_bwd(const spa_select_args* a, const spa_select_grads* g, spa::SelectLaunch* p,
                     spa::SelectGrads* sg) {
  spa_status st = check_select(a, p);
  if (st != SPA_OK) return st;
  SPA_REQUIRE(a->gate == SPA_GATE_SOFTMAX_LOG, SPA_ERR_UNSUPPORTED,
              "the selector backward needs the softmax log gate (gate = SOFTMAX_LOG)");
  SPA_REQUIRE(a->prefix_mode == SPA_PREFIX_CURRENT_BLOCK && a->erf_lambda == nullptr, SPA_ERR_UNSUPPORTED,
              "the selector backward supports current-block candidates without the erf term");
  SPA_REQUIRE(a->dtype == SPA_DTYPE_BF16, SPA_ERR_UNSUPPORTED, "the selector backward supports bf16 only");
  SPA_REQUIRE(a->kbar_scale == nullptr, SPA_ERR_UNSUPPORTED, "the selector backward takes summaries in dtype");
  SPA_REQUIRE(g != nullptr && g->dg && g->dq && g->dkbar, SPA_ERR_INVALID_ARG,
              "grads, dg, dq and dkbar must be non-NULL");
  SPA_REQUIRE(aligned16(g->dq) && aligned16(g->dkbar), SPA_ERR_INVALID_ARG, "dq and dkbar must be 16-byte aligned");
  SPA_REQUIRE((a->proj_w != nullptr) == (g->dproj_w != nullptr), SPA_ERR_INVALID_ARG,
              "dproj_w must be given exactly when the projection proj_w is");
  if (g->dk != nullptr) {
    SPA_REQUIRE(aligned16(g->dk), SPA_ERR_INVALID_ARG, "dk must be 16-byte aligned");
    SPA_REQUIRE(g->L >= a->ccap * a->b, SPA_ERR_INVALID_ARG,
                "dk holds L = %lld tokens but the summaries cover ccap * b = %lld", static_cast<long long>(g->L),
                static_cast<long long>(a->ccap * a->b));
  }
  *sg = spa::SelectGrads{g->dg, g->dq, g->dkbar, g->dproj_w, g->dk, g->L};
  return SPA_OK;
}

spa_status check_decode(const spa_decode_args* d, spa::SelectLaunch* sp, spa::AttnLaunch* ap) {
  SPA_REQUIRE(d != nullptr && d->select != nullptr && d->attn != nullptr, SPA_ERR_INVALID_ARG,
              "decode args, select and attn must be non-NULL");
  spa_status st = check_select(d->select, sp);
  if (st != SPA_OK) return st;
  st = check_attn(d->attn, ap);
  if (st != SPA_OK) return st;
  const spa_select_args* s = d->select;
  const spa_attn_args* a = d->attn;
  SPA_REQUIRE(s->nq == 1, SPA_ERR_UNSUPPORTED, "sparse_decode_step takes one query row (nq = %d)", s->nq);
  SPA_REQUIRE(s->prefix_mode == SPA_PREFIX_CURRENT_BLOCK && a->prefix_mode == SPA_PREFIX_CURRENT_BLOCK,
              SPA_ERR_UNSUPPORTED, "sparse_decode_step supports prefix_mode = CURRENT_BLOCK");
  SPA_REQUIRE(a->local == SPA_LOCAL_CURRENT_BLOCK && a->window == 0 && a->alpha == nullptr, SPA_ERR_UNSUPPORTED,
              "sparse_decode_step supports the current block + selected blocks mode");
  SPA_REQUIRE(s->q == a->q && s->B == a->B && s->Hq == a->Hq && s->Hkv == a->Hkv && s->d == a->d &&
                  s->dtype == a->dtype && s->q_pos0 == a->q_pos0 && s->b == a->b && s->K == a->K &&
                  (s->share_group != 0) == (a->share_group != 0),
              SPA_ERR_INVALID_ARG, "select and attn arguments describe different problems");
  SPA_REQUIRE(a->idx == s->idx && a->logg == s->logg, SPA_ERR_INVALID_ARG,
              "attn idx / logg must be the select outputs idx / logg");
  return SPA_OK;
}

// Selection part of the one-call step's workspace.  The u block of the
// one-call scorer sits at offset 0 on both paths: the two-call fallback keeps
// its scratch after it, so a workspace can serve steps of either path in turn
// without disturbing the u block's ready-marked words (zero between calls).
size_t decode_sel_bytes(const spa::SelectLaunch& sp) {
  const size_t two = spa::kStepFlagBytes + spa::select_workspace_bytes(sp);
  const size_t one = spa::decode_fusable(sp) ? spa::decode_step_select_bytes(sp) : 0;
  return spa::align256(two > one ? two : one);
}

static_assert(SPA_DECODE_FLAG_BYTES == spa::kStepFlagBytes, "the decode step's u block");

hipError_t run_decode_step(const spa::SelectLaunch& sp, const spa::AttnLaunch& ap, void* ws, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  char* ws_att = base + decode_sel_bytes(sp);
  if (spa::decode_fusable(sp)) return spa::launch_decode_fused_attn(sp, ws, ap, ws_att, s);
  hipError_t e = spa::launch_score_select(sp, base + spa::kStepFlagBytes, s);
  if (e == hipSuccess) e = spa::launch_attn_fwd(ap, ws_att, s);
  return e;
}

size_t decode_ws_bytes(const spa::SelectLaunch& sp, const spa::AttnLaunch& ap) {
  return decode_sel_bytes(sp) + spa::decode_step_workspace_bytes(ap);
}

spa_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return SPA_OK;
  SPA_REQUIRE(ws != nullptr && have >= need, SPA_ERR_WORKSPACE,
              "workspace of %zu bytes needed, %zu given%s", need, have, ws ? "" : " (NULL)");
  return SPA_OK;
}

spa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SPA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Address of `scratch` on each device, resolved once per device (with that
// device current) on the first no-alloc call made there.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

spa_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SPA_ERR_HIP, "sparse_decode_step_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  SPA_REQUIRE(dev >= 0 && dev < kMaxDevices, SPA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(SPA_ERR_HIP, "sparse_decode_step_noalloc: hipGetSymbolAddress on device %d: %s", dev,
                    hipGetErrorString(e));
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SPA_OK;
}

}  // namespace

extern "C" {

int sparse_abi_version(void) { return SPA_ABI_VERSION; }
int spa_abi_version(void) { return SPA_ABI_VERSION; }

spa_status spa_profile_next_call(void** events, int count) {
  SPA_REQUIRE(count >= 0 && (count == 0 || events != nullptr), SPA_ERR_INVALID_ARG,
              "events must hold 2 * count handles");
  g_profile = spa::ProfileEvents{reinterpret_cast<hipEvent_t*>(events), count, 0};
  return ok();
}

const char* sparse_last_error(void) { return g_last_error.c_str(); }
const char* spa_last_error(void) { return g_last_error.c_str(); }

spa_status sparse_block_summaries(const void* k, int dtype, int B, int Hkv, int64_t L, int d, int b,
                           int64_t first_block, int64_t num_blocks, int64_t ccap, void* kbar,
                           float* max_norm, float* centre, spa_stream_t stream) {
  ProfileScope profile_scope;
  spa_status st = check_heads(B, Hkv, Hkv, d, dtype);
  if (st != SPA_OK) return st;
  SPA_REQUIRE(k && kbar && max_norm, SPA_ERR_INVALID_ARG, "k, kbar and max_norm must be non-NULL");
  SPA_REQUIRE(aligned16(k), SPA_ERR_INVALID_ARG, "k must be 16-byte aligned");
  SPA_REQUIRE(pow2(b) && b >= 16 && b <= 128, SPA_ERR_UNSUPPORTED,
              "block size b = %d not supported (power of two in [16, 128])", b);
  SPA_REQUIRE(first_block >= 0 && num_blocks >= 0, SPA_ERR_INVALID_ARG,
              "first_block and num_blocks must be >= 0");
  SPA_REQUIRE((first_block + num_blocks) * b <= L, SPA_ERR_INVALID_ARG,
              "blocks [%lld, %lld) are not all full in L = %lld", static_cast<long long>(first_block),
              static_cast<long long>(first_block + num_blocks), static_cast<long long>(L));
  SPA_REQUIRE(first_block + num_blocks <= ccap, SPA_ERR_INVALID_ARG, "ccap = %lld too small",
              static_cast<long long>(ccap));
  SPA_REQUIRE(num_blocks < (static_cast<int64_t>(1) << 31), SPA_ERR_UNSUPPORTED, "too many blocks");
  if (num_blocks == 0) return ok();
  spa::SummaryLaunch p{k, dtype, B, Hkv, L, d, b, first_block, num_blocks, ccap, kbar, max_norm, centre};
  return hip_status(spa::launch_block_summaries(p, static_cast<hipStream_t>(stream)), "sparse_block_summaries");
}

spa_status check_pages(const spa_kv_pages* pg, int64_t blocks_needed, spa::KvPages* out) {
  SPA_REQUIRE(pg != nullptr && pg->block_table != nullptr, SPA_ERR_INVALID_ARG, "pages and block_table must be non-NULL");
  SPA_REQUIRE(pg->num_pages >= 1, SPA_ERR_INVALID_ARG, "num_pages must be >= 1");
  SPA_REQUIRE(pg->table_stride >= blocks_needed, SPA_ERR_INVALID_ARG,
              "table_stride = %lld but %lld logical blocks are addressed", static_cast<long long>(pg->table_stride),
              static_cast<long long>(blocks_needed));
  *out = spa::KvPages{pg->block_table, pg->table_stride, pg->num_pages};
  return SPA_OK;
}

spa_status sparse_block_summaries_paged(const void* k_pages, int dtype, int B, int Hkv, int64_t L, int d, int b,
                                 const spa_kv_pages* pages, int64_t first_block, int64_t num_blocks, int64_t ccap,
                                 void* kbar, float* max_norm, float* centre, spa_stream_t stream) {
  ProfileScope profile_scope;
  spa_status st = check_heads(B, Hkv, Hkv, d, dtype);
  if (st != SPA_OK) return st;
  SPA_REQUIRE(k_pages && kbar && max_norm, SPA_ERR_INVALID_ARG, "k_pages, kbar and max_norm must be non-NULL");
  SPA_REQUIRE(aligned16(k_pages), SPA_ERR_INVALID_ARG, "k_pages must be 16-byte aligned");
  SPA_REQUIRE(pow2(b) && b >= 16 && b <= 128, SPA_ERR_UNSUPPORTED,
              "block size b = %d not supported (power of two in [16, 128])", b);
  SPA_REQUIRE(first_block >= 0 && num_blocks >= 0, SPA_ERR_INVALID_ARG,
              "first_block and num_blocks must be >= 0");
  SPA_REQUIRE((first_block + num_blocks) * b <= L, SPA_ERR_INVALID_ARG,
              "blocks [%lld, %lld) are not all full in L = %lld", static_cast<long long>(first_block),
              static_cast<long long>(first_block + num_blocks), static_cast<long long>(L));
  SPA_REQUIRE(first_block + num_blocks <= ccap, SPA_ERR_INVALID_ARG, "ccap = %lld too small",
              static_cast<long long>(ccap));
  SPA_REQUIRE(num_blocks < (static_cast<int64_t>(1) << 31), SPA_ERR_UNSUPPORTED, "too many blocks");
  spa::KvPages kp;
  st = check_pages(pages, first_block + num_blocks, &kp);
  if (st != SPA_OK) return st;
  if (num_blocks == 0) return ok();
  spa::SummaryLaunch p{k_pages, dtype, B, Hkv, L, d, b, first_block, num_blocks, ccap, kbar, max_norm, centre, kp};
  return hip_status(spa::launch_block_summaries(p, static_cast<hipStream_t>(stream)),
                    "sparse_block_summaries_paged");
}

spa_status sparse_score_select(const spa_select_args* a, void* workspace, size_t ws_bytes, spa_stream_t stream) {
  ProfileScope profile_scope;
  spa::SelectLaunch p;
  spa_status st = check_select(a, &p);
  if (st != SPA_OK) return st;
  st = check_ws(workspace, ws_bytes, spa::select_workspace_bytes(p));
  if (st != SPA_OK) return st;
  return hip_status(spa::launch_score_select(p, workspace, static_cast<hipStream_t>(stream)),
                    "sparse_score_select");
}

spa_status sparse_quantize_summaries_fp8(const void* kbar, int dtype, int B, int Hkv, int64_t ccap, int d,
                                  int64_t first_block, int64_t num_blocks, uint8_t* codes, float* scales,
                                  spa_stream_t stream) {
  ProfileScope profile_scope;
  spa_status st = check_heads(B, Hkv, Hkv, d, dtype);
  if (st != SPA_OK) return st;
  SPA_REQUIRE(kbar && codes && scales, SPA_ERR_INVALID_ARG, "kbar, codes and scales must be non-NULL");
  SPA_REQUIRE(aligned16(kbar) && aligned16(codes) && aligned16(scales), SPA_ERR_INVALID_ARG,
              "kbar, codes and scales must be 16-byte aligned");
  SPA_REQUIRE(first_block >= 0 && num_blocks >= 0 && first_block + num_blocks <= ccap, SPA_ERR_INVALID_ARG,
              "blocks [%lld, %lld) outside [0, ccap = %lld)", static_cast<long long>(first_block),
              static_cast<long long>(first_block + num_blocks), static_cast<long long>(ccap));
  SPA_REQUIRE(static_cast<int64_t>(B) * Hkv * num_blocks < (static_cast<int64_t>(1) << 33), SPA_ERR_UNSUPPORTED,
              "too many blocks");
  if (num_blocks == 0) return SPA_OK;
  return hip_status(spa::launch_quantize_fp8(kbar, dtype, B, Hkv, ccap, d, first_block, num_blocks, codes, scales,
                                             static_cast<hipStream_t>(stream)),
                    "sparse_quantize_summaries_fp8");
}

spa_status sparse_dequantize_summaries_fp8(const uint8_t* codes, const float* scales, int64_t rows, int d, float* out,
                                    spa_stream_t stream) {
  ProfileScope profile_scope;
  SPA_REQUIRE(codes && scales && out, SPA_ERR_INVALID_ARG, "codes, scales and out must be non-NULL");
  SPA_REQUIRE(aligned16(codes) && aligned16(out), SPA_ERR_INVALID_ARG, "codes and out must be 16-byte aligned");
  SPA_REQUIRE(d == 64 || d == 128, SPA_ERR_UNSUPPORTED, "d = %d not supported (64 or 128)", d);
  SPA_REQUIRE(rows >= 0 && rows * (d / 16) < (static_cast<int64_t>(1) << 35), SPA_ERR_INVALID_ARG,
              "rows = %lld out of range", static_cast<long long>(rows));
  if (rows == 0) return SPA_OK;
  return hip_status(spa::launch_dequantize_fp8(codes, scales, rows, d, out, static_cast<hipStream_t>(stream)),
                    "sparse_dequantize_summaries_fp8");
}

spa_status sparse_attn_fwd(const spa_attn_args* a, void* workspace, size_t ws_bytes, spa_stream_t stream) {
  ProfileScope profile_scope;
  spa::AttnLaunch p;
  spa_status st = check_attn(a, &p);
  if (st != SPA_OK) return st;
  st = check_ws(workspace, ws_bytes, spa::attn_fwd_workspace_bytes(p));
  if (st != SPA_OK) return st;
  return hip_status(spa::launch_attn_fwd(p, workspace, static_cast<hipStream_t>(stream)), "sparse_attn_fwd");
}

spa_status sparse_attn_bwd(const spa_attn_args* a, const void* o, const void* dout, const float* lse, void* dq,
                    void* dk, void* dv, float* dg, void* workspace, size_t ws_bytes, spa_stream_t stream) {
  ProfileScope profile_scope;
  spa::BwdLaunch p;
  spa_status st = check_bwd(a, o, dout, lse, dq, dk, dv, dg, &p);
  if (st != SPA_OK) return st;
  st = check_ws(workspace, ws_bytes, spa::attn_bwd_workspace_bytes(p));
  if (st != SPA_OK) return st;
  return hip_status(spa::launch_attn_bwd(p, workspace, static_cast<hipStream_t>(stream)), "sparse_attn_bwd");
}

spa_status sparse_select_bwd(const spa_select_args* a, const spa_select_grads* g, void* workspace, size_t ws_bytes,
                      spa_stream_t stream) {
  ProfileScope profile_scope;
  spa::SelectLaunch p;
  spa::SelectGrads sg;
  spa_status st = check_select_bwd(a, g, &p, &sg);
  if (st != SPA_OK) return st;
  st = check_ws(workspace, ws_bytes, spa::select_bwd_workspace_bytes(p));
  if (st != SPA_OK) return st;
  return hip_status(spa::launch_select_bwd(p, sg, workspace, static_cast<hipStream_t>(stream)),
                    "sparse_select_bwd");
}

spa_status sparse_decode_step(const spa_decode_args* a, void* workspace, size_t ws_bytes, spa_stream_t stream) {
  ProfileScope profile_scope;
  spa::SelectLaunch sp;
  spa::AttnLaunch ap;
  spa_status st = check_decode(a, &sp, &ap);
  if (st != SPA_OK) return st;
  st = check_ws(workspace, ws_bytes, decode_ws_bytes(sp, ap));
  if (st != SPA_OK) return st;
  return hip_status(run_decode_step(sp, ap, workspace, static_cast<hipStream_t>(stream)), "sparse_decode_step");
}

spa_status sparse_decode_step_noalloc(const spa_decode_args* a, spa_stream_t stream) {
  ProfileScope profile_scope;
  spa::SelectLaunch sp;
  spa::AttnLaunch ap;
  spa_status st = check_decode(a, &sp, &ap);
  if (st != SPA_OK) return st;
  const size_t need = decode_ws_bytes(sp, ap);
  SPA_REQUIRE(need <= SPA_NOALLOC_SCRATCH_BYTES, SPA_ERR_WORKSPACE,
              "sparse_decode_step_noalloc: this step needs %zu bytes of scratch, the library holds %zu "
              "(use sparse_decode_step with a workspace)", need, static_cast<size_t>(SPA_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (need > 0) {
    st = noalloc_scratch(&ws);
    if (st != SPA_OK) return st;
  }
  return hip_status(run_decode_step(sp, ap, ws, static_cast<hipStream_t>(stream)), "sparse_decode_step_noalloc");
}

spa_status sparse_decode_step_paged(const spa_decode_args* a, const spa_kv_pages* pages, void* workspace,
                             size_t ws_bytes, spa_stream_t stream) {
  ProfileScope profile_scope;
  spa::SelectLaunch sp;
  spa::AttnLaunch ap;
  spa_status st = check_decode(a, &sp, &ap);
  if (st != SPA_OK) return st;
  st = check_pages(pages, (ap.L + ap.b - 1) / ap.b, &ap.pages);
  if (st != SPA_OK) return st;
  st = check_ws(workspace, ws_bytes, decode_ws_bytes(sp, ap));
  if (st != SPA_OK) return st;
  return hip_status(run_decode_step(sp, ap, workspace, static_cast<hipStream_t>(stream)), "sparse_decode_step_paged");
}

spa_status sparse_retain_cells(const float* max_norm, int B, int Hkv, int64_t ccap, int64_t ncand, int W, int P,
                        int32_t* cells, int32_t* count, spa_stream_t stream) {
  ProfileScope profile_scope;
  SPA_REQUIRE(max_norm && cells && count, SPA_ERR_INVALID_ARG, "max_norm, cells and count must be non-NULL");
  SPA_REQUIRE(B >= 1 && Hkv >= 1 && static_cast<int64_t>(B) * Hkv <= (static_cast<int64_t>(1) << 31) - 1,
              SPA_ERR_INVALID_ARG, "B and Hkv must be >= 1");
  SPA_REQUIRE(ncand >= 0 && ncand <= ccap, SPA_ERR_INVALID_ARG, "ncand = %lld outside [0, ccap = %lld]",
              static_cast<long long>(ncand), static_cast<long long>(ccap));
  SPA_REQUIRE(W >= 0 && P >= 0 && P <= 64 && W + P >= 1 && W + P <= 256, SPA_ERR_UNSUPPORTED,
              "W = %d, P = %d not supported (P <= 64, 1 <= W + P <= 256)", W, P);
  return hip_status(spa::launch_retain_cells(max_norm, B, Hkv, ccap, ncand, W, P, cells, count,
                                             static_cast<hipStream_t>(stream)),
                    "sparse_retain_cells");
}

spa_status sparse_score_select_subset(const spa_select_args* a, const int32_t* cells, const int32_t* count, int cap,
                               spa_stream_t stream) {
  ProfileScope profile_scope;
  spa::SelectLaunch p;
  spa_status st = check_select(a, &p);
  if (st != SPA_OK) return st;
  SPA_REQUIRE(a->proj_w == nullptr, SPA_ERR_UNSUPPORTED, "the kept-set selection takes no projection");
  SPA_REQUIRE(a->kbar_scale == nullptr, SPA_ERR_UNSUPPORTED, "the kept-set selection takes summaries in dtype");
  SPA_REQUIRE(cells && count, SPA_ERR_INVALID_ARG, "cells and count must be non-NULL");
  SPA_REQUIRE(cap >= 1 && cap <= 256, SPA_ERR_UNSUPPORTED, "cap = %d not supported (1..256)", cap);
  return hip_status(spa::launch_score_select_subset(p, cells, count, cap, static_cast<hipStream_t>(stream)),
                    "sparse_score_select_subset");
}

int64_t sparse_forest_nodes(int64_t n) { return n < 1 ? 0 : spa::forest_nodes(n); }

size_t sparse_forest_workspace_bytes(int B, int Hkv, int d, int64_t n) {
  if (B < 1 || Hkv < 1 || d < 1 || n < 1) return 0;
  return spa::forest_workspace_bytes(B, Hkv, d, n);
}

spa_status check_forest(const spa_forest* fo, int B, int Hkv, int64_t ccap, int64_t n, spa::ForestLaunch* p) {
  SPA_REQUIRE(fo != nullptr && fo->members && fo->nmem && fo->mu && fo->rad && fo->amax && fo->pmin,
              SPA_ERR_INVALID_ARG, "forest arrays must be non-NULL");
  SPA_REQUIRE(n >= 1 && n <= ccap && n < (static_cast<int64_t>(1) << 31), SPA_ERR_INVALID_ARG,
              "n = %lld outside [1, ccap = %lld]", static_cast<long long>(n), static_cast<long long>(ccap));
  SPA_REQUIRE(static_cast<int64_t>(B) * Hkv <= 65535, SPA_ERR_UNSUPPORTED, "B * Hkv exceeds 65535");
  p->B = B;
  p->Hkv = Hkv;
  p->ccap = ccap;
  p->n = n;
  p->members = fo->members;
  p->nmem = fo->nmem;
  p->mu = fo->mu;
  p->rad = fo->rad;
  p->amax = fo->amax;
  p->pmin = fo->pmin;
  return SPA_OK;
}

spa_status sparse_forest_build(const void* kbar, int dtype, const float* max_norm, const float* centre, int B, int Hkv,
                        int d, int64_t ccap, int64_t n, const spa_forest* forest, void* workspace, size_t ws_bytes,
                        spa_stream_t stream) {
  ProfileScope profile_scope;
  spa_status st = check_heads(B, Hkv, Hkv, d, dtype);
  if (st != SPA_OK) return st;
  SPA_REQUIRE(kbar && max_norm && centre, SPA_ERR_INVALID_ARG, "kbar, max_norm and centre must be non-NULL");
  spa::ForestLaunch p{};
  st = check_forest(forest, B, Hkv, ccap, n, &p);
  if (st != SPA_OK) return st;
  st = check_ws(workspace, ws_bytes, spa::forest_workspace_bytes(B, Hkv, d, n));
  if (st != SPA_OK) return st;
  p.kbar = kbar;
  p.dtype = dtype;
  p.d = d;
  p.max_norm = max_norm;
  p.centre = centre;
  p.ws = workspace;
  return hip_status(spa::launch_forest_build(p, static_cast<hipStream_t>(stream)), "sparse_forest_build");
}

spa_status sparse_forest_select(const spa_select_args* a, const void* k, int64_t L, const spa_forest* forest, int64_t n,
                         spa_stream_t stream) {
  ProfileScope profile_scope;
  spa::SelectLaunch s;
  spa_status st = check_select(a, &s);
  if (st != SPA_OK) return st;
  SPA_REQUIRE(a->gate == SPA_GATE_NONE && a->proj_w == nullptr, SPA_ERR_UNSUPPORTED,
              "the forest selection takes no gate and no projection");
  SPA_REQUIRE(a->kbar_scale == nullptr, SPA_ERR_UNSUPPORTED, "the forest selection takes summaries in dtype");
  SPA_REQUIRE(a->K <= 16, SPA_ERR_UNSUPPORTED, "K = %d not supported (<= 16)", a->K);
  SPA_REQUIRE(a->b == 16 || a->b == 32 || a->b == 64, SPA_ERR_UNSUPPORTED, "cell size b = %d not supported", a->b);
  SPA_REQUIRE(k != nullptr && aligned16(k), SPA_ERR_INVALID_ARG, "k must be non-NULL and 16-byte aligned");
  SPA_REQUIRE(L >= n * a->b, SPA_ERR_INVALID_ARG, "k holds L = %lld tokens, fewer than the n cells",
              static_cast<long long>(L));
  const int qb = a->prefix_mode == SPA_PREFIX_QUERY_BLOCK ? a->qblock : 1;
  const int64_t c_first = spa::num_candidates(a->q_pos0, a->b, a->prefix_mode, qb);
  const int64_t c_last = spa::num_candidates(a->q_pos0 + a->nq - 1, a->b, a->prefix_mode, qb);
  SPA_REQUIRE(c_first == n && c_last == n, SPA_ERR_INVALID_ARG,
              "every row must have the n = %lld cells the forests were built over as its candidates",
              static_cast<long long>(n));
  spa::ForestLaunch p{};
  st = check_forest(forest, a->B, a->Hkv, a->ccap, n, &p);
  if (st != SPA_OK) return st;
  return hip_status(spa::launch_forest_select(s, p, k, L, static_cast<hipStream_t>(stream)),
                    "sparse_forest_select");
}

size_t sparse_workspace_bytes(int op, const void* args) {
  switch (op) {
    case SPA_OP_SCORE_SELECT: {
      spa::SelectLaunch p;
      if (check_select(static_cast<const spa_select_args*>(args), &p) != SPA_OK) return 0;
      return spa::select_workspace_bytes(p);
    }
    case SPA_OP_ATTN_FWD: {
      spa::AttnLaunch p;
      if (check_attn(static_cast<const spa_attn_args*>(args), &p) != SPA_OK) return 0;
      return spa::attn_fwd_workspace_bytes(p);
    }
    case SPA_OP_ATTN_BWD: {
      spa::AttnLaunch p;
      if (check_attn(static_cast<const spa_attn_args*>(args), &p) != SPA_OK) return 0;
      spa::BwdLaunch bp{p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
      return spa::attn_bwd_workspace_bytes(bp);
    }
    case SPA_OP_DECODE_STEP: {
      spa::SelectLaunch sp;
      spa::AttnLaunch ap;
      if (check_decode(static_cast<const spa_decode_args*>(args), &sp, &ap) != SPA_OK) return 0;
      return decode_ws_bytes(sp, ap);
    }
    case SPA_OP_SELECT_BWD: {
      spa::SelectLaunch p;
      if (check_select(static_cast<const spa_select_args*>(args), &p) != SPA_OK) return 0;
      return spa::select_bwd_workspace_bytes(p);
    }
    default:
      fail(SPA_ERR_INVALID_ARG, "unknown op %d", op);
      return 0;
  }
}

spa_status sparse_workspace_init(void* workspace, size_t ws_bytes, spa_stream_t stream) {
  ProfileScope profile_scope;
  if (ws_bytes == 0) return ok();
  SPA_REQUIRE(workspace != nullptr, SPA_ERR_INVALID_ARG, "workspace is NULL");
  SPA_REQUIRE(aligned16(workspace) && ws_bytes % 16 == 0, SPA_ERR_INVALID_ARG,
              "workspace must be 16-byte aligned with a size multiple of 16");
  return hip_status(spa::launch_zero_fill(workspace, ws_bytes, static_cast<hipStream_t>(stream)),
                    "sparse_workspace_init");
}

spa_status sparse_probe_load_chase(const uint32_t* next, int64_t n, int steps, uint32_t start, uint32_t* out,
                                   spa_stream_t stream) {
  ProfileScope profile_scope;
  SPA_REQUIRE(next != nullptr && out != nullptr, SPA_ERR_INVALID_ARG, "next and out must be device pointers");
  SPA_REQUIRE(n >= 1 && n <= (int64_t{1} << 32) && (n & (n - 1)) == 0, SPA_ERR_INVALID_ARG,
              "n = %lld: a power of two in [1, 2^32]", static_cast<long long>(n));
  SPA_REQUIRE(steps >= 1, SPA_ERR_INVALID_ARG, "steps = %d: at least 1", steps);
  return hip_status(spa::launch_load_chase(next, static_cast<uint32_t>(n - 1), steps, start, out,
                                           static_cast<hipStream_t>(stream)),
                    "sparse_probe_load_chase");
}

}  // extern "C"

namespace spa {

ProfileEvents& profile_events() { return g_profile; }

__global__ void zero_fill_kernel(uint4* p, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero_fill(void* ptr, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 16;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  return launch(true, zero_fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), st,
                static_cast<uint4*>(ptr), n);
}

}  // namespace spa
