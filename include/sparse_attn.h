/*
 * sparse_attn.h -- C ABI of the MI355X (gfx950) block-sparse causal attention
 * library with learned block selection (libsparse_attn.so).
 *
 * What it computes (pages of the reference, cited by title and section):
 *  - "SAS: Simple Attention Sparsification via End-to-End Optimization of
 *    Context Ranking" (review page): §3 Eq. 1-3 (attention restricted to a
 *    selected block set; n positions split into C = n/b blocks; a selector
 *    scores every block, the top K are kept), §4.1 Eq. 4 (the current block
 *    B0 is always kept with gate 1), §4.2.2 (softmax gate
 *    log g = s - LSE(s); inner-gate gradient Eq. 5), §4.3 Eq. 9 (log g added
 *    to the logits of the selected blocks inside the softmax), Alg. 1-2.
 *  - "FreeSolo ... zero-shot retrieval up to 64x the training length"
 *    (review page), "How it works": cells of s tokens summarised by mean key,
 *    centre position and max key norm; query-block prefix of B tokens;
 *    r_ic = q_i.kbar_c/sqrt(d) + lambda_h a_c erf((i - p_c)/(2 sigma_h));
 *    top-K cells read with one softmax; sliding window of w tokens; per-head
 *    alpha_h mix of the two branches.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous:
 *      q, o, dq, dout   [B, Hq,  nq, d]
 *      k, v, dk, dv     [B, Hkv, L,  d]
 *      kbar             [B, Hkv, ccap, d]     (same dtype as k)
 *      max_norm         [B, Hkv, ccap]        fp32
 *      centre           [ccap]                fp32
 *      idx              [B, Hsel, nq, K]      int32, ascending, -1 padded
 *      logg, dg         [B, Hsel, nq, K]      fp32
 *      k_eff            [B, Hsel, nq]         int32
 *      lse              [B, Hq, nq]           fp32
 *    with Hsel = Hkv when share_group != 0 (one selection per kv head from
 *    the mean of its G = Hq/Hkv query heads) and Hsel = Hq otherwise.
 *  - Query row r sits at absolute position i = q_pos0 + r of the K/V
 *    sequence (q_pos0 + nq <= L); decode is nq = 1, q_pos0 = L - 1.
 *  - Candidates of row i: prefix_mode SPA_PREFIX_CURRENT_BLOCK: blocks
 *    c < floor(i/b); SPA_PREFIX_QUERY_BLOCK: cells with
 *    (c+1) b <= qblock floor(i/qblock).
 *  - Selection order: higher score first, lower index on equal scores;
 *    K_eff = min(K, #candidates) indices are stored ascending.
 *  - Dot products are scaled by 1/sqrt(d).
 *  - dtype: SPA_DTYPE_F32 or SPA_DTYPE_BF16; d in {64, 128}; b a power of two
 *    in [16, 128]; 1 <= K <= 64; Hq a multiple of Hkv with G <= 8.
 *
 * Ownership: the caller allocates and frees every buffer (tensors and
 * workspace).  The library never allocates, frees or synchronises, never
 * reads device memory on the host, and launches only on the given stream
 * (spa_stream_t is a hipStream_t; NULL means the null stream).  Calls are
 * safe to capture in a HIP graph.
 *
 * Errors: every entry point validates its arguments before launching
 * anything and returns a spa_status.  On error nothing is launched and
 * sparse_last_error() returns a message (per calling thread).  Launch failures
 * reported by the HIP runtime return SPA_ERR_HIP.  Kernels never trap: block
 * indices outside a row's candidate set are ignored.  NaN/Inf inputs give
 * unspecified values but never out-of-bounds accesses.
 *
 * Workspace: sparse_workspace_bytes() gives the size a call needs (device
 * memory owned by the caller, 256-byte aligned).  Its contents are scratch:
 * no initialisation is needed and nothing is kept between calls.  Calls that
 * overlap in time must use distinct workspaces.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPA_ABI_VERSION 2

typedef void *spa_stream_t;

typedef enum {
    SPA_OK = 0,
    SPA_ERR_INVALID_ARG = -1,  /* null pointer, bad shape/size, out-of-range parameter */
    SPA_ERR_UNSUPPORTED = -2,  /* valid but not implemented combination (dtype, d, mode) */
    SPA_ERR_HIP = -3,          /* the HIP runtime reported a launch error */
    SPA_ERR_WORKSPACE = -4     /* workspace null or smaller than sparse_workspace_bytes() */
} spa_status;

typedef enum { SPA_DTYPE_F32 = 0, SPA_DTYPE_BF16 = 1 } spa_dtype;
typedef enum { SPA_PREFIX_CURRENT_BLOCK = 0, SPA_PREFIX_QUERY_BLOCK = 1 } spa_prefix_mode;
typedef enum { SPA_GATE_NONE = 0, SPA_GATE_SOFTMAX_LOG = 1 } spa_gate;
typedef enum { SPA_LOCAL_CURRENT_BLOCK = 0, SPA_LOCAL_NONE = 1 } spa_local;
typedef enum {
    SPA_OP_SCORE_SELECT = 1, SPA_OP_ATTN_FWD = 2, SPA_OP_ATTN_BWD = 3, SPA_OP_SELECT_BWD = 4,
    SPA_OP_DECODE_STEP = 5
} spa_op;

/* Version of this ABI (SPA_ABI_VERSION). */
int sparse_abi_version(void);
/* The same value under the library's short prefix (kept for callers built
 * against it). */
int spa_abi_version(void);

/* Kernel timing for callers that measure it (benchmarks, profilers).  Per
 * calling thread: the next call of an entry point below launches its i-th
 * kernel (i < count) with events[2i] recorded when that kernel begins and
 * events[2i+1] when it ends, from the kernel's own dispatch timestamps
 * (hipExtLaunchKernelGGL).  events holds 2*count hipEvent_t handles created
 * by the caller; NULL entries are skipped.  The request is used up by that
 * call whether or not it launches.  Do not use under graph capture.
 * Kernels per call: summaries 1; score_select 2 on the decode path (chunk
 * scoring, merge), else 1; attn_fwd 2 on the decode path (tile partials,
 * combine), 5 for many rows where the selected units go block-major (mark,
 * count, fill, cell partials, tiles; 2 when no row has a candidate unit:
 * mark, tiles), else 1; attn_bwd 4 for bf16 with many rows (D, mark, dq and dg,
 * dk and dv), else 3 (D, dq and dg, dk and dv); decode_step 2 (scoring,
 * selection + attention + combine), or the kernels of score_select then
 * attn_fwd where the selection is not folded in; forest_build
 * 4 plus one per forest level above the first; forest_select, retain_cells,
 * score_select_subset, quantize / dequantize_summaries_fp8 1; select_bwd one
 * per stage it runs.
 * Returns SPA_ERR_INVALID_ARG if count < 0 or events is NULL with count > 0. */
spa_status spa_profile_next_call(void **events, int count);

/* Message describing the last failed call made by this thread ("" if none).
 * The pointer stays valid until the next call on the same thread. */
const char *sparse_last_error(void);
/* The same message under the library's short prefix. */
const char *spa_last_error(void);

/*
 * sparse_block_summaries -- per (batch, kv head, full block c) in
 * [first_block, first_block + num_blocks):
 *   kbar[c]     = mean of the b keys of block c, computed exactly (fp64 sum)
 *                 and rounded to nearest even in the key dtype;
 *   max_norm[c] = max over the block of ||k_j||_2 (fp64, rounded to fp32);
 *   centre[c]   = c b + (b - 1)/2 (centre may be NULL).
 * ("SAS" review §3 Eq. 3 block partition with pooled key summaries; "FreeSolo"
 * review, "How it works": mean key, centre position, max key norm.)
 * Every summarised block must be full: (first_block + num_blocks) b <= L,
 * and first_block + num_blocks <= ccap.  Decode calls it with num_blocks = 1
 * when a block closes.  Output rows outside the range are not touched.
 * Returns SPA_ERR_INVALID_ARG on null pointers or out-of-range sizes.
 */
spa_status sparse_block_summaries(const void *k, int dtype, int B, int Hkv, int64_t L, int d,
                           int b, int64_t first_block, int64_t num_blocks, int64_t ccap,
                           void *kbar, float *max_norm, float *centre,
                           spa_stream_t stream);

typedef struct spa_select_args {
    const void *q;            /* [B, Hq, nq, d], dtype */
    int dtype;                /* spa_dtype of q and kbar */
    int B, Hq, Hkv, nq, d;
    int64_t q_pos0;           /* absolute position of query row 0 */
    const void *kbar;         /* [B, Hkv, ccap, d] */
    const float *max_norm;    /* [B, Hkv, ccap]; required when erf_lambda != NULL */
    const float *centre;      /* [ccap]; required when erf_lambda != NULL */
    int64_t ccap;             /* rows allocated in kbar; must cover every candidate */
    int b;                    /* block / cell size */
    int prefix_mode;          /* spa_prefix_mode */
    int qblock;               /* query-block size for SPA_PREFIX_QUERY_BLOCK */
    int share_group;          /* 1: selection per kv head from the mean of its G q heads */
    const float *proj_w;      /* NULL or [d, d] fp32 W: score uses W kbar_c */
    const float *erf_lambda;  /* NULL or [Hsel] fp32: adds lambda a_c erf((i-p_c)/(2 sigma)) */
    const float *erf_sigma;   /* [Hsel] fp32 (required with erf_lambda), > 0 */
    int K;                    /* budget in blocks, 1..64 */
    int gate;                 /* spa_gate */
    int32_t *idx;             /* out [B, Hsel, nq, K] */
    float *logg;              /* out [B, Hsel, nq, K]: s_c - LSE over all candidates, 0 in pads;
                                 may be NULL when gate == SPA_GATE_NONE */
    int32_t *k_eff;           /* out [B, Hsel, nq], may be NULL */
    const float *kbar_scale;  /* NULL: kbar is in dtype.  Else [B, Hkv, ccap] fp32 block scales and kbar
                                 holds OCP E4M3 codes (uint8, sparse_quantize_summaries_fp8); the summary
                                 is kbar_scale[c] * decode(code).  Read only by the one-row decode scorer
                                 (nq = 1, CURRENT_BLOCK candidates, no erf term): elsewhere
                                 SPA_ERR_UNSUPPORTED */
} spa_select_args;

/*
 * sparse_score_select -- scores, optional softmax log gate and top-K block
 * selection for every query row ("SAS" review §3 Eq. 3, §4.2.2 softmax gate,
 * Alg. 1 and the worked example; "FreeSolo" review cell score with the erf
 * position bias).  Score of candidate c for row i and selection head hs:
 *   s_c = q_hat . ktilde_c / sqrt(d)  [+ lambda_hs a_c erf((i - p_c)/(2 sigma_hs))]
 * q_hat = q_hs or the mean of the G query heads of kv head hs; ktilde = kbar
 * or W kbar.  Needs a workspace of sparse_workspace_bytes(SPA_OP_SCORE_SELECT):
 * the one-row decode path keeps its chunk results there; many bf16 rows with
 * the erf term keep per-head tables of the filter there (160 KiB per
 * selection head); other row selections need none (0 bytes).
 */
spa_status sparse_score_select(const spa_select_args *a, void *workspace, size_t ws_bytes,
                        spa_stream_t stream);

/*
 * sparse_quantize_summaries_fp8 -- 8-bit block summaries for the decode
 * scorer, which then reads half the bytes (the scoring pass reads every
 * candidate's summary at every step, twice the selected K/V at 512K).  Format:
 * OCP 8-bit floating point E4M3 without infinities (bias 7, 3 mantissa bits,
 * largest finite 448).  For every (batch, kv head, block c) in
 * [first_block, first_block + num_blocks):
 *   amax = max_e |kbar_c[e]|;  scales[c] = amax / 448;
 *   codes[c][e] = E4M3(kbar_c[e] * (448 / amax)): nearest, ties to the even
 *   code, held at +-448, sign kept;
 * both quotients and the product in single precision (correctly rounded); a
 * block of zeros gets scale 0 and zero codes.  kbar [B, Hkv, ccap, d] in
 * dtype, codes [B, Hkv, ccap, d] uint8, scales [B, Hkv, ccap] fp32 (caller-
 * owned device buffers; rows outside the range are not touched).  Pass codes
 * as spa_select_args.kbar and scales as kbar_scale.  (The pages do not state
 * a summary precision; this is an optional compressed form of the mean keys
 * of "SAS" review §3 Eq. 3.)  SPA_ERR_INVALID_ARG on null pointers, unaligned
 * buffers or out-of-range blocks.
 */
spa_status sparse_quantize_summaries_fp8(const void *kbar, int dtype, int B, int Hkv, int64_t ccap, int d,
                                  int64_t first_block, int64_t num_blocks, uint8_t *codes, float *scales,
                                  spa_stream_t stream);

/* sparse_dequantize_summaries_fp8 -- the fp32 summaries the decode scorer
 * reads: out[r][e] = scales[r] * decode(codes[r][e]) (single-precision
 * product; the decode is exact), for rows r of d codes (d in {64, 128}).
 * Uses the scorer's own decode.  SPA_ERR_INVALID_ARG on null or unaligned
 * pointers. */
spa_status sparse_dequantize_summaries_fp8(const uint8_t *codes, const float *scales, int64_t rows, int d, float *out,
                                    spa_stream_t stream);

typedef struct spa_attn_args {
    const void *q;            /* [B, Hq, nq, d] */
    const void *k;            /* [B, Hkv, L, d] */
    const void *v;            /* [B, Hkv, L, d] */
    int dtype;                /* spa_dtype of q, k, v, o (and dq, dk, dv, dout) */
    int B, Hq, Hkv, nq, d;
    int64_t L;                /* tokens in K / V */
    int64_t q_pos0;           /* absolute position of query row 0 */
    int b;                    /* block / cell size of idx */
    int prefix_mode;          /* candidate rule used to validate idx entries */
    int qblock;
    const int32_t *idx;       /* [B, Hsel, nq, K] selected units (entries that are not
                                 candidates of their row are ignored) */
    const float *logg;        /* NULL (no bias) or [B, Hsel, nq, K] log gates */
    int K;
    int share_group;
    int local;                /* spa_local: SPA_LOCAL_CURRENT_BLOCK keeps B0 causally */
    int window;               /* 0, or sliding-window width w (keys i-w < j <= i) */
    const float *alpha;       /* NULL, or [Hq] mix: o = alpha o_L + (1 - alpha) o_S */
    void *o;                  /* out [B, Hq, nq, d] */
    float *lse;               /* out [B, Hq, nq] log-sum-exp of branch L, may be NULL */
} spa_attn_args;

/*
 * sparse_attn_fwd -- exact softmax attention of every query row over
 *   branch L: the current block {j : floor(j/b) = floor(i/b), j <= i}
 *             (local = SPA_LOCAL_CURRENT_BLOCK, bias 0) plus every selected
 *             unit, each logit biased by its log g ("SAS" review §4.3 Eq. 9;
 *             "Monodratic" news page: local block + exact causal softmax on
 *             the selected set);
 *   branch S: keys i - w < j <= i (window > 0), mixed with alpha
 *             ("FreeSolo" review, two-branch head).
 * Supported modes: (local = CURRENT_BLOCK, window = 0, alpha = NULL) and
 * (local = NONE, window > 0, alpha != NULL).  A row with no key in branch L
 * gets o_L = 0 and lse = -inf.  nq = 1 uses the split-K decode kernels.
 * Workspace: sparse_workspace_bytes(SPA_OP_ATTN_FWD, a).  For many rows in
 * the window mode with routed cells of 32 or 64 keys it holds the cell-major
 * branch L: a bitmap of B Hsel x cells x ceil(nq/32) words, the row lists,
 * and per (row, query head, slot) a bf16 partial of d values plus 8 bytes
 * (about B Hq nq K (2d + 8) bytes; 143 MB at 16 heads, nq = 16384, K = 4,
 * d = 64); beyond 16 GiB of partials the call walks the cells per row tile
 * instead and needs no workspace.  The selected-block mode takes the same
 * block-major form (partials of the selected blocks, the current block walked
 * per row tile, joined into one softmax) when a 32-row tile's union of
 * selected blocks would be at least 7x the K + 1 blocks a row keeps (at the
 * middle row: min(candidates, 32 K) + 1 over min(candidates, K) + 1), with
 * b of 32 or 64, at most 4 query heads per kv head sharing the selection (or
 * one) and at most 16 GiB of partials; otherwise it needs no workspace.
 */
spa_status sparse_attn_fwd(const spa_attn_args *a, void *workspace, size_t ws_bytes,
                    spa_stream_t stream);

typedef struct spa_decode_args {
    const spa_select_args *select;   /* one query row (nq = 1), prefix_mode = CURRENT_BLOCK */
    const spa_attn_args *attn;       /* same q, shapes, b, K and GQA mode; idx / logg are
                                        select's outputs; local = CURRENT_BLOCK, no window */
} spa_decode_args;

/*
 * sparse_decode_step -- one decode step of the hot path: sparse_score_select
 * then sparse_attn_fwd on its selection ("SAS" review Alg. 1 then §4.3 Eq. 9
 * for one new token; "Monodratic" news page: local block plus exact softmax
 * on the selected blocks).  Outputs: idx, logg, k_eff of `select`, o and
 * lse of `attn`, as the two calls made in sequence give them (the same
 * selection; o and lse to fp32 rounding).  With bf16 (or fp8) summaries,
 * B * Hsel <= 4096, K <= 64 and at most 16384 candidates per row, the step
 * takes two kernels: the scorer, then one workgroup per (selection head,
 * kept tile) that selects the head's top-K from the scores, attends to its
 * tile and publishes a split-K partial, the head's last workgroup combining
 * them; otherwise the two calls' kernels run in sequence.  Needs a workspace
 * of sparse_workspace_bytes(SPA_OP_DECODE_STEP, spa_decode_args*),
 * caller-owned.  Its first SPA_DECODE_FLAG_BYTES bytes hold the scorer's
 * query u, each element marked ready when published; they must read zero on
 * the first decode step with that workspace (a zero-filled allocation, or
 * sparse_workspace_init); every decode step leaves them zero again, but other
 * entry points given the same workspace may not, so clear them before going
 * back to decode steps.  The rest of the
 * workspace's contents on entry are ignored.  Errors: as the two calls, plus
 * SPA_ERR_INVALID_ARG when select and attn disagree.
 */
#define SPA_DECODE_FLAG_BYTES 16384u
spa_status sparse_decode_step(const spa_decode_args *a, void *workspace, size_t ws_bytes,
                       spa_stream_t stream);

/*
 * sparse_decode_step_noalloc -- sparse_decode_step without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc.  The
 * step's scratch (chunk winners and split-K partials) lives in a device array
 * of SPA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends; nothing is allocated or freed by the call.  Arguments,
 * outputs and results are those of sparse_decode_step (the same kernels).
 *  - Returns SPA_ERR_WORKSPACE, launching nothing, when the step needs more
 *    than SPA_NOALLOC_SCRATCH_BYTES (sparse_workspace_bytes(SPA_OP_DECODE_STEP,
 *    a) tells; about 0.6 MiB for one sequence of 8 kv heads, K = 32, d = 128).
 *  - The first call on a device looks up that device's copy of the array
 *    (hipGetSymbolAddress with the device current): make it outside graph
 *    capture.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents: the array starts zero when the library loads and each
 *    call leaves its ready-marked words (the first SPA_DECODE_FLAG_BYTES bytes) zero
 *    again, as the next call needs them.  Calls that overlap in time on one
 *    GPU, on any streams, race.  Serialise them.
 */
#define SPA_NOALLOC_SCRATCH_BYTES (8u << 20)
spa_status sparse_decode_step_noalloc(const spa_decode_args *a, spa_stream_t stream);

/*
 * Paged K / V ("SAS" review, inference setup: a paged KV cache): the key and
 * value caches are page pools [num_pages, Hkv, b, d] (one page = one block of
 * b tokens of every kv head, each head's block contiguous) and logical block
 * c of batch bi lives in page block_table[bi * table_stride + c].  Page ids
 * outside [0, num_pages) read as empty: no key of that block is attended and
 * its summary is zero.  The block summaries stay dense [B, Hkv, ccap, d].
 */
typedef struct spa_kv_pages {
    const int32_t *block_table;   /* device [B, table_stride] page ids */
    int64_t table_stride;         /* entries per batch row, >= the logical blocks addressed */
    int64_t num_pages;            /* pages in each pool */
} spa_kv_pages;

/* sparse_block_summaries over a paged key cache: k_pages is the pool,
 * L the logical tokens per batch row; otherwise as sparse_block_summaries
 * (table_stride must cover first_block + num_blocks). */
spa_status sparse_block_summaries_paged(const void *k_pages, int dtype, int B, int Hkv, int64_t L, int d,
                                 int b, const spa_kv_pages *pages, int64_t first_block,
                                 int64_t num_blocks, int64_t ccap, void *kbar, float *max_norm,
                                 float *centre, spa_stream_t stream);

/* sparse_decode_step over a paged cache: a->attn->k and a->attn->v are the
 * page pools and a->attn->L the logical tokens (table_stride >= ceil(L / b));
 * same outputs as sparse_decode_step on the cache the pages describe, and the
 * same workspace (sparse_workspace_bytes(SPA_OP_DECODE_STEP, a)). */
spa_status sparse_decode_step_paged(const spa_decode_args *a, const spa_kv_pages *pages, void *workspace,
                             size_t ws_bytes, spa_stream_t stream);

/*
 * sparse_retain_cells -- FS-L fixed-state retention ("FreeSolo" review, the
 * two variants: before any query arrives each head keeps only its W most
 * recent cells and its P cells of largest max key norm).  Of the ncand prefix
 * cells of every (batch, kv head): the W most recent (ncand-W .. ncand-1)
 * plus the P older cells of largest max_norm (lower index first on equal
 * norms), min(ncand, W + P) cells in all.  max_norm: [B, Hkv, ccap] fp32 as
 * sparse_block_summaries writes it.  Outputs: cells [B, Hkv, W + P] int32,
 * ascending, -1 padded; count [B, Hkv] int32 (caller-owned device buffers).
 * P <= 64, 1 <= W + P <= 256, else SPA_ERR_UNSUPPORTED; SPA_ERR_INVALID_ARG
 * on null pointers or ncand outside [0, ccap].  No workspace.
 * Query-independent: run it when a cell closes.
 */
spa_status sparse_retain_cells(const float *max_norm, int B, int Hkv, int64_t ccap, int64_t ncand,
                        int W, int P, int32_t *cells, int32_t *count, spa_stream_t stream);

/*
 * sparse_score_select_subset -- sparse_score_select restricted to a kept set
 * (the FS-L per-query top K inside the retained cells): each selection head
 * scores the cells listed for its kv head (cells [B, Hkv, cap], count
 * [B, Hkv], as sparse_retain_cells writes them) that are candidates of the
 * row, and the gate's LSE runs over those cells only.  Scores are formed in
 * fp64 (q_hat . kbar / sqrt(d) plus the erf position bias).  Same outputs and
 * argument struct (and checks) as sparse_score_select; a projection, fp8
 * summaries or cap outside 1..256 give SPA_ERR_UNSUPPORTED, null cells /
 * count SPA_ERR_INVALID_ARG.  No workspace.
 */
spa_status sparse_score_select_subset(const spa_select_args *a, const int32_t *cells,
                               const int32_t *count, int cap, spa_stream_t stream);

/*
 * FS-B forests ("FreeSolo" review, the two variants: no cell is dropped; each
 * head builds a forest over the whole prefix and one over the cells at or
 * above the median max key norm; nodes hold a mean key, a radius, a max norm
 * and a min position; a beam of width 16 per level descends them, the node
 * score bounding the cell scores below; the reached cells are re-ranked by
 * logsumexp over their token keys and the top K are read).
 * A forest over m member cells (ascending) has fanout 16: node j of level 1
 * groups members [16j, 16j+16), node j of level l groups nodes [16j, 16j+16)
 * of level l-1, levels being added until one has at most 16 nodes.  Node
 * fields, fp32: mu (mean of the cells' mean keys), rad (max distance of those
 * to mu), amax (max max-norm), pmin (min centre).  Node score
 *   U = q_hat . mu / sqrt(d) + ||q_hat|| rad / sqrt(d) + lambda amax erf((i - pmin) / (2 sigma)).
 * Arrays (device, caller-owned), NN = sparse_forest_nodes(n), forest f = 0
 * (whole prefix) or 1 (norm >= the ceil(n/2)-th largest):
 *   members [B, Hkv, 2, n] int32 ascending, -1 padded; nmem [B, Hkv, 2];
 *   mu [B, Hkv, 2, NN, d]; rad, amax, pmin [B, Hkv, 2, NN] (levels stored
 *   bottom-up, level 1 first; unused slots 0).
 */
typedef struct spa_forest {
    int32_t *members;
    int32_t *nmem;
    float *mu;
    float *rad;
    float *amax;
    float *pmin;
} spa_forest;

/* Internal nodes of a forest over n cells (0 for n <= 16). */
int64_t sparse_forest_nodes(int64_t n);

/* Workspace bytes of sparse_forest_build (fp64 node sums). */
size_t sparse_forest_workspace_bytes(int B, int Hkv, int d, int64_t n);

/* sparse_forest_build -- both forests of every (batch, kv head) over the n
 * prefix cells 0 .. n-1, from the cell summaries (kbar [B, Hkv, ccap, d] in
 * dtype, max_norm [B, Hkv, ccap], centre [ccap], as sparse_block_summaries
 * writes them).  1 <= n <= ccap (else SPA_ERR_INVALID_ARG, as are null
 * arrays); B Hkv <= 65535; the workspace must hold
 * sparse_forest_workspace_bytes (else SPA_ERR_WORKSPACE).  Query-independent:
 * build when a query block's prefix grows. */
spa_status sparse_forest_build(const void *kbar, int dtype, const float *max_norm, const float *centre,
                        int B, int Hkv, int d, int64_t ccap, int64_t n, const spa_forest *forest,
                        void *workspace, size_t ws_bytes, spa_stream_t stream);

/* sparse_forest_select -- the per-query top K cells by the beam search of both
 * forests and the logsumexp re-rank over token keys (k [B, Hkv, L, d], the
 * cache the cells summarise, L >= n b).  `a` as for sparse_score_select, with
 * gate NONE, no projection, K <= 16, b in {16, 32, 64}; every row must have
 * exactly the n forest cells as candidates (same query block).  Writes idx
 * (ascending, -1 padded) and k_eff; logg is not written.  Scores in fp64.
 * A gate, a projection, fp8 summaries, K > 16 or another b give
 * SPA_ERR_UNSUPPORTED; rows whose candidates are not the n cells, or L < n b,
 * SPA_ERR_INVALID_ARG.  No workspace. */
spa_status sparse_forest_select(const spa_select_args *a, const void *k, int64_t L,
                         const spa_forest *forest, int64_t n, spa_stream_t stream);

/*
 * sparse_attn_bwd -- backward of sparse_attn_fwd in the SAS mode
 * (local = CURRENT_BLOCK, window = 0, alpha = NULL), recomputing the
 * probabilities from lse:
 *   D_i = do_i . o_i,  dS_ij = p_ij (do_i . v_j - D_i),
 *   dq = sum_j dS k_j / sqrt(d), dk_j = sum_i dS q_i / sqrt(d),
 *   dv_j = sum_i p_ij do_i,
 *   dg[slot of block m] = sum_{j in B_m} dS_ij / g_m  ("SAS" review §4.2.2
 *   Eq. 5, inner gate), summed over the query heads sharing the selection.
 * o and lse are the outputs of sparse_attn_fwd on the same arguments.
 * dq, dk, dv are written (not accumulated) in the input dtype; dg in fp32
 * (0 in padded slots; with logg NULL the gradient is taken at g = 1).
 * o, dout, dq, dk and dv must be 16-byte aligned (SPA_ERR_INVALID_ARG).
 */
spa_status sparse_attn_bwd(const spa_attn_args *a, const void *o, const void *dout,
                    const float *lse, void *dq, void *dk, void *dv, float *dg,
                    void *workspace, size_t ws_bytes, spa_stream_t stream);

typedef struct spa_select_grads {
    const float *dg;          /* in  [B, Hsel, nq, K] fp32, the gate gradient of
                                 sparse_attn_bwd (slots that are not candidates
                                 of their row are ignored) */
    float *dq;                /* out [B, Hq, nq, d] fp32, written */
    float *dkbar;             /* out [B, Hkv, ccap, d] fp32, written (0 for
                                 summaries that are no row's candidate) */
    float *dproj_w;           /* out [d, d] fp32, written; required exactly when
                                 the select arguments carry proj_w */
    void *dk;                 /* in/out [B, Hkv, L, d] in the key dtype, or NULL:
                                 dk_j += dkbar_c / b for each token j of block
                                 c < ccap (the summary is the block mean) */
    int64_t L;                /* tokens in dk (>= ccap * b when dk is given) */
} spa_select_grads;

/*
 * sparse_select_bwd -- selector side of the backward: the gate gradient dg
 * carried back through log g = s - LSE(s) into the query, the block
 * summaries, the learned projection and the keys ("SAS" review, "How it
 * works" step 5: the loss reaches the selector only through the gates;
 * §4.2.2 softmax gate; §3 Eq. 3 scores, mean-key summaries).  With
 * p = softmax(s) over all candidates of a row (so g_m = p_m) and its selected
 * set S held fixed, and ktilde = kbar (or W kbar with the projection):
 *   ds_c     = p_c ([c in S] dg_c - sum_{m in S} p_m dg_m),
 *   dq       = sum_c ds_c ktilde_c / sqrt(d), given to each of the G query
 *              heads of a shared selection as dq_hat / G (q_hat is their mean),
 *   dktilde_c = sum over rows and selection heads of ds_c q_hat / sqrt(d),
 *   dkbar_c  = dktilde_c, or W^T dktilde_c;  dW = sum_c dktilde_c kbar_c^T,
 *   dk_j    += dkbar_c / b (optional; the rounding of kbar to the key dtype is
 *              passed straight through).
 * `a` is the argument struct of the sparse_score_select call that produced
 * idx, validated the same way (its outputs logg and k_eff are not read; idx
 * holds distinct entries per row, as that call writes them).  Supported:
 * bf16, gate = SOFTMAX_LOG, prefix_mode = CURRENT_BLOCK, no erf term;
 * otherwise SPA_ERR_UNSUPPORTED.  dq, dkbar and dk must be 16-byte aligned.
 * Scores are recomputed from q_hat (or W^T q_hat) rounded to bf16.  Needs a
 * workspace of sparse_workspace_bytes(SPA_OP_SELECT_BWD); caller-owned,
 * contents on entry are ignored.  Deterministic: no atomics.
 */
spa_status sparse_select_bwd(const spa_select_args *a, const spa_select_grads *g, void *workspace,
                      size_t ws_bytes, spa_stream_t stream);

/* Workspace bytes needed by `op` (spa_op) for the given argument struct
 * (spa_select_args* for SPA_OP_SCORE_SELECT and SPA_OP_SELECT_BWD,
 * spa_decode_args* for SPA_OP_DECODE_STEP, spa_attn_args* otherwise).
 * Returns 0 for invalid arguments (see spa_last_error()). */
size_t sparse_workspace_bytes(int op, const void *args);

/* Zero-fill a workspace with a kernel on `stream` (graph-capture safe).  Not
 * required by any entry point; provided for callers that want deterministic
 * scratch contents. */
spa_status sparse_workspace_init(void *workspace, size_t ws_bytes, spa_stream_t stream);

/* Measurement aid, not part of the attention path: one lane follows the
 * cyclic index list `next` (device, n uint32 entries, n a power of two in
 * [1, 2^32]) for `steps` >= 1 dependent loads from `start`, each index masked
 * to n - 1 (any contents stay in bounds), and writes the last index to out[0]
 * (device).  Timed with events on `stream`, the launch gives the round-trip
 * latency of the memory level the list occupies: a decode step is a short
 * chain of such round trips.  The caller owns both buffers.  Bad arguments
 * return SPA_ERR_INVALID_ARG. */
spa_status sparse_probe_load_chase(const uint32_t *next, int64_t n, int steps, uint32_t start, uint32_t *out,
                                   spa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
