/*
 * bsattn.h -- block-sparse, sliding-window and local+global attention on
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * Sources, cited by page title and section:
 *  [COBS]  "COBS: Cumulant Order Block Sparse Attention", explainer at
 *          gist.science/ja/paper/2607.09052, technical summary sections
 *          1 (problem: decode is bound by reading the KV cache), 2.1
 *          (selection by attention mass), 2.2 (cumulant expansion), 2.3
 *          (second-order score, low-rank covariance), 4.3 (rank <= 8).
 *  [ATT]   "LLMアテンション機構" (LLM attention mechanism), jisaku.com glossary:
 *          the four steps of scaled dot-product attention; GQA (FAQ Q2);
 *          KV cache section.
 *  [SWA]   "スライディングウィンドウアテンション" (sliding window attention),
 *          jisaku.com glossary: band matrix (概要と動作原理), sink and
 *          global extensions (SWAの拡張手法), skipping tiles outside the
 *          window (FlashAttentionとの組み合わせ).
 *  [LG]    "ローカル・グローバルアテンション" (local-global attention),
 *          jisaku.com glossary: local window, bidirectional global tokens,
 *          uniform placement of globals.
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no state between calls.  Host arrays are
 *    marked _host and are read during the call only.
 *  - Calls are asynchronous on the given HIP stream (NULL = default stream).
 *    Every argument is checked on the host before any launch; a bad argument
 *    returns BSATTN_ERR_INVALID or BSATTN_ERR_UNSUPPORTED and launches nothing.
 *    A failed launch returns BSATTN_ERR_HIP.  Faults inside a kernel surface
 *    at the caller's next synchronisation.  bsattn_last_error() gives a
 *    message for the last failure on the calling thread.
 *  - Layouts are dense, row-major (C order), 16-byte aligned base pointers:
 *      decode  Q [B, Hq, d],          O [B, Hq, d] fp32, lse [B, Hq] fp32
 *      prefill Q [B, Hq, N, d],       O [B, Hq, N, d] fp32, lse [B, Hq, N] fp32
 *      K, V    [B, Hkv, kv_capacity, d]  (token t of (b, g) at row t)
 *      mean    [B, Hkv, nblk_capacity, d] fp32 or bf16 (mean_dtype)
 *      factor  [B, Hkv, nblk_capacity, rank, e] fp32, or FP4 (factor_dtype):
 *              codes uint8 [B, Hkv, nblk_capacity, rank, e/2] (entry 2i in the
 *              low nibble of byte i, 2i+1 in the high nibble) and
 *              factor_scale [B, Hkv, nblk_capacity, rank] fp32; e = d, or
 *              sub_dim with a query-subspace basis
 *      basis   [Hkv, sub_dim, d] fp32, orthonormal rows
 *  - GQA [ATT FAQ Q2]: query head h reads K/V head h / (Hq / Hkv).
 *  - Blocks [COBS 1, 2.1]: block j holds tokens [j*S, (j+1)*S); only complete
 *    blocks ((j+1)*S <= n_ctx) have summaries and can be selected.
 *  - Softmax scale: shape.scale, or 1/sqrt(d) when it is 0 [ATT step 2].
 *    lse is the natural log of the softmax normaliser of the scaled logits.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSATTN_OK = 0,
  BSATTN_ERR_INVALID = 1,     /* argument out of range, NULL, inconsistent shape  */
  BSATTN_ERR_UNSUPPORTED = 2, /* valid request the library does not implement      */
  BSATTN_ERR_HIP = 3,         /* a HIP launch or runtime call failed               */
  BSATTN_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required        */
  BSATTN_STATUS_INT32 = 0x7fffffff /* not a status: keeps every int32 value in range */
} bsattn_status;

typedef enum {
  BSATTN_F32 = 0,
  BSATTN_BF16 = 1,
  BSATTN_FP4_E2M1 = 2 /* factor rows only: 4-bit codes + one float32 scale per row */
} bsattn_dtype;

typedef struct {
  int32_t batch;       /* B >= 1                                                   */
  int32_t n_q_heads;   /* Hq >= 1, a multiple of n_kv_heads                        */
  int32_t n_kv_heads;  /* Hkv >= 1                                                 */
  int32_t head_dim;    /* d: 64 or 128                                             */
  int32_t n_ctx;       /* decode: tokens in the cache; prefill: sequence length N  */
  int32_t kv_capacity; /* token stride of K/V per (b, kv head), >= n_ctx           */
  int32_t block_size;  /* S: 64                                                    */
  float scale;         /* softmax scale; 0 => 1/sqrt(d)                             */
  int32_t dtype;       /* bsattn_dtype of Q, K, V                                   */
} bsattn_shape;

/*
 * A paged K/V cache [ATT KV cache section: PagedAttention allocates the cache
 * page by page]: K and V are pools of pages [n_pages, Hkv, page_tokens, d]
 * (shape.dtype); token t of batch entry b is row t % page_tokens of page
 * block_table[b * max_pages + t / page_tokens], the same page number for every
 * K/V head.  page_tokens: 16, 32 or 64 (16 tokens of bf16 at d = 128 is a
 * 4 KB page per head).  block_table: device int32 [B, max_pages]; entries for
 * tokens < n_ctx must be page numbers in [0, n_pages).  Reads clamp every
 * entry into that range, so a bad entry reads a wrong row, never outside the
 * pools; bsattn_append_kv writes nothing for an entry outside it (an
 * unallocated page), so a bad entry never overwrites another sequence's page.
 * With a paged cache shape.kv_capacity must equal max_pages * page_tokens.
 * Calls that take a `paged` argument use the contiguous layout
 * [B, Hkv, kv_capacity, d] when it is NULL.  The sparse decode reads paged
 * caches in BF16 only.
 */
typedef struct {
  const int32_t* block_table;
  int32_t page_tokens;
  int32_t max_pages;
  int32_t n_pages;
} bsattn_paged_kv;

#define BSATTN_MAX_RANK 8        /* [COBS 4.3]: rank <= 8 recommended               */
#define BSATTN_MAX_GLOBAL 256    /* global token positions per call                  */
#define BSATTN_MAX_TOP_K 1024
#define BSATTN_MAX_BLOCKS 65536  /* complete blocks per (b, kv head) for selection   */
#define BSATTN_MAX_GROUP 16      /* query heads per K/V head (Hq / Hkv)              */
#define BSATTN_MAX_DILATION 65536 /* key spacing of a dilated prefill window         */

/*
 * Per-block key summaries [COBS 2.2, 2.3].
 * For every (b, g) and every block j in [first_block, first_block + n_blocks):
 *   mean[b,g,j,:]     = (1/L) sum_{t in block j} K[b,g,t,:]          (L = S)
 *   factor[b,g,j,i,:] = sqrt(lambda_i) v_i, i < rank, the i-th largest
 *                       eigenpair of Sigma = (1/L) sum (k - mean)(k - mean)^T,
 *                       sign fixed so the entry of largest magnitude is > 0;
 *                       eigenvalues below 0 clamp to 0.
 * Built once per block, as blocks fill (incremental use: pass the new range).
 * K dtype: F32 or BF16.  rank in [0, BSATTN_MAX_RANK]; factor may be NULL
 * when rank == 0.  Requires (first_block + n_blocks) * S <= n_ctx and
 * first_block + n_blocks <= nblk_capacity.  n_blocks == 0 is a no-op.
 * mean_dtype: BSATTN_F32 stores the mean in fp32; BSATTN_BF16 stores it
 * rounded to bfloat16 (nearest, ties to even), the block-mean storage of
 * [COBS 2.3, compression]; the covariance is taken about the unrounded mean
 * either way.  factor_dtype: BSATTN_F32 stores the factor rows in fp32;
 * BSATTN_FP4_E2M1 stores them as [COBS 2.3, compression] stores eigenvectors:
 * per row a float32 scale (the row's largest magnitude / 6) in factor_scale
 * and each entry as the E2M1 code nearest to entry / scale (ties to the even
 * code); factor_scale is ignored for BSATTN_F32 (may be NULL).
 * Query-subspace projection [COBS 2.3, compression]: with sub_dim > 0 and a
 * basis P_g (rows spanning K/V head g's query subspace, for instance the
 * leading eigenvectors of its queries' second moment, taken offline) the
 * factor rows are those of the projected covariance P_g Sigma P_g^T, i.e.
 * of the projected centred keys P_g (k - mean): sub_dim numbers per row
 * instead of d.  sub_dim: 0 (no basis; basis may be NULL) or a multiple of
 * 32 in [32, d], with rank >= 1; the orthonormality of the rows is the
 * caller's (not checked).  The mean is not projected.  The calls that read the
 * summaries take the same mean_dtype, factor_dtype, factor_scale, basis and
 * sub_dim.
 */
bsattn_status bsattn_build_summaries(const bsattn_shape* shape, const void* K, int32_t rank,
                                     int32_t first_block, int32_t n_blocks,
                                     int32_t nblk_capacity, void* mean, int32_t mean_dtype,
                                     void* factor, int32_t factor_dtype, float* factor_scale,
                                     const float* basis, int32_t sub_dim, const bsattn_paged_kv* paged,
                                     void* hip_stream);

/*
 * Append the decode token to the cache and keep the summaries current
 * [COBS 1 (decode reads the cache block by block); ATT KV cache]: the new
 * token is t = n_ctx - 1 (shape is the one of the decode step that follows,
 * n_ctx counting the new token; n_ctx <= kv_capacity).  For every (b, g):
 *   K[b,g,t,:] = K_new[b,g,:],  V[b,g,t,:] = V_new[b,g,:]
 * with K_new, V_new [B, Hkv, d] of shape.dtype.  When t completes block
 * j = n_ctx / S - 1 (n_ctx % S == 0), block j's summary is then built exactly
 * as bsattn_build_summaries(shape, K, rank, j, 1, ...) builds it, with the
 * summary arguments given here; they are read (and validated) only then.
 * Invalid arguments launch nothing.  Ordered after earlier calls on the stream.
 */
bsattn_status bsattn_append_kv(const bsattn_shape* shape, const void* K_new, const void* V_new, void* K,
                               void* V, int32_t rank, int32_t nblk_capacity, void* mean,
                               int32_t mean_dtype, void* factor, int32_t factor_dtype,
                               float* factor_scale, const float* basis, int32_t sub_dim,
                               const bsattn_paged_kv* paged, void* hip_stream);

/*
 * Block selection for the decode query (the last cached token, t = n_ctx - 1).
 *  1. Per query head h and complete block j, with q~ = scale * Q[b,h]:
 *       s[h,j] = q~ . mean_j                                (rank == 0) [COBS 2.2]
 *       s[h,j] = q~ . mean_j + 1/2 sum_i (factor_{j,i} . q~)^2  (rank > 0) [COBS 2.3]
 *     with a query-subspace basis the factor rows meet the projected query P_g q~.
 *  2. Group score per K/V head g: scores[b,g,j] = ln sum_{h in g} exp(s[h,j]),
 *     the log of the group's estimated attention mass [COBS 2.1].
 *  3. Forced tokens F: [0, n_sink) sinks [SWA 拡張手法], the window
 *     [t - window + 1, t] [SWA], and the global positions [LG].
 *     Candidates: complete blocks with at least one token outside F.
 *  4. sel[b,g,:] = the top_k candidates by (score descending, index
 *     ascending), written in ascending order, padded with -1.
 * Q: [B,Hq,d] of shape.dtype.  mean/factor as built above (factor NULL iff
 * rank == 0; mean_dtype, factor_dtype and factor_scale as they were built
 * with; an FP4 factor row enters the score as its codes' values times its
 * scale; basis and sub_dim as they were built with: a basis needs BF16 Q,
 * BSATTN_BF16 means and BSATTN_FP4_E2M1 factors, the explainer's compressed
 * summary, else BSATTN_ERR_UNSUPPORTED).  scores: REQUIRED [B,Hkv,nblk_capacity] fp32; entries of complete
 * blocks are written (it is also the buffer the top-k pass reads).
 * global_pos_host: sorted, unique, in [0, n_ctx), n_global <= BSATTN_MAX_GLOBAL.
 * top_k in [1, BSATTN_MAX_TOP_K]; n_ctx / S <= BSATTN_MAX_BLOCKS.
 * window >= 0 (0: no window), n_sink >= 0; sizes past n_ctx are clamped.
 */
bsattn_status bsattn_select_topk(const bsattn_shape* shape, const void* Q, const void* mean,
                                 int32_t mean_dtype, const void* factor, int32_t factor_dtype,
                                 const float* factor_scale, const float* basis, int32_t sub_dim,
                                 int32_t rank, int32_t nblk_capacity,
                                 int32_t top_k, int32_t window, int32_t n_sink,
                                 const int32_t* global_pos_host, int32_t n_global, int32_t* sel,
                                 float* scores, void* hip_stream);

/*
 * Selection by exact block mass, the selection oracle [COBS 2.1]: as
 * bsattn_select_topk (same candidates, top-k order and outputs), but the
 * group score of block j is read from the keys themselves,
 *   scores[b,g,j] = ln sum_{h in g} sum_{t in block j} exp(q~_h . K[b,g,t,:]),
 * the group's exact attention mass on the block.  It reads every key of the
 * context, so it is a reference (a quality upper bound for the summary-based
 * selectors), not a fast path.  Q [B,Hq,d] and K [B,Hkv,kv_capacity,d] BF16
 * (contiguous); scores [B,Hkv,nblk_capacity] fp32; sel [B,Hkv,top_k] int32.
 */
bsattn_status bsattn_select_exact(const bsattn_shape* shape, const void* Q, const void* K,
                                  int32_t nblk_capacity, int32_t top_k, int32_t window, int32_t n_sink,
                                  const int32_t* global_pos_host, int32_t n_global, int32_t* sel,
                                  float* scores, void* hip_stream);

/* Bytes of device workspace bsattn_decode needs for these arguments (0 if invalid, or
 * when one partial per (b, K/V head) suffices and no workspace is needed). */
size_t bsattn_decode_workspace_bytes(const bsattn_shape* shape, int32_t top_k, int32_t window,
                                     int32_t n_sink, int32_t n_global);

/*
 * Sparse decode [COBS 1, 2.1; SWA 拡張手法; LG]: for every query head h of
 * K/V head g, one softmax of scale * Q[b,h] . K[b,g,t] over the token set
 *   T = F  union  { tokens of block j : j in sel[b,g,:], j >= 0 }
 * (a set: a token reached two ways counts once), O[b,h] = sum_T p_t V[b,g,t],
 * lse[b,h] = ln sum_T exp(logit_t).  sel: [B,Hkv,top_k] int32 as written by
 * bsattn_select_topk (ascending, -1 padded, each entry a complete block).
 * dtype F32 or BF16.  workspace: device memory of at least
 * bsattn_decode_workspace_bytes(...) bytes, 256-byte aligned, holding the
 * split partials; its contents need not be initialised (NULL when that size is 0).  lse may be NULL.
 * Calls that share a workspace must be ordered (same stream); calls with
 * separate workspaces may overlap.
 */
bsattn_status bsattn_decode(const bsattn_shape* shape, const void* Q, const void* K,
                            const void* V, const int32_t* sel, int32_t top_k, int32_t window,
                            int32_t n_sink, const int32_t* global_pos_host, int32_t n_global,
                            float* O, float* lse, void* workspace, size_t ws_bytes,
                            const bsattn_paged_kv* paged, void* hip_stream);

/*
 * One decode step in one call: the selector's scores and top-k
 * (bsattn_select_topk) followed by the sparse decode (bsattn_decode), with the
 * same arguments, outputs and limits as those two calls together: sel and
 * scores are written as bsattn_select_topk writes them, O and lse as
 * bsattn_decode writes them [COBS 1, 2.1-2.3; SWA 拡張手法; LG].  workspace:
 * at least bsattn_decode_workspace_bytes(shape, top_k, window, n_sink,
 * n_global) bytes, 256-byte aligned, contents need not be initialised (NULL
 * when that size is 0).  With BF16 K/V and top_k <= 256 the top-k runs inside
 * the decode kernel while the sink and window loads are in flight (each
 * decode wave selects its pair's blocks alone up to 512 complete blocks, each
 * decode workgroup selects them together up to 2048), one launch fewer than
 * the two calls; the selection is the same exact top-k (score descending,
 * then block index ascending).  With at most 512 blocks, rank == 0 and BF16
 * means, the decode workgroups also compute the scores (the same products and
 * sums as the scoring kernel), so the step has no scoring launch.  With FP32
 * K/V, rank == 0, FP32 means, at most 256 complete blocks and at most 16
 * items per pair (top_k plus the blocks holding forced tokens), the step is
 * one launch: one decode workgroup per (b, K/V head) scores the blocks,
 * selects (the same exact order) and attends, and writes O itself.
 * Otherwise the step runs the two calls' kernels.  Calls
 * that share a workspace must be ordered (same stream).
 */
bsattn_status bsattn_decode_step(const bsattn_shape* shape, const void* Q, const void* K,
                                 const void* V, const void* mean, int32_t mean_dtype,
                                 const void* factor, int32_t factor_dtype,
                                 const float* factor_scale, const float* basis, int32_t sub_dim,
                                 int32_t rank, int32_t nblk_capacity, int32_t top_k,
                                 int32_t window, int32_t n_sink, const int32_t* global_pos_host,
                                 int32_t n_global, int32_t* sel, float* scores, float* O,
                                 float* lse, void* workspace, size_t ws_bytes,
                                 const bsattn_paged_kv* paged, void* hip_stream);

/*
 * bsattn_decode_step without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments, outputs and limits as
 * bsattn_decode_step, with the split partials kept in a static device array of
 * BSATTN_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends (its address is looked up once per device, on the
 * first call with that device current).  A call whose partials would exceed it
 * (bsattn_decode_workspace_bytes(shape, top_k, window, n_sink, n_global) >
 * BSATTN_NOALLOC_SCRATCH_BYTES) returns BSATTN_ERR_WORKSPACE and launches
 * nothing.  The call allocates nothing.  Every call on one device shares that
 * device's array: calls that overlap on one device (different streams without
 * ordering) race and give undefined results; calls ordered on a stream are
 * safe (the partials need no initialisation: each call writes every partial
 * it reads).
 */
#define BSATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
bsattn_status bsattn_decode_step_noalloc(const bsattn_shape* shape, const void* Q, const void* K,
                                         const void* V, const void* mean, int32_t mean_dtype,
                                         const void* factor, int32_t factor_dtype,
                                         const float* factor_scale, const float* basis, int32_t sub_dim,
                                         int32_t rank, int32_t nblk_capacity, int32_t top_k,
                                         int32_t window, int32_t n_sink, const int32_t* global_pos_host,
                                         int32_t n_global, int32_t* sel, float* scores, float* O,
                                         float* lse, const bsattn_paged_kv* paged, void* hip_stream);

/*
 * Masked prefill attention, BF16 Q/K/V, fp32 O and lse.  Query i sees key j iff
 *   (i - window_left <= j <= i + window_right) [and j <= i when causal]
 *   or i is a global position or j is a global position.
 * A negative window_left / window_right means no limit on that side.
 *  - Causal band [SWA 概要と動作原理]: window_left = w - 1, window_right = 0,
 *    causal = 1 (each token sees itself and the w - 1 tokens before it).
 *  - Local + global [LG]: window_left = window_right = 256, causal = 0 and
 *    the global positions (sorted, unique, in [0, N), at most BSATTN_MAX_GLOBAL).
 * Global tokens are bidirectional; causal = 1 with n_global > 0 returns
 * BSATTN_ERR_UNSUPPORTED.  Key tiles wholly outside the mask are skipped
 * [SWA FlashAttentionとの組み合わせ].  lse may be NULL.  Q/O row stride is
 * N = n_ctx; K/V row stride is kv_capacity.
 * workspace: with n_global > 0, device memory of at least
 * bsattn_prefill_workspace_bytes(shape, n_global) bytes, 256-byte aligned (the
 * key-split partials of the global query rows; contents need not be
 * initialised); with n_global == 0 it is not read and may be NULL.  Calls that
 * share a workspace must be ordered (same stream).
 */
bsattn_status bsattn_prefill(const bsattn_shape* shape, const void* Q, const void* K,
                             const void* V, int32_t window_left, int32_t window_right,
                             int32_t causal, const int32_t* global_pos_host, int32_t n_global,
                             float* O, float* lse, void* workspace, size_t ws_bytes,
                             void* hip_stream);

/*
 * Dilated sliding-window prefill [SWA 拡張手法: dilated SWA thins the window's
 * positions so the same computation covers a wider range], BF16 Q/K/V, fp32 O
 * and lse.  Query i sees key j iff
 *   (i - window_left <= j <= i + window_right) [and j <= i when causal]
 *   and (i - j) is a multiple of `dilation`.
 * A causal window of w keys at spacing s is window_left = (w - 1) s,
 * window_right = 0, causal = 1.  dilation in [1, BSATTN_MAX_DILATION]
 * (1: the plain band of bsattn_prefill); a negative window side is unlimited.
 * No global tokens.  Computed as one launch per residue class r of the
 * positions mod s: the rows and keys r, r + s, r + 2s, ... form a plain band
 * with the windows divided by s (rounded down), run by the band kernel over a
 * strided view, so the work is the allowed pairs' and no stride test runs per
 * element.  lse may be NULL.  Q/O row stride is N = n_ctx; K/V row stride is
 * kv_capacity.  Layouts and ownership as bsattn_prefill; no workspace.
 */
bsattn_status bsattn_prefill_dilated(const bsattn_shape* shape, const void* Q, const void* K,
                                     const void* V, int32_t window_left, int32_t window_right,
                                     int32_t causal, int32_t dilation, float* O, float* lse,
                                     void* hip_stream);

/*
 * Block-sparse causal prefill, NSA-style block selection shared by a query
 * tile [BLOG NSA data flow: coarse compression, then fine selection; COBS 2.1,
 * 2.2, 2.3 (COBS builds on NSA's selection branch)].  Query tiles are the
 * BSATTN_SPARSE_TILE consecutive rows [128 t, 128 t + 128) of a sequence.
 *
 * bsattn_select_prefill: for every (b, K/V head g, tile t) and complete block j,
 *   scores[b,g,t,j] = ln sum over the tile's rows i and g's query heads h of
 *                     exp(q~_{i,h} . mean_j),  q~ = scale * Q[b,h,i]
 * (written for the tile's candidates; other entries are left undefined), and
 * sel[b,g,t,:] = the top_k candidates by (score descending, index ascending),
 * ascending, -1 padded.  Candidates of tile t: complete blocks j with
 * 64 j < i_last - window_left (a key before the window of the tile's last row
 * i_last) and 64 (j + 1) > n_sink (not wholly inside the sinks).
 * Q [B, Hq, n_ctx, d] BF16; mean [B, Hkv, nblk_capacity, d] BF16 as built by
 * bsattn_build_summaries (mean_dtype must be BSATTN_BF16); scores
 * [B, Hkv, n_tiles, nblk_capacity] fp32; sel [B, Hkv, n_tiles, top_k] int32;
 * n_tiles = ceil(n_ctx / 128).  top_k in [1, BSATTN_SPARSE_MAX_TOP_K];
 * window_left >= 0; n_sink in [0, BSATTN_SPARSE_MAX_SINK].
 *
 * bsattn_sparse_prefill: row i of every query head attends, in one softmax,
 * the union of its causal window [i - window_left, i], the sinks
 * [0, min(n_sink, i + 1)) and the keys <= i of its tile's selected blocks
 * (sel as written above; entries outside the complete blocks are ignored), a
 * key reached twice counted once.  Q, K, V BF16 (K, V [B, Hkv, kv_capacity, d]);
 * O [B, Hq, n_ctx, d] fp32, lse [B, Hq, n_ctx] fp32 (may be NULL).
 */
#define BSATTN_SPARSE_TILE 128
#define BSATTN_SPARSE_MAX_TOP_K 256
#define BSATTN_SPARSE_MAX_SINK 256
bsattn_status bsattn_select_prefill(const bsattn_shape* shape, const void* Q, const void* mean,
                                    int32_t mean_dtype, int32_t nblk_capacity, int32_t top_k,
                                    int32_t window_left, int32_t n_sink, int32_t* sel, float* scores,
                                    void* hip_stream);
bsattn_status bsattn_sparse_prefill(const bsattn_shape* shape, const void* Q, const void* K,
                                    const void* V, const int32_t* sel, int32_t top_k,
                                    int32_t window_left, int32_t n_sink, float* O, float* lse,
                                    void* hip_stream);

/*
 * Gather probe, a measurement aid rather than a step of the method: the HBM
 * bandwidth a loads-only gather of K/V blocks reaches, the ceiling against
 * which the sparse decode's gathered bytes are compared (decode is bound by the
 * KV bytes it reads [COBS 1]).  For every (b, K/V head) pair p = b * Hkv + g it
 * reads the K and V rows of the blocks blocks[p, 0 .. n_blocks - 1] (device
 * int32 [B * Hkv, n_blocks]; each entry is clamped into [0, kv_capacity / 64),
 * so every access stays inside the cache; list a block twice and it is read
 * twice) and does no arithmetic with them: each thread folds the 32-bit words
 * it loaded into one XOR, written to checksum (device uint32
 * [B * Hkv * wg_per_pair * 256]); the XOR of all entries is the XOR of every
 * word of the listed blocks.  The pair's 32-token half blocks are dealt in even
 * runs to the 4 * wg_per_pair waves of its wg_per_pair workgroups (1 .. 16;
 * the decode uses 2 at the 32K, 8 K/V-head, batch-16 shape), each keeping depth
 * (1 .. 4) half blocks of K and V in flight.  shape: dtype BF16, d 64 or 128,
 * the decode's limits; the cache is contiguous [B, Hkv, kv_capacity, d].
 * Caller-owned device memory, asynchronous on hip_stream.
 */
bsattn_status bsattn_probe_gather(const bsattn_shape* shape, const void* K, const void* V,
                                  const int32_t* blocks, int32_t n_blocks, int32_t wg_per_pair,
                                  int32_t depth, uint32_t* checksum, void* hip_stream);

/* Bytes of device workspace bsattn_prefill needs with n_global global positions
 * (0 when n_global == 0 or the arguments are invalid). */
size_t bsattn_prefill_workspace_bytes(const bsattn_shape* shape, int32_t n_global);

/* Static description of a status code. */
const char* bsattn_status_string(bsattn_status status);

/* Message describing the last failed call on this thread ("" if none). */
const char* bsattn_last_error(void);

/* Library version string. */
const char* bsattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
