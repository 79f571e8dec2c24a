/*
 * kvsp — query-aware sparse block decode attention over a paged KV cache,
 * for AMD Instinct MI355X (CDNA4, gfx950).
 *
 * One decode step for a batch of sequences:
 *   1. every full KV block keeps a mean-key summary per KV head;
 *   2. a block's relevance to the current query is the sum, over query heads,
 *      of the inner product between the head's query and its KV head's
 *      summary;
 *   3. the top-k blocks are kept (never fewer than a minimum keep floor),
 *      and runs of adjacent picks form contiguous spans;
 *   4. attention runs over the kept blocks plus an exact window of recent
 *      tokens, as split-KV partial softmaxes merged by log-sum-exp;
 *   5. a sequence whose kept fraction exceeds the dense-fallback threshold γ
 *      is attended densely instead.
 *
 * Sources (titles and sections of the pages this follows; they define no API):
 *   SparPR news page ("SparPR: Runtime KV-Cache Recovery for Resource-
 *     Constrained LLM Inference on Consumer Hardware", aimodeling.com),
 *     section "Three decisions rather than one compression ratio":
 *     - paragraph "Query-Aware key-block selection" (steps 1-3: summaries
 *       resident on the GPU, head-summed inner-product score, Top-k);
 *     - paragraph "Dynamic budget control" (Minimum Keep Floor);
 *     - paragraph "On-demand local recomputation with cost-aware fallback"
 *       (adjacent blocks merged into spans; Dense Fallback Threshold γ).
 *   DKV abstract ("DKV: Anchor + Low-Rank Differential KV-Cache Compression
 *     for Scalable Long-Context Inference"): top-K block routing, an exact
 *     recency window, and the flash-style log-sum-exp merge of partial
 *     attentions (step 4).
 *   "KV cache offloading" (aiwiki), section "Why the cache leaves the GPU":
 *     a dense decode step reads every stored key and value (step 5); the
 *     paged block pool follows the PagedAttention layout it cites.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers; struct pointers are HOST pointers.
 *     k_pool and v_pool may also be host memory the device can read: pinned
 *     with hipHostMalloc(hipHostMallocMapped), passed as the address
 *     hipHostGetDevicePointer returns. The kernels then read, across PCIe,
 *     only the tiles they touch (for kvsp_sparse_decode: the kept blocks and
 *     the window), which is the offloaded-cache setting of the SparPR page;
 *     results are bit-identical to a device-resident pool. The decode entry
 *     points ask HIP (hipPointerGetAttributes) whether k_pool is host memory
 *     and then read K in whole rows, which PCIe carries in larger requests.
 *   - Work is enqueued on `stream` (0 = the null stream) and returns without
 *     waiting for it. No entry point allocates memory, synchronises the host
 *     or copies device data to the host. The library keeps no pointer after
 *     returning and holds no mutable global state, so calls on different
 *     streams may run concurrently (each with its own workspace).
 *   - The caller owns every buffer; inputs must stay valid until the stream
 *     work completes.
 *   - Host-checkable faults return a negative kvsp_status before anything is
 *     enqueued: a NULL required pointer, a non-positive size, num_q_heads not
 *     a multiple of num_kv_heads, an unsupported head_dim / block_size /
 *     dtype, keep_den or gamma_den <= 0, keep_floor == 0 together with
 *     recent_window == 0, or a workspace smaller than kvsp_workspace_bytes.
 *     A failed kernel launch returns KVSP_ERR_HIP.
 *   - Device data is trusted: block-table entries must lie in
 *     [0, num_phys_blocks), context_lens in [0, max_blocks_per_seq *
 *     block_size], values finite. Violations are undefined behaviour.
 *
 * Memory layouts (row-major, innermost last)
 *   q            [batch][num_q_heads][head_dim]                 dtype
 *   k_pool/v_pool[num_phys_blocks][num_kv_heads][block_size][head_dim] dtype
 *                 (one (block, KV head) tile is contiguous)
 *   block_table  [batch][max_blocks_per_seq] int32, logical -> physical block
 *   context_lens [batch] int32, tokens cached per sequence
 *   summaries    [num_phys_blocks][num_kv_heads][head_dim] float32
 *   out          [batch][num_q_heads][head_dim] float32
 *   lse          [batch][num_q_heads] float32 (natural log), may be NULL
 *   Query head h attends with KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef KVSP_H_
#define KVSP_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVSP_OK = 0,
  KVSP_ERR_INVALID_ARG = -1,
  KVSP_ERR_UNSUPPORTED = -2,
  KVSP_ERR_WORKSPACE = -3,
  KVSP_ERR_HIP = -4,
  KVSP_ERR_TOO_LARGE = -5 /* beyond the static scratch of kvsp_sparse_decode_noalloc */
} kvsp_status;

typedef enum { KVSP_F32 = 0, KVSP_F16 = 1, KVSP_BF16 = 2 } kvsp_dtype;

/* Shape of the batch and the pool (host struct). */
typedef struct {
  int32_t batch;              /* B: 1 .. 65536 */
  int32_t num_q_heads;        /* Hq: a multiple of num_kv_heads, <= 1024 */
  int32_t num_kv_heads;       /* Hkv >= 1 */
  int32_t head_dim;           /* D: 64 or 128 */
  int32_t block_size;         /* P: 16, 32, 64, 128 or 256 tokens */
  int32_t num_phys_blocks;    /* pool capacity in blocks */
  int32_t max_blocks_per_seq; /* row stride of block_table, <= 16384 */
                              /* also: num_kv_heads * head_dim <= 7168 */
  int32_t dtype;              /* kvsp_dtype of q, K and V */
} kvsp_layout;

/* Selection parameters (host struct).
 * For a sequence of L tokens: n = ceil(L / P) blocks; the exact recent window
 * is tokens [C*P, L) with C = floor(max(0, L - recent_window) / P), i.e. the
 * last recent_window tokens widened down to a block boundary; the C blocks
 * before it are the candidates.
 *   k_req = top_k                                   if top_k > 0
 *         = ceil(C * keep_num / keep_den)           otherwise (exact integers)
 *   k     = min(max(k_req, keep_floor), C)
 *   dense = C > 0 and k * gamma_den > gamma_num * C (kept fraction above γ) */
typedef struct {
  int32_t top_k;         /* > 0: absolute k in blocks; 0: use keep_num/keep_den */
  int32_t keep_num;      /* keep ratio numerator, >= 0 */
  int32_t keep_den;      /* keep ratio denominator, > 0 */
  int32_t keep_floor;    /* minimum blocks kept, >= 0 */
  int32_t recent_window; /* W tokens attended exactly, >= 0 */
  int32_t gamma_num;     /* dense fallback threshold γ = gamma_num / gamma_den */
  int32_t gamma_den;     /* > 0; γ >= 1 never falls back */
} kvsp_select_params;

/* Bytes of device workspace the calls below need for this layout. One
 * workspace of this size serves every entry point of one stream at a time.
 * It holds per-(sequence, KV head) completion counters for the split-KV
 * merge: zero-fill it once before its first use (any zero fill, e.g. a
 * zero-initialised allocation); every call that returns KVSP_OK leaves the
 * counters at zero again, so no per-call clearing is needed. Calls that share
 * one workspace must not overlap in time. */
size_t kvsp_workspace_bytes(const kvsp_layout* layout, const kvsp_select_params* params);

/* Dynamic budget control (SparPR, "Dynamic budget control"): the keep ratio
 * of the selection from the two prices of one block (one KV head group of
 * block_size tokens across all num_kv_heads heads):
 *   copy_s      = 2 * block_size * num_kv_heads * head_dim * E / h2d_bytes_per_s
 *                 (its data volume over host-to-device bandwidth, x2 for K and V;
 *                 E = element size of layout->dtype);
 *   recompute_s = 4 * block_size * hidden * num_kv_heads * head_dim / proj_flops_per_s
 *                 (rebuilding K and V from the block's hidden states through the
 *                 two attention projections only: two products of a
 *                 block_size x hidden matrix by a hidden x (num_kv_heads *
 *                 head_dim) one, 2 flops per multiply-add; with multi-head
 *                 attention num_kv_heads * head_dim = hidden, so the price
 *                 scales with block length times hidden squared).
 * The page leaves open how the ratio of the two prices becomes a keep ratio.
 * Reading taken: ratio = min(1, recompute_s / copy_s) — every candidate block
 * is kept while fetching it costs no more than rebuilding it, and the share
 * falls in proportion as the fetch grows dearer. It is returned as
 *   *keep_num = min(keep_den, ceil(ratio * keep_den))   (>= 1, never rounded down)
 * for kvsp_select_params.keep_num with keep_den as given; the selection's
 * keep_floor then bounds k from below (the page's Minimum Keep Floor).
 * copy_s and recompute_s may be NULL. Host arithmetic only (no device access,
 * no stream). Errors: a layout the other entry points reject gives the same
 * status; KVSP_ERR_INVALID_ARG for NULL model or keep_num, a non-finite or
 * non-positive bandwidth or throughput, hidden <= 0, or keep_den <= 0. Nothing
 * is written on error. */
typedef struct {
  double h2d_bytes_per_s;  /* measured host-to-device copy bandwidth, bytes/s */
  double proj_flops_per_s; /* measured throughput of the K/V projection GEMM, flop/s */
  int32_t hidden;          /* model hidden size: the projections' input width */
} kvsp_budget_model;

kvsp_status kvsp_budget_keep_ratio(const kvsp_layout* layout, const kvsp_budget_model* model,
                                   int32_t keep_den, double* copy_s, double* recompute_s,
                                   int32_t* keep_num);

/* Step 1 (SparPR, "Query-Aware key-block selection"): for every sequence b
 * and every full logical block j < floor(context_lens[b] / P), write
 *   summaries[block_table[b][j]][g][d] = (1/P) * sum_t K[block_table[b][j]][g][t][d]
 * for all KV heads g. The sum is exact-rounded: accumulated in double and
 * rounded once to float32. Entries of other physical blocks are not touched.
 * Run it when blocks fill, not per decode step. */
kvsp_status kvsp_build_summaries(const kvsp_layout* layout, const void* k_pool,
                                 const int32_t* block_table, const int32_t* context_lens,
                                 float* summaries, hipStream_t stream);

/* Decode-time append (SparPR, opening paragraphs: the cache gains one token
 * per decoded token; "Query-Aware key-block selection": full blocks carry a
 * summary). For every sequence b with 0 <= p = positions[b] <
 * max_blocks_per_seq * P, and phys = block_table[b][p / P] in
 * [0, num_phys_blocks):
 *   K[phys][g][p % P][:] = k_new[b][g][:],  V[phys][g][p % P][:] = v_new[b][g][:]
 * for all KV heads g; and when p % P == P - 1 (the token completes its block)
 *   summaries[phys][g][d] = (1/P) * sum_t K[phys][g][t][d]
 * with the same exact-rounded arithmetic as kvsp_build_summaries (the result
 * is bit-identical to it). Sequences whose position or block is out of range
 * are skipped on the device (no token this step); nothing else is written.
 *   k_new, v_new  [B][Hkv][D] device, layout->dtype; read only
 *   positions     [B] int32 device: the token index the new token takes (the
 *                 context length before this step); the caller advances its
 *                 context lengths afterwards
 *   k_pool, v_pool, summaries: as in the calls around it, updated in place
 * Needs no workspace. Calls on one stream run in order; a call must not
 * overlap another that reads or writes the same pool rows. */
kvsp_status kvsp_append_kv(const kvsp_layout* layout, const void* k_new, const void* v_new,
                           const int32_t* block_table, const int32_t* positions, void* k_pool,
                           void* v_pool, float* summaries, hipStream_t stream);

/* Steps 2-3 and the step-5 decision (SparPR, "Query-Aware key-block
 * selection", "Dynamic budget control", "On-demand local recomputation with
 * cost-aware fallback"). For every sequence b:
 *   scores[b][j]  = sum_{h} <q[b][h], summaries[block_table[b][j]][h / G]>, j < C
 *                   (computed in double from the float32 summaries, stored as
 *                   float32; the query heads of a group are summed first);
 *   selected[b][0..k) = the k candidates ranking highest by (score
 *                   descending, block index ascending), in ascending order;
 *                   -0.0 ranks equal to +0.0;
 *   num_selected[b] = k;
 *   spans[b][s] = {start, end} (logical blocks, half-open) for the maximal
 *                   runs of consecutive ids in selected ∪ [C, n), ascending;
 *                   the window run [C, n) comes last and absorbs a selected
 *                   run ending at C - 1; num_spans[b] of them;
 *   use_dense[b] = 1 if the kept fraction k / C exceeds γ, else 0.
 * The selection is always computed, also for sequences that fall back.
 * Output shapes: scores and selected [B][max_blocks_per_seq], spans
 * [B][max_blocks_per_seq + 1][2]; scores may be NULL (they then live in the
 * workspace). Entries past the counts are left as they are. The workspace is
 * required (kvsp_workspace_bytes): it also holds per-sequence counters. */
kvsp_status kvsp_score_topk(const kvsp_layout* layout, const kvsp_select_params* params,
                            const void* q, const float* summaries, const int32_t* block_table,
                            const int32_t* context_lens, float* scores, int32_t* selected,
                            int32_t* num_selected, int32_t* spans, int32_t* num_spans,
                            int32_t* use_dense, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Steps 4-5 (DKV abstract: attention over the routed blocks and the exact
 * recency window, partial softmaxes merged by a flash-style log-sum-exp;
 * SparPR, "On-demand local recomputation with cost-aware fallback": kept
 * blocks recovered as contiguous spans, and the dense path). For every
 * sequence b and query head h, attends over the kept blocks, given in one
 * of two forms (exactly one pair is non-NULL, else KVSP_ERR_INVALID_ARG):
 *   spans, num_spans        the span list kvsp_score_topk writes: the tokens
 *                           of logical blocks [start, end) of spans[b][0..
 *                           num_spans[b]), ascending, the window run last;
 *                           or
 *   selected, num_selected  the tokens of selected[b][0..num_selected[b])
 *                           (ascending candidate ids < C) followed by the
 *                           window tokens [C*P, L);
 * both describe the same tokens in the same order and give bit-identical
 * results. If use_dense is non-NULL and use_dense[b] != 0 the sequence
 * attends all tokens [0, L) instead. Logits are scale * <q, K> (scale <= 0
 * means 1/sqrt(head_dim)), accumulated in float32; writes the normalised
 * output and its log-sum-exp. params supplies recent_window (C depends on
 * it). Spans must cover block ceil(L/P) - 1 whenever it is partial (the
 * window always does). A sequence with no cached token attends nothing: its
 * out is 0 and its lse -inf. */
kvsp_status kvsp_sparse_decode(const kvsp_layout* layout, const kvsp_select_params* params,
                               const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const int32_t* context_lens,
                               const int32_t* spans, const int32_t* num_spans,
                               const int32_t* selected, const int32_t* num_selected,
                               const int32_t* use_dense, float scale, float* out, float* lse,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* kvsp_sparse_decode for callers that cannot allocate or pass device memory
 * of their own for scratch: code under HIP graph capture, tight serving
 * loops, and harnesses that forbid allocation. Same arguments, results (bit
 * for bit) and kernels as kvsp_sparse_decode, without the workspace: the
 * completion counters and split-KV partials live in a static device array of
 * the library (8 MiB per device that calls it, held until the process ends).
 * It allocates nothing and never calls hipMalloc or hipFree. The first call
 * on a device (the current device) looks the array up and zeroes its counter
 * region with a fill kernel enqueued on `stream`; a first call under stream
 * capture records that kernel in the graph and the next eager call enqueues
 * it again. Every call leaves the counters at zero.
 * Every call on one device shares that device's array, so calls that overlap
 * in time on one device (on different streams, or concurrent replays of
 * graphs holding this call) race and give undefined results; serialise them.
 * Errors: as kvsp_sparse_decode (no workspace error), plus KVSP_ERR_TOO_LARGE
 * when the layout has more than 16384 (sequence, KV head, head group)
 * counters or its split-KV partials exceed the array; checked on the host
 * before anything is enqueued. */
kvsp_status kvsp_sparse_decode_noalloc(const kvsp_layout* layout, const kvsp_select_params* params,
                                       const void* q, const void* k_pool, const void* v_pool,
                                       const int32_t* block_table, const int32_t* context_lens,
                                       const int32_t* spans, const int32_t* num_spans,
                                       const int32_t* selected, const int32_t* num_selected,
                                       const int32_t* use_dense, float scale, float* out,
                                       float* lse, hipStream_t stream);

/* Step 5 on its own ("KV cache offloading", "Why the cache leaves the GPU":
 * dense decode reads every key and value): attention of every query head
 * over all tokens [0, context_lens[b]) of its sequence. Same numerics and
 * outputs as kvsp_sparse_decode; the workspace size from
 * kvsp_workspace_bytes (with any params) covers it. */
kvsp_status kvsp_dense_decode(const kvsp_layout* layout, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_table,
                              const int32_t* context_lens, float scale, float* out, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- DKV variant: compressed older blocks -----------------------------------
 * DKV abstract ("DKV: Anchor + Low-Rank Differential KV-Cache Compression for
 * Scalable Long-Context Inference"): every block older than the recency window
 * is stored as one exact anchor token, a rank-32 truncated SVD of the joint
 * key|value difference of its tokens from the anchor, and a budget of exact
 * residual tokens (the rows the low-rank basis reconstructs worst). Decoding
 * attends the routed blocks through the low-rank factors (keys are never
 * decompressed), the residual tokens and the recency window exactly, and merges
 * the halves by log-sum-exp. Routing uses kvsp_build_summaries (run before the
 * blocks are compressed) and kvsp_score_topk as for the exact cache.
 *
 * Readings where the abstract is silent: the anchor is the block's first token;
 * the SVD is of X = [K - k_anchor | V - v_anchor] (block_size x 2*head_dim);
 * residual tokens are the n_resid rows of largest ||X_t - X_hat_t||.
 *
 * Record of one (physical block p, KV head g), at byte offset
 * (p * num_kv_heads + g) * kvsp_dkv_record_bytes() of `records`:
 *   anchor   [2][head_dim]            layout dtype: anchor K row, anchor V row
 *   basis    [32][2*head_dim] float32 at offset align16(2*D*E): row j is the
 *                                     j-th basis vector (K half, then V half)
 *   coef     [block_size][32] float32 right after basis: X_t projected on the
 *                                     basis (rows of residual tokens unused)
 *   resid_k  [n_resid][head_dim]      layout dtype, right after coef
 *   resid_v  [n_resid][head_dim]      layout dtype, right after resid_k
 *   resid    [n_resid] int32          ascending token offsets within the block
 *   rounds   int32                    the subspace-iteration rounds the codec ran
 *   padding to a multiple of 256 bytes.
 * E is the element size of the layout dtype. A compressed token t of the block
 * stands for the rows k_anchor + coef[t] . basis[:, :D] and
 * v_anchor + coef[t] . basis[:, D:]; a residual token stands for its exact rows.
 * Supported: block_size 64, 128 or 256; num_q_heads / num_kv_heads <= 16;
 * 0 <= n_resid <= min(64, block_size). */
typedef struct {
  int32_t rank;        /* must be 32 */
  int32_t n_resid;     /* exact residual tokens per block */
  int32_t power_iters; /* kvsp_dkv_compress rounds: > 0 exactly that many; 0 = per block
                          from its measured spectrum (see kvsp_dkv_compress) */
} kvsp_dkv_params;

/* Bytes of one record (see above); 0 for unsupported arguments. */
size_t kvsp_dkv_record_bytes(const kvsp_layout* layout, const kvsp_dkv_params* dkv);

/* Bytes of device workspace kvsp_dkv_decode needs. Same rules as
 * kvsp_workspace_bytes: zero-fill once before first use; calls that return
 * KVSP_OK leave it reusable; calls sharing one workspace must not overlap. */
size_t kvsp_dkv_workspace_bytes(const kvsp_layout* layout, const kvsp_dkv_params* dkv);

/* DKV codec: for every sequence b and every logical block j < C (C = floor(max(0,
 * L - recent_window) / P), the blocks wholly older than the window) writes the
 * record of (block_table[b][j], g) for every KV head g from the exact K/V rows
 * in the pools. The basis is the top-32 right singular subspace of X, found by
 * subspace iteration on 64 vectors (Q <- orth(X^T X Q): float32 products,
 * Cholesky QR in double) followed by a Rayleigh-Ritz step (the symmetric
 * eigenproblem of Q^T X^T X Q, cyclic Jacobi in double): the basis rows are
 * the Ritz vectors of the 32 largest Ritz values. The 64-vector iterate
 * converges to a subspace holding the top 32 at the rate (s_65 / s_32)^2 per
 * round whatever the gap between s_32 and s_33, so the result is the
 * truncated SVD's subspace wherever that is unique. Rounds: power_iters if
 * positive; otherwise 8, then a Rayleigh-Ritz step whose Ritz values
 * theta give the measured rate rho = theta_64 / theta_32, and
 * ceil(log(1e-6) / log(rho)) rounds in all (at least 8, at most 64); the
 * count is written to the record. A direction X does not have (Ritz value
 * at most 1e-10 of the largest) gives a zero basis row. coef = X basis^T;
 * residual tokens are the n_resid rows with the largest float32
 * reconstruction error ||X_t - coef_t basis|| (ties to the lower offset);
 * anchor and residual rows are bit-exact copies. Records of other blocks are
 * not touched; sequences sharing a physical block write identical records.
 * Needs no workspace. It runs off the per-step path: a block is compressed
 * once, when it leaves the window. */
kvsp_status kvsp_dkv_compress(const kvsp_layout* layout, const kvsp_dkv_params* dkv,
                              int32_t recent_window, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* context_lens,
                              void* records, hipStream_t stream);

/* DKV decode: for every sequence b and query head h, attention over the tokens of
 * the compressed blocks selected[b][0..num_selected[b]) (ascending ids < C, as
 * from kvsp_score_topk) read through their records, followed by the exact
 * window tokens [C*P, L) from the pools; logits scale * <q, k> (scale <= 0
 * means 1/sqrt(head_dim)); float32 accumulation; normalised out and natural-log
 * lse as for kvsp_sparse_decode. params supplies recent_window (the other
 * selection fields are ignored; there is no dense fallback: older blocks exist
 * only as records). An empty attended set gives out 0 and lse -inf. */
kvsp_status kvsp_dkv_decode(const kvsp_layout* layout, const kvsp_select_params* params,
                            const kvsp_dkv_params* dkv, const void* q, const void* k_pool,
                            const void* v_pool, const void* records, const int32_t* block_table,
                            const int32_t* context_lens, const int32_t* selected,
                            const int32_t* num_selected, float scale, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* kvsp_status_string(kvsp_status status);

/* ABI version of this header (bumped on any incompatible change). */
#define KVSP_ABI_VERSION 2
int32_t kvsp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVSP_H_ */
