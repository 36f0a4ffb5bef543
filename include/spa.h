/*
 * spa.h -- C ABI of the sparse paged decode-attention library (libspa.so),
 * written for AMD Instinct MI355X (gfx950).
 *
 * The library implements one decode step of LServe-style unified sparse
 * attention over a hierarchical paged KV cache:
 *   - streaming heads attend to the first `sink` tokens plus the last `window`
 *     tokens (LServe write-up, bqwf.cn, "2.1 混合稀疏注意力机制", static
 *     sparsity; the sink + local-window pattern is the StreamingLLM row of the
 *     sparse-method table in the long-context survey, xllm-io.github.io,
 *     "2.2" / sparse attention methods);
 *   - dynamic heads score every logical page from its per-channel min/max key
 *     summary, keep the best pages under a token budget, reuse that choice for
 *     several decode steps and attend only to the chosen pages (LServe
 *     write-up, "2.1" dynamic sparsity, and "3.2 解码阶段加速", reusable page
 *     selector and dynamic budget);
 *   - the KV cache lives in a pool of large physical pages, each holding
 *     several small logical pages; a per-sequence page table maps logical
 *     positions to physical pages (LServe write-up, "2.2 分层分页KV缓存").
 *
 * Conventions shared by every call
 *   - All device pointers are owned by the caller. The library never
 *     allocates, frees or synchronises device memory; every call only
 *     enqueues kernels on `stream` and returns.
 *   - Argument errors are found on the host, before anything is enqueued;
 *     the call then returns a non-zero spa_status and spa_last_error() holds
 *     a message (thread-local). A failed kernel launch returns SPA_ERR_HIP.
 *   - bf16 tensors are IEEE bfloat16 bit patterns (uint16). Inputs must be
 *     finite.
 *   - Positions: sequence b holds tokens 0 .. L_b-1, where L_b = seq_lens[b]
 *     counts the token appended in the current step. Token t of sequence b
 *     lives in physical page page_table[b][t / P] at slot t % P.
 *   - Query head i reads KV head i / G with G = H_q / H_kv (grouped-query
 *     attention, long-context survey "2.3 分组查询注意力 (GQA)"; G = H_q is
 *     multi-query attention, "2.4").
 *   - Kernels never read or write outside the buffers described here, even
 *     for bad device-side values: page ids outside [0, N) are skipped,
 *     seq_lens are clamped to [0, max_pages * P], selected page ids outside
 *     the sequence are skipped. Results for such inputs are unspecified.
 *
 * Pool layout in HBM (the method fixes only that logical pages sit inside
 * physical pages; the in-page order is ours):
 *   k_pool   bf16 [N][H_kv][P][D]        token-major: one logical page of one
 *                                        head is p*D*2 contiguous bytes
 *   v_pool   bf16 [N][H_kv][P/p][D][p]   channel-major inside each logical
 *                                        page (the page is transposed), also
 *                                        p*D*2 contiguous bytes
 *   summary  bf16 [N][H_kv][P/p][2][D]   per logical page: [0] = channel-wise
 *                                        minimum of its keys, [1] = maximum
 */
#ifndef SPA_H
#define SPA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spa_status {
  SPA_OK = 0,
  SPA_ERR_INVALID = 1,        /* bad argument: null pointer, size out of range, shapes that disagree */
  SPA_ERR_UNSUPPORTED = 2,    /* well-formed but not built: head_dim != 128, p not 16/32/64, G above
                                 16, a selection over more than 32768 logical pages per
                                 sequence (max_pages * P / p > 32768), 2^32 or more summary records */
  SPA_ERR_POOL_EXHAUSTED = 3, /* page allocator has fewer free pages than requested */
  SPA_ERR_WORKSPACE = 4,      /* workspace missing or smaller than spa_workspace_bytes() */
  SPA_ERR_HIP = 5             /* a HIP runtime call failed (kernel launch) */
} spa_status;

/* The physical-page pool of one attention layer. */
typedef struct spa_pool {
  int32_t num_kv_heads;   /* H_kv, 1..128 */
  int32_t head_dim;       /* D, must be 128 */
  int32_t logical_page;   /* p, tokens per logical page: 16, 32 or 64 (the write-up caps it at 64, "5.3") */
  int32_t physical_page;  /* P, tokens per physical page: a multiple of p, P/p <= 64 */
  int32_t num_phys_pages; /* N >= 1 */
  void* k_pool;           /* device bf16 (or fp8 codes, see kv_format) [N][S][P][D] */
  void* v_pool;           /* device bf16 (or fp8 codes) [N][S][P/p][D][p] */
  void* summary;          /* device bf16 [N][S][P/p][2][D]; may be NULL when no head is dynamic */
  /* S, head slots per physical page. 0 (or H_kv): every page holds every KV
   * head, head h in slot h. Fewer (at least the number of dynamic and of
   * streaming heads): the compact layout of window-only storage -- the page
   * table's pages hold the dynamic heads, head h in slot (dynamic heads below
   * h), and the rings of spa_batch.stream_pages hold the streaming heads, in
   * slot (streaming heads below h); every call then needs the head kinds, and
   * the rings whenever a head is streaming. With half the heads streaming this
   * halves the pool. */
  int32_t head_slots;
  /* Storage format of k_pool and v_pool. SPA_KV_BF16 (0): bf16 elements.
   * SPA_KV_FP8 (1): fp8 pages -- the same layouts with one-byte OCP E4M3
   * codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest
   * finite 448) and one fp32 scale per row in k_scale / v_scale; a row's
   * value is code value x scale. The LServe write-up ("5.2 参数调优指南")
   * sets the KV cache to fp8 and the long-text article at lshu.cn ("4.2 KV
   * Cache Quantization（INT8/FP8）") keeps K and V in E4M3; the scale rule is
   * this library's: scale = amax / 448 over the row's D values (one fp32
   * division), code = x / scale (fp32 division) rounded to the nearest E4M3
   * value, ties to even; a row of zeros has scale 0 and codes 0. The writes
   * (spa_kv_pool_write, spa_kv_pool_append) quantize the caller's bf16 rows;
   * summaries stay bf16: the exact min / max of the dequantized keys in IEEE
   * totalOrder (-0 below +0) rounded outward (min down, max up), so each
   * still bounds every q.k of its page; an append merges its key rounded
   * outward into the stored summary (the same result, rounding outward being
   * monotone). The append entry points append inside the attention and
   * scoring launches on fp8 pools as on bf16 ones. Non-finite inputs give
   * unspecified codes. */
  int32_t kv_format;
  float* k_scale;         /* SPA_KV_FP8: device fp32 [N][S][P], one scale per key row; else unused */
  float* v_scale;         /* SPA_KV_FP8: device fp32 [N][S][P], one scale per value row (token); else unused */
} spa_pool;

#define SPA_KV_BF16 0
#define SPA_KV_FP8 1

/* Which KV heads are streaming and which are dynamic, and the streaming
 * pattern. The `kind` array is read on the host during the call only. */
typedef struct spa_heads {
  int32_t num_q_heads;    /* H_q: a multiple of H_kv with G = H_q / H_kv from 1 to 16 */
  int32_t sink;           /* streaming heads attend tokens [0, min(sink, L)), sink >= 0 */
  int32_t window;         /* ... and tokens [max(sink, L - window), L), window >= 1 */
  const uint8_t* kind;    /* host [H_kv]: 0 = streaming head, 1 = dynamic head */
} spa_heads;

/* The decode batch: B sequences sharing one pool. */
typedef struct spa_batch {
  int32_t batch;              /* B >= 0; B == 0 makes every call a no-op */
  int32_t max_pages;          /* columns of page_table (physical pages per sequence), >= 1 */
  const int32_t* page_table;  /* device int32 [B][max_pages]: physical page ids in [0, N) */
  const int32_t* seq_lens;    /* device int32 [B]: L_b, tokens in sequence b after this step's append */
  /* NULL, or device int32 [B]: window-only storage of the streaming heads.
   * Sequence b keeps its streaming heads' rows in the R consecutive physical
   * pages stream_pages[b] .. stream_pages[b] + R - 1 (R from
   * spa_stream_ring_pages), not in the page table's pages: position t lives in
   * ring slot t/P while t/P < S = ceil(sink / P) (the sink's pages), else in
   * slot S + (t/P - S) mod (R - S); the window's pages reuse the slots in turn.
   * Only tokens a step can still attend are kept (the sink, and the window),
   * so a sequence's streaming heads need R pages whatever its length; the
   * page table then serves the dynamic heads only. A ring outside the pool
   * leaves the streaming heads' tokens unmapped (not attended, not written).
   * Needs the head kinds in every call that takes them (calls without them
   * return SPA_ERR_INVALID). LServe write-up "2.1" (streaming heads attend
   * the sink and a local window only); the rolling ring of a window's
   * keys and values, long-text article at lshu.cn, section "4.3"
   * (StreamingLLM rolling cache). */
  const int32_t* stream_pages;
} spa_batch;

/* ---- a1 (+ a2): append one token per sequence -------------------------
 * Writes the key and value of token L_b - 1 of every sequence b into its
 * pool slot (physical page page_table[b][(L_b-1)/P], slot (L_b-1) % P).
 *   heads: NULL, or the head kinds; when given, the same launch also rebuilds
 *          the summary of the logical page receiving the token for every
 *          dynamic head (the same result as spa_page_summary_update with
 *          first_pos NULL afterwards);
 *   k_new, v_new: device bf16 [B][H_kv][D], read only.
 * Sequences with L_b < 1 are skipped.
 * LServe write-up "2.2 分层分页KV缓存" (pool of physical pages holding
 * logical pages); paged store of the long-context survey "3.4 KV 缓存分页";
 * min-max page summaries, write-up "2.1". */
spa_status spa_kv_pool_append(const spa_pool* pool, const spa_heads* heads,
                              const spa_batch* batch, const void* k_new,
                              const void* v_new, hipStream_t stream);

/* Bulk write of tokens [start, start + count) of ONE sequence (prefill, or a
 * chunk of it).
 *   stream_base: -1, or the first page of the sequence's ring (its
 *          stream_pages entry, see spa_batch; needs `heads`): the streaming
 *          heads then keep only the sink's pages and the last R - S pages of
 *          the range, in their ring slots;
 *   heads: NULL, or the head kinds; when given, the same pass also builds the
 *          summary of every logical page it writes into, for every dynamic
 *          head, over the page's tokens below start + count (tokens of the
 *          page before `start` are read from the pool): the same result as
 *          spa_page_summary_update with first_pos = start and
 *          L = start + count afterwards;
 *   page_table_row: device int32 [max_pages], that sequence's row;
 *   k, v: device bf16 [H_kv][count][D] in logical (position) order.
 * Tokens of the pool outside the range are left as they are.
 * Requires 0 <= start, count >= 0, start + count <= max_pages * P.
 * LServe write-up "2.1" (min-max pooling of the keys at prefill) and "2.2"
 * (pages of the pool through the page table). */
spa_status spa_kv_pool_write(const spa_pool* pool, const spa_heads* heads,
                             const int32_t* page_table_row, int32_t max_pages,
                             int32_t stream_base, int64_t start, int64_t count,
                             const void* k, const void* v, hipStream_t stream);

/* ---- a2: page summaries ------------------------------------------------
 * For every dynamic KV head and every logical page j that overlaps positions
 * [first_pos[b], L_b) of sequence b, recomputes the page's summary from the
 * keys in the pool: channel-wise minimum and maximum over the page's valid
 * tokens [j*p, min(j*p + p, L_b)). Min and max use IEEE totalOrder
 * (-0 < +0), so the result is exact and independent of evaluation order.
 * LServe write-up "2.1" (min-max pooling of each block's features).
 *   first_pos: device int32 [B], or NULL meaning L_b - 1 (the decode case:
 *              only the page holding the new token);
 *   max_tokens: host bound, L_b - first_pos[b] <= max_tokens for every b
 *              (1 when first_pos is NULL). Pages beyond the bound are not
 *              refreshed. */
spa_status spa_page_summary_update(const spa_pool* pool, const spa_heads* heads,
                                   const spa_batch* batch, const int32_t* first_pos,
                                   int32_t max_tokens, hipStream_t stream);

/* ---- a3 + a4: page selection for dynamic heads --------------------------
 * For sequence b and dynamic KV head h with query group g = 0..G-1, page j
 * (0 <= j < n_b = ceil(L_b / p)) scores
 *     s_j = max_g RN32( sum_c max(q[g][c] * kmax[j][c], q[g][c] * kmin[j][c]) ),
 * the largest value q_g . k can take for any key inside the page's min/max
 * box (LServe write-up "2.1": query-to-pooled-feature similarity; the
 * upper-bound form is the Quest row of the long-context survey's sparse-method
 * table). The sum is accumulated in fp64 from exact bf16 products and rounded
 * once to fp32; no 1/sqrt(D) factor. Then
 *     k_b = min(n_b, max(1, budget_tokens[b] / p), k_max)
 * pages are kept: the first k_b in the order (score descending, page id
 * ascending), written to sel_pages[b][h][0..k_b) in ascending page id, with
 * sel_count[b][h] = k_b and sel_len[b] = L_b (the length the selection was
 * made at). Rows of streaming heads are not written.
 *   q:             device bf16 [B][H_q][D]
 *   budget_tokens: device int32 [B], token budget per sequence (the write-up's
 *                  rule min(4096, L/32) is spa_default_budget)
 *   k_max:         host int, capacity of a sel_pages row, >= 1
 *   sel_pages:     device int32 [B][H_kv][k_max]  (written)
 *   sel_count:     device int32 [B][H_kv]         (written)
 *   sel_len:       device int32 [B]               (written)
 *   sel_phys:      device int32 [B][H_kv][k_max] or NULL; when given,
 *                  receives page_table[b][id / (P / p)] for each selected id
 *                  (the physical page holding it), which lets
 *                  spa_sparse_decode_attn skip the page-table look-up
 *   scores:        device fp32 [B][H_kv][max_pages * P / p] or NULL; when
 *                  given, receives s_j for dynamic heads (entries j >= n_b
 *                  unspecified)
 *   ws, ws_bytes:  device workspace of at least spa_workspace_bytes() bytes
 * Limit: a page-table row may address at most 32768 logical pages
 * (max_pages * P / p <= 32768, e.g. 524288 tokens at p = 16); larger rows
 * return SPA_ERR_UNSUPPORTED before anything is enqueued.
 * Reuse across steps (write-up "3.2": rerun selection every C tokens) is the
 * caller's: call this only on steps that select and keep the outputs. */
spa_status spa_select_pages(const spa_pool* pool, const spa_heads* heads,
                            const spa_batch* batch, const void* q,
                            const int32_t* budget_tokens, int32_t k_max,
                            int32_t* sel_pages, int32_t* sel_count, int32_t* sel_len,
                            int32_t* sel_phys, float* scores, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* ---- a1 + a2 + a3 + a4 in one launch pair -----------------------------
 * The same pool state and outputs as spa_kv_pool_append(pool, heads, batch,
 * k_new, v_new) followed by spa_select_pages with the other arguments: the
 * scoring launch also writes token L_b - 1 (k_new, v_new: device bf16
 * [B][H_kv][D], read only) into its pool slot and rebuilds the summary of its
 * logical page for every dynamic head, and scores that page with the new key
 * merged into its summary (the step order of the LServe write-up "3.2
 * 解码阶段加速": append, then select on the updated summaries). For steps that
 * select; the pool rows it writes are read by spa_sparse_decode_attn
 * afterwards. Same workspace as spa_select_pages. */
spa_status spa_append_select_pages(const spa_pool* pool, const spa_heads* heads,
                                   const spa_batch* batch, const void* k_new, const void* v_new,
                                   const void* q, const int32_t* budget_tokens, int32_t k_max,
                                   int32_t* sel_pages, int32_t* sel_count, int32_t* sel_len,
                                   int32_t* sel_phys, float* scores, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* ---- a6 + a7 + a8: unified sparse decode attention ----------------------
 * For every sequence b and query head i (KV head h = i / G):
 *     out[b][i] = sum_{t in T} softmax_t(q_i . K_t / sqrt(D)) V_t,
 *     lse[b][i] = natural log of sum_{t in T} exp(q_i . K_t / sqrt(D)),
 * with the attended token set T
 *   streaming head: [0, min(sink, L)) U [max(sink, L - window), L);
 *   dynamic head:   { t < L : t / p in sel_pages[b][h][0..sel_count) }
 *                   U [sel_len[b], L)   (tokens appended since the selection).
 * bf16 inputs, fp32 accumulation. Work is split over the attended tokens and
 * the split results are merged with the running-max / running-sum rule of
 * online softmax (FlashAttention, long-context survey "2.1"; the max and sum
 * outputs of the Novita vLLM article, "2. 注意力机制修改").
 *   out: device fp32 [B][H_q][D]; lse: device fp32 [B][H_q] or NULL.
 *   sel_pages / sel_count / sel_len: as written by spa_select_pages (page
 *          ids distinct; not read for streaming heads);
 *   sel_phys: as written by the same spa_select_pages call, or NULL to look
 *          the selected pages up in the page table here. When given, the
 *          page-table entries of the selected pages must not have changed
 *          since the selection (pages are only ever added at the end);
 *   k_max: capacity of a sel_pages row.
 * A sequence with L_b < 1 gets out = 0 and lse = -inf. */
spa_status spa_sparse_decode_attn(const spa_pool* pool, const spa_heads* heads,
                                  const spa_batch* batch, const void* q,
                                  const int32_t* sel_pages, const int32_t* sel_count,
                                  const int32_t* sel_len, const int32_t* sel_phys, int32_t k_max,
                                  float* out, float* lse, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* ---- a6 + a7 + a8 for callers that cannot allocate ----------------------
 * For callers that cannot call hipMalloc or hand in a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The same results as spa_sparse_decode_attn with the same arguments (the
 * same kernels), but the split partials live in a static scratch array of the
 * library instead of a caller's workspace: SPA_NOALLOC_SCRATCH_BYTES (32 MiB)
 * per GPU, held from the first call on that GPU until the process ends. Shapes
 * whose partials need more return SPA_ERR_WORKSPACE before anything is
 * enqueued (the benchmark's 4 x 131072-token batch at 32 / 8 heads needs
 * about 3.6 MB). The first call on a device looks the array's device address
 * up, with that device current. Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and give unspecified results. Allocates nothing: no hipMalloc, hipFree or
 * allocating library routine, and needs no zeroed memory. */
#define SPA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
spa_status spa_sparse_decode_attn_noalloc(const spa_pool* pool, const spa_heads* heads,
                                          const spa_batch* batch, const void* q,
                                          const int32_t* sel_pages, const int32_t* sel_count,
                                          const int32_t* sel_len, const int32_t* sel_phys,
                                          int32_t k_max, float* out, float* lse, hipStream_t stream);

/* ---- a1 + a2 + a6 + a7 + a8 in one launch -------------------------------
 * The same pool state and outputs as spa_kv_pool_append(pool, heads, batch,
 * k_new, v_new) followed by spa_sparse_decode_attn with the other arguments:
 * token L_b - 1 of every sequence (k_new, v_new: device bf16 [B][H_kv][D],
 * read only) is written into its pool slot, the summary of the logical page
 * receiving it is rebuilt for every dynamic head, and the attention takes that
 * token from k_new / v_new instead of the pool (the step order of the LServe
 * write-up "3.2 解码阶段加速": the new token is appended, then attended).
 * For steps that do not select: the selection passed in must have been made
 * before this token, i.e. sel_len[b] <= L_b - 1 (a larger sel_len is read as
 * L_b - 1). Same workspace as spa_sparse_decode_attn. */
spa_status spa_append_decode_attn(const spa_pool* pool, const spa_heads* heads,
                                  const spa_batch* batch, const void* k_new, const void* v_new,
                                  const void* q, const int32_t* sel_pages,
                                  const int32_t* sel_count, const int32_t* sel_len,
                                  const int32_t* sel_phys, int32_t k_max, float* out, float* lse,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- prefill: block-sparse attention over a whole prompt ----------------
 * LServe write-up "3.1 预填充阶段优化": for every query head i (KV head
 * h = i / G) and position t of a sequence of L tokens,
 *     out[i][t] = sum_{s in T(t)} softmax_s(q_i,t . k_h,s / sqrt(D)) v_h,s,
 *     lse[i][t] = natural log of the softmax denominator,
 * with blocks of b = 64 tokens and T(t) depending on the head's kind:
 *   streaming head: s <= t with s < sink or s > t - window (sink + window);
 *   dynamic head, L < dense_below: every s <= t (the write-up's dense
 *       fallback below 32K tokens);
 *   dynamic head otherwise: s <= t inside the key blocks selected for t's
 *       block j: block j itself and the kb - 1 (kb = max(1, budget / 64)) best
 *       earlier blocks by the low-rank importance score
 *           S(j, i) = RN32( (qbar_j W_q) . (kbar_i W_k) / sqrt(D) ),
 *       qbar_j the mean query of block j over the KV head's G query heads and
 *       the block's tokens, kbar_i the mean key of block i, the projections
 *       W_q, W_k bf16 [D][D / 8], evaluated in fp64 (the mean of the low-rank
 *       logits (q W_q)(k W_k)^T / sqrt(D) over the block pair); best = score
 *       descending, block id ascending; one selection per KV head serves its
 *       whole query group.
 * Inputs are the prompt's activations in position order (before they are
 * written into the page pool): q bf16 [H_q][L][D], k and v bf16 [H_kv][L][D].
 *   out: device fp32 [H_q][L][D]; lse: device fp32 [H_q][L] or NULL;
 *   sel_blocks, sel_count: NULL, or device int32 [H_kv][nb][kb] and
 *       [H_kv][nb] (nb = ceil(L / 64)) receiving each dynamic head's attended
 *       blocks, ascending (written only when the heads select);
 *   block_scores: NULL, or device fp32 [H_kv][nb][nb] receiving S(j, i) for
 *       i < j of the dynamic heads (other entries unspecified);
 *   ws, ws_bytes: workspace of spa_prefill_workspace_bytes() bytes.
 * head_dim 128 and blocks of 64 only; with selection L <= 524288 (longer:
 * SPA_ERR_UNSUPPORTED). L == 0 is a no-op. */
typedef struct spa_prefill {
  int32_t head_dim;      /* D, 128 */
  int32_t block;         /* b, 64 */
  int32_t budget;        /* tokens of key blocks per query block, the diagonal block included, >= 1 */
  int32_t dense_below;   /* dynamic heads attend densely when L < dense_below (the write-up: 32768) */
} spa_prefill;

spa_status spa_prefill_attn(const spa_heads* heads, int32_t num_kv_heads, const spa_prefill* cfg,
                            int64_t seq_len, const void* q, const void* k, const void* v,
                            const void* w_q, const void* w_k, float* out, float* lse,
                            int32_t* sel_blocks, int32_t* sel_count, float* block_scores,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes of spa_prefill_attn for these shapes (0 for invalid
 * arguments). Needs no initialisation; calls sharing it must not overlap. */
size_t spa_prefill_workspace_bytes(const spa_heads* heads, int32_t num_kv_heads, const spa_prefill* cfg,
                                   int64_t seq_len);

/* Workspace bytes needed by spa_select_pages and spa_sparse_decode_attn for
 * these shapes (one buffer serves both). Returns 0 for invalid arguments.
 * The workspace needs no initialisation and holds nothing between calls;
 * calls that share a workspace must not run concurrently. */
size_t spa_workspace_bytes(const spa_pool* pool, const spa_heads* heads,
                           int32_t batch, int32_t max_pages, int32_t k_max);

/* Tuning of spa_sparse_decode_attn's work split (no effect on results
 * beyond floating-point summation order): the attended tokens of a head are
 * cut into items of `blocks` 16-token blocks, one work-group per item, and
 * the item partials are merged afterwards. 0 (the default) picks the size
 * per call so that the busiest compute unit has the fewest blocks; 4, 5, 6,
 * 7, 8, 9, 10, 12 or 16 fixes it (as does the SPA_ATTN_BLOCKS_PER_ITEM
 * environment variable, read once). Any other value: SPA_ERR_INVALID.
 * Process-wide; takes effect from the next call. */
spa_status spa_set_attn_blocks_per_item(int32_t blocks);

/* The write-up's dynamic budget rule ("3.2"): min(4096, L / 32) tokens,
 * integer division; 0 for L < 32. */
int32_t spa_default_budget(int64_t context_len);

/* Pages of one sequence's ring for window-only storage of the streaming
 * heads (spa_batch.stream_pages): ceil(sink / P) + ceil(window / P) + 1.
 * Returns 0 for invalid arguments. */
int32_t spa_stream_ring_pages(const spa_pool* pool, const spa_heads* heads);

/* ---- physical-page allocator (host) -------------------------------------
 * A free list over page ids 0..N-1 (LServe write-up "2.2": free list of
 * physical pages; long-context survey "3.4": allocate_page raises when no
 * page is free). Pages are handed out lowest id first from a fresh
 * allocator. Not thread-safe. */
typedef struct spa_allocator spa_allocator;

/* num_pages >= 1; *out receives the handle. */
spa_status spa_alloc_create(int32_t num_pages, spa_allocator** out);
/* All-or-nothing: either `count` ids are written to ids_out (host int32
 * [count]) or SPA_ERR_POOL_EXHAUSTED is returned and nothing changes. */
spa_status spa_alloc_pages(spa_allocator* a, int32_t count, int32_t* ids_out);
/* Returns pages to the free list. An id out of range or not allocated makes
 * the whole call fail with SPA_ERR_INVALID and nothing changes. */
spa_status spa_alloc_free(spa_allocator* a, int32_t count, const int32_t* ids);
/* Number of free pages, or -1 for a NULL handle. */
int32_t spa_alloc_num_free(const spa_allocator* a);
void spa_alloc_destroy(spa_allocator* a);

/* Static text for a status code. */
const char* spa_status_string(spa_status s);
/* Message of the last failing call on this thread ("" if none). */
const char* spa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SPA_H */
