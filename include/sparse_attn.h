/*
 * sparse_attn.h -- C ABI of the indexer-selected block-sparse attention library
 * for AMD Instinct MI355X (gfx950).  Library: libsparse_attn.so.
 *
 * The method (llama.cpp commit "llama: QSA sparse attention for qwen4exp", in the
 * Qwen3.8-Flash-Next / qwen4exp series #27742): an indexer keeps one raw key per
 * cached token; every block of compress_ratio consecutive positions gets one
 * mean-pooled key; each query token scores every complete block as the sum over
 * indexer heads of ReLU(q_h . kbar_b); it keeps the best blocks up to a budget of
 * indexer_top_k tokens plus the tail of tokens not yet forming a complete block
 * (exactly dense below indexer_top_k + compress_ratio - 1 visible tokens); and
 * attention softmax(scale * Q K^T) V runs over the kept rows only (llama.cpp PR
 * #27970 "CUDA + ggml: add sparse-fa for DSV4/GLM": gather through an ascending
 * int32 index list, many query heads per KV head, V optionally a view of K).
 *
 * Four calls, one per step, all asynchronous on the caller's HIP stream (and one that
 * joins the last two):
 *   sparse_attn_pool   -- incremental block mean-pool of the raw indexer keys
 *   sparse_attn_score  -- indexer block scores per query token
 *   sparse_attn_select -- kept blocks + tail -> ascending position list per query
 *   sparse_attn_fwd    -- gather-fused attention over the position lists
 *   sparse_attn_select_fwd -- the two above in one call (one launch where it fits)
 *
 * Conventions shared by every call
 *  - Ownership: the caller allocates every buffer; the library never allocates,
 *    frees or synchronises.  Every pointer in sa_cache and every array argument
 *    is DEVICE memory unless stated otherwise; sa_dims / sa_cache themselves are
 *    host structs read during the call only.
 *  - Stream: `stream` is a hipStream_t (NULL = the default stream).  Calls return
 *    after enqueueing; results are ready when the stream reaches them.
 *  - Errors: 0 on success or a negative SA_ERR_* code.  Every argument error is
 *    detected on the host before any HIP call, so nothing is enqueued on error.
 *    SA_ERR_HIP reports a failed launch (hipGetLastError after the launch).
 *  - Positions: row seq_row0[s] + t of a cache holds position t of sequence s.
 *    A query token i (sequence q_seq[i], position q_pos[i]) sees position t iff
 *    t <= q_pos[i] and t < seq_len[q_seq[i]]; n_vis = number of such positions.
 *    Block b of sequence s covers positions [b*c, (b+1)*c); it is complete for a
 *    query when (b+1)*c <= n_vis.  NB = n_vis / c; tail = n_vis - NB*c.
 *  - Element types: every cache and query tensor has the one dtype of sa_dims;
 *    scores, outputs and workspaces are float32; lists are int32.
 *  - Calls that overlap on one stream are ordered; calls on different streams that
 *    write the same buffers race (as with any kernel).
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the caches and query tensors. */
typedef enum { SA_F32 = 0, SA_F16 = 1, SA_BF16 = 2 } sa_dtype;

/* Error codes. */
enum {
  SA_OK = 0,
  SA_ERR_NULL = -1,      /* a required pointer is NULL                                   */
  SA_ERR_DIMS = -2,      /* dimensions unsupported or inconsistent (see sparse_attn_check_dims) */
  SA_ERR_ARG = -3,       /* another argument out of range (count, leading dimension, size) */
  SA_ERR_WORKSPACE = -4, /* workspace NULL or smaller than sparse_attn_workspace_bytes     */
  SA_ERR_HIP = -5,       /* a kernel launch failed                                        */
  SA_ERR_SCRATCH = -6    /* sparse_attn_fwd_noalloc: the call needs more than the static scratch */
};

/* Shape of one attention layer and its indexer. */
typedef struct {
  int32_t h_q;            /* query heads                                                   */
  int32_t h_kv;           /* KV heads; h_q % h_kv == 0; query head h reads KV head h/(h_q/h_kv) */
  int32_t d_kq;           /* K and Q head size                                             */
  int32_t d_v;            /* V head size                                                   */
  int32_t h_idx;          /* indexer heads                                                 */
  int32_t d_idx;          /* indexer head size (one indexer key head)                      */
  int32_t compress_ratio; /* c: tokens per pooled block, >= 1                              */
  int32_t top_k;          /* indexer_top_k: token budget of kept blocks, a multiple of c    */
  int32_t dtype;          /* sa_dtype of K, V, raw/pooled indexer keys, q, indexer queries  */
} sa_dims;

/* One layer's caches for n_seq sequences (all pointers device memory, caller-owned).
 * Element (row r, KV head g, dim d) of K is k[r*k_ld + g*k_head_stride + d]; V
 * likewise.  V may alias K (v == k, v_ld == k_ld, v_head_stride == k_head_stride):
 * V is then the first d_v elements of each K head, as in MLA's latent cache
 * (llama.cpp "Create V as a view of K" in the llm_graph_input_attn_k_iswa fix).   */
typedef struct {
  int32_t n_seq;            /* sequences                                                     */
  int32_t max_len;          /* host-side upper bound on every seq_len[s] (sizes the grids)   */
  const int64_t* seq_row0;  /* [n_seq] first cache row of sequence s                          */
  const int64_t* seq_blk0;  /* [n_seq] first pooled-key row of sequence s                     */
  const int32_t* seq_len;   /* [n_seq] cached tokens L_s (positions 0..L_s-1)                 */
  const void* k;            /* K cache, d_kq per head                                        */
  int64_t k_ld;             /* row stride of K in elements (>= h_kv*d_kq when unaliased)      */
  int64_t k_head_stride;    /* KV-head stride of K in elements                               */
  const void* v;            /* V cache, d_v per head (may alias k)                           */
  int64_t v_ld;
  int64_t v_head_stride;
  const void* kidx;         /* raw indexer keys, one head of d_idx per row                   */
  int64_t kidx_ld;
  void* kpool;              /* pooled indexer keys, d_idx per pooled row (written by pool)   */
  int64_t kpool_ld;
} sa_cache;

/* Host-only validation of the dimensions: 0 or SA_ERR_NULL / SA_ERR_DIMS.
 * Supported: dtype in {F32, F16, BF16}; h_q, h_kv >= 1 with h_q % h_kv == 0 and
 * h_q / h_kv <= 16; 1 <= d_kq <= 1024; 1 <= d_v <= 1024; 1 <= h_idx <= 128;
 * d_idx in [8, 512] and a multiple of 8; 1 <= compress_ratio <= 64; top_k >= c and
 * top_k % c == 0; top_k + c - 1 <= 65536.  Makes no HIP call.                        */
int sparse_attn_check_dims(const sa_dims* dims);

/* Bytes at the start of a workspace that hold state between calls. */
#define SA_WS_STATE_BYTES ((size_t)1056768)

/* Bytes of device workspace that sparse_attn_select, sparse_attn_fwd and
 * sparse_attn_select_fwd need for n_q query tokens over caches whose sa_cache.max_len
 * is max_len; one buffer of this size serves every call (after the state, room for
 * the chunked selection's candidates, the attention's split partials and, for fewer
 * than 64 tokens over rows of at most 32768 blocks, the candidate list of
 * sparse_attn_pool_score_select_fwd, side by side).  Returns 0 on bad arguments or when no workspace is needed.
 * Host only, no HIP call.
 * Contract: zero-fill the buffer once before its first use (e.g. hipMemset when it is
 * allocated).  Its first SA_WS_STATE_BYTES bytes hold histograms
 * that every call returns to zero, so later calls need no re-initialisation; the rest
 * is scratch that each call overwrites.  Calls that share a workspace must not run
 * concurrently (use one workspace per stream).                                     */
size_t sparse_attn_workspace_bytes(const sa_dims* dims, int32_t n_q, int32_t max_len);

/* Incremental block mean-pool (pages: the indexer cache holds raw keys because
 * pooling happens before the norm and the rotation; one pooled key per block of
 * compress_ratio tokens).  For each sequence s, pools blocks
 * [n_pooled_in[s], n_new) where n_new = min(seq_len[s] / c, n_pooled_in[s] + max_new_blocks):
 *     kpool[seq_blk0[s] + b] = (sum_{i<c} kidx[seq_row0[s] + b*c + i]) / c,
 * summed in float32 in position order and rounded to the cache dtype (RNE), and
 * writes n_pooled_out[s] = n_new (device arrays of n_seq int32; they may alias --
 * the update is ordered after every read).  Resuming from raw keys = n_pooled_in 0.
 * A sequence whose seq_len shrank below n_pooled_in*c gets n_pooled_out = seq_len/c.
 * Errors: SA_ERR_NULL, SA_ERR_DIMS, SA_ERR_ARG (n_seq < 1, max_new_blocks < 0,
 * kidx_ld / kpool_ld < d_idx, max_len < 0), SA_ERR_HIP.                            */
int sparse_attn_pool(const sa_dims* dims, const sa_cache* cache, const int32_t* n_pooled_in,
                     int32_t* n_pooled_out, int32_t max_new_blocks, void* stream);

/* Indexer block scores (pages: each head's dot product is rectified before the sum
 * over heads; scoring is batched per sequence so a sequence's queries meet only its
 * own blocks).  For query token i and every complete block b < NB(i):
 *     scores[i*scores_ld + b] = sum_{h<h_idx} max(0, sum_d qidx[i][h][d] * kpool[seq_blk0[s]+b][d])
 * accumulated in float32, written as +0.0 when no head is positive.  Entries
 * b >= NB(i) are not written.  qidx is [n_q][h_idx][d_idx] contiguous, in the
 * cache dtype.  The pooled keys of blocks < NB(i) must be current (sparse_attn_pool).
 * Requires scores_ld >= max_len / c.  Errors: SA_ERR_NULL, SA_ERR_DIMS, SA_ERR_ARG
 * (n_q < 0, scores_ld too small), SA_ERR_HIP.  n_q == 0 is a no-op.                  */
int sparse_attn_score(const sa_dims* dims, const sa_cache* cache, const void* qidx,
                      const int32_t* q_seq, const int32_t* q_pos, int32_t n_q,
                      float* scores, int64_t scores_ld, void* stream);

/* sparse_attn_pool followed by sparse_attn_score, with the same arguments and the
 * same results (kpool, n_pooled_out and scores bit for bit), in one launch where
 * the decode scoring kernel applies (f16/bf16, h_idx a multiple of 32 up to 128,
 * d_idx 64/128/256, fewer than 64 query tokens, aligned rows, n_pooled_in and
 * n_pooled_out distinct): the workgroups that score a new block pool it from the raw
 * keys themselves, while others write the cache.  Otherwise it makes the two calls.
 * Errors: those of sparse_attn_pool and sparse_attn_score.                           */
int sparse_attn_pool_score(const sa_dims* dims, const sa_cache* cache, const int32_t* n_pooled_in,
                           int32_t* n_pooled_out, int32_t max_new_blocks, const void* qidx,
                           const int32_t* q_seq, const int32_t* q_pos, int32_t n_q, float* scores,
                           int64_t scores_ld, void* stream);

/* Block selection (pages: keep a budget of the best blocks plus the tail; exactly
 * dense below top_k + c - 1 tokens; block scores are expanded to tokens and the cut
 * lands on a block boundary).  For query token i with K_blk = top_k / c:
 *   kept = all NB blocks if NB <= K_blk, else the first K_blk blocks in the order
 *          (score descending, block index ascending) -- ties go to the lower index,
 *          and +0.0 / -0.0 compare equal;
 *   sel[i*sel_ld + j], j < n_sel[i] = the positions of the kept blocks (c each) in
 *          ascending order, followed by the tail positions [NB*c, n_vis);
 *   sel[i*sel_ld + j], n_sel[i] <= j < sel_ld = -1.
 * n_sel[i] = min(NB, K_blk)*c + tail <= top_k + c - 1 (the list cannot overflow).
 * Requires sel_ld >= top_k + c - 1 and scores_ld >= max_len / c.  Scores must not be
 * NaN.  ws: workspace of sparse_attn_workspace_bytes(dims, n_q, max_len) bytes (may
 * be NULL when that is 0).  Errors: SA_ERR_NULL, SA_ERR_DIMS, SA_ERR_ARG,
 * SA_ERR_WORKSPACE, SA_ERR_HIP.                                                      */
int sparse_attn_select(const sa_dims* dims, const sa_cache* cache, const float* scores,
                       int64_t scores_ld, const int32_t* q_seq, const int32_t* q_pos, int32_t n_q,
                       int32_t* sel, int64_t sel_ld, int32_t* n_sel, void* ws, size_t ws_bytes,
                       void* stream);

/* Gather-fused attention over the selected rows (pages: the sparse flash-attention
 * kernel loads K/V rows through the index list; rows -1 contribute nothing).  For
 * query token i, query head h (KV head g = h / (h_q/h_kv)):
 *     out[i][h][:] = sum_t softmax_t(scale * q[i][h] . K[t][g]) V[t][g][:]
 * over t in { seq_row0[s] + sel[i*sel_ld + j] : j < min(n_sel[i], sel_ld, top_k + c - 1),
 *             0 <= sel[...] < seq_len[s] } (other entries are skipped), accumulated
 * in float32; out = 0 when the set is empty.  q is [n_q][h_q][d_kq] contiguous in
 * the cache dtype; out is [n_q][h_q][d_v] float32 contiguous.  ws: workspace of
 * sparse_attn_workspace_bytes(dims, n_q, cache->max_len) bytes (split-KV partials).
 * Errors: SA_ERR_NULL, SA_ERR_DIMS, SA_ERR_ARG, SA_ERR_WORKSPACE, SA_ERR_HIP.        */
int sparse_attn_fwd(const sa_dims* dims, const sa_cache* cache, const void* q,
                    const int32_t* q_seq, const int32_t* sel, int64_t sel_ld, const int32_t* n_sel,
                    int32_t n_q, float scale, float* out, void* ws, size_t ws_bytes, void* stream);

/* sparse_attn_select followed by sparse_attn_fwd (pages: the indexer's block selection
 * of the QSA commit, then the sparse flash attention of PR #27970 over the list it
 * writes), for the same n_q query tokens: writes sel, n_sel and out exactly as the two
 * calls would, bit for bit.  When every (token, KV head, split) workgroup of the
 * attention has a compute unit of its own -- few decode tokens, the MLA shapes with V
 * inside K (d_v 512, d_kq 512 or 576, f16 / bf16), lists of at most 3072 entries --
 * the selection runs inside the attention's launch (each workgroup selects its token's
 * list into LDS): all of it for rows of at most 32768 blocks, the finishing pass of
 * the chunked selection for longer rows of at most 256 chunks of 2048 blocks (its
 * histogram and candidate launches run first), saving a launch and the list's round
 * trip through memory; otherwise the call makes the two calls.  Arguments are those of
 * the two calls (scores/scores_ld/q_pos as in sparse_attn_select; q/scale/out as in
 * sparse_attn_fwd); ws: sparse_attn_workspace_bytes(dims, n_q, cache->max_len) bytes,
 * one buffer for both parts.
 * Errors: those of sparse_attn_select and of sparse_attn_fwd.                        */
int sparse_attn_select_fwd(const sa_dims* dims, const sa_cache* cache, const float* scores,
                           int64_t scores_ld, const int32_t* q_seq, const int32_t* q_pos, const void* q,
                           int32_t n_q, float scale, int32_t* sel, int64_t sel_ld, int32_t* n_sel,
                           float* out, void* ws, size_t ws_bytes, void* stream);

/* Which form sparse_attn_select_fwd takes for these arguments on the current device,
 * with a workspace of sparse_attn_workspace_bytes: 1 = the selection (or its finishing
 * pass) inside the attention's launch, 0 = the two calls; a negative SA_ERR_* on bad
 * arguments (n_q < 1 is SA_ERR_ARG).  Host only: reads the device's compute-unit
 * count, launches nothing.                                                           */
int sparse_attn_select_fwd_is_fused(const sa_dims* dims, const sa_cache* cache, const void* q, int32_t n_q);

/* The decode step's first links: sparse_attn_pool_score followed by
 * sparse_attn_select_fwd (pages: the indexer's pooled keys and block scores, the
 * top-k block selection, then the sparse attention over the list), with the
 * arguments of the two calls (ws: sparse_attn_workspace_bytes(dims, n_q,
 * cache->max_len) bytes) and their results bit for bit (kpool, n_pooled_out, scores,
 * sel, n_sel, out).  Where the pooled scoring launch and a selection inside the
 * attention's launch both apply (see sparse_attn_pool_score_select_fwd_uses_list:
 * fewer than 64 tokens of the MLA shapes, at most 8192 groups of 32 blocks in all,
 * rows of at most 262144 blocks), the scoring launch also writes, for every 32
 * consecutive blocks of each token's row, the 8 best (4 for rows of more than 131072
 * blocks; ties to the lower block) into the workspace's last part, and each attention
 * workgroup selects from that list instead of the row: the list's cut is the row's cut
 * exactly when every block it leaves out scores below that cut, which each group's
 * last listed key bounds; where it does not, the groups whose listed keys reach the cut
 * (at most 32; 64 for rows of more than 32768 blocks) are read whole from the row and
 * the cut taken again, and where that does not decide
 * either (or the token's row is too short for the list to be likely to decide), the
 * workgroup selects over the row.  The list part ends with one int32 per token: 1 when
 * the list (with any groups read whole) decided its selection, 0 when the row did (or
 * the token was dense).
 * Errors: those of sparse_attn_pool_score and sparse_attn_select_fwd; n_q == 0 makes
 * the pooling alone.                                                                 */
int sparse_attn_pool_score_select_fwd(const sa_dims* dims, const sa_cache* cache, const int32_t* n_pooled_in,
                                      int32_t* n_pooled_out, int32_t max_new_blocks, const void* qidx,
                                      const int32_t* q_seq, const int32_t* q_pos, int32_t n_q, float* scores,
                                      int64_t scores_ld, const void* q, float scale, int32_t* sel, int64_t sel_ld,
                                      int32_t* n_sel, float* out, void* ws, size_t ws_bytes, void* stream);

/* 1 when sparse_attn_pool_score_select_fwd with these arguments and a workspace of
 * sparse_attn_workspace_bytes writes the candidate list and selects from it, 0 when it
 * makes the two calls unchanged; a negative SA_ERR_* on bad arguments.  Host only.   */
int sparse_attn_pool_score_select_fwd_uses_list(const sa_dims* dims, const sa_cache* cache,
                                                const int32_t* n_pooled_in, const int32_t* n_pooled_out,
                                                const void* qidx, const void* q, int32_t n_q);

/* Bytes of the library's static scratch (per GPU), used by sparse_attn_fwd_noalloc:
 * the split partials of 512 workgroups of 16 query heads with d_v = 512 (the most the
 * split plan makes), 512 * 16 * (512 + 2) * 4 bytes, so every call with
 * h_q / h_kv <= 16 and d_v <= 512 fits.                                              */
#define SA_STATIC_SCRATCH_BYTES ((size_t)16842752)

/* sparse_attn_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments (less ws / ws_bytes), same kernels and the same
 * results as sparse_attn_fwd.  The split-KV partials go to a static device array of
 * SA_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on until the
 * process ends; its device address is looked up on the first call on each device.
 * The call allocates nothing (no hipMalloc / hipFree, no allocating library call).
 * The scratch needed is that of the split partials (0 when unsplit; at most
 * sparse_attn_workspace_bytes(dims, n_q, max_len) minus SA_WS_STATE_BYTES, which also
 * counts the selection's scratch and the candidate list); a call needing more than SA_STATIC_SCRATCH_BYTES
 * returns SA_ERR_SCRATCH before any HIP call; that cannot happen for d_v <= 512 (e.g.
 * one decode token of 16 heads 576/512 with top_k 2048 needs 1.09 MB, 32 sequences
 * of 8 heads 512/512 8.4 MB), but can for wider V heads.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (on any streams) race, so
 * issue them in one stream order.  Nothing in the array needs to start at zero.
 * Errors: those of sparse_attn_fwd (no SA_ERR_WORKSPACE), SA_ERR_SCRATCH.           */
int sparse_attn_fwd_noalloc(const sa_dims* dims, const sa_cache* cache, const void* q,
                            const int32_t* q_seq, const int32_t* sel, int64_t sel_ld, const int32_t* n_sel,
                            int32_t n_q, float scale, float* out, void* stream);

/* The additive-mask form of the attention (pages: PR #27970, the sparse mode of the
 * flash-attention op: the finite entries of each query's mask row are its K/V set
 * and their values are added to the logits; the caller bounds the finite entries per
 * row, which sizes the index list).  This call turns masks into the index lists the
 * attention consumes -- the same form the block selection writes.
 *   mask:     device, [n_q][mask_ld] of mask_dtype (SA_F16 or SA_F32); column p of row
 *             i is position p of query token i's sequence.  Entries that are not
 *             finite (-inf, +inf, NaN) are excluded.  May be NULL when n_kv == 0.
 *   sel:      device, [n_q][sel_ld] int32 out: row i's finite columns in ascending
 *             order, then -1 up to sel_ld.
 *   n_sel:    device, [n_q] int32 out: the number of finite entries of row i; a count
 *             above sel_ld means the row was cut to its first sel_ld positions.
 *   sel_bias: device, [n_q][sel_ld] float out, optional (NULL): the mask value at each
 *             listed position, 0 for the padding -- the bias input of
 *             sparse_attn_fwd_bias.
 * Errors: SA_ERR_ARG (bad dtype, negative sizes, sel_ld < 1, mask_ld < n_kv),
 *         SA_ERR_NULL, SA_ERR_HIP.                                                     */
int sparse_attn_mask_to_indices(const void* mask, int32_t mask_dtype, int64_t mask_ld, int32_t n_q,
                                int32_t n_kv, int32_t* sel, int64_t sel_ld, int32_t* n_sel, float* sel_bias,
                                void* stream);

/* sparse_attn_fwd with an additive logit bias per list entry (pages: PR #27970, the
 * mask value added to the logit in the mask-driven sparse mode): the logit of list
 * entry j of query token i, for every head, is
 *     scale * q[i][h] . K[row][g] + sel_bias[i*sel_ld + j].
 * sel_bias: device, [n_q][sel_ld] float, or NULL for no bias (then identical to
 * sparse_attn_fwd).  Entries must be finite or -inf (-inf drops the row).  All other
 * arguments, the workspace and the errors are those of sparse_attn_fwd.             */
int sparse_attn_fwd_bias(const sa_dims* dims, const sa_cache* cache, const void* q,
                         const int32_t* q_seq, const int32_t* sel, int64_t sel_ld, const int32_t* n_sel,
                         const float* sel_bias, int32_t n_q, float scale, float* out, void* ws,
                         size_t ws_bytes, void* stream);

/* sparse_attn_fwd over the selected rows together with a dense window: the
 * `window` most recent visible positions of each query token (t in [n_vis - window,
 * n_vis), n_vis = min(seq_len[s], q_pos[i] + 1)), each position once -- list
 * entries inside the window are covered by it (pages: PR #27970 review thread, the
 * dense attention over the contiguous recent keys plus sparse attention over the
 * selected keys, merged; reading: the contiguous block is the most recent window).
 * The window rows are contiguous and need no list.  q_pos: device [n_q] int32,
 * required when window > 0.  window = 0 gives sparse_attn_fwd.  The workspace of
 * sparse_attn_workspace_bytes suffices; one of sparse_attn_workspace_bytes_window
 * bytes lets the window rows take workgroups of their own instead of lengthening
 * every split (same results up to rounding order).
 * Errors: those of sparse_attn_fwd; SA_ERR_ARG for window < 0 or > 2^24.            */
/* Workspace for sparse_attn_fwd_window with this window (>= that of
 * sparse_attn_workspace_bytes; same contract).  0 on invalid arguments.             */
size_t sparse_attn_workspace_bytes_window(const sa_dims* dims, int32_t n_q, int32_t max_len, int32_t window);

int sparse_attn_fwd_window(const sa_dims* dims, const sa_cache* cache, const void* q,
                           const int32_t* q_seq, const int32_t* q_pos, const int32_t* sel, int64_t sel_ld,
                           const int32_t* n_sel, int32_t window, int32_t n_q, float scale, float* out,
                           void* ws, size_t ws_bytes, void* stream);

/* ---- q8_0 K/V cache (pages: the qwen4exp commit series, a quantized KV cache on the
 * QSA attention path, served with K and V caches of type q8_0).  q8_0 is ggml's
 * block format: per 32 consecutive elements of a row one float16 scale d and 32
 * signed 8-bit codes c; element = d * c.  Here codes and scales are separate planes
 * (codes [rows][h_kv][d] int8, scales [rows][h_kv][d / 32] float16 bits), so a row's
 * codes are one contiguous run.  Strides are in elements of each plane.  V may be the
 * same planes as K (v == k, v_scale == k_scale, equal strides): V is then the first
 * d_v elements of each K head, as in MLA.  d_kq and d_v must be multiples of 32.    */
typedef struct sa_kv_q8_0 {
  const int8_t*   k;        /* K codes                                                     */
  int64_t         k_ld;     /* codes per cache row (>= (h_kv-1)*k_head_stride + d_kq)      */
  int64_t         k_head_stride;
  const uint16_t* k_scale;  /* K scales (float16)                                          */
  int64_t         k_scale_ld;     /* scales per cache row (>= (h_kv-1)*stride + d_kq/32)   */
  int64_t         k_scale_head_stride;
  const int8_t*   v;        /* V codes                                                     */
  int64_t         v_ld;
  int64_t         v_head_stride;
  const uint16_t* v_scale;  /* V scales (float16)                                          */
  int64_t         v_scale_ld;
  int64_t         v_scale_head_stride;
} sa_kv_q8_0;

/* Quantize rows to q8_0: for row r < n_rows and block b < n_cols / 32, with
 * x_b = x[r*x_ld + 32b .. 32b + 31]:
 *     d = max|x_b| / 127,  codes[r*codes_ld + 32b + e] = round(x_b[e] / d)
 * (round half away from zero; all codes 0 when d = 0), scales[r*scales_ld + b] =
 * float16(d).  The codes are decided in float32 (the division by 127, then 1/d, then
 * x * (1/d), each correctly rounded).  x: device [n_rows][x_ld] of x_dtype (SA_F32,
 * SA_F16 or SA_BF16); codes: device int8 [n_rows][codes_ld], 4-byte aligned rows;
 * scales: device float16 [n_rows][scales_ld].  This is the cache write: a step's new
 * K/V rows are quantized into the cache planes (for h_kv heads, view each cache row
 * as h_kv rows when the heads are contiguous).
 * Errors: SA_ERR_ARG (bad dtype, n_cols % 32, negative sizes, lds too small,
 *         codes pointer or codes_ld not 4-byte aligned), SA_ERR_NULL, SA_ERR_HIP.    */
int sparse_attn_quantize_q8_0(const void* x, int32_t x_dtype, int64_t n_rows, int32_t n_cols, int64_t x_ld,
                              int8_t* codes, int64_t codes_ld, uint16_t* scales, int64_t scales_ld,
                              void* stream);

/* sparse_attn_fwd over a q8_0 K/V cache: K[t][g][e] = k_scale[...][e / 32] *
 * k[...][e] (likewise V), otherwise as sparse_attn_fwd.  cache supplies the sequence
 * layout (seq_row0, seq_len, max_len); its k and v are not read.  q is in
 * dims->dtype.  The MLA shapes (V = K prefix, d_v 512, d_kq 512 or 576, f16/bf16
 * queries, 16-byte aligned code rows, 4-byte aligned scale rows) run the LDS-gather
 * MFMA kernel; everything else the generic kernel.  Workspace: that of
 * sparse_attn_fwd.  Errors: those of sparse_attn_fwd; SA_ERR_ARG when d_kq or d_v is
 * not a multiple of 32 or a stride is too small.                                     */
int sparse_attn_fwd_q8_0(const sa_dims* dims, const sa_cache* cache, const sa_kv_q8_0* kv, const void* q,
                         const int32_t* q_seq, const int32_t* sel, int64_t sel_ld, const int32_t* n_sel,
                         int32_t n_q, float scale, float* out, void* ws, size_t ws_bytes, void* stream);

/* Static description of an error code (never NULL). */
const char* sparse_attn_strerror(int code);

/* Library version string, e.g. "sparse_attn 0.1 gfx950". */
const char* sparse_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
