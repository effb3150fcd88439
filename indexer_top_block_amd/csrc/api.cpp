// C ABI of libsparse_attn: argument validation on the host, then the launchers.
// Every argument error is reported before any HIP call is made.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "sa_launch.hpp"
#include "sparse_attn.h"

namespace {

using sa::CacheArgs;

bool dtype_ok(int32_t t) { return t == SA_F32 || t == SA_F16 || t == SA_BF16; }

int check_dims(const sa_dims* d) {
  if (!d) return SA_ERR_NULL;
  if (!dtype_ok(d->dtype)) return SA_ERR_DIMS;
  if (d->h_q < 1 || d->h_kv < 1 || d->h_q % d->h_kv != 0 || d->h_q / d->h_kv > 16) return SA_ERR_DIMS;
  if (d->d_kq < 1 || d->d_kq > 1024 || d->d_v < 1 || d->d_v > 1024) return SA_ERR_DIMS;
  if (d->h_idx < 1 || d->h_idx > 128) return SA_ERR_DIMS;
  if (d->d_idx < 8 || d->d_idx > 512 || d->d_idx % 8 != 0) return SA_ERR_DIMS;
  if (d->compress_ratio < 1 || d->compress_ratio > 64) return SA_ERR_DIMS;
  if (d->top_k < d->compress_ratio || d->top_k % d->compress_ratio != 0) return SA_ERR_DIMS;
  if ((int64_t)d->top_k + d->compress_ratio - 1 > 65536) return SA_ERR_DIMS;
  return SA_OK;
}

// Checks shared by every call that reads the cache struct.
int check_cache_common(const sa_dims* d, const sa_cache* c) {
  if (!c) return SA_ERR_NULL;
  if (!c->seq_row0 || !c->seq_len) return SA_ERR_NULL;
  if (c->n_seq < 1 || c->max_len < 0) return SA_ERR_ARG;
  (void)d;
  return SA_OK;
}

CacheArgs to_args(const sa_cache* c) {
  CacheArgs a;
  a.n_seq = c->n_seq;
  a.max_len = c->max_len;
  a.seq_row0 = c->seq_row0;
  a.seq_blk0 = c->seq_blk0;
  a.seq_len = c->seq_len;
  a.k = c->k;
  a.k_ld = c->k_ld;
  a.k_hs = c->k_head_stride;
  a.v = c->v;
  a.v_ld = c->v_ld;
  a.v_hs = c->v_head_stride;
  a.kidx = c->kidx;
  a.kidx_ld = c->kidx_ld;
  a.kpool = c->kpool;
  a.kpool_ld = c->kpool_ld;
  return a;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_HIP; }

constexpr int kMaxGridY = 65535;

}  // namespace

extern "C" {

int sparse_attn_check_dims(const sa_dims* dims) { return check_dims(dims); }

size_t sparse_attn_workspace_bytes(const sa_dims* dims, int32_t n_q, int32_t max_len) {
  if (check_dims(dims) != SA_OK || n_q < 0 || max_len < 0) return 0;
  return sa::workspace_bytes(*dims, n_q, max_len);
}

size_t sparse_attn_workspace_bytes_window(const sa_dims* dims, int32_t n_q, int32_t max_len, int32_t window) {
  if (check_dims(dims) != SA_OK || n_q < 0 || max_len < 0 || window < 0 || window > (1 << 24)) return 0;
  return sa::workspace_bytes_window(*dims, n_q, max_len, window);
}

int sparse_attn_pool(const sa_dims* dims, const sa_cache* cache, const int32_t* n_pooled_in, int32_t* n_pooled_out,
                     int32_t max_new_blocks, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_cache_common(dims, cache))) return rc;
  if (!cache->seq_blk0 || !cache->kidx || !cache->kpool || !n_pooled_in || !n_pooled_out) return SA_ERR_NULL;
  if (max_new_blocks < 0 || cache->kidx_ld < dims->d_idx || cache->kpool_ld < dims->d_idx) return SA_ERR_ARG;
  if (cache->n_seq > kMaxGridY) return SA_ERR_ARG;
  (void)hipGetLastError();  // clear a stale error so that a failure below is this call's own
  return hip_status(sa::launch_pool(*dims, to_args(cache), n_pooled_in, n_pooled_out, max_new_blocks,
                                    (hipStream_t)stream));
}

int sparse_attn_score(const sa_dims* dims, const sa_cache* cache, const void* qidx, const int32_t* q_seq,
                      const int32_t* q_pos, int32_t n_q, float* scores, int64_t scores_ld, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_cache_common(dims, cache))) return rc;
  if (n_q < 0 || n_q > kMaxGridY) return SA_ERR_ARG;
  if (n_q == 0) return SA_OK;
  if (!cache->seq_blk0 || !cache->kpool || !qidx || !q_seq || !q_pos || !scores) return SA_ERR_NULL;
  if (cache->kpool_ld < dims->d_idx) return SA_ERR_ARG;
  if (scores_ld < (int64_t)(cache->max_len / dims->compress_ratio) || scores_ld < 0) return SA_ERR_ARG;
  (void)hipGetLastError();
  return hip_status(
      sa::launch_score(*dims, to_args(cache), qidx, q_seq, q_pos, n_q, scores, scores_ld, (hipStream_t)stream));
}

int sparse_attn_pool_score(const sa_dims* dims, const sa_cache* cache, const int32_t* n_pooled_in,
                           int32_t* n_pooled_out, int32_t max_new_blocks, const void* qidx, const int32_t* q_seq,
                           const int32_t* q_pos, int32_t n_q, float* scores, int64_t scores_ld, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_cache_common(dims, cache))) return rc;
  if (!cache->seq_blk0 || !cache->kidx || !cache->kpool || !n_pooled_in || !n_pooled_out) return SA_ERR_NULL;
  if (max_new_blocks < 0 || cache->kidx_ld < dims->d_idx || cache->kpool_ld < dims->d_idx) return SA_ERR_ARG;
  if (cache->n_seq > kMaxGridY) return SA_ERR_ARG;
  if (n_q < 0 || n_q > kMaxGridY) return SA_ERR_ARG;
  if (n_q > 0) {
    if (!qidx || !q_seq || !q_pos || !scores) return SA_ERR_NULL;
    if (scores_ld < (int64_t)(cache->max_len / dims->compress_ratio) || scores_ld < 0) return SA_ERR_ARG;
  }
  (void)hipGetLastError();
  const sa::CacheArgs a = to_args(cache);
  if (n_q == 0)
    return hip_status(sa::launch_pool(*dims, a, n_pooled_in, n_pooled_out, max_new_blocks, (hipStream_t)stream));
  return hip_status(sa::launch_pool_score(*dims, a, n_pooled_in, n_pooled_out, max_new_blocks, qidx, q_seq, q_pos,
                                          n_q, scores, scores_ld, (hipStream_t)stream));
}

int sparse_attn_select(const sa_dims* dims, const sa_cache* cache, const float* scores, int64_t scores_ld,
                       const int32_t* q_seq, const int32_t* q_pos, int32_t n_q, int32_t* sel, int64_t sel_ld,
                       int32_t* n_sel, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_cache_common(dims, cache))) return rc;
  if (n_q < 0) return SA_ERR_ARG;
  if (n_q == 0) return SA_OK;
  if (!scores || !q_seq || !q_pos || !sel || !n_sel) return SA_ERR_NULL;
  if (sel_ld < (int64_t)dims->top_k + dims->compress_ratio - 1) return SA_ERR_ARG;
  if (scores_ld < (int64_t)(cache->max_len / dims->compress_ratio) || scores_ld < 0) return SA_ERR_ARG;
  if (sa::select_scratch_bytes(*dims, n_q, cache->max_len) > 0) {
    const size_t need = sa::workspace_bytes(*dims, n_q, cache->max_len);
    if (!ws || ws_bytes < need) return SA_ERR_WORKSPACE;
  }
  (void)hipGetLastError();
  return hip_status(sa::launch_select(*dims, to_args(cache), scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld,
                                      n_sel, ws, (hipStream_t)stream));
}

// Checks of the attention's arguments (those sel/n_sel/q_pos/window shared with the
// select are the caller's), then its split plan for this device and the partials'
// scratch.  use_static: the partials go to the library's static scratch, ws is unused.
static int fwd_prepare(const sa_dims* dims, const sa_cache* cache, const void* q, const int32_t* q_seq,
                       const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, const int32_t* q_pos, int32_t window,
                       int32_t n_q, float scale, float* out, void* ws, size_t ws_bytes, bool use_static,
                       sa::FwdPlan* plan, void** scratch) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_cache_common(dims, cache))) return rc;
  if (n_q < 0 || (int64_t)n_q * dims->h_kv > kMaxGridY) return SA_ERR_ARG;
  if (n_q == 0) return SA_OK;
  if (!cache->k || !cache->v || !q || !q_seq || !sel || !n_sel || !out) return SA_ERR_NULL;
  if (sel_ld < 1) return SA_ERR_ARG;
  if (cache->k_ld < 1 || cache->v_ld < 1 || cache->k_head_stride < 0 || cache->v_head_stride < 0) return SA_ERR_ARG;
  if (dims->h_kv > 1 && (cache->k_head_stride < dims->d_kq || cache->v_head_stride < dims->d_v)) return SA_ERR_ARG;
  if (cache->k_ld < (int64_t)(dims->h_kv - 1) * cache->k_head_stride + dims->d_kq) return SA_ERR_ARG;
  const bool alias = cache->v == cache->k;
  if (alias && dims->d_v > dims->d_kq) return SA_ERR_ARG;
  if (cache->v_ld < (int64_t)(dims->h_kv - 1) * cache->v_head_stride + dims->d_v) return SA_ERR_ARG;
  if (!(scale == scale)) return SA_ERR_ARG;  // NaN
  if (window < 0 || window > (1 << 24)) return SA_ERR_ARG;
  if (window > 0 && !q_pos) return SA_ERR_NULL;
  const size_t ws_avail = use_static ? SA_STATIC_SCRATCH_BYTES
                                     : ((ws && ws_bytes > SA_WS_STATE_BYTES) ? ws_bytes - SA_WS_STATE_BYTES : 0);
  // The workspace is checked against the plan for the most workgroups any device
  // takes (host only); the plan for this device never needs more.
  const sa::FwdPlan bound = sa::plan_fwd_window(*dims, n_q, window, ws_avail, sa::kPlanSlots);
  if (bound.ws_bytes > 0) {
    if (use_static) {
      if (bound.ws_bytes > SA_STATIC_SCRATCH_BYTES) return SA_ERR_SCRATCH;
    } else if (!ws || ws_bytes < SA_WS_STATE_BYTES + bound.ws_bytes) {
      return SA_ERR_WORKSPACE;
    }
  }
  (void)hipGetLastError();
  *plan = sa::plan_fwd_window(*dims, n_q, window, ws_avail, sa::fwd_slots(*dims, to_args(cache), q));
  *scratch = nullptr;
  if (plan->ws_bytes > 0) {
    if (use_static) {
      if (sa::static_scratch(scratch) != hipSuccess) return SA_ERR_HIP;
    } else {
      *scratch = (char*)ws + SA_WS_STATE_BYTES;
    }
  }
  return SA_OK;
}

static int fwd_common(const sa_dims* dims, const sa_cache* cache, const void* q, const int32_t* q_seq,
                      const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, const float* sel_bias,
                      const int32_t* q_pos, int32_t window, int32_t n_q, float scale, float* out, void* ws,
                      size_t ws_bytes, void* stream, bool use_static = false) {
  sa::FwdPlan plan{};
  void* scratch = nullptr;
  const int rc = fwd_prepare(dims, cache, q, q_seq, sel, sel_ld, n_sel, q_pos, window, n_q, scale, out, ws, ws_bytes,
                             use_static, &plan, &scratch);
  if (rc != SA_OK || n_q == 0) return rc;
  return hip_status(sa::launch_fwd(*dims, to_args(cache), q, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window,
                                   n_q, scale, out, scratch, plan, (hipStream_t)stream));
}

int sparse_attn_select_fwd(const sa_dims* dims, const sa_cache* cache, const float* scores, int64_t scores_ld,
                           const int32_t* q_seq, const int32_t* q_pos, const void* q, int32_t n_q, float scale,
                           int32_t* sel, int64_t sel_ld, int32_t* n_sel, float* out, void* ws, size_t ws_bytes,
                           void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_cache_common(dims, cache))) return rc;
  if (n_q < 0) return SA_ERR_ARG;
  if (n_q == 0) return SA_OK;
  // the select's checks
  if (!scores || !q_seq || !q_pos || !sel || !n_sel) return SA_ERR_NULL;
  if (sel_ld < (int64_t)dims->top_k + dims->compress_ratio - 1) return SA_ERR_ARG;
  if (scores_ld < (int64_t)(cache->max_len / dims->compress_ratio) || scores_ld < 0) return SA_ERR_ARG;
  if (sa::select_scratch_bytes(*dims, n_q, cache->max_len) > 0) {
    const size_t need = sa::workspace_bytes(*dims, n_q, cache->max_len);
    if (!ws || ws_bytes < need) return SA_ERR_WORKSPACE;
  }
  // the attention's
  sa::FwdPlan plan{};
  void* scratch = nullptr;
  rc = fwd_prepare(dims, cache, q, q_seq, sel, sel_ld, n_sel, q_pos, 0, n_q, scale, out, ws, ws_bytes, false, &plan,
                   &scratch);
  if (rc != SA_OK) return rc;
  return hip_status(sa::launch_select_fwd(*dims, to_args(cache), scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld,
                                          n_sel, q, scale, out, ws, ws ? ws_bytes : 0, scratch, plan,
                                          (hipStream_t)stream));
}

int sparse_attn_pool_score_select_fwd(const sa_dims* dims, const sa_cache* cache, const int32_t* n_pooled_in,
                                      int32_t* n_pooled_out, int32_t max_new_blocks, const void* qidx,
                                      const int32_t* q_seq, const int32_t* q_pos, int32_t n_q, float* scores,
                                      int64_t scores_ld, const void* q, float scale, int32_t* sel, int64_t sel_ld,
                                      int32_t* n_sel, float* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_cache_common(dims, cache))) return rc;
  if (n_q < 0 || n_q > kMaxGridY) return SA_ERR_ARG;
  if (n_q == 0)                                      // nothing to score or select: the pooling alone
    return sparse_attn_pool(dims, cache, n_pooled_in, n_pooled_out, max_new_blocks, stream);
  // the pooling's and the scoring's checks
  if (!cache->seq_blk0 || !cache->kidx || !cache->kpool || !n_pooled_in || !n_pooled_out) return SA_ERR_NULL;
  if (max_new_blocks < 0 || cache->kidx_ld < dims->d_idx || cache->kpool_ld < dims->d_idx) return SA_ERR_ARG;
  if (cache->n_seq > kMaxGridY) return SA_ERR_ARG;
  if (!qidx || !q_seq || !q_pos || !scores) return SA_ERR_NULL;
  if (scores_ld < (int64_t)(cache->max_len / dims->compress_ratio) || scores_ld < 0) return SA_ERR_ARG;
  // the select's
  if (!sel || !n_sel) return SA_ERR_NULL;
  if (sel_ld < (int64_t)dims->top_k + dims->compress_ratio - 1) return SA_ERR_ARG;
  if (sa::select_scratch_bytes(*dims, n_q, cache->max_len) > 0) {
    const size_t need = sa::workspace_bytes(*dims, n_q, cache->max_len);
    if (!ws || ws_bytes < need) return SA_ERR_WORKSPACE;
  }
  // the attention's
  sa::FwdPlan plan{};
  void* scratch = nullptr;
  rc = fwd_prepare(dims, cache, q, q_seq, sel, sel_ld, n_sel, q_pos, 0, n_q, scale, out, ws, ws_bytes, false, &plan,
                   &scratch);
  if (rc != SA_OK) return rc;
  return hip_status(sa::launch_pool_score_select_fwd(*dims, to_args(cache), n_pooled_in, n_pooled_out,
                                                     max_new_blocks, qidx, q_seq, q_pos, n_q, scores, scores_ld, q,
                                                     scale, sel, sel_ld, n_sel, out, ws, ws ? ws_bytes : 0, scratch,
                                                     plan, (hipStream_t)stream));
}

int sparse_attn_pool_score_select_fwd_uses_list(const sa_dims* dims, const sa_cache* cache,
                                                const int32_t* n_pooled_in, const int32_t* n_pooled_out,
                                                const void* qidx, const void* q, int32_t n_q) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_cache_common(dims, cache))) return rc;
  if (n_q < 1 || (int64_t)n_q * dims->h_kv > kMaxGridY) return SA_ERR_ARG;
  if (!cache->k || !cache->v || !q || !qidx || !n_pooled_in || !n_pooled_out) return SA_ERR_NULL;
  const sa::CacheArgs a = to_args(cache);
  const sa::FwdPlan plan = sa::plan_fwd_window(*dims, n_q, 0, SIZE_MAX, sa::fwd_slots(*dims, a, q));
  return sa::step_uses_cand(*dims, a, qidx, q, n_q, n_pooled_in, n_pooled_out, plan,
                            sa::workspace_bytes(*dims, n_q, cache->max_len))
             ? 1
             : 0;
}

int sparse_attn_select_fwd_is_fused(const sa_dims* dims, const sa_cache* cache, const void* q, int32_t n_q) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_cache_common(dims, cache))) return rc;
  if (n_q < 1 || (int64_t)n_q * dims->h_kv > kMaxGridY) return SA_ERR_ARG;
  if (!cache->k || !cache->v || !q) return SA_ERR_NULL;
  const sa::CacheArgs a = to_args(cache);
  const sa::FwdPlan plan = sa::plan_fwd_window(*dims, n_q, 0, SIZE_MAX, sa::fwd_slots(*dims, a, q));
  // with a workspace of sparse_attn_workspace_bytes
  return sa::select_fwd_fused(*dims, a, q, n_q, plan, sa::workspace_bytes(*dims, n_q, cache->max_len)) ? 1 : 0;
}

int sparse_attn_fwd(const sa_dims* dims, const sa_cache* cache, const void* q, const int32_t* q_seq,
                    const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, int32_t n_q, float scale, float* out,
                    void* ws, size_t ws_bytes, void* stream) {
  return fwd_common(dims, cache, q, q_seq, sel, sel_ld, n_sel, nullptr, nullptr, 0, n_q, scale, out, ws, ws_bytes,
                    stream);
}

int sparse_attn_fwd_noalloc(const sa_dims* dims, const sa_cache* cache, const void* q, const int32_t* q_seq,
                            const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, int32_t n_q, float scale,
                            float* out, void* stream) {
  return fwd_common(dims, cache, q, q_seq, sel, sel_ld, n_sel, nullptr, nullptr, 0, n_q, scale, out, nullptr, 0,
                    stream, /*use_static=*/true);
}

int sparse_attn_fwd_window(const sa_dims* dims, const sa_cache* cache, const void* q, const int32_t* q_seq,
                           const int32_t* q_pos, const int32_t* sel, int64_t sel_ld, const int32_t* n_sel,
                           int32_t window, int32_t n_q, float scale, float* out, void* ws, size_t ws_bytes,
                           void* stream) {
  return fwd_common(dims, cache, q, q_seq, sel, sel_ld, n_sel, nullptr, q_pos, window, n_q, scale, out, ws,
                    ws_bytes, stream);
}

int sparse_attn_fwd_bias(const sa_dims* dims, const sa_cache* cache, const void* q, const int32_t* q_seq,
                         const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, const float* sel_bias,
                         int32_t n_q, float scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  return fwd_common(dims, cache, q, q_seq, sel, sel_ld, n_sel, sel_bias, nullptr, 0, n_q, scale, out, ws, ws_bytes,
                    stream);
}

int sparse_attn_mask_to_indices(const void* mask, int32_t mask_dtype, int64_t mask_ld, int32_t n_q, int32_t n_kv,
                                int32_t* sel, int64_t sel_ld, int32_t* n_sel, float* sel_bias, void* stream) {
  if (mask_dtype != SA_F16 && mask_dtype != SA_F32) return SA_ERR_ARG;
  if (n_q < 0 || n_kv < 0 || sel_ld < 1 || mask_ld < n_kv) return SA_ERR_ARG;
  if (n_q == 0) return SA_OK;
  if ((n_kv > 0 && !mask) || !sel || !n_sel) return SA_ERR_NULL;
  (void)hipGetLastError();
  return hip_status(sa::launch_mask_to_indices(mask, mask_dtype, mask_ld, n_q, n_kv, sel, sel_ld, n_sel, sel_bias,
                                               (hipStream_t)stream));
}

int sparse_attn_quantize_q8_0(const void* x, int32_t x_dtype, int64_t n_rows, int32_t n_cols, int64_t x_ld,
                              int8_t* codes, int64_t codes_ld, uint16_t* scales, int64_t scales_ld, void* stream) {
  if (!dtype_ok(x_dtype)) return SA_ERR_ARG;
  if (n_rows < 0 || n_cols < 0 || n_cols % 32 != 0) return SA_ERR_ARG;
  if (n_rows == 0 || n_cols == 0) return SA_OK;
  if (!x || !codes || !scales) return SA_ERR_NULL;
  if (x_ld < n_cols || codes_ld < n_cols || scales_ld < n_cols / 32) return SA_ERR_ARG;
  if ((uintptr_t)codes % 4 != 0 || codes_ld % 4 != 0) return SA_ERR_ARG;
  if (n_rows > ((int64_t)1 << 40) / (n_cols / 32)) return SA_ERR_ARG;
  (void)hipGetLastError();
  return hip_status(sa::launch_quantize_q8_0(x, x_dtype, n_rows, n_cols, x_ld, codes, codes_ld, scales, scales_ld,
                                             (hipStream_t)stream));
}

int sparse_attn_fwd_q8_0(const sa_dims* dims, const sa_cache* cache, const sa_kv_q8_0* kv, const void* q,
                         const int32_t* q_seq, const int32_t* sel, int64_t sel_ld, const int32_t* n_sel,
                         int32_t n_q, float scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_cache_common(dims, cache))) return rc;
  if (!kv) return SA_ERR_NULL;
  if (dims->d_kq % 32 != 0 || dims->d_v % 32 != 0) return SA_ERR_ARG;
  if (n_q < 0 || (int64_t)n_q * dims->h_kv > kMaxGridY) return SA_ERR_ARG;
  if (n_q == 0) return SA_OK;
  if (!kv->k || !kv->k_scale || !kv->v || !kv->v_scale || !q || !q_seq || !sel || !n_sel || !out) return SA_ERR_NULL;
  if (sel_ld < 1) return SA_ERR_ARG;
  if (kv->k_head_stride < 0 || kv->v_head_stride < 0 || kv->k_scale_head_stride < 0 || kv->v_scale_head_stride < 0)
    return SA_ERR_ARG;
  const int64_t hk = dims->h_kv - 1;
  if (dims->h_kv > 1 && (kv->k_head_stride < dims->d_kq || kv->v_head_stride < dims->d_v ||
                         kv->k_scale_head_stride < dims->d_kq / 32 || kv->v_scale_head_stride < dims->d_v / 32))
    return SA_ERR_ARG;
  if (kv->k_ld < hk * kv->k_head_stride + dims->d_kq || kv->v_ld < hk * kv->v_head_stride + dims->d_v) return SA_ERR_ARG;
  if (kv->k_scale_ld < hk * kv->k_scale_head_stride + dims->d_kq / 32 ||
      kv->v_scale_ld < hk * kv->v_scale_head_stride + dims->d_v / 32)
    return SA_ERR_ARG;
  if (kv->v == kv->k && dims->d_v > dims->d_kq) return SA_ERR_ARG;
  if (!(scale == scale)) return SA_ERR_ARG;  // NaN
  const sa::FwdPlan plan = sa::plan_fwd(*dims, n_q);
  void* scratch = nullptr;
  if (plan.ws_bytes > 0) {
    if (!ws || ws_bytes < SA_WS_STATE_BYTES + plan.ws_bytes) return SA_ERR_WORKSPACE;
    scratch = (char*)ws + SA_WS_STATE_BYTES;
  }
  sa::Q8Args a;
  a.k = kv->k;
  a.k_ld = kv->k_ld;
  a.k_hs = kv->k_head_stride;
  a.ks = kv->k_scale;
  a.ks_ld = kv->k_scale_ld;
  a.ks_hs = kv->k_scale_head_stride;
  a.v = kv->v;
  a.v_ld = kv->v_ld;
  a.v_hs = kv->v_head_stride;
  a.vs = kv->v_scale;
  a.vs_ld = kv->v_scale_ld;
  a.vs_hs = kv->v_scale_head_stride;
  (void)hipGetLastError();
  return hip_status(sa::launch_fwd_q8(*dims, to_args(cache), a, q, q_seq, sel, sel_ld, n_sel, n_q, scale, out,
                                      scratch, plan, (hipStream_t)stream));
}

const char* sparse_attn_strerror(int code) {
  switch (code) {
    case SA_OK: return "success";
    case SA_ERR_NULL: return "a required pointer is NULL";
    case SA_ERR_DIMS: return "unsupported or inconsistent dimensions";
    case SA_ERR_ARG: return "argument out of range";
    case SA_ERR_WORKSPACE: return "workspace missing or too small";
    case SA_ERR_HIP: return "HIP kernel launch failed";
    case SA_ERR_SCRATCH: return "the call needs more than the library's static scratch (SA_STATIC_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

const char* sparse_attn_version(void) { return "sparse_attn 0.1 gfx950"; }

}  // extern "C"
