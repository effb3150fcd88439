// Host-side launchers of the sparse-attention kernels.  Internal to the library:
// the C ABI in api.cpp validates every argument, then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

// Plain-old-data view of sa_cache with typed-agnostic pointers, as the kernels see it.
struct CacheArgs {
  int n_seq;
  int max_len;
  const int64_t* seq_row0;
  const int64_t* seq_blk0;
  const int32_t* seq_len;
  const void* k;
  int64_t k_ld, k_hs;
  const void* v;
  int64_t v_ld, v_hs;
  const void* kidx;
  int64_t kidx_ld;
  void* kpool;
  int64_t kpool_ld;
};

hipError_t launch_pool(const sa_dims& d, const CacheArgs& c, const int32_t* n_pooled_in,
                       int32_t* n_pooled_out, int max_new_blocks, hipStream_t stream);

hipError_t launch_score(const sa_dims& d, const CacheArgs& c, const void* qidx, const int32_t* q_seq,
                        const int32_t* q_pos, int n_q, float* scores, int64_t scores_ld, hipStream_t stream);

// Workspace bytes of the selection (0 when one workgroup per query token is used).
size_t select_ws_bytes(const sa_dims& d, int n_q, int max_len);

hipError_t launch_select(const sa_dims& d, const CacheArgs& c, const float* scores, int64_t scores_ld,
                         const int32_t* q_seq, const int32_t* q_pos, int n_q, int32_t* sel, int64_t sel_ld,
                         int32_t* n_sel, void* ws, hipStream_t stream);

// Split-KV partition of the attention for n_q query tokens: rows of each query's
// list handled per split (a multiple of 32) and the number of splits.
struct FwdPlan {
  int n_split;
  int rows_per_split;
  size_t ws_bytes;
};
FwdPlan plan_fwd(const sa_dims& d, int n_q);

hipError_t launch_fwd(const sa_dims& d, const CacheArgs& c, const void* q, const int32_t* q_seq,
                      const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, int n_q, float scale, float* out,
                      void* ws, const FwdPlan& plan, hipStream_t stream);

// Which implementation a call takes (exposed for tests and reports).
bool score_uses_mfma(const sa_dims& d, const CacheArgs& c, const void* qidx);
bool fwd_uses_mfma(const sa_dims& d, const CacheArgs& c, const void* q);

}  // namespace sa
