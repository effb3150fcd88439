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
// sparse_attn_pool then sparse_attn_score, in one launch when the decode scoring
// kernel applies (else the two launches).
// cand (optional): the candidate list of the fused select (the cand_keep <= kCandKeep
// best blocks of every kCandTile, select_wide.hpp), cand_ld words per query token;
// only the pooling scoring launch writes it (pool_score_fused), else the call fails.
hipError_t launch_pool_score(const sa_dims& d, const CacheArgs& c, const int32_t* n_in, int32_t* n_out, int max_new,
                             const void* qidx, const int32_t* q_seq, const int32_t* q_pos, int n_q, float* scores,
                             int64_t scores_ld, hipStream_t stream, uint32_t* cand = nullptr, int64_t cand_ld = 0,
                             int cand_keep = 0, int cand_tpt = 0);
bool pool_score_fused(const sa_dims& d, const CacheArgs& c, const void* qidx, int n_q, const int32_t* n_in,
                      const int32_t* n_out);

// Workspace layout shared by sparse_attn_select and sparse_attn_fwd:
//   [0, SA_WS_STATE_BYTES)   state -- zero before the first call, left zero by every call
//                            (the chunked selection's histograms);
//   [SA_WS_STATE_BYTES, ...) scratch -- overwritten by each call.
constexpr int kStateQueries = 64;          // query tokens the chunked selection keeps state for
struct WsState {
  uint32_t ghist[kStateQueries][4096];     // per-query histogram of the top 12 key bits
};
static_assert(sizeof(WsState) <= SA_WS_STATE_BYTES, "state region too small");

// Scratch bytes of the chunked selection (0 when one workgroup per query token is used).
size_t select_scratch_bytes(const sa_dims& d, int n_q, int max_len);

// ws: the whole workspace (state at offset 0).
hipError_t launch_select(const sa_dims& d, const CacheArgs& c, const float* scores, int64_t scores_ld,
                         const int32_t* q_seq, const int32_t* q_pos, int n_q, int32_t* sel, int64_t sel_ld,
                         int32_t* n_sel, void* ws, hipStream_t stream);
// Whether the selection takes the chunked passes, and over how many chunks.
bool select_chunked(const sa_dims& d, int n_q, int max_len);
int select_chunk_count(const sa_dims& d, int max_len);
// The chunked selection's first two launches (histogram, candidates); the finishing
// pass is the caller's.  ws: the whole workspace.
hipError_t launch_chunk_passes(const sa_dims& d, const CacheArgs& c, const float* scores, int64_t scores_ld,
                               const int32_t* q_seq, const int32_t* q_pos, int n_q, int32_t* sel, int64_t sel_ld,
                               int32_t* n_sel, void* ws, hipStream_t stream);

// Split-KV partition of the attention for n_q query tokens: rows of each query's
// list handled per split (a multiple of 32) and the number of splits.
struct FwdPlan {
  int n_split;
  int rows_per_split;
  int list_max;                            // list entries attended at most (top_k + c - 1)
  size_t ws_bytes;                         // scratch bytes (partial results), 0 when unsplit
};
FwdPlan plan_fwd(const sa_dims& d, int n_q);
constexpr long long kPlanSlots = 512;      // the most workgroups a split plan aims at
// A q8_0 K/V cache: int8 code planes and float16 scale planes (one scale per 32
// codes), strides in elements.
struct Q8Args {
  const void* k;
  int64_t k_ld, k_hs;
  const void* ks;
  int64_t ks_ld, ks_hs;
  const void* v;
  int64_t v_ld, v_hs;
  const void* vs;
  int64_t vs_ld, vs_hs;
};
bool fwd_q8_uses_lds(const sa_dims& d, const Q8Args& kv, const void* q);
hipError_t launch_fwd_q8(const sa_dims& d, const CacheArgs& c, const Q8Args& kv, const void* q, const int32_t* q_seq,
                         const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, int n_q, float scale, float* out,
                         void* ws, const FwdPlan& plan, hipStream_t stream);
hipError_t launch_quantize_q8_0(const void* x, int x_dtype, int64_t n_rows, int n_cols, int64_t x_ld, int8_t* codes,
                                int64_t codes_ld, void* scales, int64_t scales_ld, hipStream_t stream);
// Compute units of the current device (cached per device; 0 if unknown).
int device_cus();
// Merges the split partials (ws_o, ws_ml) into out; nothing when unsplit.
hipError_t launch_combine(const sa_dims& d, int n_q, float* out, const float* ws_o, const float* ws_ml,
                          const FwdPlan& plan, hipStream_t stream);
FwdPlan plan_fwd_window(const sa_dims& d, int n_q, int window, size_t ws_avail, long long slots);
// Workgroups that fill the chip for the attention kernel this call takes.
long long fwd_slots(const sa_dims& d, const CacheArgs& c, const void* q);

// ws: the scratch part of the workspace.
hipError_t launch_mask_to_indices(const void* mask, int mask_dtype, int64_t mask_ld, int n_q, int n_kv,
                                  int32_t* sel, int64_t sel_ld, int32_t* n_sel, float* sel_bias, hipStream_t stream);

hipError_t launch_fwd(const sa_dims& d, const CacheArgs& c, const void* q, const int32_t* q_seq,
                      const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, const float* sel_bias,
                      const int32_t* q_pos, int window, int n_q, float scale, float* out, void* ws,
                      const FwdPlan& plan, hipStream_t stream);

// sparse_attn_select then sparse_attn_fwd (plain form) for the same query tokens, with
// the selection (or its finishing pass) inside the attention's launch when
// select_fwd_fused says so (select_fwd.hip).  ws / ws_bytes: the whole workspace (the
// select's); scratch: its partials part for the two calls (null when unsplit).
bool select_fwd_fused(const sa_dims& d, const CacheArgs& c, const void* q, int n_q, const FwdPlan& plan,
                      size_t ws_bytes);
// cand (optional): the scoring launch's candidate list (cand_ld words per query token,
// then a word per query token that the launch sets to 1 when the list decided that
// token's selection, else 0); only for the one-workgroup form, else the call fails.
hipError_t launch_select_fwd(const sa_dims& d, const CacheArgs& c, const float* scores, int64_t scores_ld,
                             const int32_t* q_seq, const int32_t* q_pos, int n_q, int32_t* sel, int64_t sel_ld,
                             int32_t* n_sel, const void* q, float scale, float* out, void* ws, size_t ws_bytes,
                             void* scratch, const FwdPlan& plan, hipStream_t stream, const uint32_t* cand = nullptr,
                             int64_t cand_ld = 0);

// The candidate list (select_fwd.hip): the best blocks it keeps per 32-block tile (8,
// or 4 for rows of 131073-262144 blocks; 0: no list), the tiles each select thread
// reads (1 for rows of up to 32768 blocks, else 32 / keep), its words per query token, and
// its bytes for n_q tokens with the decided flags (0 when the list is never used: rows
// that are always dense or longer than 262144 blocks, more query tokens than the
// pooling scoring launch takes, or more than 8192 tiles in all); it is the workspace's
// last part.
int cand_keep(const sa_dims& d, int max_len);
int cand_tpt(const sa_dims& d, int max_len);
int64_t cand_words(const sa_dims& d, int max_len);
size_t cand_bytes(const sa_dims& d, int n_q, int max_len);

// sparse_attn_pool_score then sparse_attn_select_fwd; where the pooling scoring launch
// and a fused select both apply and ws holds workspace_bytes, the scoring launch also
// writes the candidate list and the select starts from it (rows of up to 32768 blocks
// in select_fwd_kernel, longer ones in list_fwd_kernel).
hipError_t launch_pool_score_select_fwd(const sa_dims& d, const CacheArgs& c, const int32_t* n_in, int32_t* n_out,
                                        int max_new, const void* qidx, const int32_t* q_seq, const int32_t* q_pos,
                                        int n_q, float* scores, int64_t scores_ld, const void* q, float scale,
                                        int32_t* sel, int64_t sel_ld, int32_t* n_sel, float* out, void* ws,
                                        size_t ws_bytes, void* scratch, const FwdPlan& plan, hipStream_t stream);
// Whether launch_pool_score_select_fwd starts the select from the candidate list.
bool step_uses_cand(const sa_dims& d, const CacheArgs& c, const void* qidx, const void* q, int n_q,
                    const int32_t* n_in, const int32_t* n_out, const FwdPlan& plan, size_t ws_bytes);

// Device address of this device's copy of the static scratch array
// (SA_STATIC_SCRATCH_BYTES), looked up on first use per device (fwd_static.hip).
hipError_t static_scratch(void** ptr);

// Total workspace bytes for n_q query tokens (state, then the chunked selection's
// scratch, the attention's partials and the candidate list side by side), 0 if none.
size_t workspace_bytes(const sa_dims& d, int n_q, int max_len);
size_t workspace_bytes_window(const sa_dims& d, int n_q, int max_len, int window);

// Which implementation a call takes (exposed for tests and reports).
bool score_uses_mfma(const sa_dims& d, const CacheArgs& c, const void* qidx);
bool fwd_uses_mfma(const sa_dims& d, const CacheArgs& c, const void* q);

}  // namespace sa
