// Index lists from additive attention masks.
//
// In the pages' mask-driven sparse flash attention the finite entries of a query's
// mask row are the K/V set and their values are added to the logits; a bound on the
// finite count per row sizes an ascending int32 index list, -1 padded, that the
// attention kernel gathers by (llama.cpp PR #27970 "CUDA + ggml: add sparse-fa for
// DSV4/GLM": ggml_flash_attn_ext_set_sparse and the mask-to-indices kernel).  Here
// that list is the same one the block selection produces, and the mask values of
// the listed positions are written beside it for sparse_attn_fwd_bias.
//
// One 256-thread workgroup per mask row streams the row in chunks: thread t examines
// 16 consecutive columns, a workgroup prefix sum over the per-thread finite counts
// gives each thread its output offset, so positions come out in ascending order.
#include "sa_common.hpp"
#include "sa_launch.hpp"

namespace sa {

constexpr int kMaskThreads = 256;
constexpr int kMaskPer = 16;                         // columns per thread per chunk

template <typename M>
__global__ void __launch_bounds__(kMaskThreads)
mask_to_indices_kernel(const M* __restrict__ mask, int64_t mask_ld, int n_kv, int32_t* __restrict__ sel,
                       int64_t sel_ld, int32_t* __restrict__ n_sel, float* __restrict__ sel_bias) {
  __shared__ int scan[kMaskThreads / kWave + 1];
  const int i = blockIdx.x, tid = threadIdx.x;
  const M* row = mask + (int64_t)i * mask_ld;
  int32_t* out = sel + (int64_t)i * sel_ld;
  float* bout = sel_bias ? sel_bias + (int64_t)i * sel_ld : nullptr;
  int64_t base = 0;                                  // finite entries in earlier chunks
  for (int c0 = 0; c0 < n_kv; c0 += kMaskThreads * kMaskPer) {
    const int p0 = c0 + tid * kMaskPer;
    float v[kMaskPer];
    uint32_t fin = 0;
#pragma unroll
    for (int j = 0; j < kMaskPer; ++j) {
      v[j] = (float)row[min(p0 + j, n_kv - 1)];     // clamped: the loads need no guard
      if (p0 + j < n_kv && __builtin_isfinite(v[j])) fin |= 1u << j;
    }
    int total;
    int64_t o = base + block_exclusive_scan<kMaskThreads>(__popc(fin), scan, &total);
    while (fin != 0u) {
      const int j = __ffs(fin) - 1;
      fin &= fin - 1u;
      if (o < sel_ld) {
        out[o] = p0 + j;
        if (bout) bout[o] = v[j];
      }
      ++o;
    }
    base += total;
  }
  for (int64_t j = min(base, sel_ld) + tid; j < sel_ld; j += kMaskThreads) {
    out[j] = -1;
    if (bout) bout[j] = 0.f;
  }
  if (tid == 0) n_sel[i] = (int32_t)min(base, (int64_t)0x7fffffff);
}

hipError_t launch_mask_to_indices(const void* mask, int mask_dtype, int64_t mask_ld, int n_q, int n_kv,
                                  int32_t* sel, int64_t sel_ld, int32_t* n_sel, float* sel_bias, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  if (n_kv == 0) {                                   // no columns: every list is empty
    hipLaunchKernelGGL((mask_to_indices_kernel<float>), dim3(n_q), dim3(kMaskThreads), 0, stream,
                       (const float*)mask, mask_ld, 0, sel, sel_ld, n_sel, sel_bias);
  } else if (mask_dtype == SA_F16) {
    hipLaunchKernelGGL((mask_to_indices_kernel<f16>), dim3(n_q), dim3(kMaskThreads), 0, stream, (const f16*)mask,
                       mask_ld, n_kv, sel, sel_ld, n_sel, sel_bias);
  } else {
    hipLaunchKernelGGL((mask_to_indices_kernel<float>), dim3(n_q), dim3(kMaskThreads), 0, stream,
                       (const float*)mask, mask_ld, n_kv, sel, sel_ld, n_sel, sel_bias);
  }
  return hipGetLastError();
}

}  // namespace sa
