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
// One 1024-thread workgroup per mask row streams the row in chunks of 32768 columns,
// two chunks' loads in flight at a time (one for fp32): thread t examines 32 consecutive columns of
// a chunk (16-byte loads when the rows are aligned), and a workgroup prefix sum over
// the per-thread finite counts gives each thread its output offset, so positions come
// out in ascending order.
#include "sa_common.hpp"
#include "sa_launch.hpp"

namespace sa {

constexpr int kMaskThreads = 1024;
constexpr int kMaskPer = 32;                         // consecutive columns per thread per chunk

// VEC: the row is 16-byte aligned (checked on the host), so whole per-thread spans
// are read with 16-byte loads.  Only a bitmask of the finite columns is kept; the
// values of the (few) listed entries are read again when they are written.
template <typename M, bool VEC>
__global__ void __launch_bounds__(kMaskThreads)
mask_to_indices_kernel(const M* __restrict__ mask, int64_t mask_ld, int n_kv, int32_t* __restrict__ sel,
                       int64_t sel_ld, int32_t* __restrict__ n_sel, float* __restrict__ sel_bias) {
  constexpr int EV = 16 / sizeof(M);                 // elements per 16-byte load
  constexpr int CHUNK = kMaskThreads * kMaskPer;
  constexpr int kMaskGroup = 4 / (int)sizeof(M);     // chunks in flight: 32 registers of raw data
  typedef M vec_t __attribute__((ext_vector_type(EV)));
  __shared__ int scan[kMaskThreads / kWave + 1];
  const int i = blockIdx.x, tid = threadIdx.x;
  const M* row = mask + (int64_t)i * mask_ld;
  int32_t* out = sel + (int64_t)i * sel_ld;
  float* bout = sel_bias ? sel_bias + (int64_t)i * sel_ld : nullptr;
  int64_t base = 0;                                  // finite entries in earlier chunks
  for (int g0 = 0; g0 < n_kv; g0 += kMaskGroup * CHUNK) {
    // every load of the group first (clamped, not guarded) ...
    vec_t raw[kMaskGroup][kMaskPer / EV];
#pragma unroll
    for (int c = 0; c < kMaskGroup; ++c) {
      const int p0 = g0 + c * CHUNK + tid * kMaskPer;
#pragma unroll
      for (int u = 0; u < kMaskPer / EV; ++u) {
        if (VEC && p0 + kMaskPer <= n_kv) {
          raw[c][u] = *reinterpret_cast<const vec_t*>(row + p0 + u * EV);
        } else {
#pragma unroll
          for (int e = 0; e < EV; ++e) raw[c][u][e] = row[min(p0 + u * EV + e, n_kv - 1)];
        }
      }
    }
    // ... then per chunk: finite bitmask, offsets, writes
#pragma unroll
    for (int c = 0; c < kMaskGroup; ++c) {
      const int p0 = g0 + c * CHUNK + tid * kMaskPer;
      uint32_t fin = 0;
#pragma unroll
      for (int u = 0; u < kMaskPer / EV; ++u)
#pragma unroll
        for (int e = 0; e < EV; ++e) {
          const int j = u * EV + e;
          if (p0 + j < n_kv && __builtin_isfinite((float)raw[c][u][e])) fin |= 1u << j;
        }
      int total;
      int64_t o = base + block_exclusive_scan<kMaskThreads>(__popc(fin), scan, &total);
      while (fin != 0u) {
        const int j = __ffs(fin) - 1;
        fin &= fin - 1u;
        if (o < sel_ld) {
          out[o] = p0 + j;
          if (bout) bout[o] = (float)row[p0 + j];
        }
        ++o;
      }
      base += total;
    }
  }
  for (int64_t j = min(base, sel_ld) + tid; j < sel_ld; j += kMaskThreads) {
    out[j] = -1;
    if (bout) bout[j] = 0.f;
  }
  if (tid == 0) n_sel[i] = (int32_t)min(base, (int64_t)0x7fffffff);
}

template <typename M>
static void launch_m(const void* mask, int64_t mask_ld, int n_q, int n_kv, int32_t* sel, int64_t sel_ld,
                     int32_t* n_sel, float* sel_bias, hipStream_t stream) {
  const bool vec = ((uintptr_t)mask % 16 == 0) && ((mask_ld * (int64_t)sizeof(M)) % 16 == 0);
  if (vec)
    hipLaunchKernelGGL((mask_to_indices_kernel<M, true>), dim3(n_q), dim3(kMaskThreads), 0, stream, (const M*)mask,
                       mask_ld, n_kv, sel, sel_ld, n_sel, sel_bias);
  else
    hipLaunchKernelGGL((mask_to_indices_kernel<M, false>), dim3(n_q), dim3(kMaskThreads), 0, stream, (const M*)mask,
                       mask_ld, n_kv, sel, sel_ld, n_sel, sel_bias);
}

hipError_t launch_mask_to_indices(const void* mask, int mask_dtype, int64_t mask_ld, int n_q, int n_kv,
                                  int32_t* sel, int64_t sel_ld, int32_t* n_sel, float* sel_bias, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  if (mask_dtype == SA_F16) launch_m<f16>(mask, mask_ld, n_q, n_kv, sel, sel_ld, n_sel, sel_bias, stream);
  else launch_m<float>(mask, mask_ld, n_q, n_kv, sel, sel_ld, n_sel, sel_bias, stream);
  return hipGetLastError();
}

}  // namespace sa
