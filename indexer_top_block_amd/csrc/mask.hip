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
// the loads of four chunks (two for fp32) in flight at a time: thread t examines 32
// consecutive columns of each chunk (16-byte loads when the rows are aligned) and
// keeps a bitmask of the finite ones.  One workgroup exchange of per-wave counts per
// group of chunks gives every thread its output offset in each chunk, so positions
// come out in ascending order.  The values of the listed entries come from an LDS copy
// of the thread's own span (laid out [quad][thread], so its writes are conflict-free
// and a thread reads back only what it wrote: no barrier), not from a second read of
// the row.  Lists that fit (kMaskListCap) are assembled in LDS and written out
// coalesced at the end instead of as scattered stores of a few lanes each.
#include "sa_common.hpp"
#include "sa_launch.hpp"

namespace sa {

constexpr int kMaskThreads = 1024;
constexpr int kMaskPer = 32;                         // consecutive columns per thread per chunk
// list entries assembled in LDS (beside the 64 KiB (f16) or 128 KiB (fp32) value copy)
template <typename M> constexpr int kMaskListCap = sizeof(M) == 2 ? 8192 : 2048;

__device__ __forceinline__ bool finite_bits(f16 x) { return (__builtin_bit_cast(uint16_t, x) & 0x7c00u) != 0x7c00u; }
__device__ __forceinline__ bool finite_bits(float x) { return (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u; }

// VEC: the row is 16-byte aligned (checked on the host), so whole per-thread spans
// are read with 16-byte loads.
template <typename M, bool VEC>
__global__ void __launch_bounds__(kMaskThreads)
mask_to_indices_kernel(const M* __restrict__ mask, int64_t mask_ld, int n_kv, int32_t* __restrict__ sel,
                       int64_t sel_ld, int32_t* __restrict__ n_sel, float* __restrict__ sel_bias) {
  constexpr int EV = 16 / sizeof(M);                 // elements per 16-byte load
  constexpr int NQ = kMaskPer / EV;                  // 16-byte quads per thread per chunk
  constexpr int CHUNK = kMaskThreads * kMaskPer;
  constexpr int G = (VEC ? 8 : 4) / (int)sizeof(M);  // chunks in flight: 64 (32 unaligned) registers of raw data
  constexpr int NW = kMaskThreads / kWave;
  typedef M vec_t __attribute__((ext_vector_type(EV)));
  __shared__ int wtot[2][G][NW];                     // per-wave finite counts, alternating by group
  __shared__ __attribute__((aligned(16))) vec_t vstage[NQ][kMaskThreads];   // this chunk's values, [quad][thread]
  constexpr int LCAP = kMaskListCap<M>;
  __shared__ int32_t lpos[LCAP];                     // the list, when it fits
  __shared__ float lval[LCAP];
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const M* row = mask + (int64_t)i * mask_ld;
  int32_t* out = sel + (int64_t)i * sel_ld;
  float* bout = sel_bias ? sel_bias + (int64_t)i * sel_ld : nullptr;
  const M* vals = reinterpret_cast<const M*>(vstage);
  const bool staged = sel_ld <= LCAP;                // the list is assembled in LDS
  int64_t base = 0;                                  // finite entries in earlier groups
  int par = 0;
  for (int g0 = 0; g0 < n_kv; g0 += G * CHUNK, par ^= 1) {
    // every load of the group first (clamped, not guarded) ...
    // (a group wholly inside the row needs no bounds checks: the common case)
    const bool whole = VEC && g0 + G * CHUNK <= n_kv;
    vec_t raw[G][NQ];
    if (whole) {
#pragma unroll
      for (int c = 0; c < G; ++c)
#pragma unroll
        for (int u = 0; u < NQ; ++u)
          raw[c][u] = *reinterpret_cast<const vec_t*>(row + g0 + c * CHUNK + tid * kMaskPer + u * EV);
    } else {
#pragma unroll
      for (int c = 0; c < G; ++c) {
        const int p0 = g0 + c * CHUNK + tid * kMaskPer;
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
          if (VEC && p0 + kMaskPer <= n_kv) {
            raw[c][u] = *reinterpret_cast<const vec_t*>(row + p0 + u * EV);
          } else {
#pragma unroll
            for (int e = 0; e < EV; ++e) raw[c][u][e] = row[min(p0 + u * EV + e, n_kv - 1)];
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ... then the finite bitmasks and one exchange of the per-wave counts ...
    uint32_t fin[G];
    int incl[G];
#pragma unroll
    for (int c = 0; c < G; ++c) {
      const int p0 = g0 + c * CHUNK + tid * kMaskPer;
      fin[c] = 0u;
      if (whole) {
#pragma unroll
        for (int u = 0; u < NQ; ++u)
#pragma unroll
          for (int e = 0; e < EV; ++e) fin[c] |= finite_bits(raw[c][u][e]) ? 1u << (u * EV + e) : 0u;
      } else {
#pragma unroll
        for (int u = 0; u < NQ; ++u)
#pragma unroll
          for (int e = 0; e < EV; ++e)
            fin[c] |= (p0 + u * EV + e < n_kv && finite_bits(raw[c][u][e])) ? 1u << (u * EV + e) : 0u;
      }
      incl[c] = wave_inclusive_scan(__popc(fin[c]), lane);
      if (lane == kWave - 1) wtot[par][c][wave] = incl[c];
    }
    __syncthreads();
    // ... then each chunk's positions (and values) at the thread's offset
#pragma unroll
    for (int c = 0; c < G; ++c) {
      int tot = 0, before = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int v = wtot[par][c][w];
        tot += v;
        before += w < wave ? v : 0;
      }
      int64_t o = base + before + incl[c] - __popc(fin[c]);
      const int p0 = g0 + c * CHUNK + tid * kMaskPer;
      uint32_t f = fin[c];
      if (bout) {
#pragma unroll
        for (int u = 0; u < NQ; ++u) vstage[u][tid] = raw[c][u];
      }
      if (staged) {
        int oo = (int)min(o, (int64_t)LCAP);         // entries past sel_ld (<= LCAP) are counted only
        while (f != 0u && oo < sel_ld) {
          const int j = __ffs(f) - 1;
          f &= f - 1u;
          lpos[oo] = p0 + j;
          if (bout) lval[oo] = (float)vals[((j / EV) * kMaskThreads + tid) * EV + j % EV];
          ++oo;
        }
      } else {
        while (f != 0u) {
          const int j = __ffs(f) - 1;
          f &= f - 1u;
          if (o < sel_ld) {
            out[o] = p0 + j;
            if (bout) bout[o] = (float)vals[((j / EV) * kMaskThreads + tid) * EV + j % EV];
          }
          ++o;
        }
      }
      base += tot;
    }
  }
  const int n_list = (int)min(base, sel_ld);
  if (staged) {
    __syncthreads();
    for (int j = tid; j < n_list; j += kMaskThreads) {
      out[j] = lpos[j];
      if (bout) bout[j] = lval[j];
    }
  }
  for (int64_t j = n_list + tid; j < sel_ld; j += kMaskThreads) {
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
