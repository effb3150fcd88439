// q8_0 quantization of K/V rows, the write side of a q8_0 cache.
//
// The pages serve the sparse graph with K and V caches of type q8_0 (qwen4exp commit
// series: a quantized KV cache on the QSA attention path).  q8_0 is ggml's block
// format: per 32 consecutive elements d = max|x| / 127 (stored as float16) and codes
// x / d rounded half away from zero (all zero for an all-zero block).  The codes are
// decided in float32: max|x| exactly, one correctly rounded division for d and one
// for 1/d, one product per element, then the rounding.
//
// One thread per block of 32: it reads the block's 32 elements, writes 32 codes and
// one scale.  Codes go to a plane [n_rows][codes_ld] of int8, scales to a plane
// [n_rows][scales_ld] of float16.
#include "sa_common.hpp"
#include "sa_launch.hpp"

namespace sa {

constexpr int kQuantThreads = 256;

template <typename T>
__global__ void __launch_bounds__(kQuantThreads)
quantize_q8_0_kernel(const T* __restrict__ x, int64_t x_ld, int64_t n_rows, int n_blk, int8_t* __restrict__ codes,
                     int64_t codes_ld, f16* __restrict__ scales, int64_t scales_ld) {
  const int64_t b = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (b >= n_rows * n_blk) return;
  const int64_t row = b / n_blk;
  const int blk = (int)(b - row * n_blk);
  const T* src = x + row * x_ld + (int64_t)blk * 32;
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    v[e] = (float)src[e];
    amax = fmaxf(amax, fabsf(v[e]));
  }
  const float d = amax / 127.0f;
  const float id = d != 0.f ? 1.0f / d : 0.f;
  uint32_t w[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    uint32_t acc = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = (int)roundf(v[4 * u + e] * id);
      acc |= (uint32_t)(uint8_t)(int8_t)c << (8 * e);
    }
    w[u] = acc;
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(codes + row * codes_ld + (int64_t)blk * 32);
#pragma unroll
  for (int u = 0; u < 8; ++u) dst[u] = w[u];
  scales[row * scales_ld + blk] = (f16)d;
}

hipError_t launch_quantize_q8_0(const void* x, int x_dtype, int64_t n_rows, int n_cols, int64_t x_ld, int8_t* codes,
                                int64_t codes_ld, void* scales, int64_t scales_ld, hipStream_t stream) {
  const int n_blk = n_cols / 32;
  const int64_t n = n_rows * n_blk;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + kQuantThreads - 1) / kQuantThreads));
  switch (x_dtype) {
    case SA_F32:
      hipLaunchKernelGGL(quantize_q8_0_kernel<float>, grid, dim3(kQuantThreads), 0, stream, (const float*)x, x_ld,
                         n_rows, n_blk, codes, codes_ld, (f16*)scales, scales_ld);
      break;
    case SA_F16:
      hipLaunchKernelGGL(quantize_q8_0_kernel<f16>, grid, dim3(kQuantThreads), 0, stream, (const f16*)x, x_ld, n_rows,
                         n_blk, codes, codes_ld, (f16*)scales, scales_ld);
      break;
    default:
      hipLaunchKernelGGL(quantize_q8_0_kernel<bf16>, grid, dim3(kQuantThreads), 0, stream, (const bf16*)x, x_ld,
                         n_rows, n_blk, codes, codes_ld, (f16*)scales, scales_ld);
      break;
  }
  return hipGetLastError();
}

}  // namespace sa
