// Measurement probe (not part of the sparse-attention library): the dense bf16
// matrix-core rate of the chip, measured with a plain loop of independent
// v_mfma_f32_32x32x16_bf16 chains and no memory traffic, to be reported beside the
// vendor's peak figure.  Built as its own library, libsa_probe.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kChains = 8;   // independent accumulators per wave: covers the MFMA latency

__global__ void __launch_bounds__(kThreads) mfma_loop_kernel(const bf16x8* __restrict__ ab, int iters,
                                                             float* __restrict__ out) {
  const bf16x8 a = ab[threadIdx.x % 64];
  const bf16x8 b = ab[64 + threadIdx.x % 64];
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Launches n_wg workgroups of 256 threads, each wave running `iters` rounds of 8
// independent 32x32x16 bf16 products (2*32*32*16 FLOP each).
//   ab:  device, 128 vectors of 8 bf16 (the operands; any finite values)
//   out: device, n_wg * 256 floats (written, to keep the products live)
// Returns 0, -1 on bad arguments, -2 on a failed launch.  Asynchronous on `stream`.
int sa_probe_mfma_bf16(int n_wg, int iters, const void* ab, float* out, void* stream) {
  if (n_wg < 1 || iters < 1 || !ab || !out) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(n_wg), dim3(kThreads), 0, (hipStream_t)stream, (const bf16x8*)ab, iters,
                     out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// FLOP one call performs.
double sa_probe_mfma_bf16_flop(int n_wg, int iters) {
  return (double)n_wg * (kThreads / 64) * iters * kChains * (2.0 * 32 * 32 * 16);
}

}  // extern "C"
