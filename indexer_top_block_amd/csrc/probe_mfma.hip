// Measurement probes (not part of the sparse-attention library): the dense bf16
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

// ---------------------------------------------------------------------------------
// HBM read probes: the read bandwidth the chip delivers to a plain streaming kernel
// and to a gather of random 1 KiB rows (the access pattern of the attention's row
// gathers), reported beside the 8 TB/s peak.

namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// Every thread reads UNR 16-byte vectors per round, grid-stride, and keeps an xor.
template <int UNR>
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4v* __restrict__ src, int64_t n_vec,
                                                          uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4v acc = {0, 0, 0, 0};
  for (; i + (UNR - 1) * stride < n_vec; i += UNR * stride) {
    u32x4v v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < UNR; ++u) acc ^= v[u];
  }
  for (; i < n_vec; i += stride) acc ^= src[i];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Each wave reads whole 1 KiB rows (one 16-byte vector per lane) at row indices
// rows[] (UNR rows in flight per wave), grid-stride over the index list.
template <int UNR>
__global__ void __launch_bounds__(256) gather_read_kernel(const u32x4v* __restrict__ src,
                                                          const int32_t* __restrict__ rows, int64_t n_rows,
                                                          uint32_t* __restrict__ out) {
  const int lane = threadIdx.x % 64;
  const int64_t waves = (int64_t)gridDim.x * 4;
  int64_t w = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  u32x4v acc = {0, 0, 0, 0};
  for (; w + (UNR - 1) * waves < n_rows; w += UNR * waves) {
    u32x4v v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) v[u] = src[(int64_t)rows[w + u * waves] * 64 + lane];
#pragma unroll
    for (int u = 0; u < UNR; ++u) acc ^= v[u];
  }
  for (; w < n_rows; w += waves) acc ^= src[(int64_t)rows[w] * 64 + lane];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

// Streams `bytes` (a multiple of 16, 16-byte aligned) from src with n_wg workgroups
// of 256 threads; out: device, n_wg * 256 uint32.  0, or -1 / -2 as above.
int sa_probe_stream_read(const void* src, int64_t bytes, int n_wg, uint32_t* out, void* stream) {
  if (!src || !out || bytes < 16 || bytes % 16 || n_wg < 1) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(stream_read_kernel<8>, dim3(n_wg), dim3(256), 0, (hipStream_t)stream, (const u32x4v*)src,
                     bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Gathers n_rows rows of 1 KiB from src (rows[j] < the number of rows src holds;
// the caller guarantees it) with n_wg workgroups; out: device, n_wg * 256 uint32.
int sa_probe_gather_read(const void* src, const int32_t* rows, int64_t n_rows, int n_wg, uint32_t* out,
                         void* stream) {
  if (!src || !rows || !out || n_rows < 1 || n_wg < 1) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(gather_read_kernel<8>, dim3(n_wg), dim3(256), 0, (hipStream_t)stream, (const u32x4v*)src,
                     rows, n_rows, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"

// ---------------------------------------------------------------------------------
// Latency probes: what a graph node and a dependent memory round trip cost, the
// floors of a chain of small kernels.

namespace {

__global__ void empty_kernel(uint32_t* __restrict__ out) {
  if (threadIdx.x == 0 && blockIdx.x == 0 && out == nullptr) out[0] = 1u;   // never taken; keeps the argument
}

// One thread per workgroup follows `hops` dependent loads through next[] (each index
// read decides the next address), starting at start[blockIdx.x].
__global__ void chain_kernel(const int32_t* __restrict__ next, const int32_t* __restrict__ start, int hops,
                             int32_t* __restrict__ out) {
  if (threadIdx.x != 0) return;
  int32_t i = start[blockIdx.x];
  for (int h = 0; h < hops; ++h) i = __builtin_nontemporal_load(&next[i]);
  out[blockIdx.x] = i;
}

}  // namespace

extern "C" {

// An empty kernel of n_wg workgroups of 64 threads.
int sa_probe_empty(int n_wg, void* stream) {
  if (n_wg < 1) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(empty_kernel, dim3(n_wg), dim3(64), 0, (hipStream_t)stream, (uint32_t*)nullptr);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// n_wg workgroups each follow `hops` dependent loads; next[] and start[] hold valid
// indices into next[] (the caller guarantees it); out: device, n_wg int32.
int sa_probe_chain(const int32_t* next, const int32_t* start, int hops, int n_wg, int32_t* out, void* stream) {
  if (!next || !start || !out || hops < 0 || n_wg < 1) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(chain_kernel, dim3(n_wg), dim3(64), 0, (hipStream_t)stream, next, start, hops, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
