// Device-side helpers shared by the sparse-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16;
typedef _Float16 f16;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Eight 16-bit elements as the MFMA operand type of T.
template <typename T> struct vec8;
template <> struct vec8<bf16> { typedef bf16x8 type; };
template <> struct vec8<f16> { typedef f16x8 type; };

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave, with DPP: shifts by 1, 2, 4, 8
// within each row of 16 lanes, then the last lane of rows 0 and 2 is added to rows 1
// and 3 (row_bcast:15) and lane 31 to rows 2 and 3 (row_bcast:31).  `lane` is unused
// and kept for the call sites' readability.
__device__ __forceinline__ int wave_inclusive_scan(int x, int /*lane*/) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive prefix sum of one int per thread over the workgroup; returns the
// exclusive value and writes the total to *total.  `scratch` holds >= BLOCK/64 ints.
template <int BLOCK>
__device__ __forceinline__ int block_exclusive_scan(int x, int* scratch, int* total) {
  constexpr int W = BLOCK / kWave;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int inc = wave_inclusive_scan(x, lane);
  __syncthreads();
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int v = scratch[w];
    base += (w < wave) ? v : 0;
    tot += v;
  }
  *total = tot;
  return base + inc - x;
}

// The pooling sum of one element over a block's c raw rows (row stride ld): float
// adds in row order.  Rows are loaded 8 at a time (clamped, not guarded), so a block
// of up to 8 rows costs one memory round trip.
template <typename T>
__device__ __forceinline__ float pool_sum(const T* src, int64_t ld, int c) {
  float acc = 0.f;
  for (int r0 = 0; r0 < c; r0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (float)src[(int64_t)min(r0 + u, c - 1) * ld];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (r0 + u < c) acc += v[u];
  }
  return acc;
}

// The same for 8 consecutive elements (one 16-byte load per row; src 16-byte aligned).
template <typename T>
__device__ __forceinline__ void pool_sum8(const T* src, int64_t ld, int c, float (&acc)[8]) {
  typedef typename vec8<T>::type V8;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int r0 = 0; r0 < c; r0 += 8) {
    V8 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const V8*>(src + (int64_t)min(r0 + u, c - 1) * ld);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (r0 + u < c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (float)v[u][e];
      }
  }
}

// 2^x with the hardware exponential (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sequence metadata of query token i.  Sequence 0's entries are read together with
// q_seq[i] (one memory round trip instead of two when, as in single-sequence decode,
// the token belongs to sequence 0); other sequences take a second read.
struct SeqMeta {
  int s;
  int len;
  int64_t row0;
  int64_t blk0;
};
__device__ __forceinline__ SeqMeta seq_meta(const int32_t* __restrict__ q_seq, const int32_t* __restrict__ seq_len,
                                            const int64_t* __restrict__ seq_row0,
                                            const int64_t* __restrict__ seq_blk0, int i) {
  SeqMeta m;
  m.s = q_seq[i];
  m.len = seq_len[0];
  m.row0 = seq_row0 ? seq_row0[0] : 0;
  m.blk0 = seq_blk0 ? seq_blk0[0] : 0;
  if (m.s != 0) {
    m.len = seq_len[m.s];
    m.row0 = seq_row0 ? seq_row0[m.s] : 0;
    m.blk0 = seq_blk0 ? seq_blk0[m.s] : 0;
  }
  return m;
}

// Visible cached positions for a query: t <= q_pos and t < seq_len.
__device__ __forceinline__ int visible_tokens(int seq_len, int q_pos) {
  long long v = (long long)q_pos + 1;
  if (v > seq_len) v = seq_len;
  return v < 0 ? 0 : (int)v;
}

}  // namespace sa
