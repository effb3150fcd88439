// Device pieces shared by the attention kernels of fwd.hip (caches in the query
// dtype) and fwd_q8.hip (q8_0 caches): row bookkeeping, MFMA wrappers, the LDS-only
// barrier, and the generic VALU kernel, which reads K/V through an element reader.
#pragma once

#include "sa_common.hpp"
#include "sa_launch.hpp"

namespace sa {

constexpr int kRowTile = 32;

// ------------------------------------------------------------------- shared helpers

// Cache row of list entry j holding position `pos`, or -1 when j is past the
// query's count or pos is padding / not a cached position.
__device__ __forceinline__ int64_t tile_row(int pos, int j, int r_end, int seq_len, int64_t row0) {
  return (j < r_end && pos >= 0 && pos < seq_len) ? row0 + pos : -1;
}

// Position of row j of a query's attended rows: the list entries first (an entry
// inside the dense window is dropped there, the window covers it), then the window's
// wlen positions w0 .. w0 + wlen - 1.  Without a window (wlen 0) it is the entry.
__device__ __forceinline__ int row_pos(int entry, int j, int cnt, int w0, int wlen) {
  if (j < cnt) return (wlen > 0 && entry >= w0) ? -1 : entry;
  return w0 + (j - cnt);
}

template <typename T>
__device__ __forceinline__ f32x4 mfma16x16x32(const typename vec8<T>::type& a, const typename vec8<T>::type& b,
                                              const f32x4& c);
template <>
__device__ __forceinline__ f32x4 mfma16x16x32<bf16>(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16x16x32<f16>(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// P^T V^T as one 16x16x32 product (the full-rate bf16 / f16 shape) over two 16-row
// chunks of a tile: A = two transposing reads of V (4 rows each; lane i of a 16-lane
// group: dim i), B = the matching two 4-row pieces of P.  The rows a lane group
// contributes as its 8 k-values need not be contiguous, only the same in A and B.
typedef short i16x8 __attribute__((ext_vector_type(8)));
template <typename T>
__device__ __forceinline__ f32x4 pv_mfma32(const i16x4& a_lo, const i16x4& a_hi, const T (&b_lo)[4],
                                           const T (&b_hi)[4], const f32x4& c) {
  typedef typename vec8<T>::type V8;
  const i16x8 a = __builtin_shufflevector(a_lo, a_hi, 0, 1, 2, 3, 4, 5, 6, 7);
  const V8 b = {b_lo[0], b_lo[1], b_lo[2], b_lo[3], b_hi[0], b_hi[1], b_hi[2], b_hi[3]};
  return mfma16x16x32<T>(__builtin_bit_cast(V8, a), b, c);
}

// ---------------------------------------------------------------------------- MFMA

constexpr int kMfmaTile = 64;        // rows per workgroup tile: S for 16 per wave

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations but
// not for its global loads (a __syncthreads fence waits for those too).  The memory
// clobber keeps the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// A lane's value and that of the lane 16 (32) apart, by the permlane swaps: each lane
// of a pair receives both values in lane order, so max and sum come out the same in
// both lanes (and equal to those of a shuffle: the operations commute).  VALU
// operations, where a shuffle is an LDS round trip on the softmax's critical path.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane `src` (wave-uniform) of a 64-bit per-lane value.
__device__ __forceinline__ int64_t readlane64(int64_t x, int src) {
  const int lo = __builtin_amdgcn_readlane((int)(uint32_t)x, src);
  const int hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), src);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// ---------------------------------------------------------------------------- VALU

// K/V element readers of the generic kernel: a plain cache in the query dtype, or a
// q8_0 cache (int8 codes with one float16 scale per 32 consecutive elements).
template <typename T>
struct KvPlain {
  const T* k;
  int64_t k_ld, k_hs;
  const T* v;
  int64_t v_ld, v_hs;
  __device__ __forceinline__ float key(int64_t row, int g, int d) const { return (float)k[row * k_ld + g * k_hs + d]; }
  __device__ __forceinline__ float val(int64_t row, int g, int d) const { return (float)v[row * v_ld + g * v_hs + d]; }
};

struct KvQ8 {
  const int8_t* k;
  int64_t k_ld, k_hs;
  const f16* ks;
  int64_t ks_ld, ks_hs;
  const int8_t* v;
  int64_t v_ld, v_hs;
  const f16* vs;
  int64_t vs_ld, vs_hs;
  __device__ __forceinline__ float key(int64_t row, int g, int d) const {
    return (float)k[row * k_ld + g * k_hs + d] * (float)ks[row * ks_ld + g * ks_hs + d / 32];
  }
  __device__ __forceinline__ float val(int64_t row, int g, int d) const {
    return (float)v[row * v_ld + g * v_hs + d] * (float)vs[row * vs_ld + g * vs_hs + d / 32];
  }
};


template <typename T, int ACC, typename KV>
__global__ void __launch_bounds__(256)
fwd_valu_kernel(const T* __restrict__ q, const KV kv, const int64_t* __restrict__ seq_row0,
                const int32_t* __restrict__ seq_len, const int32_t* __restrict__ q_seq,
                const int32_t* __restrict__ sel, int64_t sel_ld, const int32_t* __restrict__ n_sel,
                const float* __restrict__ sel_bias, const int32_t* __restrict__ q_pos, int window, int list_max, int h_q,
                int h_kv, int d_kq, int d_v, float scale_log2, int n_split, int rows_per_split,
                float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  __shared__ int64_t rows[kRowTile];
  __shared__ float rbias[kRowTile];                  // additive logit bias of each row (log2 units)
  __shared__ float p[16][kRowTile];
  __shared__ float m_s[16], l_s[16], a_s[16];
  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int i = blockIdx.y / h_kv, g = blockIdx.y % h_kv;
  const int G = h_q / h_kv;
  const SeqMeta sm = seq_meta(q_seq, seq_len, seq_row0, nullptr, i);
  const int L = sm.len;
  const int64_t row0 = sm.row0;
  const int cnt = max(0, (int)min((int64_t)n_sel[i], min(sel_ld, (int64_t)list_max)));
  const int r_begin = split * rows_per_split;
  int w0 = 0, wlen = 0;                              // dense window of the most recent positions
  if (window > 0) {
    const int n_vis = visible_tokens(L, q_pos[i]);
    wlen = min(window, n_vis);
    w0 = n_vis - wlen;
  }
  // the last split takes every remaining row (the tail rows when they have no split of their own)
  const int r_end = split == n_split - 1 ? cnt + wlen : min(cnt + wlen, r_begin + rows_per_split);
  const int32_t* list = sel + (int64_t)i * sel_ld;
  const float* blist = sel_bias ? sel_bias + (int64_t)i * sel_ld : nullptr;
  const T* qg = q + ((int64_t)i * h_q + (int64_t)g * G) * d_kq;
  if (tid < 16) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  float acc[ACC];
#pragma unroll
  for (int a = 0; a < ACC; ++a) acc[a] = 0.f;

  for (int r0 = r_begin; r0 < r_end; r0 += kRowTile) {
    __syncthreads();
    if (tid < kRowTile) {
      const int j = r0 + tid;
      const int entry = list[min(j, (int)min(sel_ld, (int64_t)list_max) - 1)];
      rows[tid] = tile_row(row_pos(entry, j, cnt, w0, wlen), j, r_end, L, row0);
      rbias[tid] = (blist && j < min(r_end, cnt)) ? blist[j] * kLog2e : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < G * kRowTile; e += 256) {
      const int h = e / kRowTile, r = e % kRowTile;
      const int64_t row = rows[r];
      float xv = -INFINITY;
      if (row >= 0) {
        const T* qr = qg + (int64_t)h * d_kq;
        float dot = 0.f;
        for (int d = 0; d < d_kq; ++d) dot += (float)qr[d] * kv.key(row, g, d);
        xv = dot * scale_log2 + rbias[r];
      }
      p[h][r] = xv;
    }
    __syncthreads();
    if (tid < G) {
      const int h = tid;
      float mx = -INFINITY;
      for (int r = 0; r < kRowTile; ++r) mx = fmaxf(mx, p[h][r]);
      const float m_new = fmaxf(m_s[h], mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_s[h] - m_new);
      float sum = 0.f;
      for (int r = 0; r < kRowTile; ++r) {
        const float pr = (p[h][r] == -INFINITY) ? 0.f : fast_exp2(p[h][r] - m_new);
        p[h][r] = pr;
        sum += pr;
      }
      l_s[h] = l_s[h] * alpha + sum;
      m_s[h] = m_new;
      a_s[h] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < ACC; ++a) {
      const int e = tid + 256 * a;
      if (e < G * d_v) {
        const int h = e / d_v, dv = e % d_v;
        float o = acc[a] * a_s[h];
        for (int r = 0; r < kRowTile; ++r) {
          const int64_t row = rows[r];
          if (row >= 0) o += p[h][r] * kv.val(row, g, dv);
        }
        acc[a] = o;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < ACC; ++a) {
    const int e = tid + 256 * a;
    if (e < G * d_v) {
      const int h = e / d_v, dv = e % d_v;
      const int64_t qh = (int64_t)i * h_q + (int64_t)g * G + h;
      if (n_split == 1) {
        out[qh * d_v + dv] = l_s[h] > 0.f ? acc[a] / l_s[h] : 0.f;
      } else {
        ws_o[(qh * n_split + split) * d_v + dv] = acc[a];
      }
    }
  }
  if (n_split > 1 && tid < G) {
    const int64_t qh = (int64_t)i * h_q + (int64_t)g * G + tid;
    ws_ml[(qh * n_split + split) * 2 + 0] = m_s[tid];
    ws_ml[(qh * n_split + split) * 2 + 1] = l_s[tid];
  }
}

}  // namespace sa
