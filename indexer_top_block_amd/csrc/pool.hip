// Incremental block mean-pool of the raw indexer keys.
//
// One pooled key per block of compress_ratio consecutive positions; the cache keeps
// raw keys and pooling comes before any norm or rotation (llama.cpp commit "llama:
// QSA sparse attention for qwen4exp", the paragraph on the indexer key cache).
// Pooled keys persist, so a decode step pools at most the one block that has just
// completed instead of re-reading the whole raw cache.
#include "sa_common.hpp"
#include "sa_launch.hpp"

namespace sa {

// grid = (wgs per sequence, n_seq); every thread handles (block, dim) elements with
// the dim fastest, so a wave reads consecutive elements of the same raw-key rows.
template <typename T>
__global__ void __launch_bounds__(256)
pool_kernel(const T* __restrict__ kidx, int64_t kidx_ld, T* __restrict__ kpool, int64_t kpool_ld,
            const int64_t* __restrict__ seq_row0, const int64_t* __restrict__ seq_blk0,
            const int32_t* __restrict__ seq_len, const int32_t* n_pooled_in, int32_t* n_pooled_out, int c,
            int d_idx, int max_new, int update_here) {
  const int s = blockIdx.y;
  // Read the pooled count before anything writes it (the arrays may alias).
  const int start = max(n_pooled_in[s], 0);
  const int target = max(seq_len[s], 0) / c;
  const int end = (int)min((long long)target, (long long)start + max_new);
  const long long total = (long long)max(end - start, 0) * d_idx;
  const int64_t row0 = seq_row0[s], blk0 = seq_blk0[s];
  const float den = (float)c;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const int64_t b = start + e / d_idx;
    const int d = (int)(e % d_idx);
    const T* src = kidx + (row0 + b * c) * kidx_ld + d;
    kpool[(blk0 + b) * kpool_ld + d] = (T)(pool_sum(src, kidx_ld, c) / den);
  }
  if (update_here) {  // one workgroup per sequence: every thread has read `start`
    __syncthreads();
    if (threadIdx.x == 0) n_pooled_out[s] = end;
  }
}

__global__ void pool_count_kernel(const int32_t* n_pooled_in, int32_t* n_pooled_out, const int32_t* seq_len,
                                  int n_seq, int c, int max_new) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n_seq) return;
  const int start = max(n_pooled_in[s], 0);
  const int target = max(seq_len[s], 0) / c;
  n_pooled_out[s] = (int)min((long long)target, (long long)start + max_new);
}

template <typename T>
static hipError_t launch_pool_t(const sa_dims& d, const CacheArgs& c, const int32_t* n_in, int32_t* n_out,
                                int max_new, hipStream_t stream) {
  const int cr = d.compress_ratio;
  const long long max_blocks = (long long)c.max_len / cr;
  const long long blocks = max_new < max_blocks ? max_new : max_blocks;
  const long long elems = blocks * d.d_idx;
  long long wgs = (elems + 255) / 256;
  if (wgs < 1) wgs = 1;
  if (wgs > 2048) wgs = 2048;
  const int update_here = (wgs == 1);
  dim3 grid((unsigned)wgs, (unsigned)c.n_seq);
  hipLaunchKernelGGL(pool_kernel<T>, grid, dim3(256), 0, stream, (const T*)c.kidx, c.kidx_ld, (T*)c.kpool,
                     c.kpool_ld, c.seq_row0, c.seq_blk0, c.seq_len, n_in, n_out, cr, d.d_idx, max_new, update_here);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || update_here) return err;
  hipLaunchKernelGGL(pool_count_kernel, dim3((c.n_seq + 255) / 256), dim3(256), 0, stream, n_in, n_out, c.seq_len,
                     c.n_seq, cr, max_new);
  return hipGetLastError();
}

hipError_t launch_pool(const sa_dims& d, const CacheArgs& c, const int32_t* n_in, int32_t* n_out, int max_new,
                       hipStream_t stream) {
  switch (d.dtype) {
    case SA_F32: return launch_pool_t<float>(d, c, n_in, n_out, max_new, stream);
    case SA_F16: return launch_pool_t<f16>(d, c, n_in, n_out, max_new, stream);
    default: return launch_pool_t<bf16>(d, c, n_in, n_out, max_new, stream);
  }
}

}  // namespace sa
