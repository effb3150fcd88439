// Block selection: the kept blocks of each query token plus its tail, as an
// ascending list of positions.
//
// The indexer keeps the best blocks up to an indexer_top_k token budget plus the
// tail of tokens not yet forming a complete block; below top_k + c - 1 visible
// tokens every block fits and the result is dense (llama.cpp commit "llama: QSA
// sparse attention for qwen4exp").  The list has the form the sparse flash
// attention consumes: int32, ascending, -1 padded, never longer than its capacity
// (llama.cpp PR #27970, flash_attn_mask_to_sparse_indices).  Ties go to the lower
// block index, which is where the pages' token-level top-k over expanded block
// scores cuts as well (members of a block tie, the budget is whole blocks).
//
// Design: one workgroup per query token.  Scores are mapped to order-preserving
// 32-bit keys (+0/-0 identical).  The K_blk-th largest key T is found exactly by a
// 4-pass radix select over 8-bit digits (most significant first); each pass builds
// a histogram of the digit among the keys that match the digits fixed so far.  The
// histogram is privatised per lane (32 copies, padded by one word) so that keys
// that share a digit -- the common case, scores crowd into a few binades -- land
// on different LDS banks instead of serialising on one address.  Then the kept
// blocks (key > T, or key == T among the first r such in index order) are compacted
// in index order with two workgroup prefix sums and written as positions.  Keys
// live in registers (thread t owns blocks [t*KPT, (t+1)*KPT) of a chunk); a query
// with more blocks than BLOCK*KPT streams its chunks from global memory per pass.
#include "sa_common.hpp"
#include "sa_launch.hpp"

namespace sa {

constexpr int kCopies = 32;
constexpr int kBins = 256;
constexpr int kCopyStride = kBins + 1;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;                       // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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

template <int BLOCK, int KPT>
__global__ void __launch_bounds__(BLOCK)
select_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
              const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk,
              int32_t* __restrict__ sel, int64_t sel_ld, int32_t* __restrict__ n_sel) {
  constexpr int CH = BLOCK * KPT;                    // blocks per chunk
  __shared__ int hist[kCopies * kCopyStride];
  __shared__ int total[kBins];
  __shared__ int scan_scratch[BLOCK / kWave + 1];
  __shared__ int pick[2];

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int s = q_seq[i];
  const int n_vis = visible_tokens(seq_len[s], q_pos[i]);
  const int nb = n_vis / c;
  const int tail = n_vis - nb * c;
  int32_t* out = sel + (int64_t)i * sel_ld;

  if (nb <= k_blk) {                                 // every block fits: dense
    for (int64_t j = tid; j < sel_ld; j += BLOCK) out[j] = j < n_vis ? (int32_t)j : -1;
    if (tid == 0) n_sel[i] = n_vis;
    return;
  }

  const float* row = scores + (int64_t)i * scores_ld;
  const int n_chunks = (nb + CH - 1) / CH;
  const bool resident = (n_chunks == 1);
  uint32_t key[KPT];
  auto load_chunk = [&](int ch) {
    const int base = ch * CH + tid * KPT;
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = (base + j < nb) ? order_key(row[base + j]) : 0u;
  };
  if (resident) load_chunk(0);

  // ---- exact K_blk-th largest key by 4 radix passes -------------------------------
  uint32_t prefix = 0;
  int k_rem = k_blk;
  int* my_hist = hist + (lane & (kCopies - 1)) * kCopyStride;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int e = tid; e < kCopies * kCopyStride; e += BLOCK) hist[e] = 0;
    __syncthreads();
#pragma unroll 1
    for (int ch = 0; ch < n_chunks; ++ch) {
      if (!resident) load_chunk(ch);
      const int base = ch * CH + tid * KPT;
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const uint32_t k = key[j];
        const bool match = (base + j < nb) && (uint32_t)((uint64_t)k >> (shift + 8)) == prefix;
        if (match) atomicAdd(&my_hist[(k >> shift) & 0xFFu], 1);
      }
    }
    __syncthreads();
    for (int v = tid; v < kBins; v += BLOCK) {
      int sum = 0;
#pragma unroll 8
      for (int cp = 0; cp < kCopies; ++cp) sum += hist[cp * kCopyStride + v];
      total[v] = sum;
    }
    __syncthreads();
    // Suffix sums over the 256 bins, highest bin first: thread t < 256 takes bin
    // 255 - t; a wave-level inclusive scan gives the keys in bins >= v within the
    // wave's span and the per-wave totals are added after a barrier.  The thread
    // whose bin holds the k_rem-th largest matching key publishes it.
    int ge_in_wave = 0;
    if (tid < kBins) {                               // whole waves 0..3
      ge_in_wave = wave_inclusive_scan(total[kBins - 1 - tid], lane);
      if (lane == kWave - 1) scan_scratch[tid / kWave] = ge_in_wave;
    }
    __syncthreads();
    if (tid < kBins) {
      const int v = kBins - 1 - tid;
      int base = 0;
      for (int w = 0; w < tid / kWave; ++w) base += scan_scratch[w];
      const int ge = base + ge_in_wave;              // matching keys in bins >= v
      const int gt = ge - total[v];                  // matching keys in bins > v
      if (gt < k_rem && ge >= k_rem) {
        pick[0] = v;
        pick[1] = k_rem - gt;
      }
    }
    __syncthreads();
    prefix = (prefix << 8) | (uint32_t)pick[0];
    k_rem = pick[1];
    __syncthreads();
  }
  const uint32_t T = prefix;                         // the K_blk-th largest key
  const int r_eq = k_rem;                            // keys equal to T that are kept

  // ---- compaction in block-index order --------------------------------------------
  int eq_base = 0, out_base = 0;
#pragma unroll 1
  for (int ch = 0; ch < n_chunks; ++ch) {
    if (!resident) load_chunk(ch);
    const int base = ch * CH + tid * KPT;
    int n_eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) n_eq += (base + j < nb && key[j] == T) ? 1 : 0;
    int eq_tot;
    const int eq_before = eq_base + block_exclusive_scan<BLOCK>(n_eq, scan_scratch, &eq_tot);
    int n_take = 0, e = eq_before;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool ok = base + j < nb;
      const bool gt = ok && key[j] > T;
      const bool eq = ok && key[j] == T;
      const bool take = gt || (eq && e < r_eq);
      e += eq ? 1 : 0;
      n_take += take ? 1 : 0;
    }
    int take_tot;
    int o = out_base + block_exclusive_scan<BLOCK>(n_take, scan_scratch, &take_tot);
    e = eq_before;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool ok = base + j < nb;
      const bool gt = ok && key[j] > T;
      const bool eq = ok && key[j] == T;
      const bool take = gt || (eq && e < r_eq);
      e += eq ? 1 : 0;
      if (take) {
        const int32_t p0 = (int32_t)(base + j) * c;
        int32_t* dst = out + (int64_t)o * c;
        for (int t = 0; t < c; ++t) dst[t] = p0 + t;
        ++o;
      }
    }
    eq_base += eq_tot;
    out_base += take_tot;
  }
  // ---- tail and padding -------------------------------------------------------------
  const int body = k_blk * c;
  for (int j = tid; j < tail; j += BLOCK) out[body + j] = nb * c + j;
  for (int64_t j = body + tail + tid; j < sel_ld; j += BLOCK) out[j] = -1;
  if (tid == 0) n_sel[i] = body + tail;
}

template <int BLOCK, int KPT>
static void launch_select_t(const sa_dims& d, const float* scores, int64_t scores_ld, const CacheArgs& c,
                            const int32_t* q_seq, const int32_t* q_pos, int n_q, int32_t* sel, int64_t sel_ld,
                            int32_t* n_sel, hipStream_t stream) {
  hipLaunchKernelGGL((select_kernel<BLOCK, KPT>), dim3(n_q), dim3(BLOCK), 0, stream, scores, scores_ld, c.seq_len,
                     q_seq, q_pos, d.compress_ratio, d.top_k / d.compress_ratio, sel, sel_ld, n_sel);
}

hipError_t launch_select(const sa_dims& d, const CacheArgs& c, const float* scores, int64_t scores_ld,
                         const int32_t* q_seq, const int32_t* q_pos, int n_q, int32_t* sel, int64_t sel_ld,
                         int32_t* n_sel, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  const long long max_blocks = (long long)c.max_len / d.compress_ratio;
  if (n_q <= 64) {                                   // few queries: wide workgroups
    if (max_blocks <= 1024 * 8) launch_select_t<1024, 8>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
    else if (max_blocks <= 1024 * 16) launch_select_t<1024, 16>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
    else launch_select_t<1024, 32>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
  } else {
    if (max_blocks <= 256 * 8) launch_select_t<256, 8>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
    else if (max_blocks <= 256 * 16) launch_select_t<256, 16>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
    else if (max_blocks <= 256 * 32) launch_select_t<256, 32>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
    else launch_select_t<256, 64>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
  }
  return hipGetLastError();
}

}  // namespace sa
