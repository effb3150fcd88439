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
// Scores are mapped to order-preserving 32-bit keys (+0/-0 identical).  Two designs:
//
// Per-query workgroup (many query tokens, e.g. a prefill chunk): one workgroup per
// query finds the K_blk-th largest key T exactly by a 4-pass radix select over 8-bit
// digits, most significant first; each pass histograms the digit among the keys
// that match the digits fixed so far.  The histogram is privatised per lane (32
// copies, padded by one word) so that keys sharing a digit -- scores crowd into a
// few binades -- hit different LDS banks instead of serialising on one address.
// The kept blocks (key > T, or key == T among the first r such in index order) are
// then compacted in index order with two workgroup prefix sums.  Thread t owns
// blocks [t*KPT, (t+1)*KPT) of a chunk; longer rows stream chunk by chunk.
//
// Chunked (few query tokens over long rows, i.e. decode): the row is cut into
// chunks of 2048 blocks, one workgroup each, so the whole GPU takes part.
//   zero   clear the per-query histogram and counters in the workspace;
//   hist   each chunk histograms the top 12 bits of its keys in LDS and adds the
//          non-empty bins to the query's histogram (device-scope atomics);
//   cand   every chunk finds the bin b holding the K_blk-th largest key, counts its
//          keys above b and appends its keys inside b to a candidate list as
//          (key << 32 | ~index) -- unique 64-bit values whose order is exactly
//          (score desc, index asc), so ties need no special case;
//   final  one workgroup radix-selects the cut among the candidates (8-bit digits
//          below the 12 shared bits, stopping as soon as the cut's bin holds one
//          value), tallies the kept blocks per chunk and turns the tallies into
//          output offsets; it also writes the tail, the padding and n_sel;
//   emit   each chunk writes its kept blocks' positions at its offset.
// If the candidates overflow their buffer (massive exact ties), `final` runs the
// per-query algorithm above over the whole row instead and `emit` does nothing.
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

// Positions of the dense case (every block fits): 0 .. n_vis-1, then -1.
template <int BLOCK>
__device__ __forceinline__ void write_dense(int32_t* out, int64_t sel_ld, int n_vis, int32_t* n_sel_out) {
  for (int64_t j = threadIdx.x; j < sel_ld; j += BLOCK) out[j] = j < n_vis ? (int32_t)j : -1;
  if (threadIdx.x == 0) *n_sel_out = n_vis;
}

// Tail positions after the K_blk kept blocks, then -1, then the count.
template <int BLOCK>
__device__ __forceinline__ void write_tail(int32_t* out, int64_t sel_ld, int nb, int n_vis, int c, int k_blk,
                                           int32_t* n_sel_out) {
  const int body = k_blk * c, tail = n_vis - nb * c;
  for (int j = threadIdx.x; j < tail; j += BLOCK) out[body + j] = nb * c + j;
  for (int64_t j = body + tail + threadIdx.x; j < sel_ld; j += BLOCK) out[j] = -1;
  if (threadIdx.x == 0) *n_sel_out = body + tail;
}

// ------------------------------------------------------- per-query workgroup select

struct WgSmem {
  int hist[kCopies * kCopyStride];
  int total[kBins];
  int scan_scratch[1024 / kWave + 1];
  int pick[2];
};

// One workgroup selects for one query whose scores are row[0 .. nb).  Requires nb > k_blk.
template <int BLOCK, int KPT>
__device__ void select_one_query(const float* __restrict__ row, int nb, int n_vis, int c, int k_blk,
                                 int32_t* __restrict__ out, int64_t sel_ld, int32_t* n_sel_out, WgSmem& sm) {
  constexpr int CH = BLOCK * KPT;                    // blocks per chunk
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
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
  int* my_hist = sm.hist + (lane & (kCopies - 1)) * kCopyStride;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int e = tid; e < kCopies * kCopyStride; e += BLOCK) sm.hist[e] = 0;
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
      for (int cp = 0; cp < kCopies; ++cp) sum += sm.hist[cp * kCopyStride + v];
      sm.total[v] = sum;
    }
    __syncthreads();
    // Suffix sums over the 256 bins, highest bin first: thread t < 256 takes bin
    // 255 - t; a wave-level inclusive scan gives the keys in bins >= v within the
    // wave's span and the per-wave totals are added after a barrier.  The thread
    // whose bin holds the k_rem-th largest matching key publishes it.
    int ge_in_wave = 0;
    if (tid < kBins) {                               // whole waves 0..3
      ge_in_wave = wave_inclusive_scan(sm.total[kBins - 1 - tid], lane);
      if (lane == kWave - 1) sm.scan_scratch[tid / kWave] = ge_in_wave;
    }
    __syncthreads();
    if (tid < kBins) {
      const int v = kBins - 1 - tid;
      int base = 0;
      for (int w = 0; w < tid / kWave; ++w) base += sm.scan_scratch[w];
      const int ge = base + ge_in_wave;              // matching keys in bins >= v
      const int gt = ge - sm.total[v];               // matching keys in bins > v
      if (gt < k_rem && ge >= k_rem) {
        sm.pick[0] = v;
        sm.pick[1] = k_rem - gt;
      }
    }
    __syncthreads();
    prefix = (prefix << 8) | (uint32_t)sm.pick[0];
    k_rem = sm.pick[1];
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
    const int eq_before = eq_base + block_exclusive_scan<BLOCK>(n_eq, sm.scan_scratch, &eq_tot);
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
    int o = out_base + block_exclusive_scan<BLOCK>(n_take, sm.scan_scratch, &take_tot);
    e = eq_before;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool ok = base + j < nb;
      const bool gt = ok && key[j] > T;
      const bool eq = ok && key[j] == T;
      const bool take = gt || (eq && e < r_eq);
      e += eq ? 1 : 0;
      if (take && o < k_blk) {                       // o < k_blk always; the bound only guards memory
        const int32_t p0 = (int32_t)(base + j) * c;
        int32_t* dst = out + (int64_t)o * c;
        for (int t = 0; t < c; ++t) dst[t] = p0 + t;
        ++o;
      }
    }
    eq_base += eq_tot;
    out_base += take_tot;
  }
  write_tail<BLOCK>(out, sel_ld, nb, n_vis, c, k_blk, n_sel_out);
}

template <int BLOCK, int KPT>
__global__ void __launch_bounds__(BLOCK)
select_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
              const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk,
              int32_t* __restrict__ sel, int64_t sel_ld, int32_t* __restrict__ n_sel) {
  __shared__ WgSmem sm;
  const int i = blockIdx.x;
  const int n_vis = visible_tokens(seq_len[q_seq[i]], q_pos[i]);
  const int nb = n_vis / c;
  int32_t* out = sel + (int64_t)i * sel_ld;
  if (nb <= k_blk) {
    write_dense<BLOCK>(out, sel_ld, n_vis, n_sel + i);
    return;
  }
  select_one_query<BLOCK, KPT>(scores + (int64_t)i * scores_ld, nb, n_vis, c, k_blk, out, sel_ld, n_sel + i, sm);
}

// ------------------------------------------------------------------ chunked select

constexpr int kChunk = 2048;                         // blocks per chunk workgroup
constexpr int kChunkThreads = 256;
constexpr int kChunkKpt = kChunk / kChunkThreads;   // 8
constexpr int kTopBits = 12;
constexpr int kBins1 = 1 << kTopBits;                // 4096 bins of the top 12 bits
constexpr int kHistCopies = 4;
constexpr int kCandCap = 16384;                      // candidates the final step holds in LDS
constexpr int kMaxChunks = 2048;                     // chunks per query the final step tallies
constexpr int kFinalThreads = 1024;

// Per-query control words in the workspace.
enum { CT_FALLBACK = 0, CT_T = 1, CT_CUT = 2, CT_WORDS = 16 };

struct ChunkWs {
  // per query: ghist[kBins1] | ctrl[CT_WORDS] | n_above[g] | n_cand[g] | offsets[g] | cand[g][kChunk] (u64)
  char* base;
  size_t q_stride;
  int g;
  __device__ __host__ uint32_t* ghist(int q) const { return (uint32_t*)(base + q * q_stride); }
  __device__ __host__ uint32_t* ctrl(int q) const { return ghist(q) + kBins1; }
  __device__ __host__ uint32_t* n_above(int q) const { return ctrl(q) + CT_WORDS; }
  __device__ __host__ uint32_t* n_cand(int q) const { return n_above(q) + g; }
  __device__ __host__ uint32_t* offsets(int q) const { return n_cand(q) + g; }
  static __device__ __host__ size_t head_bytes(int g) {
    return ((size_t)(kBins1 + CT_WORDS + 3 * (size_t)g) * 4 + 255) / 256 * 256;
  }
  __device__ __host__ uint64_t* cand(int q, int w) const {
    return (uint64_t*)(base + q * q_stride + head_bytes(g)) + (size_t)w * kChunk;
  }
  static __host__ size_t query_bytes(int g) { return head_bytes(g) + (size_t)g * kChunk * 8; }
};

struct QueryRow {
  int nb, n_vis;
};
__device__ __forceinline__ QueryRow query_row(const int32_t* seq_len, const int32_t* q_seq, const int32_t* q_pos,
                                              int q, int c) {
  const int n_vis = visible_tokens(seq_len[q_seq[q]], q_pos[q]);
  return QueryRow{n_vis / c, n_vis};
}

// Keys of this chunk, read before the query's length is known (indices up to the
// row's capacity are valid memory; those past nb are masked by the caller).
// `contiguous`: thread t holds blocks [t*8, t*8+8) (index order); otherwise
// j*256 + t (coalesced).
template <bool contiguous>
__device__ __forceinline__ void load_chunk_keys(const float* __restrict__ row, int64_t row_cap, int base,
                                                uint32_t (&key)[kChunkKpt], int (&idx)[kChunkKpt]) {
#pragma unroll
  for (int j = 0; j < kChunkKpt; ++j) {
    idx[j] = contiguous ? base + (int)threadIdx.x * kChunkKpt + j : base + j * kChunkThreads + (int)threadIdx.x;
    key[j] = idx[j] < row_cap ? order_key(row[idx[j]]) : 0u;
  }
}

__global__ void __launch_bounds__(256) chunk_zero_kernel(ChunkWs ws) {
  uint32_t* h = ws.ghist(blockIdx.x);
  for (int e = threadIdx.x; e < kBins1 + CT_WORDS; e += blockDim.x) h[e] = 0u;  // ghist and ctrl are adjacent
}

__global__ void __launch_bounds__(kChunkThreads)
chunk_hist_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
                  const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk, ChunkWs ws) {
  constexpr int kStride = kBins1 + 1;
  __shared__ uint32_t h[kHistCopies * kStride];
  const int q = blockIdx.y, tid = threadIdx.x;
  const int base = blockIdx.x * kChunk;
  uint32_t key[kChunkKpt];
  int idx[kChunkKpt];
  load_chunk_keys<false>(scores + (int64_t)q * scores_ld, scores_ld, base, key, idx);
  for (int e = tid; e < kHistCopies * kStride; e += kChunkThreads) h[e] = 0u;
  const QueryRow qr = query_row(seq_len, q_seq, q_pos, q, c);
  if (qr.nb <= k_blk || base >= qr.nb) return;      // uniform over the workgroup
  __syncthreads();
  uint32_t* mine = h + (tid & (kHistCopies - 1)) * kStride;
#pragma unroll
  for (int j = 0; j < kChunkKpt; ++j)
    if (idx[j] < qr.nb) atomicAdd(&mine[key[j] >> (32 - kTopBits)], 1u);
  __syncthreads();
  uint32_t* g = ws.ghist(q);
  for (int b = tid; b < kBins1; b += kChunkThreads) {
    uint32_t n = 0;
#pragma unroll
    for (int cp = 0; cp < kHistCopies; ++cp) n += h[cp * kStride + b];
    if (n) atomicAdd(&g[b], n);
  }
}

// Bin holding the k-th largest key of the query histogram (`cnt` = this thread's 16
// bins [t*16, t*16+16)), and the number of keys in higher bins, to all threads.
__device__ __forceinline__ void find_top_bin(const uint32_t (&cnt)[kBins1 / kChunkThreads], int k, int* lds_scan,
                                             int* out_bin, int* out_above) {
  constexpr int PER = kBins1 / kChunkThreads;
  const int tid = threadIdx.x;
  int sum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) sum += (int)cnt[j];
  int total;
  const int below_incl = block_exclusive_scan<kChunkThreads>(sum, lds_scan, &total) + sum;
  int above = total - below_incl;                    // keys in bins >= (t+1)*16
#pragma unroll
  for (int j = PER - 1; j >= 0; --j) {
    const int gt = above, ge = above + (int)cnt[j];
    if (gt < k && ge >= k) {
      out_bin[0] = tid * PER + j;
      out_above[0] = gt;
    }
    above = ge;
  }
  __syncthreads();
}

__global__ void __launch_bounds__(kChunkThreads)
chunk_cand_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
                  const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk, ChunkWs ws) {
  constexpr int PER = kBins1 / kChunkThreads;
  constexpr int W = kChunkThreads / kWave;
  __shared__ int scan[W + 1];
  __shared__ int sh_bin, sh_above;
  __shared__ int wave_cand[W], wave_gt[W];
  const int q = blockIdx.y, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int base = blockIdx.x * kChunk;
  uint32_t key[kChunkKpt];
  int idx[kChunkKpt];
  load_chunk_keys<false>(scores + (int64_t)q * scores_ld, scores_ld, base, key, idx);
  uint32_t hc[PER];
  const uint32_t* gh = ws.ghist(q);
#pragma unroll
  for (int j = 0; j < PER; ++j) hc[j] = gh[tid * PER + j];
  const QueryRow qr = query_row(seq_len, q_seq, q_pos, q, c);
  if (qr.nb <= k_blk || base >= qr.nb) return;
  find_top_bin(hc, k_blk, scan, &sh_bin, &sh_above);
  const uint32_t bin = (uint32_t)sh_bin;
  // this thread's candidates (top bits == bin) and keys above the bin
  uint64_t masks[kChunkKpt];
  int n_gt = 0, n_c = 0;
#pragma unroll
  for (int j = 0; j < kChunkKpt; ++j) {
    const bool ok = idx[j] < qr.nb;
    const uint32_t kb = key[j] >> (32 - kTopBits);
    n_gt += (ok && kb > bin) ? 1 : 0;
    masks[j] = __ballot(ok && kb == bin);
    n_c += __popcll(masks[j]);                       // the wave's candidates (same in every lane)
  }
  n_gt = wave_sum_int(n_gt);
  if (lane == 0) {
    wave_cand[wave] = n_c;
    wave_gt[wave] = n_gt;
  }
  __syncthreads();
  int slot = 0, tot_c = 0, tot_gt = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    slot += w < wave ? wave_cand[w] : 0;
    tot_c += wave_cand[w];
    tot_gt += wave_gt[w];
  }
  uint64_t* seg = ws.cand(q, blockIdx.x);
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < kChunkKpt; ++j) {
    if ((masks[j] >> lane) & 1ull)
      seg[slot + __popcll(masks[j] & below)] = ((uint64_t)key[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx[j]);
    slot += __popcll(masks[j]);
  }
  if (tid == 0) {
    ws.n_above(q)[blockIdx.x] = (uint32_t)tot_gt;
    ws.n_cand(q)[blockIdx.x] = (uint32_t)tot_c;
  }
}

struct FinalSmem {
  uint64_t cand[kCandCap];                           // 128 KiB
  uint32_t hist[8 * kCopyStride];
  uint32_t tally[kMaxChunks];                        // kept blocks per chunk
  uint32_t cpre[kMaxChunks + 1];                     // exclusive prefix of candidates per chunk
  int scan[kFinalThreads / kWave + 1];
  int pick[3];
  uint64_t cut;
};

__global__ void __launch_bounds__(kFinalThreads)
chunk_final_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
                   const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk,
                   int32_t* __restrict__ sel, int64_t sel_ld, int32_t* __restrict__ n_sel, ChunkWs ws) {
  __shared__ union {
    FinalSmem f;
    WgSmem w;
  } sm;
  constexpr int PER = kMaxChunks / kFinalThreads;    // chunks per thread, contiguous
  const int q = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave;
  // per-chunk counts, read before the query's length is known (entries past the
  // query's chunks are ignored)
  uint32_t na[PER], nc[PER];
  const int gcap = ws.g < kMaxChunks ? ws.g : kMaxChunks;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int w = tid * PER + j;
    na[j] = w < gcap ? ws.n_above(q)[w] : 0u;
    nc[j] = w < gcap ? ws.n_cand(q)[w] : 0u;
  }
  const QueryRow qr = query_row(seq_len, q_seq, q_pos, q, c);
  int32_t* out = sel + (int64_t)q * sel_ld;
  if (qr.nb <= k_blk) {
    write_dense<kFinalThreads>(out, sel_ld, qr.n_vis, n_sel + q);
    return;
  }
  uint32_t* ctrl = ws.ctrl(q);
  const int n_chunks = (qr.nb + kChunk - 1) / kChunk;
  int la = 0, lc = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int w = tid * PER + j;
    if (w >= n_chunks) na[j] = nc[j] = 0u;
    la += (int)na[j];
    lc += (int)nc[j];
  }
  int tot_above, n_cand;
  (void)block_exclusive_scan<kFinalThreads>(la, sm.f.scan, &tot_above);
  int cp = block_exclusive_scan<kFinalThreads>(lc, sm.f.scan, &n_cand);
  if (n_cand > kCandCap || n_chunks > kMaxChunks) {
    if (tid == 0) ctrl[CT_FALLBACK] = 1u;
    select_one_query<kFinalThreads, 8>(scores + (int64_t)q * scores_ld, qr.nb, qr.n_vis, c, k_blk, out, sel_ld,
                                       n_sel + q, sm.w);
    return;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int w = tid * PER + j;
    sm.f.cpre[w] = (uint32_t)cp;
    sm.f.tally[w] = na[j];
    cp += (int)nc[j];
  }
  if (tid == 0) sm.f.cpre[kMaxChunks] = (uint32_t)n_cand;
  __syncthreads();
  // gather the candidates: entry e lives in the chunk whose prefix range holds it
  for (int e = tid; e < n_cand; e += kFinalThreads) {
    int lo = 0, hi = n_chunks - 1;                   // largest w with cpre[w] <= e
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int)sm.f.cpre[mid] <= e) lo = mid;
      else hi = mid - 1;
    }
    sm.f.cand[e] = ws.cand(q, lo)[e - (int)sm.f.cpre[lo]];
  }
  int k_rem = k_blk - tot_above;                     // >= 1 by the choice of the bin
  if (tid == 0) sm.f.pick[2] = 0;
  __syncthreads();
  // Radix select of the k_rem-th largest candidate over the 52 bits below the
  // shared top 12, 8 bits at a time (the last digit has 4), stopping once the
  // chosen bin holds a single value -- values are unique, so it always ends.
  uint64_t prefix = sm.f.cand[0] >> (64 - kTopBits);
  for (int shift = 64 - kTopBits; shift > 0;) {
    const int width = shift >= 8 ? 8 : shift;
    shift -= width;
    const uint32_t dmask = (1u << width) - 1u;
    for (int e = tid; e < 8 * kCopyStride; e += kFinalThreads) sm.f.hist[e] = 0u;
    __syncthreads();
    uint32_t* mine = sm.f.hist + (lane & 7) * kCopyStride;
    for (int e = tid; e < n_cand; e += kFinalThreads) {
      const uint64_t v = sm.f.cand[e];
      if ((v >> (shift + width)) == prefix) atomicAdd(&mine[(uint32_t)(v >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (tid < kBins) {                               // 4 whole waves
      uint32_t n = 0;
#pragma unroll
      for (int cpy = 0; cpy < 8; ++cpy) n += sm.f.hist[cpy * kCopyStride + tid];
      sm.f.hist[tid] = n;                            // copy 0 now holds the totals
    }
    __syncthreads();
    int ge_in_wave = 0;
    if (tid < kBins) {
      ge_in_wave = wave_inclusive_scan((int)sm.f.hist[kBins - 1 - tid], lane);
      if (lane == kWave - 1) sm.f.scan[tid / kWave] = ge_in_wave;
    }
    __syncthreads();
    if (tid < kBins) {
      const int v = kBins - 1 - tid;
      int b = 0;
      for (int w = 0; w < tid / kWave; ++w) b += sm.f.scan[w];
      const int ge = b + ge_in_wave, cnt = (int)sm.f.hist[v], gt = ge - cnt;
      if (gt < k_rem && ge >= k_rem) {
        sm.f.pick[0] = v;
        sm.f.pick[1] = k_rem - gt;
        sm.f.pick[2] = cnt;
      }
    }
    __syncthreads();
    prefix = (prefix << width) | (uint64_t)sm.f.pick[0];
    k_rem = sm.f.pick[1];
    const int cnt = sm.f.pick[2];
    __syncthreads();
    if (cnt == 1 || shift == 0) {                    // the cut is the single value left in the bin
      for (int e = tid; e < n_cand; e += kFinalThreads) {
        const uint64_t v = sm.f.cand[e];
        if ((v >> shift) == prefix) sm.f.cut = v;
      }
      __syncthreads();
      break;
    }
  }
  const uint64_t cut = sm.f.cut;
  // kept blocks per chunk: those above the bin plus the kept candidates
  for (int e = tid; e < n_cand; e += kFinalThreads) {
    const uint64_t v = sm.f.cand[e];
    if (v >= cut) atomicAdd(&sm.f.tally[(0xFFFFFFFFu - (uint32_t)v) / kChunk], 1u);
  }
  __syncthreads();
  int loc = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) loc += (int)sm.f.tally[tid * PER + j];   // entries past n_chunks are 0
  int tot;
  int run = block_exclusive_scan<kFinalThreads>(loc, sm.f.scan, &tot);
  uint32_t* offs = ws.offsets(q);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int w = tid * PER + j;
    if (w < n_chunks) offs[w] = (uint32_t)run;
    run += (int)sm.f.tally[w];
  }
  if (tid == 0) {
    ctrl[CT_T] = (uint32_t)(cut >> 32);
    ctrl[CT_CUT] = 0xFFFFFFFFu - (uint32_t)cut;
  }
  write_tail<kFinalThreads>(out, sel_ld, qr.nb, qr.n_vis, c, k_blk, n_sel + q);
}

__global__ void __launch_bounds__(kChunkThreads)
chunk_emit_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
                  const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk,
                  int32_t* __restrict__ sel, int64_t sel_ld, ChunkWs ws) {
  __shared__ int scan[kChunkThreads / kWave + 1];
  const int q = blockIdx.y;
  const int base = blockIdx.x * kChunk;
  uint32_t key[kChunkKpt];
  int idx[kChunkKpt];
  load_chunk_keys<true>(scores + (int64_t)q * scores_ld, scores_ld, base, key, idx);
  const uint32_t* ctrl = ws.ctrl(q);
  const uint32_t fallback = ctrl[CT_FALLBACK], T = ctrl[CT_T], cut = ctrl[CT_CUT];
  const int off = (int)ws.offsets(q)[blockIdx.x];
  const QueryRow qr = query_row(seq_len, q_seq, q_pos, q, c);
  if (qr.nb <= k_blk || base >= qr.nb || fallback) return;
  bool take[kChunkKpt];
  int n = 0;
#pragma unroll
  for (int j = 0; j < kChunkKpt; ++j) {
    take[j] = idx[j] < qr.nb && (key[j] > T || (key[j] == T && (uint32_t)idx[j] <= cut));
    n += take[j] ? 1 : 0;
  }
  int tot;
  int o = off + block_exclusive_scan<kChunkThreads>(n, scan, &tot);
  int32_t* out = sel + (int64_t)q * sel_ld;
#pragma unroll
  for (int j = 0; j < kChunkKpt; ++j) {
    if (take[j] && o < k_blk) {                      // o < k_blk always; the bound only guards memory
      const int32_t p0 = (int32_t)idx[j] * c;
      int32_t* dst = out + (int64_t)o * c;
      for (int t = 0; t < c; ++t) dst[t] = p0 + t;
      ++o;
    }
  }
}

// ---------------------------------------------------------------------------- host

static bool use_chunked(const sa_dims& d, int n_q, int max_len) {
  const long long max_blocks = (long long)max_len / d.compress_ratio;
  return n_q <= 64 && max_blocks > 4096 && max_blocks > d.top_k / d.compress_ratio;
}

static int chunks_for(const sa_dims& d, int max_len) {
  const long long max_blocks = (long long)max_len / d.compress_ratio;
  return (int)((max_blocks + kChunk - 1) / kChunk);
}

size_t select_ws_bytes(const sa_dims& d, int n_q, int max_len) {
  if (!use_chunked(d, n_q, max_len)) return 0;
  return (size_t)n_q * ChunkWs::query_bytes(chunks_for(d, max_len));
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
                         int32_t* n_sel, void* ws, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  const int cr = d.compress_ratio, k_blk = d.top_k / d.compress_ratio;
  const long long max_blocks = (long long)c.max_len / cr;
  if (use_chunked(d, n_q, c.max_len)) {
    const int g = chunks_for(d, c.max_len);
    ChunkWs cw{(char*)ws, ChunkWs::query_bytes(g), g};
    hipLaunchKernelGGL(chunk_zero_kernel, dim3(n_q), dim3(256), 0, stream, cw);
    dim3 grid(g, n_q);
    hipLaunchKernelGGL(chunk_hist_kernel, grid, dim3(kChunkThreads), 0, stream, scores, scores_ld, c.seq_len, q_seq,
                       q_pos, cr, k_blk, cw);
    hipLaunchKernelGGL(chunk_cand_kernel, grid, dim3(kChunkThreads), 0, stream, scores, scores_ld, c.seq_len, q_seq,
                       q_pos, cr, k_blk, cw);
    hipLaunchKernelGGL(chunk_final_kernel, dim3(n_q), dim3(kFinalThreads), 0, stream, scores, scores_ld, c.seq_len,
                       q_seq, q_pos, cr, k_blk, sel, sel_ld, n_sel, cw);
    hipLaunchKernelGGL(chunk_emit_kernel, grid, dim3(kChunkThreads), 0, stream, scores, scores_ld, c.seq_len, q_seq,
                       q_pos, cr, k_blk, sel, sel_ld, cw);
    return hipGetLastError();
  }
  if (n_q <= 64) {                                   // few queries, short rows: wide workgroups
    if (max_blocks <= 1024 * 4) launch_select_t<1024, 4>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
    else launch_select_t<1024, 8>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
  } else {
    if (max_blocks <= 256 * 8) launch_select_t<256, 8>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
    else if (max_blocks <= 256 * 16) launch_select_t<256, 16>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
    else if (max_blocks <= 256 * 32) launch_select_t<256, 32>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
    else launch_select_t<256, 64>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
  }
  return hipGetLastError();
}

}  // namespace sa
