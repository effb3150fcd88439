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
// Scores are mapped to order-preserving 32-bit keys (+0/-0 identical).  Three designs,
// by row length and number of query tokens:
//
// Rows of up to 32768 blocks (any number of query tokens): one 1024-thread workgroup
// per query holds the whole row in registers and radix-selects over them (see the
// wide kernel below); no workspace.
//
// Longer rows, many query tokens: one workgroup per query finds the K_blk-th largest
// key T exactly by a 4-pass radix select over 8-bit digits, most significant first;
// each pass histograms the digit among the keys that match the digits fixed so far.
// The histogram is privatised per lane (32 copies, padded by one word) so that keys
// sharing a digit -- scores crowd into a few binades -- hit different LDS banks
// instead of serialising on one address.  The kept blocks (key > T, or key == T among
// the first r such in index order) are then compacted in index order with two
// workgroup prefix sums.  Thread t owns blocks [t*KPT, (t+1)*KPT) of a chunk; longer
// rows stream chunk by chunk.
//
// Longer rows, few query tokens (long-context decode), chunked: the row is cut into
// chunks of 2048 blocks, one workgroup each, so the whole GPU takes part; three
// launches, whose boundaries order them (no workgroup ever waits on another):
//   hist    each chunk histograms the top 12 bits of its keys in LDS and adds the
//           non-empty bins to the query's histogram in the workspace (device-scope
//           atomics);
//   select  each chunk finds, from that (complete) histogram, the bin b holding the
//           K_blk-th largest key and the number of keys above it -- every chunk
//           alike -- and writes its keys in b or above, in index order, to its own
//           segment as (key << 32 | ~index): unique 64-bit values whose order is
//           exactly (score desc, index asc), so ties need no special case;
//   finish  one workgroup per query gathers the segments, radix-selects the cut
//           among the values inside b (11-bit digits below the 12 shared bits,
//           stopping once the chosen bin holds one value), writes every value at or
//           above the cut as positions in index order, then the tail, the padding
//           and n_sel, and returns the histogram to zero for the next call.
// If the values in b and above overflow what that workgroup holds (massive exact
// ties), it runs the 4-pass algorithm above over the whole row instead.
#include "select_chunk.hpp"

namespace sa {

// ------------------------------------------------------- per-query workgroup select

template <int BLOCK, int KPT>
__global__ void __launch_bounds__(BLOCK)
select_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
              const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk,
              int32_t* __restrict__ sel, int64_t sel_ld, int32_t* __restrict__ n_sel) {
  __shared__ WgSmem sm;
  const int i = blockIdx.x;
  const int n_vis = visible_tokens(seq_meta(q_seq, seq_len, nullptr, nullptr, i).len, q_pos[i]);
  const int nb = n_vis / c;
  int32_t* out = sel + (int64_t)i * sel_ld;
  if (nb <= k_blk) {
    write_dense<BLOCK>(out, sel_ld, n_vis, n_sel + i);
    return;
  }
  select_one_query<BLOCK, KPT>(scores + (int64_t)i * scores_ld, nb, c, k_blk, out, sm);
  write_tail<BLOCK>(out, sel_ld, nb, n_vis, c, k_blk, n_sel + i);
}

// ------------------------------------------------------------------ chunked select

// Bin holding the k-th largest key of a histogram split as PER bins per thread
// (thread t holds bins [t*PER, t*PER+PER)), and the number of keys in higher bins,
// to all threads of the BLOCK-thread workgroup.
template <int BLOCK, int PER>
__device__ __forceinline__ void find_top_bin(const uint32_t (&cnt)[PER], int k, int* lds_scan, int* out_bin,
                                             int* out_above) {
  const int tid = threadIdx.x;
  int sum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) sum += (int)cnt[j];
  int total;
  const int below_incl = block_exclusive_scan<BLOCK>(sum, lds_scan, &total) + sum;
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

__device__ __forceinline__ uint32_t coherent_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Pass 1 (one workgroup per chunk): the chunk's histogram of the top 12 key bits is
// added to the query's histogram.
__global__ void __launch_bounds__(kHistThreads)
chunk_hist_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
                  const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk,
                  WsState* __restrict__ st, ChunkScratch sc) {
  constexpr int kStride = kBins1 + 1;
  __shared__ uint32_t h[kHistCopies * kStride];
  const int q = blockIdx.y, tid = threadIdx.x;
  const int base = blockIdx.x * kChunk;
  const float* row = scores + (int64_t)q * scores_ld;
  // keys read before the query's length is known (indices below scores_ld are valid)
  uint32_t key[kHistKpt];
  int idx[kHistKpt];
#pragma unroll
  for (int j = 0; j < kHistKpt; ++j) {
    idx[j] = base + j * kHistThreads + tid;
    key[j] = key_clamped(row, idx[j], (int)scores_ld - 1);
  }
  for (int e = tid; e < kHistCopies * kStride; e += kHistThreads) h[e] = 0u;
  const QueryRowInfo qr = query_blocks(seq_len, q_seq, q_pos, q, c);
  if (qr.nb <= k_blk || base >= qr.nb) return;      // uniform over the workgroup
  __syncthreads();
  uint32_t* mine = h + (tid & (kHistCopies - 1)) * kStride;
#pragma unroll
  for (int j = 0; j < kHistKpt; ++j)
    if (idx[j] < qr.nb) atomicAdd(&mine[key[j] >> (32 - kTopBits)], 1u);
  __syncthreads();
  uint32_t* g = st->ghist[q];
  for (int b = tid; b < kBins1; b += kHistThreads) {
    uint32_t n = 0;
#pragma unroll
    for (int cp = 0; cp < kHistCopies; ++cp) n += h[cp * kStride + b];
    if (n) atomicAdd(&g[b], n);
  }
}

// Pass 2 (one workgroup per chunk): the chunk finds the bin holding the K_blk-th
// largest key from the query's histogram and keeps, in index order, every block whose
// key lies in that bin or above as (key << 32 | ~index) -- unique values ordered
// exactly as (score desc, index asc).  Chunk 0 records the bin and the number still
// to take inside it for pass 3; the dense case is written here.
__global__ void __launch_bounds__(kSelThreads)
chunk_select_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
                    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk,
                    int32_t* __restrict__ sel, int64_t sel_ld, int32_t* __restrict__ n_sel, WsState* __restrict__ st,
                    ChunkScratch sc) {
  __shared__ int scan[kSelThreads / kWave + 1];
  __shared__ int pick[2];
  const int q = blockIdx.y, tid = threadIdx.x;
  const int base = blockIdx.x * kChunk;
  const float* row = scores + (int64_t)q * scores_ld;
  uint32_t key[kSelKpt];
  int idx[kSelKpt];
#pragma unroll
  for (int j = 0; j < kSelKpt; ++j) {
    idx[j] = base + tid * kSelKpt + j;               // contiguous: index order across threads
    key[j] = key_clamped(row, idx[j], (int)scores_ld - 1);
  }
  uint32_t* ghist = st->ghist[q];
  constexpr int PER1 = kBins1 / kSelThreads;         // histogram bins per thread
  uint32_t hc[PER1];
#pragma unroll
  for (int j = 0; j < PER1; ++j) hc[j] = coherent_load(&ghist[tid * PER1 + j]);
  const QueryRowInfo qr = query_blocks(seq_len, q_seq, q_pos, q, c);
  int32_t* out = sel + (int64_t)q * sel_ld;
  if (qr.nb <= k_blk) {                              // every block fits: dense
    if (blockIdx.x == 0) write_dense<kSelThreads>(out, sel_ld, qr.n_vis, n_sel + q);
    return;
  }
  if (base >= qr.nb) return;
  // the bin b holding the K_blk-th largest key, and how many to take inside it
  find_top_bin<kSelThreads, PER1>(hc, k_blk, scan, &pick[0], &pick[1]);
  const uint32_t bin = (uint32_t)pick[0];
  int k_rem = k_blk - pick[1];
  // this chunk's entries, in index order
  bool keep[kSelKpt];
  int n = 0;
#pragma unroll
  for (int j = 0; j < kSelKpt; ++j) {
    keep[j] = idx[j] < qr.nb && (key[j] >> (32 - kTopBits)) >= bin;
    n += keep[j] ? 1 : 0;
  }
  int tot;
  int slot = block_exclusive_scan<kSelThreads>(n, scan, &tot);
  uint64_t* seg = sc.ent(q, blockIdx.x);
#pragma unroll
  for (int j = 0; j < kSelKpt; ++j)
    if (keep[j]) seg[slot++] = ((uint64_t)key[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx[j]);
  if (tid == 0) {
    sc.n_ent(q)[blockIdx.x] = (uint32_t)tot;
    if (blockIdx.x == 0) {
      sc.ctrl(q)[0] = bin;
      sc.ctrl(q)[1] = (uint32_t)k_rem;
    }
  }
}

// ------------------------------------------------------ one wide workgroup per row

// Decode rows of up to 32768 blocks: one 1024-thread workgroup holds the whole row in
// registers and needs no workspace (the radix select of select_wide.hpp).
constexpr int kWideThreads = 1024;
constexpr int kWideMaxKpt = 32;

template <int KPT>
__global__ void __launch_bounds__(kWideThreads)
select_wide_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
                   const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk,
                   int32_t* __restrict__ sel, int64_t sel_ld, int32_t* __restrict__ n_sel) {
  constexpr int NT = kWideThreads, COPIES = WideCfg<NT, KPT>::copies;
  __shared__ WideSmem<NT, KPT> sm;
  const int q = blockIdx.x, tid = threadIdx.x;
  const float* row = scores + (int64_t)q * scores_ld;
  // The whole row is loaded up front and kept in registers for every pass; the
  // query's length arrives with it (indices below scores_ld are valid memory).
  float raw[KPT];
  wide_load_row<NT, KPT>(row, scores_ld, raw);
  const QueryRowInfo qr = query_blocks(seq_len, q_seq, q_pos, q, c);
  for (int e = tid; e < kP1Bins * COPIES / 4; e += NT) ((uint4*)sm.h1)[e] = uint4{0u, 0u, 0u, 0u};
  for (int e = tid; e < kWideBins; e += NT) sm.h2[e] = 0u;
  __builtin_amdgcn_sched_barrier(0);                 // every load in flight before the first is used
  int32_t* out = sel + (int64_t)q * sel_ld;
  if (qr.nb <= k_blk) {
    write_dense<NT>(out, sel_ld, qr.n_vis, n_sel + q);
    return;
  }
  __syncthreads();                                   // the histograms are clear (the loads may still fly)
  const int body = k_blk * c;
  int32_t* list = body <= kP1Bins * COPIES ? (int32_t*)sm.h1 : nullptr;   // pass 1's histogram is free by then
  wide_select_rows<NT, KPT>(raw, qr.nb, c, k_blk, sm, list, out);
  if (list)
    for (int i = tid; i < body; i += NT) out[i] = list[i];
  write_tail<NT>(out, sel_ld, qr.nb, qr.n_vis, c, k_blk, n_sel + q);
}

// ------------------------------------------------------------ chunked: finish

// Pass 3 (one workgroup per query, after every chunk's entries are written): gather
// the entries, cut inside the bin, write the list, return the histogram to zero.
__global__ void __launch_bounds__(kSelThreads)
chunk_finish_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
                    const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk,
                    int32_t* __restrict__ sel, int64_t sel_ld, int32_t* __restrict__ n_sel, WsState* __restrict__ st,
                    ChunkScratch sc) {
  __shared__ union {
    FinSmem<kEntCap, kMaxChunks> f;
    WgSmem w;
  } sm;
  const int q = blockIdx.x;
  ChunkSpec sp;
  sp.issue(sc, q);
  const uint32_t bin = sc.ctrl(q)[0];
  const int k_rem = (int)sc.ctrl(q)[1];
  const QueryRowInfo qr = query_blocks(seq_len, q_seq, q_pos, q, c);
  if (qr.nb <= k_blk) return;                        // dense: written by the selection pass
  uint32_t* ghist = st->ghist[q];
  for (int b = threadIdx.x; b < kBins1; b += kSelThreads) ghist[b] = 0u;   // every chunk has read it
  int32_t* out = sel + (int64_t)q * sel_ld;
  chunk_cut<kEntCap, kMaxChunks>(sp, sc, q, scores + (int64_t)q * scores_ld, qr, c, k_blk, bin, k_rem, sm.f, sm.w,
                                 out);
  write_tail<kSelThreads>(out, sel_ld, qr.nb, qr.n_vis, c, k_blk, n_sel + q);
}

// ---------------------------------------------------------------------------- host

constexpr long long kWideMax = (long long)kWideThreads * kWideMaxKpt;   // blocks one wide workgroup holds

bool select_chunked(const sa_dims& d, int n_q, int max_len) {
  const long long max_blocks = (long long)max_len / d.compress_ratio;
  return n_q <= kStateQueries && max_blocks > kWideMax && max_blocks > d.top_k / d.compress_ratio;
}

int select_chunk_count(const sa_dims& d, int max_len) {
  const long long max_blocks = (long long)max_len / d.compress_ratio;
  return (int)((max_blocks + kChunk - 1) / kChunk);
}

size_t select_scratch_bytes(const sa_dims& d, int n_q, int max_len) {
  if (!select_chunked(d, n_q, max_len)) return 0;
  return (size_t)n_q * ChunkScratch::query_bytes(select_chunk_count(d, max_len));
}

ChunkScratch chunk_scratch(const sa_dims& d, const CacheArgs& c, void* ws) {
  const int g = select_chunk_count(d, c.max_len);
  return ChunkScratch{(char*)ws + SA_WS_STATE_BYTES, ChunkScratch::query_bytes(g), g};
}

hipError_t launch_chunk_passes(const sa_dims& d, const CacheArgs& c, const float* scores, int64_t scores_ld,
                               const int32_t* q_seq, const int32_t* q_pos, int n_q, int32_t* sel, int64_t sel_ld,
                               int32_t* n_sel, void* ws, hipStream_t stream) {
  const int cr = d.compress_ratio, k_blk = d.top_k / d.compress_ratio;
  WsState* st = (WsState*)ws;
  const ChunkScratch sc = chunk_scratch(d, c, ws);
  const dim3 grid(sc.g, n_q);
  hipLaunchKernelGGL(chunk_hist_kernel, grid, dim3(kHistThreads), 0, stream, scores, scores_ld, c.seq_len, q_seq,
                     q_pos, cr, k_blk, st, sc);
  hipLaunchKernelGGL(chunk_select_kernel, grid, dim3(kSelThreads), 0, stream, scores, scores_ld, c.seq_len, q_seq,
                     q_pos, cr, k_blk, sel, sel_ld, n_sel, st, sc);
  return hipGetLastError();
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
  if (select_chunked(d, n_q, c.max_len)) {
    const hipError_t err = launch_chunk_passes(d, c, scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld, n_sel, ws,
                                               stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(chunk_finish_kernel, dim3(n_q), dim3(kSelThreads), 0, stream, scores, scores_ld, c.seq_len,
                       q_seq, q_pos, cr, k_blk, sel, sel_ld, n_sel, (WsState*)ws, chunk_scratch(d, c, ws));
    return hipGetLastError();
  }
  if (max_blocks <= kWideMax) {                      // rows that fit one workgroup's registers
#define SA_WIDE(KPT_)                                                                                         \
  hipLaunchKernelGGL(select_wide_kernel<KPT_>, dim3(n_q), dim3(kWideThreads), 0, stream, scores, scores_ld,  \
                     c.seq_len, q_seq, q_pos, cr, k_blk, sel, sel_ld, n_sel)
    if (max_blocks <= 1024 * 4) SA_WIDE(4);
    else if (max_blocks <= 1024 * 8) SA_WIDE(8);
    else if (max_blocks <= 1024 * 16) SA_WIDE(16);
    else SA_WIDE(32);
#undef SA_WIDE
  } else {
    if (max_blocks <= 256 * 8) launch_select_t<256, 8>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
    else if (max_blocks <= 256 * 16) launch_select_t<256, 16>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
    else if (max_blocks <= 256 * 32) launch_select_t<256, 32>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
    else launch_select_t<256, 64>(d, scores, scores_ld, c, q_seq, q_pos, n_q, sel, sel_ld, n_sel, stream);
  }
  return hipGetLastError();
}

}  // namespace sa