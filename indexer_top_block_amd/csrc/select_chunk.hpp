// Pieces of the block selection shared by select.hip and select_fwd.hip: the
// per-query radix select over a streamed row, and the finishing pass of the chunked
// selection (gather the candidates the chunks kept, cut inside the bin, write the
// kept blocks' positions), as device functions over global or LDS output.
//
// The kept blocks are the K_blk best of the query's complete blocks (ties to the lower
// block index), plus the tail, dense below top_k + c - 1 visible tokens (llama.cpp
// commit "llama: QSA sparse attention for qwen4exp"); the list is int32, ascending,
// -1 padded (llama.cpp PR #27970, flash_attn_mask_to_sparse_indices).
#pragma once

#include "sa_common.hpp"
#include "sa_launch.hpp"
#include "select_wide.hpp"

namespace sa {

constexpr int kCopies = 32;
constexpr int kBins = 256;
constexpr int kCopyStride = kBins + 1;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;                       // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Key of row[min(idx, last)]: the index is clamped rather than the load guarded, so
// consecutive loads issue back to back instead of each waiting behind a branch.
// Callers mask keys past the row's end themselves.
__device__ __forceinline__ uint32_t key_clamped(const float* __restrict__ row, int idx, int last) {
  return order_key(row[idx < last ? idx : last]);
}

// ------------------------------------------------------- per-query workgroup select

struct WgSmem {
  int hist[kCopies * kCopyStride];
  int total[kBins];
  int scan_scratch[1024 / kWave + 1];
  int pick[2];
};

// One workgroup selects for one query whose scores are row[0 .. nb): the k_blk kept
// blocks' positions, k_blk * c ascending entries, to out (global memory or LDS).
// Requires nb > k_blk.  The tail and the padding are the caller's.
template <int BLOCK, int KPT>
__device__ void select_one_query(const float* __restrict__ row, int nb, int c, int k_blk, int32_t* __restrict__ out,
                                 WgSmem& sm) {
  constexpr int CH = BLOCK * KPT;                    // blocks per chunk
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int n_chunks = (nb + CH - 1) / CH;
  const bool resident = (n_chunks == 1);
  uint32_t key[KPT];
  auto load_chunk = [&](int ch) {
    const int base = ch * CH + tid * KPT;
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = key_clamped(row, base + j, nb - 1);
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
        if (c == 1) {
          dst[0] = p0;
        } else {
          for (int t = 0; t < c; ++t) dst[t] = p0 + t;
        }
        ++o;
      }
    }
    eq_base += eq_tot;
    out_base += take_tot;
  }
}

// ------------------------------------------------------------------ chunked select

constexpr int kChunk = 2048;                         // blocks per chunk workgroup
constexpr int kHistThreads = 256;
constexpr int kHistKpt = kChunk / kHistThreads;      // 8
constexpr int kSelThreads = 1024;
constexpr int kSelKpt = kChunk / kSelThreads;        // 2
constexpr int kTopBits = 12;
constexpr int kBins1 = 1 << kTopBits;                // 4096 bins of the top 12 bits
constexpr int kHistCopies = 4;
constexpr int kEntCap = 16384;                       // entries the finishing workgroup holds in LDS
constexpr int kMaxChunks = 2048;                     // chunks per query it tallies

// Scratch of one query: bin and remaining count from the histogram pass, the
// number of entries each chunk kept, and each chunk's entries (index order).
struct ChunkScratch {
  char* base;
  size_t q_stride;
  int g;
  static __device__ __host__ size_t head_bytes(int g) { return ((size_t)(16 + g) * 4 + 255) / 256 * 256; }
  __device__ uint32_t* ctrl(int q) const { return (uint32_t*)(base + q * q_stride); }
  __device__ uint32_t* n_ent(int q) const { return ctrl(q) + 16; }
  __device__ uint64_t* ent(int q, int w) const {
    return (uint64_t*)(base + q * q_stride + head_bytes(g)) + (size_t)w * kChunk;
  }
  static __host__ size_t query_bytes(int g) { return head_bytes(g) + (size_t)g * kChunk * 8; }
};

// The chunk segments of a workspace (host).
ChunkScratch chunk_scratch(const sa_dims& d, const CacheArgs& c, void* ws);

constexpr int kFinBins = 2048;                      // 11-bit digits of the cut inside the bin

// LDS of the finishing pass: ENT_CAP candidates, MAX_CHUNKS chunk prefixes.
template <int ENT_CAP, int MAX_CHUNKS>
struct FinSmem {
  uint64_t ent[ENT_CAP];                             // the candidates, (key << 32 | ~index)
  uint32_t h[2][kFinBins];                           // alternating digit histograms
  uint32_t cpre[MAX_CHUNKS + 1];                     // exclusive prefix of entries per chunk
  int scan[kSelThreads / kWave + 1];
  int wsum[2][kSelThreads / kWave];                  // per-wave totals of the picks
  int pick[4];
  uint64_t cut;
};

// The finishing pass's first reads, issued before the query's length (and so its
// chunk count) is known, so that they share one round trip: the entry count and the
// first entries of each of up to kSelThreads / 4 chunks.  Thread t serves chunk
// t / tpc, entries t % tpc + tpc * i.
struct ChunkSpec {
  static constexpr int kB = 4;
  bool on;
  int tpc, cw, cr;
  uint32_t ne;
  uint64_t v[kB];
  __device__ __forceinline__ void issue(const ChunkScratch& sc, int q) {
    const int tid = threadIdx.x;
    on = sc.g <= kSelThreads / 4;
    tpc = 1;                                         // a power of two, <= kChunk / kB
    while (tpc * 2 * sc.g <= kSelThreads && tpc * 2 * kB <= kChunk) tpc *= 2;
    cw = tid / tpc;
    cr = tid % tpc;
    ne = 0u;
    if (on && cw < sc.g) {
      ne = sc.n_ent(q)[cw];
      const uint64_t* seg = sc.ent(q, cw);
#pragma unroll
      for (int i = 0; i < kB; ++i) v[i] = seg[cr + tpc * i];   // < kChunk: inside the segment
    }
  }
};

// The finishing pass for query q, whose nb > k_blk blocks the chunks have cut to the
// candidates in bin `bin` and above (k_rem still to take inside the bin): gathers the
// candidates, finds the k_rem-th largest inside the bin, and writes the k_blk kept
// blocks' positions (k_blk * c ascending entries) to dst, global memory or LDS.
// Candidates beyond ENT_CAP (massive exact ties), or more chunks than MAX_CHUNKS, take
// the per-query select over the row instead.  The tail and the padding are the
// caller's; dst is complete once every thread has returned.
template <int ENT_CAP, int MAX_CHUNKS>
__device__ __forceinline__ void chunk_cut(ChunkSpec& sp, const ChunkScratch& sc, int q, const float* __restrict__ row,
                                          const QueryRowInfo& qr, int c, int k_blk, uint32_t bin, int k_rem,
                                          FinSmem<ENT_CAP, MAX_CHUNKS>& f, WgSmem& w, int32_t* dst) {
  const int tid = threadIdx.x;
  const int n_chunks = min((qr.nb + kChunk - 1) / kChunk, sc.g);   // (a length beyond max_len is clamped)

  // ---- gather ------------------------------------------------------------------------
  int n_ent;
  if (sp.on) {
    if (sp.cw >= n_chunks) sp.ne = 0u;
    // exclusive prefix over the chunks: only each chunk's first thread contributes
    const int cp = block_exclusive_scan<kSelThreads>(sp.cr == 0 ? (int)sp.ne : 0, f.scan, &n_ent);
    if (n_ent > ENT_CAP) {                           // massive exact ties: per-query select over the row
      select_one_query<kSelThreads, 8>(row, qr.nb, c, k_blk, dst, w);
      return;
    }
    if (sp.cr == 0 && sp.cw < n_chunks) f.cpre[sp.cw] = (uint32_t)cp;
    __syncthreads();
    if (sp.cw < n_chunks && sp.ne > 0u) {
      const int base_e = (int)f.cpre[sp.cw];
#pragma unroll
      for (int i = 0; i < ChunkSpec::kB; ++i)
        if (sp.cr + sp.tpc * i < (int)sp.ne) f.ent[base_e + sp.cr + sp.tpc * i] = sp.v[i];
      const uint64_t* seg = sc.ent(q, sp.cw);
      for (int k = sp.cr + sp.tpc * ChunkSpec::kB; k < (int)sp.ne; k += sp.tpc) f.ent[base_e + k] = seg[k];
    }
  } else if constexpr (MAX_CHUNKS > kSelThreads / 4) {
    constexpr int PER = MAX_CHUNKS / kSelThreads;    // chunk counts per thread
    const int gcap = n_chunks < MAX_CHUNKS ? n_chunks : MAX_CHUNKS;
    uint32_t ne[PER];
    int loc = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int wj = tid * PER + j;
      ne[j] = wj < gcap ? sc.n_ent(q)[wj] : 0u;
      loc += (int)ne[j];
    }
    int cp = block_exclusive_scan<kSelThreads>(loc, f.scan, &n_ent);
    if (n_ent > ENT_CAP || n_chunks > MAX_CHUNKS) {  // massive exact ties: per-query select over the row
      select_one_query<kSelThreads, 8>(row, qr.nb, c, k_blk, dst, w);
      return;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      f.cpre[tid * PER + j] = (uint32_t)cp;
      cp += (int)ne[j];
    }
    __syncthreads();
    for (int e = tid; e < n_ent; e += kSelThreads) {
      int lo = 0, hi = n_chunks - 1;                 // largest chunk whose prefix is <= e
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int)f.cpre[mid] <= e) lo = mid;
        else hi = mid - 1;
      }
      f.ent[e] = sc.ent(q, lo)[e - (int)f.cpre[lo]];
    }
  } else {                                           // more chunks than this form reads at once
    select_one_query<kSelThreads, 8>(row, qr.nb, c, k_blk, dst, w);
    return;
  }
  __syncthreads();
  // k_rem-th largest value among the entries inside the bin (top 12 bits == bin):
  // 11-bit digits below them, each bin found with the hierarchical pick; two
  // histograms, each cleared while the other counts; stop once the chosen bin holds
  // one value (values are unique).
  for (int b = tid; b < kFinBins; b += kSelThreads) {
    f.h[0][b] = 0u;
    f.h[1][b] = 0u;
  }
  __syncthreads();
  uint64_t prefix = bin;
  for (int shift = 64 - kTopBits, pass = 0; shift > 0; ++pass) {
    const int width = shift >= 11 ? 11 : shift;
    shift -= width;
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t* h = f.h[pass & 1];
    for (int e = tid; e < n_ent; e += kSelThreads) {
      const uint64_t v = f.ent[e];
      if ((v >> (shift + width)) == prefix) atomicAdd(&h[(uint32_t)(v >> shift) & dmask], 1u);
    }
    if (pass > 0)                                    // the previous pass's (read before its pick), for the next
      for (int b = tid; b < kFinBins; b += kSelThreads) f.h[(pass + 1) & 1][b] = 0u;
    __syncthreads();
    uint32_t cnt2[2] = {h[2 * tid], h[2 * tid + 1]};
    wide_pick<kSelThreads, 2>(cnt2, k_rem, 0, f.wsum[pass & 1], f.pick);
    prefix = (prefix << width) | (uint64_t)f.pick[0];
    k_rem -= f.pick[1];
    if (f.pick[2] == 1 || shift == 0) {              // the cut is the single value left in the bin
      for (int e = tid; e < n_ent; e += kSelThreads) {
        const uint64_t v = f.ent[e];
        if ((v >> shift) == prefix) f.cut = v;
      }
      __syncthreads();
      break;
    }
  }
  const uint64_t cut = f.cut;
  // kept entries (value >= cut) in index order -> positions
  const int per = (n_ent + kSelThreads - 1) / kSelThreads;
  const int e0 = tid * per, e1 = min(n_ent, e0 + per);
  int nk = 0;
  for (int e = e0; e < e1; ++e) nk += f.ent[e] >= cut ? 1 : 0;
  int ktot;
  int o = block_exclusive_scan<kSelThreads>(nk, f.scan, &ktot);
  for (int e = e0; e < e1; ++e) {
    const uint64_t v = f.ent[e];
    if (v >= cut && o < k_blk) {                     // o < k_blk always; the bound only guards memory
      const int32_t p0 = (int32_t)(0xFFFFFFFFu - (uint32_t)v) * c;
      int32_t* d = dst + (int64_t)o * c;
      if (c == 1) {
        d[0] = p0;
      } else {
        for (int t = 0; t < c; ++t) d[t] = p0 + t;
      }
      ++o;
    }
  }
}

}  // namespace sa
