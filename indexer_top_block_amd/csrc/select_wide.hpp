// Block selection of one query row held in a workgroup's registers: the radix
// select of the one-workgroup decode kernel (select.hip) and of the fused select +
// attention kernel (select_fwd.hip), for NT threads of KPT keys each.
//
// The indexer keeps the K_blk best blocks of the row (ties to the lower block index,
// where the pages' token-level top-k over expanded block scores cuts as well: members
// of a block tie, the budget is whole blocks), plus the tail; below top_k + c - 1
// visible tokens every block fits and the result is dense (llama.cpp commit "llama:
// QSA sparse attention for qwen4exp").  The list is int32, ascending, -1 padded
// (llama.cpp PR #27970, flash_attn_mask_to_sparse_indices).
//
// Thread t owns blocks j*NT + t (j < KPT), so every load is coalesced.  The K_blk-th
// largest key T is found by radix select over the registers, most significant digit
// first (10, 11, then 11 bits), each pass histogramming the keys that match the
// digits fixed so far; a pass whose chosen bin is taken whole (its count equals the
// number still to take) ends the search early, and the remaining digits do not
// matter.
//
// One compute unit runs the whole row, so the cost is the vector instructions spent
// per key in each pass (about 0.2 us per instruction per key at 32768 keys), and the
// passes are written for few of them:
//   - keys are formed with two integer operations after an add that folds -0 into +0;
//   - the first pass, which counts every key, adds into 32 copies of its histogram
//     laid out [bin][copy] (the address is the digit shifted onto the lane's copy, no
//     other arithmetic), so keys sharing a digit -- scores crowd into a few binades --
//     hit different copies; a 10-bit first digit keeps 32 copies within the LDS that
//     16 copies of an 11-bit digit took, and halves the lanes sharing each copy;
//   - later passes test membership in the running bin with one subtract and compare;
//   - kept blocks (key at or above a threshold) and, when the search ran to the full
//     32 bits, the keys equal to T go to bitmaps of the row with one compare and one
//     wave ballot per register (64 consecutive blocks); every wave then places its
//     bitmap words itself, counting the bits of the words before its own, so the
//     output needs no workgroup-wide prefix sum.  Only the first keys equal to T in
//     index order are taken.
#pragma once

#include <type_traits>

#include "sa_common.hpp"

namespace sa {

struct QueryRowInfo {
  int nb, n_vis;                                     // visible complete blocks, visible positions
};

// Visible complete blocks of query q.
__device__ __forceinline__ QueryRowInfo query_blocks(const int32_t* seq_len, const int32_t* q_seq,
                                                     const int32_t* q_pos, int q, int c) {
  const SeqMeta m = seq_meta(q_seq, seq_len, nullptr, nullptr, q);
  const int n_vis = visible_tokens(m.len, q_pos[q]);
  return QueryRowInfo{n_vis / c, n_vis};
}

constexpr int kWideBins = 2048;                      // passes 2 and 3 (11-bit digits)
constexpr int kP1Bins = 1024;                        // pass 1 (10-bit digit)

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

// Pass-1 histogram copies and bitmap words by row size: rows of fewer than 32768
// keys take 16 copies, so that a 1024-thread workgroup's LDS (< 80 KiB) and registers
// leave room for a second workgroup on the CU (prefill: many rows).
template <int NT, int KPT>
struct WideCfg {
  static_assert(NT % kWave == 0 && kP1Bins % NT == 0 && kWideBins % NT == 0, "thread count");
  static_assert(KPT <= kWave, "one ballot register per lane");
  static constexpr int copies = KPT * NT >= 32768 ? 32 : 16;   // lanes l, l+copies, ... share a copy
  static constexpr int words = KPT * NT / 32;        // bitmap words (32 blocks each)
  static constexpr int waves = NT / kWave;
  static constexpr int wpl = words > NT ? words / NT : 1;       // bitmap words each lane places
  static_assert(wpl == 1 || wpl == 2, "at most two bitmap words per lane");
  static_assert(4 * (waves - 1) * wpl <= kWave, "bits_before reads 16 words per lane");
};

template <int NT, int KPT>
struct alignas(16) WideSmem {
  uint32_t h2[kWideBins];                            // pass 2 (first: its bins' addresses need no base)
  uint32_t h1[kP1Bins * WideCfg<NT, KPT>::copies];  // pass 1 [bin][copy]; pass 3: words 0..2047; a staged list
  uint32_t keep[WideCfg<NT, KPT>::words];            // blocks at or above the threshold
  uint32_t tie[WideCfg<NT, KPT>::words];             // blocks equal to T (full-width search)
  int wsum[2][NT / kWave];                           // per-wave totals, alternating between picks
  int pick[4];
};

// The scoring launch's candidate list (optional): for each tile of kCandTile
// consecutive blocks of a query's row, its keep (kCandKeep or kCandKeep / 2) largest
// keys (ties to the lower block; key 0 in the slots of a tile with fewer blocks) and
// then their block indices.  Every block outside a tile's list scores at most the
// smallest key in it.
constexpr int kCandTile = 32, kCandKeep = 8;
constexpr int kCandThreads = 1024;                   // threads of the workgroup that reads the list

// Word offset in a token's list of word r (keys 0..keep-1, then the indices) of tile
// g's record, for a reader whose thread t holds tiles [tpt t, tpt t + tpt): thread
// t's 16-byte piece q (piece r / 4 of tile tpt t + j, whose record is keep / 2 pieces,
// is q = j keep / 2 + r / 4) sits at q * kCandThreads + t, so that each of the
// reader's loads is one contiguous run across its lanes.
__host__ __device__ __forceinline__ int64_t cand_offset(int g, int r, int keep, int tpt) {
  const int t = g / tpt, q = (g % tpt) * (keep / 2) + r / 4;
  return ((int64_t)q * kCandThreads + t) * 4 + r % 4;
}

// Maximum / minimum over the wave by DPP and permlane exchanges, the same value in
// every lane (lane ^ 1, lane ^ 2, the mirror in 8, lane ^ 8, then the 16- and 32-lane
// swaps: each step combines two halves that already hold their own extremes).  HALF:
// over each 32-lane half only (the 32-lane swap left out).
template <bool MAX, bool HALF = false>
__device__ __forceinline__ uint32_t wave_extreme_u32(uint32_t x) {
  auto f = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  x = f(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false));   // lane ^ 1
  x = f(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, false));   // lane ^ 2
  x = f(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xf, 0xf, false));  // 7 - lane in 8
  x = f(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xf, 0xf, false));  // lane ^ 8 in 16
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = f(a[0], a[1]);
  if constexpr (HALF) return x;
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return f(b[0], b[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) { return wave_extreme_u32<true>(x); }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return wave_extreme_u32<false>(x); }

// Order-preserving 32-bit key of a score: +0 and -0 give the same key, negative
// scores map below positive ones.
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);      // -0 + +0 = +0
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// The bin holding the k-th largest of the counted keys, for a histogram held as PER
// consecutive bins per thread (thread t: bins [t*PER, t*PER + PER)), with `pad` keys
// taken back out of bin 0.  Writes bin, keys in higher bins and keys in the bin to
// pick[0..2] and synchronises.  `wsum` must not be in use by the previous pick.
// Every wave posts its total; each then finds, from the wave totals, the one wave
// whose range holds the k-th key, and only that wave scans its lanes.
template <int NT, int PER>
__device__ __forceinline__ void wide_pick(uint32_t (&cnt)[PER], int k, int pad, int* wsum, int* pick) {
  constexpr int kWaves = NT / kWave;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  if (tid == 0) cnt[0] -= (uint32_t)pad;
  int sum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) sum += (int)cnt[j];
  const int incl = wave_inclusive_scan(sum, lane);
  const int wave_total = __builtin_amdgcn_readlane(incl, kWave - 1);
  if (lane == 0) wsum[wave] = wave_total;
  __syncthreads();
  // lanes 0..kWaves-1: keys in the waves above wave `lane`, and whether the k-th is in it
  const int v = lane < kWaves ? wsum[lane] : 0;
  const int v_incl = wave_inclusive_scan(v, lane);
  const int v_after = __builtin_amdgcn_readlane(v_incl, kWave - 1) - v_incl;
  const uint64_t hit = __ballot(lane < kWaves && v_after < k && v_after + v >= k);
  const int w_hit = (int)__builtin_ctzll(hit | (1ull << 63));   // exactly one wave when 0 < k <= keys
  if (wave == w_hit) {
    int above = __builtin_amdgcn_readlane(v_after, w_hit) + wave_total - incl;   // keys in bins >= (t+1)*PER
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {
      const int gt = above, ge = above + (int)cnt[j];
      if (gt < k && ge >= k) {
        pick[0] = tid * PER + j;
        pick[1] = gt;
        pick[2] = (int)cnt[j];
      }
      above = ge;
    }
  }
  __syncthreads();
}

// Set bits in the bitmap words before word 64 * WPL * wave (lane l reads words
// [16 l, 16 l + 16)); the bitmap holds `words` words.
template <int WPL>
__device__ __forceinline__ int bits_before(const uint32_t* bm, int words, int wave, int lane) {
  int n = 0;
  if (lane < 4 * WPL * wave && lane * 16 < words) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = *(const uint4*)&bm[lane * 16 + i * 4];
      n += __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
    }
  }
  return __builtin_amdgcn_readlane(wave_inclusive_scan(n, lane), kWave - 1);
}

// The compiler's lane write (v_writelane_b32: lane `lane` of `old` replaced by the
// wave-uniform `x`), declared by its intrinsic name so that the compiler, which
// knows its wait-state rules, schedules it.
__device__ int amdgcn_writelane(int x, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// Lane j < N of (lo, hi) receives the wave's ballot of pred(j): the low and the
// high 32 lanes' bits.
template <int N, int J = 0, typename P>
__device__ __forceinline__ void ballot_rows(P pred, uint32_t& lo, uint32_t& hi) {
  if constexpr (J < N) {
    const uint64_t m = __ballot(pred(J));
    lo = (uint32_t)amdgcn_writelane((int)(uint32_t)m, J, (int)lo);
    hi = (uint32_t)amdgcn_writelane((int)(uint32_t)(m >> 32), J, (int)hi);
    ballot_rows<N, J + 1>(pred, lo, hi);
  }
}

// Positions p0 .. p0 + c - 1 of one kept block.
__device__ __forceinline__ void store_block(int32_t* dst, int32_t p0, int c) {
  if (c == 4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) dst[t] = p0 + t;
  } else if (c == 1) {
    dst[0] = p0;
  } else {
    for (int t = 0; t < c; ++t) dst[t] = p0 + t;
  }
}

__device__ __forceinline__ int popcount(uint32_t x) { return __popc(x); }
__device__ __forceinline__ int popcount(uint64_t x) { return __popcll(x); }
__device__ __forceinline__ int lowest_bit(uint32_t x) { return __ffs(x) - 1; }
__device__ __forceinline__ int lowest_bit(uint64_t x) { return __ffsll((unsigned long long)x) - 1; }

// The row's scores into registers, thread t register j holding block j*NT + t, all
// loads issued before the first is used; each index is clamped to the row's last
// readable entry rather than the load guarded (callers mask the entries past the
// row's blocks themselves).  (Buffer loads with a scalar offset per register, which
// spend no vector instruction on addresses, measured 0.3-0.4 us later to the first
// pass at 32768 keys.)
template <int NT, int KPT>
__device__ __forceinline__ void wide_load_row(const float* __restrict__ row, int64_t ld, float (&raw)[KPT]) {
  const int tid = threadIdx.x;
  const int last = (int)min(ld, (int64_t)KPT * NT) - 1;
#pragma unroll
  for (int j = 0; j < KPT; ++j) raw[j] = row[min(j * NT + tid, last)];
}

// The cut of a radix select after its first pass has counted every key (keys in
// registers, KC per thread, key(j) the j-th; each key's top 10 bits added into the
// pass-1 histogram h1 laid out [bin][copy]): the first pick, then the 11-bit passes 2 and 3 among
// the keys still in the running, stopping once a pass's bin is taken whole.  Returns
// the prefix of the k_blk-th largest key at `shift` (the kept keys are those >=
// prefix << shift when whole; else shift is 0, prefix is that key T, and k_rem keys
// equal to T are kept besides those above it).  n_pad keys of 0 are padding.
struct WideCut {
  uint32_t prefix;
  int shift;
  bool whole;
  int k_rem;
};
template <int NT, int KPT, int KC, typename KeyOf>
__device__ __forceinline__ WideCut wide_cut(const KeyOf& key, int k_blk, int n_pad, WideSmem<NT, KPT>& sm) {
  constexpr int COPIES = WideCfg<NT, KPT>::copies;
  constexpr int PER1 = kP1Bins / NT, PER2 = kWideBins / NT;
  const int tid = threadIdx.x;
  __syncthreads();
  {
    // thread t: bins t*PER1 ..; each bin's copies read as quads from a lane-rotated
    // start, so that consecutive lanes spread over the banks
    constexpr int NQD = COPIES / 4;
    uint32_t cnt[PER1];
#pragma unroll
    for (int p = 0; p < PER1; ++p) {
      cnt[p] = 0u;
      const uint4* h = (const uint4*)(sm.h1 + (tid * PER1 + p) * COPIES);
#pragma unroll
      for (int i = 0; i < NQD; ++i) {
        const uint4 v = h[(i + tid) & (NQD - 1)];
        cnt[p] += v.x + v.y + v.z + v.w;
      }
    }
    wide_pick<NT, PER1>(cnt, k_blk, n_pad, sm.wsum[0], sm.pick);
  }
  uint32_t prefix = (uint32_t)sm.pick[0];            // key >> shift of the keys still in the running
  int k_rem = k_blk - sm.pick[1];
  int shift = 22;
  bool whole = sm.pick[2] == k_rem && prefix != 0u;
  // ---- pass 2: next 11 bits among keys in the bin -----------------------------------------
  if (!whole) {
    if constexpr (PER2 == 2) ((uint2*)sm.h1)[tid] = uint2{0u, 0u};   // words 0..2047 serve pass 3
    else if constexpr (PER2 == 4) ((uint4*)sm.h1)[tid] = uint4{0u, 0u, 0u, 0u};
    else
      for (int e = tid; e < kWideBins; e += NT) sm.h1[e] = 0u;
    const uint32_t lo = prefix << 22;
    uint32_t one = 1u;
    asm volatile("" : "+v"(one));                    // one register for every add, not one per key
#pragma unroll
    for (int j = 0; j < KC; ++j)
      if (key(j) - lo < (1u << 22)) atomicAdd(&sm.h2[(key(j) >> 11) & (kWideBins - 1)], one);
    __syncthreads();
    uint32_t cnt[PER2];
#pragma unroll
    for (int p = 0; p < PER2; ++p) cnt[p] = sm.h2[tid * PER2 + p];
    wide_pick<NT, PER2>(cnt, k_rem, prefix == 0u ? n_pad : 0, sm.wsum[1], sm.pick);
    prefix = (prefix << 11) | (uint32_t)sm.pick[0];
    k_rem -= sm.pick[1];
    shift = 11;
    whole = sm.pick[2] == k_rem && prefix != 0u;
    // ---- pass 3: last 11 bits ------------------------------------------------------------
    if (!whole) {
      const uint32_t lo3 = prefix << 11;
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (key(j) - lo3 < (1u << 11)) atomicAdd(&sm.h1[key(j) & 2047u], 1u);
      __syncthreads();
      uint32_t cnt3[PER2];
#pragma unroll
      for (int p = 0; p < PER2; ++p) cnt3[p] = sm.h1[tid * PER2 + p];
      wide_pick<NT, PER2>(cnt3, k_rem, prefix == 0u ? n_pad : 0, sm.wsum[0], sm.pick);
      prefix = (prefix << 11) | (uint32_t)sm.pick[0];
      k_rem -= sm.pick[1];
      shift = 0;
      whole = sm.pick[2] == k_rem && prefix != 0u;
    }
  }
  return WideCut{prefix, shift, whole, k_rem};
}

// The kept blocks' positions, k_blk * c ascending entries, from the workgroup's keep
// and tie bitmaps (bit b of word b / 32: block b): every block in keep, then, when the
// cut fell inside one key value (!whole), the first k_rem blocks of tie in index
// order.  Into the LDS array `list` when it is given (complete and visible to the
// whole workgroup on return), else straight to `out` (global).
template <int NT, int KPT>
__device__ __forceinline__ void wide_list(const WideSmem<NT, KPT>& sm, bool whole, int k_rem, int c, int k_blk,
                                          int32_t* list, int32_t* out) {
  constexpr int WORDS = WideCfg<NT, KPT>::words, WPL = WideCfg<NT, KPT>::wpl;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  // ---- this wave's words -> positions in index order ------------------------------------------
  // Lane word w (WPL bitmap words, 32*WPL blocks) of this lane: w = 64 * wave + lane.
  typedef typename std::conditional<WPL == 2, uint64_t, uint32_t>::type Word;
  constexpr int LW = WORDS / WPL, BPW = 32 * WPL;
  const int w = wave * kWave + lane;
  Word word = w < LW ? ((const Word*)sm.keep)[w] : Word(0);
  int o = bits_before<WPL>(sm.keep, WORDS, wave, lane);
  if (!whole) {                                      // the first k_rem tied blocks in index order
    Word t = w < LW ? ((const Word*)sm.tie)[w] : Word(0);
    const int t_before = bits_before<WPL>(sm.tie, WORDS, wave, lane);
    o += min(k_rem, t_before);
    int take = k_rem - t_before - (wave_inclusive_scan(popcount(t), lane) - popcount(t));
    while (t != Word(0) && take > 0) {
      const Word low = t & (Word(0) - t);
      word |= low;
      t ^= low;
      --take;
    }
  }
  o += wave_inclusive_scan(popcount(word), lane) - popcount(word);
  if (list) {
    // the list is assembled in LDS and written out coalesced by the caller, rather
    // than as scattered stores of a few lanes each
    if (c == 4) {
      while (word != Word(0) && o < k_blk) {         // o < k_blk always; the bound only guards memory
        const int32_t p0 = (w * BPW + lowest_bit(word)) * 4;
        word &= word - Word(1);
        *(int4*)&list[o * 4] = int4{p0, p0 + 1, p0 + 2, p0 + 3};
        ++o;
      }
    } else if (c == 1) {
      while (word != Word(0) && o < k_blk) {
        list[o++] = w * BPW + lowest_bit(word);
        word &= word - Word(1);
      }
    } else {
      while (word != Word(0) && o < k_blk) {
        const int32_t p0 = (w * BPW + lowest_bit(word)) * c;
        word &= word - Word(1);
        for (int t = 0; t < c; ++t) list[o * c + t] = p0 + t;
        ++o;
      }
    }
    __syncthreads();
  } else {
    while (word != Word(0) && o < k_blk) {           // o < k_blk always; the bound only guards memory
      const int b = lowest_bit(word);
      word &= word - Word(1);
      store_block(out + (int64_t)o * c, (w * BPW + b) * c, c);
      ++o;
    }
  }
}

// The K_blk kept blocks of a row of nb > k_blk complete blocks whose scores the
// threads hold in raw[] (thread t, register j: block j*NT + t; entries past nb are
// ignored), as k_blk*c ascending positions: into the LDS array `list` when it is
// given, else straight to `out` (global).  The histograms h1 and h2 must be zero on
// entry.  Ends with the list complete and visible to the whole workgroup.
template <int NT, int KPT>
__device__ __forceinline__ void wide_select_rows(const float (&raw)[KPT], int nb_vis, int c, int k_blk,
                                                 WideSmem<NT, KPT>& sm, int32_t* list, int32_t* out) {
  constexpr int COPIES = WideCfg<NT, KPT>::copies;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int nb = min(nb_vis, KPT * NT);              // the launch guarantees nb_vis fits; the bitmap relies on it
  const int n_pad = KPT * NT - nb;

  // ---- pass 1: the top 10 bits, each key counted as it arrives ---------------------------
  // Keys past the row's end become 0 -- below every key a score can have except
  // negative NaNs -- so the passes need no bounds checks: the picks take the n_pad
  // padding keys back out of bin 0, and a prefix of 0 (the only one they can match)
  // never takes its bin whole, so they are never kept.
  uint32_t key[KPT];
  {
    uint32_t* mine = sm.h1 + (lane & (COPIES - 1));
    if (n_pad == 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        key[j] = score_key(raw[j]);
        atomicAdd(&mine[(key[j] >> 22) * COPIES], 1u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        key[j] = j * NT + tid < nb ? score_key(raw[j]) : 0u;
        atomicAdd(&mine[(key[j] >> 22) * COPIES], 1u);
      }
    }
  }
  const WideCut cut = wide_cut<NT, KPT, KPT>([&](int j) { return key[j]; }, k_blk, n_pad, sm);
  const uint32_t prefix = cut.prefix;
  const int shift = cut.shift, k_rem = cut.k_rem;
  const bool whole = cut.whole;
  // ---- kept blocks -> bitmaps -----------------------------------------------------------
  // Kept for sure: key >> shift above the prefix, or equal to it when its bin is
  // taken whole, i.e. key >= thr.  A search that did not end whole ran to the full
  // width (shift 0): keys above T are kept, keys equal to T are ties.  Padding keys
  // are 0: below every threshold of a prefix other than 0, which is never whole.
  // Register j of the wave's lanes holds blocks j*NT + 64*wave + [0, 64): bitmap
  // words j*NT/32 + 2 wave + {0, 1}, collected in lane j.
  {
    uint32_t k_lo = 0u, k_hi = 0u, t_lo = 0u, t_hi = 0u;
    if (whole || prefix != 0xffffffffu) {
      const uint32_t thr = whole ? prefix << shift : prefix + 1u;
      ballot_rows<KPT>([&](int j) { return key[j] >= thr; }, k_lo, k_hi);
    }
    if (!whole) ballot_rows<KPT>([&](int j) { return key[j] == prefix; }, t_lo, t_hi);
    if (lane < KPT) {
      *(uint2*)&sm.keep[lane * (NT / 32) + wave * 2] = uint2{k_lo, k_hi};
      *(uint2*)&sm.tie[lane * (NT / 32) + wave * 2] = uint2{t_lo, t_hi};
    }
  }
  __syncthreads();
  wide_list<NT, KPT>(sm, whole, k_rem, c, k_blk, list, out);
}

}  // namespace sa
