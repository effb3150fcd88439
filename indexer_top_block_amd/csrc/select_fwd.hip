// Block selection and attention in one launch (sparse_attn_select_fwd).
//
// The decode chain is a row of dependent launches (score -> select -> attention ->
// combine), each of which costs a launch and at least one memory round trip before
// its work starts.  When every (query token, KV head, split) workgroup of the
// attention has a compute unit to itself, the select can ride along: each
// workgroup runs its query's selection with 16 waves, keeps the list in LDS, and then
// attends over its own split's rows with 4 of them (fwd_lds.hpp) -- every workgroup
// of a query computes the same list.  That removes the select's launch (or, for rows
// too long for one workgroup, the chunked selection's finishing launch) and the list's
// trip through memory; the split partials are merged by the usual combine launch.  A
// 1024-thread workgroup leaves 128 registers per lane, so the attention reads its
// query operand from LDS at every Q.K^T step instead of holding it in registers.
//
// Two forms:
//   rows of up to 32768 blocks: the one-workgroup radix select over the row in
//     registers (select_wide.hpp);
//   longer rows of few query tokens: the chunked selection's histogram and candidate
//     launches run first, and the finishing pass (select_chunk.hpp) runs in every
//     attention workgroup; the attention's partials go after the candidates in the
//     workspace.
//
// Workgroup (split 0, KV head 0) of each query also writes the list, the padding and
// the count (and returns the chunked selection's histogram to zero), so the call
// leaves exactly what sparse_attn_select followed by sparse_attn_fwd leaves, bit for
// bit (the same select, the same split plan, the same attention arithmetic).  Calls
// that do not fit (more workgroups than compute units, shapes other than the MLA ones
// with V inside K, lists longer than kFusedListMax, more chunks than the finishing
// pass reads at once) take those two calls instead.
//
// With the scoring launch's candidate list (sparse_attn_pool_score_select_fwd: the
// best 8 -- or 4 -- of every 32 blocks), the select starts from the list instead of
// the row: select_fwd_kernel's list form for rows of up to 32768 blocks, and
// list_fwd_kernel for rows of up to 262144, where it replaces the chunked selection.
// The list's cut is the row's exactly when no block it leaves out reaches the cut
// (cand_select); otherwise the workgroup selects over the row, with the same result.
#include <cmath>

#include "fwd_lds.hpp"
#include "select_chunk.hpp"
#include "select_wide.hpp"

namespace sa {

constexpr int kFusedThreads = 1024;          // 16 waves select; waves 0..3 then attend
constexpr int kFusedMaxKpt = 32;             // keys per thread: rows of up to 32768 blocks
constexpr int kFusedListMax = 3072;          // list entries held in LDS (top_k + c - 1)
constexpr int kFusedMaxChunks = kSelThreads / 4;   // chunks whose counts the finishing pass reads at once
constexpr int kCandMaxQueries = 63;         // query tokens of the pooling scoring launch
constexpr long long kCandMaxTiles = 8192;   // listed tiles of all tokens of a call
static_assert(kSelThreads == kFusedThreads, "the finishing pass runs on the fused workgroup");
static_assert(kCandThreads == kFusedThreads, "the list is laid out for the fused workgroup's loads");

// The list the workgroup selected, in LDS: cnt entries (kept blocks, then the tail),
// read clamped so that every lane reads valid memory.
struct LdsList {
  const int32_t* lds;
  int cnt;
  SeqMeta sm;                                        // read at the start, while the select ran
  __device__ __forceinline__ int at(int j) const { return cnt > 0 ? lds[min(j, cnt - 1)] : -1; }
  __device__ __forceinline__ float bias(int) const { return 0.f; }
  __device__ __forceinline__ bool has_bias() const { return false; }
  __device__ __forceinline__ int count() const { return cnt; }
  __device__ __forceinline__ SeqMeta meta(const int32_t*, const int32_t*, const int64_t*, int) const { return sm; }
};

// The select's LDS and the attention's LDS share the same bytes: the select is done
// (and its list copied out of them) before the attention's first gather lands.
template <typename T, int DKQ, int KPT>
union FusedSmem {
  WideSmem<kFusedThreads, KPT> sel;
  FwdLdsSmem<T, DKQ, true> att;
};

// The kept blocks' positions into the LDS list from each thread's tile words (bit b of
// kw[j] / tw[j]: block b of the thread's tile j kept / tied) and their counts: every
// kept block and the first k_rem tied blocks in index order, placed from the counts of
// the threads before (wave scans, then the wave totals in h2, which the picks no
// longer use).  Ends with the list complete and visible to the workgroup -- except
// for the tiles of skip (bit j: tile j): for each of those, in tile order, the first
// list entry its blocks take and the tied blocks it still takes at most go to at[0],
// at[1], then at += 2, and the caller places its blocks.
template <int NT, int KPT, int TPT>
__device__ __forceinline__ void place_words(const uint32_t (&kw)[TPT], const uint32_t (&tw)[TPT], int kc, int tc,
                                            int k_rem, int c, int k_blk, WideSmem<NT, KPT>& sm, int32_t* list,
                                            uint32_t skip = 0u, uint32_t* at = nullptr) {
  constexpr int WAVES = NT / kWave;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int k_incl = wave_inclusive_scan(kc, lane), t_incl = wave_inclusive_scan(tc, lane);
  if (lane == kWave - 1) {
    sm.h2[wave] = (uint32_t)k_incl;
    sm.h2[WAVES + wave] = (uint32_t)t_incl;
  }
  lds_barrier();
  const int wk = lane < WAVES ? (int)sm.h2[lane] : 0, wt = lane < WAVES ? (int)sm.h2[WAVES + lane] : 0;
  const int wk_incl = wave_inclusive_scan(wk, lane), wt_incl = wave_inclusive_scan(wt, lane);
  const int k_before = (wave > 0 ? __builtin_amdgcn_readlane(wk_incl, wave - 1) : 0) + k_incl - kc;
  const int t_before = (wave > 0 ? __builtin_amdgcn_readlane(wt_incl, wave - 1) : 0) + t_incl - tc;
  int o = k_before + min(k_rem, t_before);
  int want = k_rem - t_before;                       // tied blocks still wanted at this thread's first tile
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    uint32_t word = kw[j], t = tw[j];
    if (skip & (1u << j)) {
      const int take = min(max(want, 0), __popc(t));
      at[0] = (uint32_t)o;
      at[1] = (uint32_t)max(want, 0);
      at += 2;
      o += __popc(word) + take;
      want -= take;
      continue;
    }
    for (; want > 0 && t != 0u; --want) {            // the first tied blocks still wanted, in index order
      word |= t & (0u - t);
      t &= t - 1u;
    }
    const int32_t b0 = (tid * TPT + j) * kCandTile;
    if (c == 4) {
      while (word != 0u && o < k_blk) {              // o < k_blk always; the bound only guards memory
        const int32_t p0 = (b0 + __ffs(word) - 1) * 4;
        word &= word - 1u;
        *(int4*)&list[o * 4] = int4{p0, p0 + 1, p0 + 2, p0 + 3};
        ++o;
      }
    } else if (c == 1) {
      while (word != 0u && o < k_blk) {
        list[o++] = b0 + __ffs(word) - 1;
        word &= word - 1u;
      }
    } else {
      while (word != 0u && o < k_blk) {
        const int32_t p0 = (b0 + __ffs(word) - 1) * c;
        word &= word - 1u;
        for (int u = 0; u < c; ++u) list[o * c + u] = p0 + u;
        ++o;
      }
    }
  }
  __syncthreads();
}

// The select from the scoring launch's candidate list: thread t holds tiles
// [TPT t, TPT t + TPT), each tile's KEEP largest keys and their block indices (keys 0
// past the row), counts the keys into the pass-1 histogram and runs the passes over
// them.  The result is the row's select exactly when every block left out of the list
// falls below the cut: below the cut's bin when the bin is taken whole, below the cut
// key T otherwise (a block equal to T, left out, could be a tie the row's select
// takes).  Each tile's smallest listed key bounds those it left out, so the largest
// of those bounds is compared with the cut (false: the caller selects over the row).
// The kept blocks of a tile are then its own candidates: each thread places its
// tiles' kept blocks in the list from the counts of the tiles before it (kept blocks,
// and the first k_rem tied blocks in index order).  Requires nb > k_blk and at least
// k_blk listed blocks; the histograms are clear on entry and dirty on return.  On
// failure failed_bound is the cut the list reached (the keys of cv are then those the
// cut counted: 0 past the row).
template <int NT, int KPT, int KEEP, int TPT>
__device__ __forceinline__ bool cand_select(uint4 (&cv)[KEEP * TPT / 2], int nb, int c, int k_blk,
                                            WideSmem<NT, KPT>& sm, int32_t* list, uint32_t& failed_bound) {
  constexpr int COPIES = WideCfg<NT, KPT>::copies, WAVES = NT / kWave, KC = KEEP * TPT;
  static_assert(KEEP % 4 == 0 && WideCfg<NT, KPT>::words >= WAVES && kWideBins >= 2 * WAVES,
                "tile records in 16-byte pieces; LDS words reused for the wave totals");
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  nb = min(nb, NT * TPT * kCandTile);                // the launch guarantees nb fits; the list relies on it
  // tile j: KEEP keys, then KEEP block indices; the keys of tiles past the row become
  // 0 in place (no second copy of 32 keys in registers)
  uint32_t* w = reinterpret_cast<uint32_t*>(cv);
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    const bool in_row = (tid * TPT + j) * kCandTile < nb;
#pragma unroll
    for (int e = 0; e < KEEP; ++e) w[j * 2 * KEEP + e] = in_row ? w[j * 2 * KEEP + e] : 0u;
  }
  auto key = [&](int j) -> uint32_t { return w[(j / KEEP) * 2 * KEEP + j % KEEP]; };
  // blocks listed: KEEP per whole tile, all of a last tile shorter than that
  const int n_listed = nb / kCandTile * KEEP + min(KEEP, nb % kCandTile);
  {
    uint32_t* mine = sm.h1 + (lane & (COPIES - 1));
#pragma unroll
    for (int j = 0; j < KC; ++j) atomicAdd(&mine[(key(j) >> 22) * COPIES], 1u);
  }
  // the bound on the keys left out (each tile's smallest listed key, the largest of
  // them): per wave into keep[wave] (free until the list), ordered before its reads by
  // the picks' barriers
  uint32_t bound_out = 0u;
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    uint32_t least = key(j * KEEP);
#pragma unroll
    for (int e = 1; e < KEEP; ++e) least = min(least, key(j * KEEP + e));
    bound_out = max(bound_out, least);
  }
  bound_out = wave_max_u32(bound_out);
  if (lane == 0) sm.keep[wave] = bound_out;
  const WideCut cut = wide_cut<NT, KPT, KC>(key, k_blk, NT * KC - n_listed, sm);
  const uint32_t bound = cut.whole ? cut.prefix << cut.shift : cut.prefix;
  uint32_t left_out = 0u;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) left_out = max(left_out, sm.keep[v]);
  if (left_out >= bound) {                           // (bound 0: never taken)
    failed_bound = bound;
    return false;
  }
  // keep: key >= thr (thr > 0: bound > 0 here); tie: key == T (the cut inside a key)
  const uint32_t thr = cut.whole ? bound : bound + 1u;
  const bool full = !cut.whole && bound == 0xffffffffu;   // nothing above T
  uint32_t kw[TPT], tw[TPT];
  int kc = 0, tc = 0;
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    kw[j] = 0u;
    tw[j] = 0u;
#pragma unroll
    for (int e = 0; e < KEEP; ++e) {
      const uint32_t k = key(j * KEEP + e), bit = 1u << (w[j * 2 * KEEP + KEEP + e] % kCandTile);
      kw[j] |= (!full && k >= thr) ? bit : 0u;
      if (!cut.whole) tw[j] |= k == bound ? bit : 0u;
    }
    kc += __popc(kw[j]);
    tc += __popc(tw[j]);
  }
  place_words<NT, KPT, TPT>(kw, tw, kc, tc, cut.k_rem, c, k_blk, sm, list);
  return true;
}

// The list could not decide: some tiles' smallest listed key reached the cut bound0,
// so a block such a tile left out might be kept.  Those tiles (at most 32) are read
// whole from the row, one block per thread of 32 consecutive threads each, in place of
// their listed keys, and the cut is taken again over them and the other tiles' listed
// keys (9 keys per thread at most): adding keys only raises it, so the other tiles'
// left-out blocks stay below it -- unless the new cut's whole bin starts at or below one
// of their smallest listed keys, which is checked again (false: the caller selects over
// the row).  The kept and tied blocks then go to the keep and tie bitmaps and the list
// is made from them in index order (wide_list).  For the one-tile-per-thread list (rows
// of up to 32768 blocks); cv as cand_select left it.
template <int NT, int KPT>
__device__ __forceinline__ bool cand_complete(const uint4 (&cv)[kCandKeep / 2], const float* __restrict__ row, int nb,
                                              int c, int k_blk, uint32_t bound0, WideSmem<NT, KPT>& sm,
                                              int32_t* list) {
  constexpr int COPIES = WideCfg<NT, KPT>::copies, WAVES = NT / kWave, MAX_OVER = NT / kCandTile;
  static_assert(WideCfg<NT, KPT>::words >= 2 * WAVES + MAX_OVER, "LDS words reused for counts and tile numbers");
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  nb = min(nb, KPT * NT);                            // the launch guarantees nb fits; the bitmaps rely on it
  const uint32_t* w = reinterpret_cast<const uint32_t*>(cv);
  uint32_t least = w[0];
#pragma unroll
  for (int e = 1; e < kCandKeep; ++e) least = min(least, w[e]);
  const bool over = tid * kCandTile < nb && least >= bound0;   // this thread's tile is read whole
  // the tiles read whole, numbered in tile order: per-wave counts, then their offsets
  const uint64_t ob = __ballot(over);
  __syncthreads();                                   // the first cut's LDS reads are done
  if (lane == 0) sm.tie[wave] = (uint32_t)__popcll(ob);
  __syncthreads();
  int n_over = 0, before = 0;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) {
    const int n = (int)sm.tie[v];
    before += v < wave ? n : 0;
    n_over += n;
  }
  if (n_over > MAX_OVER) return false;               // (uniform) too many: the row's select
  if (over) sm.tie[2 * WAVES + before + __popcll(ob & ((1ull << lane) - 1ull))] = (uint32_t)tid;
  for (int e = tid; e < kP1Bins * COPIES / 4; e += NT) ((uint4*)sm.h1)[e] = uint4{0u, 0u, 0u, 0u};
  for (int e = tid; e < kWideBins; e += NT) sm.h2[e] = 0u;
  const uint32_t bound_out = wave_max_u32(over ? 0u : least);        // completed tiles leave nothing out
  if (lane == 0) sm.keep[wave] = bound_out;
  __syncthreads();
  // keys: this tile's listed 8 (none when it is read whole), and block tid % 32 of the
  // (tid / 32)-th tile read whole
  uint32_t key[kCandKeep + 1];
#pragma unroll
  for (int e = 0; e < kCandKeep; ++e) key[e] = over ? 0u : w[e];
  const int xo = tid / kCandTile;
  const int xtile = xo < n_over ? (int)sm.tie[2 * WAVES + xo] : -1;
  const int xb = xtile * kCandTile + tid % kCandTile;
  key[kCandKeep] = (xtile >= 0 && xb < nb) ? score_key(row[xtile >= 0 ? min(xb, nb - 1) : 0]) : 0u;
  int zeros = 0;                                     // padding: key 0 (no score has it)
#pragma unroll
  for (int e = 0; e <= kCandKeep; ++e) zeros += key[e] == 0u ? 1 : 0;
  {
    uint32_t* mine = sm.h1 + (lane & (COPIES - 1));
#pragma unroll
    for (int e = 0; e <= kCandKeep; ++e) atomicAdd(&mine[(key[e] >> 22) * COPIES], 1u);
  }
  const int z_incl = wave_inclusive_scan(zeros, lane);
  if (lane == kWave - 1) sm.tie[WAVES + wave] = (uint32_t)z_incl;
  __syncthreads();
  int n_pad = 0;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) n_pad += (int)sm.tie[WAVES + v];
  const WideCut cut = wide_cut<NT, KPT, kCandKeep + 1>([&](int e) { return key[e]; }, k_blk, n_pad, sm);
  const uint32_t bound = cut.whole ? cut.prefix << cut.shift : cut.prefix;
  uint32_t left_out = 0u;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) left_out = max(left_out, sm.keep[v]);
  if (left_out >= bound) return false;
  // kept and tied blocks into the bitmaps (bit b % 32 of word b / 32)
  const uint32_t thr = cut.whole ? bound : bound + 1u;
  const bool full = !cut.whole && bound == 0xffffffffu;
  __syncthreads();                                   // every wave has read keep[]
  for (int e = tid; e < WideCfg<NT, KPT>::words; e += NT) {
    sm.keep[e] = 0u;
    sm.tie[e] = 0u;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e <= kCandKeep; ++e) {
    const int b = e < kCandKeep ? tid * kCandTile + (int)(w[kCandKeep + e] % kCandTile) : xb;
    if (key[e] != 0u && !full && key[e] >= thr) atomicOr(&sm.keep[b / kCandTile], 1u << (b % kCandTile));
    if (key[e] != 0u && !cut.whole && key[e] == bound) atomicOr(&sm.tie[b / kCandTile], 1u << (b % kCandTile));
  }
  __syncthreads();
  wide_list<NT, KPT>(sm, cut.whole, cut.k_rem, c, k_blk, list, nullptr);
  return true;
}

// cand_complete for the lists of rows longer than one workgroup's registers hold
// (TPT tiles per thread): the crowded tiles (at most 32 * XPT) are read whole, XPT
// blocks per thread, and the cut taken again over them and the other tiles' listed
// keys, with the same check.  A crowded tile's kept and tied blocks are collected
// into LDS words by the threads that read its blocks; its own thread counts them in
// index order with its other tiles (place_words) and leaves their first list entry,
// from which the threads that read them place them.  src: this thread's first list
// piece, as the launch loaded it; the list is read again here (the keys first, the
// block indices after the cut) rather than held in registers through the common path.
template <int NT, int KPT, int KEEP, int TPT, int XPT>
__device__ __forceinline__ bool cand_complete_tiles(const uint4* __restrict__ src, const float* __restrict__ row,
                                                    int nb, int c, int k_blk, uint32_t bound0, WideSmem<NT, KPT>& sm,
                                                    int32_t* list) {
  constexpr int COPIES = WideCfg<NT, KPT>::copies, WAVES = NT / kWave, KC = KEEP * TPT, KP = KEEP / 4;
  constexpr int MAX_OVER = NT * XPT / kCandTile;
  // keep[] words: [0, WAVES) bounds, [WAVES, 2 WAVES) crowded tiles per wave, then the
  // crowded tiles' numbers, their kept words, their tied words and their (first list
  // entry, tied blocks wanted) pairs; tie[]: zero counts
  constexpr int OT = 2 * WAVES, OK = OT + MAX_OVER, OTW = OK + MAX_OVER, OP = OTW + MAX_OVER;
  static_assert(WideCfg<NT, KPT>::words >= OP + 2 * MAX_OVER, "LDS words for the crowded tiles");
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  nb = min(nb, NT * TPT * kCandTile);
  // the addresses are formed anew (an empty asm hides src's origin), so the common
  // path keeps none of its own load addresses live for this one
  asm volatile("" : "+v"(src));
  uint4 kv[TPT * KP];                                // tile j's keys: pieces j * 2 KP .. + KP of the record
#pragma unroll
  for (int j = 0; j < TPT; ++j)
#pragma unroll
    for (int p = 0; p < KP; ++p) kv[j * KP + p] = src[(j * 2 * KP + p) * kCandThreads];
  uint32_t* w = reinterpret_cast<uint32_t*>(kv);     // key e of tile j: w[j * KEEP + e]
#pragma unroll
  for (int j = 0; j < TPT; ++j)                      // tiles past the row list nothing
#pragma unroll
    for (int e = 0; e < KEEP; ++e) w[j * KEEP + e] = (tid * TPT + j) * kCandTile < nb ? w[j * KEEP + e] : 0u;
  uint32_t ov = 0u;                                  // bit j: this thread's tile j is read whole
  uint32_t bmax = 0u;                                // the largest smallest-key of the others
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    uint32_t x = w[j * KEEP];
#pragma unroll
    for (int e = 1; e < KEEP; ++e) x = min(x, w[j * KEEP + e]);
    const bool o = (tid * TPT + j) * kCandTile < nb && x >= bound0;
    ov |= o ? 1u << j : 0u;
    bmax = max(bmax, o ? 0u : x);
  }
  const int n_mine = __popc(ov);
  const int incl = wave_inclusive_scan(n_mine, lane);
  bmax = wave_max_u32(bmax);
  __syncthreads();                                   // the first cut's LDS reads are done
  if (lane == kWave - 1) sm.keep[WAVES + wave] = (uint32_t)incl;
  if (lane == 0) sm.keep[wave] = bmax;
  __syncthreads();
  int n_over = 0, first = incl - n_mine;             // this thread's first crowded tile's rank
#pragma unroll
  for (int v = 0; v < WAVES; ++v) {
    const int n = (int)sm.keep[WAVES + v];
    first += v < wave ? n : 0;
    n_over += n;
  }
  if (n_over > MAX_OVER) return false;               // (uniform) too many: the row's select
  {
    int r = first;
#pragma unroll
    for (int j = 0; j < TPT; ++j)
      if (ov & (1u << j)) sm.keep[OT + r++] = (uint32_t)(tid * TPT + j);
  }
  for (int e = tid; e < kP1Bins * COPIES / 4; e += NT) ((uint4*)sm.h1)[e] = uint4{0u, 0u, 0u, 0u};
  for (int e = tid; e < kWideBins; e += NT) sm.h2[e] = 0u;
  for (int e = tid; e < 2 * MAX_OVER; e += NT) sm.keep[OK + e] = 0u;
  // the crowded tiles' listed keys leave the count (their blocks come whole below)
#pragma unroll
  for (int j = 0; j < TPT; ++j)
#pragma unroll
    for (int e = 0; e < KEEP; ++e) w[j * KEEP + e] = (ov & (1u << j)) ? 0u : w[j * KEEP + e];
  __syncthreads();
  // extra keys: slot x * NT + tid is block slot % 32 of the (slot / 32)-th crowded tile
  uint32_t xkey[XPT];
#pragma unroll
  for (int x = 0; x < XPT; ++x) {
    const int slot = x * NT + tid, k = slot / kCandTile;
    const int xtile = k < n_over ? (int)sm.keep[OT + k] : -1;
    const int b = xtile * kCandTile + slot % kCandTile;
    const bool ok = xtile >= 0 && b < nb;
    const uint32_t rk = score_key(row[ok ? b : 0]);
    xkey[x] = ok ? rk : 0u;
  }
  auto key = [&](int j) -> uint32_t { return j < KC ? w[j] : xkey[j - KC]; };
  int zeros = 0;                                     // padding: key 0 (no score has it)
#pragma unroll
  for (int j = 0; j < KC + XPT; ++j) zeros += key(j) == 0u ? 1 : 0;
  {
    uint32_t* mine = sm.h1 + (lane & (COPIES - 1));
#pragma unroll
    for (int j = 0; j < KC + XPT; ++j) atomicAdd(&mine[(key(j) >> 22) * COPIES], 1u);
  }
  const int z_incl = wave_inclusive_scan(zeros, lane);
  if (lane == kWave - 1) sm.tie[wave] = (uint32_t)z_incl;
  __syncthreads();
  int n_pad = 0;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) n_pad += (int)sm.tie[v];
  const WideCut cut = wide_cut<NT, KPT, KC + XPT>(key, k_blk, n_pad, sm);
  const uint32_t bound = cut.whole ? cut.prefix << cut.shift : cut.prefix;
  uint32_t left_out = 0u;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) left_out = max(left_out, sm.keep[v]);
  if (left_out >= bound) return false;
  const uint32_t thr = cut.whole ? bound : bound + 1u;
  const bool full = !cut.whole && bound == 0xffffffffu;
  // the other tiles' block indices (their keys' order)
  uint4 iv[TPT * KP];
#pragma unroll
  for (int j = 0; j < TPT; ++j)
#pragma unroll
    for (int p = 0; p < KP; ++p) iv[j * KP + p] = src[(j * 2 * KP + KP + p) * kCandThreads];
  const uint32_t* wi = reinterpret_cast<const uint32_t*>(iv);
  // the crowded tiles' kept and tied blocks, collected by the threads that read them
#pragma unroll
  for (int x = 0; x < XPT; ++x) {
    if (xkey[x] == 0u) continue;
    const int slot = x * NT + tid, k = slot / kCandTile;
    const uint32_t bit = 1u << (slot % kCandTile);
    if (!full && xkey[x] >= thr) atomicOr(&sm.keep[OK + k], bit);
    if (!cut.whole && xkey[x] == bound) atomicOr(&sm.keep[OTW + k], bit);
  }
  __syncthreads();
  uint32_t kw[TPT], tw[TPT];
  int kc = 0, tc = 0, r = first;
#pragma unroll
  for (int j = 0; j < TPT; ++j) {
    kw[j] = 0u;
    tw[j] = 0u;
    if (ov & (1u << j)) {
      kw[j] = sm.keep[OK + r];
      tw[j] = sm.keep[OTW + r];
      ++r;
    } else {
#pragma unroll
      for (int e = 0; e < KEEP; ++e) {
        const uint32_t k = w[j * KEEP + e], bit = 1u << (wi[j * KEEP + e] % kCandTile);
        kw[j] |= (!full && k >= thr) ? bit : 0u;
        if (!cut.whole) tw[j] |= k == bound ? bit : 0u;
      }
    }
    kc += __popc(kw[j]);
    tc += __popc(tw[j]);
  }
  place_words<NT, KPT, TPT>(kw, tw, kc, tc, cut.k_rem, c, k_blk, sm, list, ov, &sm.keep[OP + 2 * first]);
  // the crowded tiles' blocks, each placed by the thread that read it: after the kept
  // and taken tied blocks before it in its tile
#pragma unroll
  for (int x = 0; x < XPT; ++x) {
    const int slot = x * NT + tid, k = slot / kCandTile;
    if (xkey[x] == 0u) continue;
    const uint32_t below = (1u << (slot % kCandTile)) - 1u, bit = below + 1u;
    const uint32_t kwt = sm.keep[OK + k], twt = sm.keep[OTW + k];
    const int want = (int)sm.keep[OP + 2 * k + 1], tb = __popc(twt & below);
    const int o = (int)sm.keep[OP + 2 * k] + __popc(kwt & below) + min(want, tb);
    if (((kwt & bit) != 0u || ((twt & bit) != 0u && tb < want)) && o < k_blk) {
      const int32_t p0 = ((int)sm.keep[OT + k] * kCandTile + slot % kCandTile) * c;
      for (int u = 0; u < c; ++u) list[o * c + u] = p0 + u;
    }
  }
  __syncthreads();
  return true;
}

// CAND: the select starts from the scoring launch's candidate list (cand, cand_ld
// words per query token) for rows of at least cand_min_groups whole groups, and takes
// the row when the list cannot decide it; decided[i] records which (1: the list).
// Otherwise cand, cand_min_groups and decided are unused.
template <typename T, int DKQ, int KPT, bool CAND>
__global__ void __launch_bounds__(kFusedThreads, 1)
select_fwd_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
                  const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk,
                  int32_t* __restrict__ sel, int64_t sel_ld, int32_t* __restrict__ n_sel, const T* __restrict__ q,
                  const T* __restrict__ k, int64_t k_ld, int64_t k_hs, const int64_t* __restrict__ seq_row0, int h_q,
                  int h_kv, float scale_log2, int n_split, int rows_per_split, float* __restrict__ out,
                  float* __restrict__ ws_o, float* __restrict__ ws_ml, const uint32_t* __restrict__ cand,
                  int64_t cand_ld, int cand_min_groups, uint32_t* __restrict__ decided) {
  constexpr int NT = kFusedThreads, COPIES = WideCfg<NT, KPT>::copies;
  __shared__ FusedSmem<T, DKQ, KPT> sm;
  __shared__ int32_t list[kFusedListMax];
  const int i = blockIdx.y / h_kv, tid = threadIdx.x;
  const bool writer = blockIdx.x == 0 && blockIdx.y % h_kv == 0;   // writes sel and n_sel of query i
  const float* row = scores + (int64_t)i * scores_ld;
  // the whole row, loaded up front (indices below scores_ld are valid memory); with
  // the candidate list, this thread's tile of it instead (clamped to the last tile)
  float raw[KPT];
  uint4 cv[4];
  if constexpr (CAND) {                              // coalesced: piece q of thread t at q * kCandThreads + t
    const uint4* src = (const uint4*)(cand + (int64_t)i * cand_ld) + tid;
#pragma unroll
    for (int q = 0; q < 4; ++q) cv[q] = src[q * kCandThreads];
  } else {
    wide_load_row<NT, KPT>(row, scores_ld, raw);
  }
  // the query's sequence (its cache rows too, for the attention) and visible blocks
  const SeqMeta meta = seq_meta(q_seq, seq_len, seq_row0, nullptr, i);
  const int n_vis = visible_tokens(meta.len, q_pos[i]);
  const QueryRowInfo qr{n_vis / c, n_vis};
  for (int e = tid; e < kP1Bins * COPIES / 4; e += NT) ((uint4*)sm.sel.h1)[e] = uint4{0u, 0u, 0u, 0u};
  for (int e = tid; e < kWideBins; e += NT) sm.sel.h2[e] = 0u;
  __builtin_amdgcn_sched_barrier(0);                 // every load in flight before the first is used
  int32_t* gsel = sel + (int64_t)i * sel_ld;
  int cnt;
  if (qr.nb <= k_blk) {                              // dense: every visible position
    cnt = qr.n_vis;
    for (int j = tid; j < cnt; j += NT) list[j] = j;
    if (writer) write_dense<NT>(gsel, sel_ld, qr.n_vis, n_sel + i);
    if (CAND && writer && tid == 0) decided[i] = 0u;
  } else {
    __syncthreads();                                 // the histograms are clear
    bool done = false;
    if constexpr (CAND) {
      // only rows of enough groups for the list to be likely to decide (cand_min_groups)
      uint32_t failed = 0u;
      if (qr.nb / kCandTile >= cand_min_groups)
        done = cand_select<NT, KPT, kCandKeep, 1>(cv, qr.nb, c, k_blk, sm.sel, list, failed);
      // a few tiles held more of the kept blocks than they list: read them whole
      if (!done && failed != 0u) done = cand_complete<NT, KPT>(cv, row, qr.nb, c, k_blk, failed, sm.sel, list);
      if (!done) {                                   // the row's select: fresh histograms, the row's keys
        __syncthreads();
        for (int e = tid; e < kP1Bins * COPIES / 4; e += NT) ((uint4*)sm.sel.h1)[e] = uint4{0u, 0u, 0u, 0u};
        for (int e = tid; e < kWideBins; e += NT) sm.sel.h2[e] = 0u;
        wide_load_row<NT, KPT>(row, scores_ld, raw);
        __syncthreads();
      }
    }
    if (!done) wide_select_rows<NT, KPT>(raw, qr.nb, c, k_blk, sm.sel, list, nullptr);
    if (CAND && writer && tid == 0) decided[i] = done ? 1u : 0u;
    const int body = k_blk * c, tail = qr.n_vis - qr.nb * c;
    cnt = body + tail;
    for (int j = tid; j < tail; j += NT) list[body + j] = qr.nb * c + j;
    if (writer) {
      for (int j = tid; j < body; j += NT) gsel[j] = list[j];
      write_tail<NT>(gsel, sel_ld, qr.nb, qr.n_vis, c, k_blk, n_sel + i);
    }
  }
  __syncthreads();                                   // the list is whole; the select's LDS is free
  // Waves 4..15 are done (a barrier waits only for the waves still running).
  if (__builtin_amdgcn_readfirstlane(tid / kWave) >= 4) return;
  const LdsList ls{list, cnt, meta};
  fwd_lds_body<T, DKQ, true, LdsList, true>(sm.att, ls, q, k, k_ld, k_hs, seq_row0, seq_len, q_seq, q_pos, 0, h_q,
                                            h_kv, scale_log2, n_split, rows_per_split, out, ws_o, ws_ml);
}

// Rows longer than one workgroup's registers hold (more than 32768 blocks), from the
// scoring launch's list of the KEEP best of every 32 blocks (KEEP 8: rows of up to
// 131072 blocks; 4: up to 262144), 32 listed keys per thread; where the list cannot
// decide, the per-query select over the row (select_chunk.hpp) runs instead.
template <typename T, int DKQ>
union ListLongSmem {
  WideSmem<kFusedThreads, kFusedMaxKpt> sel;
  WgSmem one;                                        // the per-query select over the row
  FwdLdsSmem<T, DKQ, true> att;
};

template <typename T, int DKQ, int KEEP>
__global__ void __launch_bounds__(kFusedThreads, 1)
list_fwd_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
                const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk,
                int32_t* __restrict__ sel, int64_t sel_ld, int32_t* __restrict__ n_sel, const T* __restrict__ q,
                const T* __restrict__ k, int64_t k_ld, int64_t k_hs, const int64_t* __restrict__ seq_row0, int h_q,
                int h_kv, float scale_log2, int n_split, int rows_per_split, float* __restrict__ out,
                float* __restrict__ ws_o, float* __restrict__ ws_ml, const uint32_t* __restrict__ cand,
                int64_t cand_ld, int cand_min_groups, uint32_t* __restrict__ decided) {
  constexpr int NT = kFusedThreads, KPT = kFusedMaxKpt, COPIES = WideCfg<NT, KPT>::copies;
  constexpr int TPT = KPT / KEEP;                    // tiles per thread (32 listed keys)
  __shared__ ListLongSmem<T, DKQ> sm;
  __shared__ int32_t list[kFusedListMax];
  const int i = blockIdx.y / h_kv, tid = threadIdx.x;
  const bool writer = blockIdx.x == 0 && blockIdx.y % h_kv == 0;   // writes sel and n_sel of query i
  // this thread's tiles of the list, coalesced: piece q of thread t at q * kCandThreads + t
  uint4 cv[KEEP * TPT / 2];
  const uint4* cand_src = (const uint4*)(cand + (int64_t)i * cand_ld) + tid;
#pragma unroll
  for (int q = 0; q < KEEP * TPT / 2; ++q) cv[q] = cand_src[q * kCandThreads];
  const SeqMeta meta = seq_meta(q_seq, seq_len, seq_row0, nullptr, i);
  const int n_vis = visible_tokens(meta.len, q_pos[i]);
  const QueryRowInfo qr{n_vis / c, n_vis};
  for (int e = tid; e < kP1Bins * COPIES / 4; e += NT) ((uint4*)sm.sel.h1)[e] = uint4{0u, 0u, 0u, 0u};
  for (int e = tid; e < kWideBins; e += NT) sm.sel.h2[e] = 0u;
  int32_t* gsel = sel + (int64_t)i * sel_ld;
  int cnt;
  if (qr.nb <= k_blk) {                              // dense: every visible position
    cnt = qr.n_vis;
    for (int j = tid; j < cnt; j += NT) list[j] = j;
    if (writer) write_dense<NT>(gsel, sel_ld, qr.n_vis, n_sel + i);
    if (writer && tid == 0) decided[i] = 0u;
  } else {
    __syncthreads();                                 // the histograms are clear
    bool done = false;
    uint32_t failed = 0u;
    if (qr.nb / kCandTile >= cand_min_groups)
      done = cand_select<NT, KPT, KEEP, TPT>(cv, qr.nb, c, k_blk, sm.sel, list, failed);
    // a few tiles held more of the kept blocks than they list: read them whole
    if (!done && failed != 0u)
      done = cand_complete_tiles<NT, KPT, KEEP, TPT, 2>(cand_src, scores + (int64_t)i * scores_ld, qr.nb, c, k_blk, failed,
                                                        sm.sel, list);
    if (!done) {                                     // the row's select, streamed (rare)
      __syncthreads();
      select_one_query<NT, 8>(scores + (int64_t)i * scores_ld, qr.nb, c, k_blk, list, sm.one);
      __syncthreads();
    }
    if (writer && tid == 0) decided[i] = done ? 1u : 0u;
    const int body = k_blk * c, tail = qr.n_vis - qr.nb * c;
    cnt = body + tail;
    for (int j = tid; j < tail; j += NT) list[body + j] = qr.nb * c + j;
    if (writer) {
      for (int j = tid; j < body; j += NT) gsel[j] = list[j];
      write_tail<NT>(gsel, sel_ld, qr.nb, qr.n_vis, c, k_blk, n_sel + i);
    }
  }
  __syncthreads();                                   // the list is whole; the select's LDS is free
  if (__builtin_amdgcn_readfirstlane(tid / kWave) >= 4) return;   // waves 4..15 are done
  const LdsList ls{list, cnt, meta};
  fwd_lds_body<T, DKQ, true, LdsList, true>(sm.att, ls, q, k, k_ld, k_hs, seq_row0, seq_len, q_seq, q_pos, 0, h_q,
                                            h_kv, scale_log2, n_split, rows_per_split, out, ws_o, ws_ml);
}

template <typename T, int DKQ>
union FinishFusedSmem {
  FinSmem<kEntCap, kFusedMaxChunks> fin;
  WgSmem one;                                        // the per-query select (massive exact ties)
  FwdLdsSmem<T, DKQ, true> att;
};

// Rows longer than one workgroup holds: the chunked selection's histogram and
// candidate launches have run; each attention workgroup runs the finishing pass into
// LDS, then attends.
template <typename T, int DKQ>
__global__ void __launch_bounds__(kFusedThreads, 1)
finish_fwd_kernel(const float* __restrict__ scores, int64_t scores_ld, const int32_t* __restrict__ seq_len,
                  const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int k_blk,
                  int32_t* __restrict__ sel, int64_t sel_ld, int32_t* __restrict__ n_sel, WsState* __restrict__ st,
                  ChunkScratch sc, const T* __restrict__ q, const T* __restrict__ k, int64_t k_ld, int64_t k_hs,
                  const int64_t* __restrict__ seq_row0, int h_q, int h_kv, float scale_log2, int n_split,
                  int rows_per_split, float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  constexpr int NT = kFusedThreads;
  __shared__ FinishFusedSmem<T, DKQ> sm;
  __shared__ int32_t list[kFusedListMax];
  const int i = blockIdx.y / h_kv, tid = threadIdx.x;
  const bool writer = blockIdx.x == 0 && blockIdx.y % h_kv == 0;   // writes sel and n_sel of query i
  ChunkSpec sp;
  sp.issue(sc, i);                                   // the candidates' first round trip, with the metadata's
  const uint32_t bin = sc.ctrl(i)[0];
  const int k_rem = (int)sc.ctrl(i)[1];
  const SeqMeta meta = seq_meta(q_seq, seq_len, seq_row0, nullptr, i);
  const int n_vis = visible_tokens(meta.len, q_pos[i]);
  const QueryRowInfo qr{n_vis / c, n_vis};
  int cnt;
  if (qr.nb <= k_blk) {                              // dense: the candidate launch wrote sel and n_sel
    cnt = qr.n_vis;
    for (int j = tid; j < cnt; j += NT) list[j] = j;
  } else {
    if (writer)                                      // every chunk has read it
      for (int b = tid; b < kBins1; b += NT) st->ghist[i][b] = 0u;
    chunk_cut<kEntCap, kFusedMaxChunks>(sp, sc, i, scores + (int64_t)i * scores_ld, qr, c, k_blk, bin, k_rem, sm.fin,
                                        sm.one, list);
    const int body = k_blk * c, tail = qr.n_vis - qr.nb * c;
    cnt = body + tail;
    for (int j = tid; j < tail; j += NT) list[body + j] = qr.nb * c + j;
    __syncthreads();                                 // the list is whole
    if (writer) {
      int32_t* gsel = sel + (int64_t)i * sel_ld;
      for (int j = tid; j < body; j += NT) gsel[j] = list[j];
      write_tail<NT>(gsel, sel_ld, qr.nb, qr.n_vis, c, k_blk, n_sel + i);
    }
  }
  __syncthreads();                                   // the list is whole; the selection's LDS is free
  if (__builtin_amdgcn_readfirstlane(tid / kWave) >= 4) return;   // waves 4..15 are done
  const LdsList ls{list, cnt, meta};
  fwd_lds_body<T, DKQ, true, LdsList, true>(sm.att, ls, q, k, k_ld, k_hs, seq_row0, seq_len, q_seq, q_pos, 0, h_q,
                                            h_kv, scale_log2, n_split, rows_per_split, out, ws_o, ws_ml);
}

// ---------------------------------------------------------------------------- host

static bool alias_of(const CacheArgs& c) { return c.v == c.k && c.v_ld == c.k_ld && c.v_hs == c.k_hs; }

enum class FusedForm { kTwoCalls, kWide, kChunked };

// What every form with the selection inside the attention's launch needs: the MLA
// shapes with V inside K, a list that fits LDS, one workgroup per compute unit.
static bool fused_base(const sa_dims& d, const CacheArgs& c, const void* q, int n_q, const FwdPlan& plan) {
  if (n_q < 1 || !fwd_uses_mfma(d, c, q) || !alias_of(c)) return false;
  if (d.d_v != 512 || (d.d_kq != 576 && d.d_kq != 512)) return false;
  if ((long long)d.top_k + d.compress_ratio - 1 > kFusedListMax) return false;
  const int cus = device_cus();
  return cus > 0 && (long long)plan.n_split * n_q * d.h_kv <= cus;   // one per CU
}

static FusedForm fused_form(const sa_dims& d, const CacheArgs& c, const void* q, int n_q, const FwdPlan& plan,
                            size_t ws_bytes) {
  if (!fused_base(d, c, q, n_q, plan)) return FusedForm::kTwoCalls;
  const long long max_blocks = (long long)c.max_len / d.compress_ratio;
  if (max_blocks <= (long long)kFusedThreads * kFusedMaxKpt) return FusedForm::kWide;
  if (!select_chunked(d, n_q, c.max_len) || select_chunk_count(d, c.max_len) > kFusedMaxChunks)
    return FusedForm::kTwoCalls;
  // the partials go after the candidates, which the launch is still reading (the
  // workspace the calls require has room for both)
  if (SA_WS_STATE_BYTES + select_scratch_bytes(d, n_q, c.max_len) + plan.ws_bytes > ws_bytes)
    return FusedForm::kTwoCalls;
  return FusedForm::kChunked;
}

bool select_fwd_fused(const sa_dims& d, const CacheArgs& c, const void* q, int n_q, const FwdPlan& plan,
                      size_t ws_bytes) {
  return fused_form(d, c, q, n_q, plan, ws_bytes) != FusedForm::kTwoCalls;
}

// P(X >= k) for X ~ Poisson(lam).
static double poisson_tail(double lam, int k) {
  double term = std::exp(-lam), below = 0.0;
  for (int j = 0; j < k; ++j) {
    below += term;
    term *= lam / (j + 1);
  }
  return below >= 1.0 ? 0.0 : 1.0 - below;
}

// The candidate list's best blocks per 32-block tile for rows of max_len tokens: the
// larger of 8 and 4 for which the list holds at most 32768 keys (one workgroup's) and
// a row of independent scores would rarely hold more than that many kept blocks in
// some tile (fewer than 1 row in 10 falls back to its row select: the list's attempt
// costs about twice what it saves); 0: no list (also for rows that are always dense).
int cand_keep(const sa_dims& d, int max_len) {
  const long long max_blocks = (long long)max_len / d.compress_ratio, k_blk = d.top_k / d.compress_ratio;
  if (max_blocks <= k_blk) return 0;
  const long long tiles = (max_blocks + kCandTile - 1) / kCandTile;
  const long long cap = (long long)kFusedThreads * kFusedMaxKpt;   // listed keys one workgroup holds
  for (int keep = kCandKeep; keep >= kCandKeep / 2; keep /= 2)
    if (tiles * keep <= cap && (double)tiles * poisson_tail((double)k_blk / tiles, keep + 1) < 0.1) return keep;
  return 0;
}

// The fewest whole groups a token's row must have for the list to be tried: with
// fewer, a row of independent scores would fall back once in 10 or more (the same
// rule as cand_keep's, for the token's own row), and the list would hold less than
// twice the cut.  The fallback rate falls as the groups grow past k_blk / keep.
static int cand_min_groups(const sa_dims& d, int keep) {
  const long long k_blk = d.top_k / d.compress_ratio, cap = (long long)kFusedThreads * kFusedMaxKpt / keep;
  auto ok = [&](long long g) { return (double)g * poisson_tail((double)k_blk / g, keep + 1) < 0.1; };
  long long lo = std::max(1LL, (2 * k_blk + keep - 1) / keep), hi = cap;
  if (lo > hi || !ok(hi)) return (int)(cap + 1);
  while (lo < hi) {
    const long long mid = (lo + hi) / 2;
    if (ok(mid)) hi = mid;
    else lo = mid + 1;
  }
  return (int)lo;
}

int cand_tpt(const sa_dims& d, int max_len) {
  const int keep = cand_keep(d, max_len);
  if (keep == 0) return 0;
  return (long long)max_len / d.compress_ratio <= (long long)kFusedThreads * kFusedMaxKpt ? 1 : kFusedMaxKpt / keep;
}

// Room for kCandThreads * tpt tiles: every reader's load is in bounds.
int64_t cand_words(const sa_dims& d, int max_len) {
  return (int64_t)kCandThreads * cand_tpt(d, max_len) * 2 * cand_keep(d, max_len);
}

// The tiles of n_q tokens, then one decided flag per token (n_q * cand_words + n_q
// words).
size_t cand_bytes(const sa_dims& d, int n_q, int max_len) {
  if (n_q < 1 || n_q > kCandMaxQueries) return 0;
  // Each scoring wave's tile search costs ~0.3-0.45 us per round of workgroups on the
  // chip; past 8192 tiles in all (the 1M decode token) the rounds cost more than the
  // selection saves (32 batched tokens of 16384 blocks: 67.4 us against 63.0)
  const long long tiles = ((long long)max_len / d.compress_ratio + kCandTile - 1) / kCandTile;
  if ((long long)n_q * tiles > kCandMaxTiles) return 0;
  const size_t words = (size_t)n_q * cand_words(d, max_len);
  return words == 0 ? 0 : (words + n_q) * 4;
}

template <typename T, int DKQ, int KPT, bool CAND>
static void launch_fused_t(const sa_dims& d, const CacheArgs& c, const float* scores, int64_t scores_ld,
                           const int32_t* q_seq, const int32_t* q_pos, int n_q, int32_t* sel, int64_t sel_ld,
                           int32_t* n_sel, const void* q, float scale_log2, float* out, float* ws_o, float* ws_ml,
                           const uint32_t* cand, int64_t cand_ld, const FwdPlan& plan, hipStream_t stream) {
  const dim3 grid(plan.n_split, n_q * d.h_kv);
  // the decided flags: the n_q words that end the workspace's candidate part
  uint32_t* decided = cand ? (uint32_t*)(cand + (int64_t)n_q * cand_ld) : nullptr;
  hipLaunchKernelGGL((select_fwd_kernel<T, DKQ, KPT, CAND>), grid, dim3(kFusedThreads), 0, stream, scores,
                     scores_ld, c.seq_len, q_seq, q_pos, d.compress_ratio, d.top_k / d.compress_ratio, sel, sel_ld,
                     n_sel, (const T*)q, (const T*)c.k, c.k_ld, c.k_hs, c.seq_row0, d.h_q, d.h_kv, scale_log2,
                     plan.n_split, plan.rows_per_split, out, ws_o, ws_ml, cand, cand_ld,
                     cand ? cand_min_groups(d, kCandKeep) : 0, decided);
}

template <typename T, int DKQ>
static void dispatch_fused(const sa_dims& d, const CacheArgs& c, const float* scores, int64_t scores_ld,
                           const int32_t* q_seq, const int32_t* q_pos, int n_q, int32_t* sel, int64_t sel_ld,
                           int32_t* n_sel, const void* q, float scale_log2, float* out, float* ws_o, float* ws_ml,
                           const uint32_t* cand, int64_t cand_ld, const FwdPlan& plan, hipStream_t stream) {
  const long long max_blocks = (long long)c.max_len / d.compress_ratio;
#define SA_FUSED(KPT_, CAND_)                                                                                   \
  launch_fused_t<T, DKQ, KPT_, CAND_>(d, c, scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld, n_sel, q,        \
                                      scale_log2, out, ws_o, ws_ml, cand, cand_ld, plan, stream)
  if (cand) {
    if (max_blocks <= (long long)kFusedThreads * 4) SA_FUSED(4, true);
    else if (max_blocks <= (long long)kFusedThreads * 8) SA_FUSED(8, true);
    else if (max_blocks <= (long long)kFusedThreads * 16) SA_FUSED(16, true);
    else SA_FUSED(32, true);
  } else {
    if (max_blocks <= (long long)kFusedThreads * 4) SA_FUSED(4, false);
    else if (max_blocks <= (long long)kFusedThreads * 8) SA_FUSED(8, false);
    else if (max_blocks <= (long long)kFusedThreads * 16) SA_FUSED(16, false);
    else SA_FUSED(32, false);
  }
#undef SA_FUSED
}

template <typename T, int DKQ>
static void launch_finish_fwd_t(const sa_dims& d, const CacheArgs& c, const float* scores, int64_t scores_ld,
                                const int32_t* q_seq, const int32_t* q_pos, int n_q, int32_t* sel, int64_t sel_ld,
                                int32_t* n_sel, void* ws, const void* q, float scale_log2, float* out, float* ws_o,
                                float* ws_ml, const FwdPlan& plan, hipStream_t stream) {
  const dim3 grid(plan.n_split, n_q * d.h_kv);
  hipLaunchKernelGGL((finish_fwd_kernel<T, DKQ>), grid, dim3(kFusedThreads), 0, stream, scores, scores_ld, c.seq_len,
                     q_seq, q_pos, d.compress_ratio, d.top_k / d.compress_ratio, sel, sel_ld, n_sel, (WsState*)ws,
                     chunk_scratch(d, c, ws), (const T*)q, (const T*)c.k, c.k_ld, c.k_hs, c.seq_row0, d.h_q, d.h_kv,
                     scale_log2, plan.n_split, plan.rows_per_split, out, ws_o, ws_ml);
}

hipError_t launch_select_fwd(const sa_dims& d, const CacheArgs& c, const float* scores, int64_t scores_ld,
                             const int32_t* q_seq, const int32_t* q_pos, int n_q, int32_t* sel, int64_t sel_ld,
                             int32_t* n_sel, const void* q, float scale, float* out, void* ws, size_t ws_bytes,
                             void* scratch, const FwdPlan& plan, hipStream_t stream, const uint32_t* cand,
                             int64_t cand_ld) {
  if (n_q == 0) return hipSuccess;
  const FusedForm form = fused_form(d, c, q, n_q, plan, ws_bytes);
  if (cand && (form != FusedForm::kWide || cand_ld < cand_words(d, c.max_len)))
    return hipErrorInvalidValue;                     // the candidate list serves the one-workgroup select only
  if (form == FusedForm::kTwoCalls) {
    hipError_t err = launch_select(d, c, scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld, n_sel, ws, stream);
    if (err != hipSuccess) return err;
    return launch_fwd(d, c, q, q_seq, sel, sel_ld, n_sel, nullptr, nullptr, 0, n_q, scale, out, scratch, plan,
                      stream);
  }
  const float scale_log2 = scale * kLog2e;
  float* ws_o = (float*)scratch;
  if (form == FusedForm::kChunked) {
    hipError_t err = launch_chunk_passes(d, c, scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld, n_sel, ws, stream);
    if (err != hipSuccess) return err;
    ws_o = (float*)((char*)ws + SA_WS_STATE_BYTES + select_scratch_bytes(d, n_q, c.max_len));
  }
  float* ws_ml = plan.n_split > 1 ? ws_o + (size_t)n_q * d.h_q * plan.n_split * d.d_v : nullptr;
  if (form == FusedForm::kChunked) {
#define SA_FIN(T_, DKQ_)                                                                                      \
  launch_finish_fwd_t<T_, DKQ_>(d, c, scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld, n_sel, ws, q, scale_log2, \
                                out, ws_o, ws_ml, plan, stream)
    if (d.dtype == SA_BF16) {
      if (d.d_kq == 576) SA_FIN(bf16, 576);
      else SA_FIN(bf16, 512);
    } else {
      if (d.d_kq == 576) SA_FIN(f16, 576);
      else SA_FIN(f16, 512);
    }
#undef SA_FIN
  } else if (d.dtype == SA_BF16) {
    if (d.d_kq == 576) dispatch_fused<bf16, 576>(d, c, scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld, n_sel, q, scale_log2, out, ws_o, ws_ml, cand, cand_ld, plan, stream);
    else dispatch_fused<bf16, 512>(d, c, scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld, n_sel, q, scale_log2, out, ws_o, ws_ml, cand, cand_ld, plan, stream);
  } else {
    if (d.d_kq == 576) dispatch_fused<f16, 576>(d, c, scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld, n_sel, q, scale_log2, out, ws_o, ws_ml, cand, cand_ld, plan, stream);
    else dispatch_fused<f16, 512>(d, c, scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld, n_sel, q, scale_log2, out, ws_o, ws_ml, cand, cand_ld, plan, stream);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine(d, n_q, out, ws_o, ws_ml, plan, stream);
}

enum class StepForm { kNoList, kListWide, kListLong };

// The form of pool + score + select + attention: with the candidate list where the
// pooling scoring launch and a fused select both apply and the workspace has the list's
// room; rows of up to 32768 blocks in the one-workgroup kernel, longer ones in
// list_fwd_kernel.  (Where the attention runs as a launch of its own, a selection from
// the list in a launch of its own measured no faster than the row's.)
static StepForm step_form(const sa_dims& d, const CacheArgs& c, const void* qidx, const void* q, int n_q,
                          const int32_t* n_in, const int32_t* n_out, const FwdPlan& plan, size_t ws_bytes) {
  if (cand_bytes(d, n_q, c.max_len) == 0 || ws_bytes < workspace_bytes(d, n_q, c.max_len)) return StepForm::kNoList;
  if (!pool_score_fused(d, c, qidx, n_q, n_in, n_out)) return StepForm::kNoList;
  const long long max_blocks = (long long)c.max_len / d.compress_ratio;
  if (!fused_base(d, c, q, n_q, plan)) return StepForm::kNoList;
  return max_blocks <= (long long)kFusedThreads * kFusedMaxKpt ? StepForm::kListWide : StepForm::kListLong;
}

bool step_uses_cand(const sa_dims& d, const CacheArgs& c, const void* qidx, const void* q, int n_q,
                    const int32_t* n_in, const int32_t* n_out, const FwdPlan& plan, size_t ws_bytes) {
  return step_form(d, c, qidx, q, n_q, n_in, n_out, plan, ws_bytes) != StepForm::kNoList;
}

template <typename T, int DKQ>
static void launch_list_long_t(const sa_dims& d, const CacheArgs& c, const float* scores, int64_t scores_ld,
                               const int32_t* q_seq, const int32_t* q_pos, int n_q, int32_t* sel, int64_t sel_ld,
                               int32_t* n_sel, const void* q, float scale_log2, float* out, float* ws_o, float* ws_ml,
                               const uint32_t* cand, int64_t cand_ld, int keep, const FwdPlan& plan,
                               hipStream_t stream) {
  const dim3 grid(plan.n_split, n_q * d.h_kv);
  uint32_t* decided = (uint32_t*)(cand + (int64_t)n_q * cand_ld);
#define SA_LIST_LONG(KEEP_)                                                                                          \
  hipLaunchKernelGGL((list_fwd_kernel<T, DKQ, KEEP_>), grid, dim3(kFusedThreads), 0, stream, scores, scores_ld,      \
                     c.seq_len, q_seq, q_pos, d.compress_ratio, d.top_k / d.compress_ratio, sel, sel_ld, n_sel,     \
                     (const T*)q, (const T*)c.k, c.k_ld, c.k_hs, c.seq_row0, d.h_q, d.h_kv, scale_log2,            \
                     plan.n_split, plan.rows_per_split, out, ws_o, ws_ml, cand, cand_ld, min_groups, decided)
  const int min_groups = cand_min_groups(d, keep);
  if (keep == kCandKeep) SA_LIST_LONG(kCandKeep);
  else SA_LIST_LONG(kCandKeep / 2);
#undef SA_LIST_LONG
}

hipError_t launch_pool_score_select_fwd(const sa_dims& d, const CacheArgs& c, const int32_t* n_in, int32_t* n_out,
                                        int max_new, const void* qidx, const int32_t* q_seq, const int32_t* q_pos,
                                        int n_q, float* scores, int64_t scores_ld, const void* q, float scale,
                                        int32_t* sel, int64_t sel_ld, int32_t* n_sel, float* out, void* ws,
                                        size_t ws_bytes, void* scratch, const FwdPlan& plan, hipStream_t stream) {
  const StepForm form = ws ? step_form(d, c, qidx, q, n_q, n_in, n_out, plan, ws_bytes) : StepForm::kNoList;
  if (form == StepForm::kNoList) {
    hipError_t err = launch_pool_score(d, c, n_in, n_out, max_new, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream);
    if (err != hipSuccess) return err;
    return launch_select_fwd(d, c, scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld, n_sel, q, scale, out, ws,
                             ws_bytes, scratch, plan, stream);
  }
  // the list: the workspace's last part (after the partials, which the select's launch writes)
  const size_t need = workspace_bytes(d, n_q, c.max_len);
  uint32_t* cand = (uint32_t*)((char*)ws + need - cand_bytes(d, n_q, c.max_len));
  const int64_t cand_ld = cand_words(d, c.max_len);
  const int keep = cand_keep(d, c.max_len);
  hipError_t err = launch_pool_score(d, c, n_in, n_out, max_new, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream,
                                     cand, cand_ld, keep, cand_tpt(d, c.max_len));
  if (err != hipSuccess) return err;
  if (form == StepForm::kListWide)
    return launch_select_fwd(d, c, scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld, n_sel, q, scale, out, ws,
                             ws_bytes, scratch, plan, stream, cand, cand_ld);
  const float scale_log2 = scale * kLog2e;
  float* ws_o = (float*)scratch;
  float* ws_ml = plan.n_split > 1 ? ws_o + (size_t)n_q * d.h_q * plan.n_split * d.d_v : nullptr;
#define SA_LL(T_, DKQ_)                                                                                         \
  launch_list_long_t<T_, DKQ_>(d, c, scores, scores_ld, q_seq, q_pos, n_q, sel, sel_ld, n_sel, q, scale_log2, out, \
                               ws_o, ws_ml, cand, cand_ld, keep, plan, stream)
  if (d.dtype == SA_BF16) {
    if (d.d_kq == 576) SA_LL(bf16, 576);
    else SA_LL(bf16, 512);
  } else {
    if (d.d_kq == 576) SA_LL(f16, 576);
    else SA_LL(f16, 512);
  }
#undef SA_LL
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine(d, n_q, out, ws_o, ws_ml, plan, stream);
}

}  // namespace sa
