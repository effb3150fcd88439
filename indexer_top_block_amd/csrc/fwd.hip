// Gather-fused attention over each query token's selected rows, with split-KV
// partial results and an online-softmax combine.
//
// The pages' sparse flash attention loads K/V rows through an ascending int32 index
// list inside the attention kernel instead of materialising a dense copy (llama.cpp
// PR #27970 "CUDA + ggml: add sparse-fa for DSV4/GLM": the gather-vs-get_rows review
// exchange, and the index-guarded row loads); V may be the first DV elements of each
// K row (MLA latent cache).  Shapes of note: DKQ/DV = 576/512 with 16 query heads per
// KV head, 512/512 with 8.
//
// MFMA path (f16 / bf16, up to 16 query heads per KV head, DKQ % 32 == 0, DV % 64 == 0):
//   one workgroup = 4 waves = one (query token, KV head, split).  Per 64-row tile the
//   workgroup gathers K rows (and V rows when separate) into LDS with 16-byte loads,
//   holding the next tile's rows in registers meanwhile.  Wave w computes S^T = K Q^T
//   for rows [16w, 16w+16) with v_mfma_f32_16x16x32 (rows as M, the up-to-16 heads as
//   N, Q^T kept in registers) and writes it, scaled, to a small transposed LDS tile;
//   every wave then reads the whole tile back in the B-operand layout of
//   v_mfma_f32_16x16x16 (a head's rows in one lane column), runs the same online
//   softmax, and accumulates its own quarter of DV as O^T = V^T P^T, with V^T read
//   from LDS column-wise.  Splitting DV rather than rows keeps one accumulator per
//   output element (32 registers per lane), so two workgroups share a CU and their
//   gathers overlap.
// MLA shapes with V inside K (DV 512, DKQ 512 or 576): fwd_lds_kernel, rows gathered
// straight into LDS (described at the kernel).
// VALU path (any dtype; fwd_common.hpp): the same tiles with plain float dot products.
// Entry forms: plain, with a bias per list entry, and with a dense window of recent
// positions appended to the list (row_pos in fwd_common.hpp).
//
// Partial results: o (unnormalised, float32), m (running max, log2 units) and l
// (sum of weights) per (query, head, split); the combine kernel merges the splits.
#include <type_traits>

#include "fwd_common.hpp"
#include "fwd_lds.hpp"

namespace sa {

template <typename T, int DKQ, int DV, bool ALIAS>
__global__ void __launch_bounds__(256, 1)
fwd_mfma_kernel(const T* __restrict__ q, const T* __restrict__ k, int64_t k_ld, int64_t k_hs,
                const T* __restrict__ v, int64_t v_ld, int64_t v_hs, const int64_t* __restrict__ seq_row0,
                const int32_t* __restrict__ seq_len, const int32_t* __restrict__ q_seq,
                const int32_t* __restrict__ sel, int64_t sel_ld, const int32_t* __restrict__ n_sel,
                const float* __restrict__ sel_bias, const int32_t* __restrict__ q_pos, int window, int list_max, int h_q,
                int h_kv, float scale_log2, int n_split, int rows_per_split, float* __restrict__ out,
                float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  typedef typename vec8<T>::type V8;
  constexpr int RT = kMfmaTile;       // = 64: one list entry per lane
  constexpr int KST = DKQ / 32;       // QK^T MFMA steps
  constexpr int KP = DKQ + 16;        // LDS row pitches (elements): 8 dwords mod 64 banks (40 for DKQ 576)
  constexpr int VP = ALIAS ? KP : DV + 16;
  constexpr int DVW = DV / 4;         // output dims owned by one wave
  constexpr int NTW = DVW / 16;       // its 16-dim MFMA tiles
  constexpr int KCH = DKQ / 8;        // 16-byte chunks per K row
  constexpr int VCH = DV / 8;
  constexpr int KLD = RT * KCH / 256;                 // K chunks per thread per tile
  constexpr int VLD = ALIAS ? 1 : RT * VCH / 256;     // V chunks per thread per tile
  constexpr int SP = RT + 4;                          // pitch of the transposed score tile (floats)
  static_assert(RT == kWave, "one list entry per lane");
  static_assert(RT * KCH % 256 == 0 && (ALIAS || RT * VCH % 256 == 0), "tile must split evenly");
  static_assert(DV % 64 == 0, "four waves split DV in 16-dim tiles");
  __shared__ __attribute__((aligned(16))) T ks[RT * KP];
  __shared__ __attribute__((aligned(16))) T vs_sep[ALIAS ? 8 : RT * VP];
  __shared__ __attribute__((aligned(16))) float st[16 * SP];   // scaled scores, [head][row]
  const T* vs = ALIAS ? ks : vs_sep;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 15, grp = lane >> 4;
  const int split = blockIdx.x;
  const int i = blockIdx.y / h_kv, g = blockIdx.y % h_kv;
  const int G = h_q / h_kv;
  const int32_t* list = sel + (int64_t)i * sel_ld;
  const float* blist = sel_bias ? sel_bias + (int64_t)i * sel_ld : nullptr;   // additive logit bias per entry
  const int r_begin = split * rows_per_split;
  // Every wave reads the list itself, lane l taking entry l of a tile.  Indices are
  // clamped into the row rather than guarded, so the loads issue back to back;
  // entries at or past the query's count are discarded once it is known.  The
  // first four tiles' entries are read alongside the query's metadata.
  const int lim = (int)min(sel_ld, (int64_t)list_max) - 1;
  auto list_at = [&](int t) { return list[min(r_begin + t * RT + lane, lim)]; };
  const int pre0 = list_at(0), pre1 = list_at(1), pre2 = list_at(2), pre3 = list_at(3);
  const SeqMeta sm = seq_meta(q_seq, seq_len, seq_row0, nullptr, i);
  const int L = sm.len;
  const int64_t row0 = sm.row0;
  const int cnt = max(0, (int)min((int64_t)n_sel[i], min(sel_ld, (int64_t)list_max)));
  int w0 = 0, wlen = 0;                              // dense window of the most recent positions
  if (window > 0) {
    const int n_vis = visible_tokens(L, q_pos[i]);
    wlen = min(window, n_vis);
    w0 = n_vis - wlen;
  }
  // the last split takes every remaining row (the tail rows when they have no split of their own)
  const int r_end = split == n_split - 1 ? cnt + wlen : min(cnt + wlen, r_begin + rows_per_split);
  const int n_tiles = r_end > r_begin ? (r_end - r_begin + RT - 1) / RT : 0;
  const T* kg = k + (int64_t)g * k_hs;
  const T* vg = v + (int64_t)g * v_hs;

  // Q^T as the B operand: lane (col = head, grp) holds dims st*32 + grp*8 .. +8.
  // Lanes past the group's heads read head 0 and zero the values.
  const T* qbase = q + ((int64_t)i * h_q + (int64_t)g * G) * DKQ;
  V8 qf[KST];
  {
    const T* qh = qbase + (col < G ? col : 0) * DKQ + grp * 8;
#pragma unroll
    for (int st_ = 0; st_ < KST; ++st_) qf[st_] = *reinterpret_cast<const V8*>(qh + st_ * 32);
    if (col >= G) {
#pragma unroll
      for (int st_ = 0; st_ < KST; ++st_) qf[st_] = V8{};
    }
  }
  // Running max (log2 units) and weight sum of head `col` over all rows so far: every
  // wave sees the whole score tile, so every wave holds the same values.
  float m = -INFINITY, lsum = 0.f;
  f32x4 o[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A tile's rows as held by every wave: lane l has row l's gather offsets (element
  // offsets from kg / vg), and a 64-bit mask marks the selected rows.  Rows that are
  // not selected gather this query's own Q row instead (finite values, and their
  // scores are masked to -inf, so they add exactly zero), so every gather is an
  // unconditional load.
  struct TileRows {
    int64_t ko, vo;
    uint64_t valid;
    float bias;                                      // lane l: the bias of entry l (0 without one)
  };
  const int64_t safe_k = qbase - kg, safe_v = qbase - vg;
  auto tile_rows = [&](int pos, int t) {
    const int j = r_begin + t * RT + lane;
    const int64_t row = tile_row(row_pos(pos, j, cnt, w0, wlen), j, r_end, L, row0);
    TileRows tr;
    tr.ko = row >= 0 ? row * k_ld : safe_k;
    tr.vo = ALIAS ? 0 : (row >= 0 ? row * v_ld : safe_v);
    tr.valid = __ballot(row >= 0);
    tr.bias = blist ? blist[min(r_begin + t * RT + lane, lim)] : 0.f;
    return tr;
  };
  // Offset of chunk e's row: the chunks of one wave instruction span at most NR rows
  // starting at the wave-uniform row R, whose offsets are read from their lanes.
  auto chunk_off = [&](int64_t per_lane, int e0, int e, int CH) -> int64_t {
    const int R = e0 / CH;
    const int r = e / CH;
    int64_t off = readlane64(per_lane, R);
    const int nr = (kWave + CH - 1) / CH + 1;
    for (int u = 1; u < nr; ++u) {
      const int64_t o2 = readlane64(per_lane, min(R + u, RT - 1));
      off = (r == R + u) ? o2 : off;
    }
    return off;
  };

  // Gathered rows of the next PD tiles are held in registers (PD buffers, used in
  // turn) while the current tile is computed from LDS, so PD tiles' gathers are in
  // flight at a time; the row list runs two tiles further ahead still.  With V
  // aliasing K a tile is 18 registers of 16 bytes per thread and two fit; with a
  // separate V tile only one does.
  constexpr int PD = ALIAS ? 2 : 1;
  V8 kbuf[PD][KLD], vbuf[PD][VLD];
  auto issue = [&](V8 (&kr)[KLD], V8 (&vr)[VLD], const TileRows& tr) {
#pragma unroll
    for (int j = 0; j < KLD; ++j) {
      const int e0 = wave * kWave + 256 * j, e = e0 + lane;
      const int cc = e % KCH;
      kr[j] = *reinterpret_cast<const V8*>(kg + chunk_off(tr.ko, e0, e, KCH) + cc * 8);
    }
    if (!ALIAS) {
#pragma unroll
      for (int j = 0; j < VLD; ++j) {
        const int e0 = wave * kWave + 256 * j, e = e0 + lane;
        const int cc = e % VCH;
        vr[j] = *reinterpret_cast<const V8*>(vg + chunk_off(tr.vo, e0, e, VCH) + cc * 8);
      }
    }
  };
  auto land = [&](const V8 (&kr)[KLD], const V8 (&vr)[VLD]) {
#pragma unroll
    for (int j = 0; j < KLD; ++j) {
      const int e = tid + 256 * j, r = e / KCH, cc = e % KCH;
      *reinterpret_cast<V8*>(ks + r * KP + cc * 8) = kr[j];
    }
    if (!ALIAS) {
#pragma unroll
      for (int j = 0; j < VLD; ++j) {
        const int e = tid + 256 * j, r = e / VCH, cc = e % VCH;
        *reinterpret_cast<V8*>(vs_sep + r * VP + cc * 8) = vr[j];
      }
    }
  };

  const int wr = wave * 16;                          // this wave's 16 rows of S
  const int dvb = wave * DVW;                        // this wave's output dims
  auto compute = [&](uint64_t valid, float bias) {
    // S^T[row][head] for this wave's 16 rows, as two independent accumulation chains,
    // scaled to log2 units (-inf for rows not selected) and shared through LDS.
    {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      const T* arow = ks + (wr + col) * KP + grp * 8;
#pragma unroll
      for (int st_ = 0; st_ + 1 < KST; st_ += 2) {
        s0 = mfma16x16x32<T>(*reinterpret_cast<const V8*>(arow + st_ * 32), qf[st_], s0);
        s1 = mfma16x16x32<T>(*reinterpret_cast<const V8*>(arow + (st_ + 1) * 32), qf[st_ + 1], s1);
      }
      if (KST & 1) s0 = mfma16x16x32<T>(*reinterpret_cast<const V8*>(arow + (KST - 1) * 32), qf[KST - 1], s0);
      const f32x4 sacc = s0 + s1;
      f32x4 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float b = blist ? __shfl(bias, wr + 4 * grp + j) * kLog2e : 0.f;
        x[j] = ((valid >> (wr + 4 * grp + j)) & 1ull) ? sacc[j] * scale_log2 + b : -INFINITY;
      }
      *reinterpret_cast<f32x4*>(st + col * SP + wr + 4 * grp) = x;
    }
    __syncthreads();
    // Online softmax of head `col` over the whole tile; this lane takes rows
    // 16*kk + 4*grp + j, which is the B-operand layout of the P^T MFMA steps below.
    f32x4 xs[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) xs[kk] = *reinterpret_cast<const f32x4*>(st + col * SP + 16 * kk + 4 * grp);
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = fmaxf(mx, xs[kk][j]);
    mx = max_xor32(max_xor16(mx));
    const float m_new = fmaxf(m, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m - m_new);
    T pb[4][4];
    float psum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = (xs[kk][j] == -INFINITY) ? 0.f : fast_exp2(xs[kk][j] - m_new);
        psum += p;
        pb[kk][j] = (T)p;
      }
    psum = sum_xor32(sum_xor16(psum));
    lsum = lsum * alpha + psum;
    m = m_new;
    // O^T[dv][head] = alpha * O^T + V^T[dv][row] P^T[row][head] for this wave's dims.
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) o[nt] *= alpha;
    // V^T operand by transposing LDS reads: in each 16-lane group, lane r reads 4
    // dims at row 4*grp + r/4, dims 4*(r%4) .. +4 of the 16-dim tile, and lane i then
    // holds dim i of rows 4*grp .. 4*grp+3 -- the A-operand layout.  Two such reads,
    // 16 rows apart, make a lane group's 8 k-values of one 16x16x32 product.
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      const T* vrow0 = vs + (32 * kk2 + 4 * grp + (col >> 2)) * VP + dvb + 4 * (col & 3);
      const T* vrow1 = vrow0 + 16 * VP;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vrow0 + nt * 16));
        const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vrow1 + nt * 16));
        o[nt] = pv_mfma32<T>(a0, a1, pb[2 * kk2], pb[2 * kk2 + 1], o[nt]);
      }
    }
  };

  // Pipeline: while tile t is computed, tiles t+1 .. t+PD are in flight and the list
  // entries of tiles t+PD+1 and t+PD+2 are in registers.  Inside the loop every step
  // issues its next tile unconditionally (past the end a tile has no selected rows
  // and gathers the Q row), so the number of loads in flight behind each tile is
  // the same on every path and the wait before landing a tile leaves the next
  // tile's loads outstanding; the last tile is landed by a step that issues nothing.
  uint64_t vq[PD];                                   // selected-row masks of tiles t .. t+PD-1
  float bq[PD];                                      // and the lanes' entry biases
#pragma unroll
  for (int u = 0; u < PD; ++u) {
    vq[u] = 0;
    bq[u] = 0.f;
  }
  int rawA = PD == 2 ? pre2 : pre1;                  // list entries of tile t+PD
  int rawB = PD == 2 ? pre3 : pre2;                  // and of tile t+PD+1
  auto step = [&](int t, V8 (&kr)[KLD], V8 (&vr)[VLD], auto issue_next) {
    land(kr, vr);
    __syncthreads();
    if constexpr (decltype(issue_next)::value) {
      const int raw_new = list_at(t + PD + 2);       // before the gathers: waiting for it must not wait for them
      const TileRows rn = tile_rows(rawA, t + PD);
      issue(kr, vr, rn);
      compute(vq[0], bq[0]);
#pragma unroll
      for (int u = 0; u + 1 < PD; ++u) {
        vq[u] = vq[u + 1];
        bq[u] = bq[u + 1];
      }
      vq[PD - 1] = rn.valid;
      bq[PD - 1] = rn.bias;
      rawA = rawB;
      rawB = raw_new;
    } else {
      compute(vq[0], bq[0]);
#pragma unroll
      for (int u = 0; u + 1 < PD; ++u) {
        vq[u] = vq[u + 1];
        bq[u] = bq[u + 1];
      }
    }
    __syncthreads();
  };
  using issue_t = std::integral_constant<bool, true>;
  using final_t = std::integral_constant<bool, false>;
  if constexpr (PD == 2) {
    if (n_tiles >= 2) {
      const TileRows r0 = tile_rows(pre0, 0), r1 = tile_rows(pre1, 1);
      vq[0] = r0.valid;
      vq[1] = r1.valid;
      bq[0] = r0.bias;
      bq[1] = r1.bias;
      issue(kbuf[0], vbuf[0], r0);
      issue(kbuf[1], vbuf[1], r1);
      int t = 0;
      for (; t + 1 < n_tiles; t += 2) {
        step(t, kbuf[0], vbuf[0], issue_t{});
        step(t + 1, kbuf[1], vbuf[1], issue_t{});
      }
      if (t < n_tiles) step(t, kbuf[0], vbuf[0], final_t{});
    } else if (n_tiles == 1) {
      const TileRows r0 = tile_rows(pre0, 0);
      vq[0] = r0.valid;
      bq[0] = r0.bias;
      issue(kbuf[0], vbuf[0], r0);
      step(0, kbuf[0], vbuf[0], final_t{});
    }
  } else {
    // One buffer: only one tile is ever in flight, so the plain loop (conditional
    // issue, conservative waits) loses nothing.
    if (n_tiles >= 1) {
      const TileRows r0 = tile_rows(pre0, 0);
      vq[0] = r0.valid;
      bq[0] = r0.bias;
      issue(kbuf[0], vbuf[0], r0);
      for (int t = 0; t < n_tiles; ++t) {
        land(kbuf[0], vbuf[0]);
        __syncthreads();
        const int raw_new = list_at(t + 3);
        const TileRows rn = tile_rows(rawA, t + 1);
        if (t + 1 < n_tiles) issue(kbuf[0], vbuf[0], rn);
        compute(vq[0], bq[0]);
        __syncthreads();
        vq[0] = rn.valid;
        bq[0] = rn.bias;
        rawA = rawB;
        rawB = raw_new;
      }
    }
  }

  // ---- this wave's dims of the result (or of the split's partial) ------------------
  if (col < G) {
    const int hq = g * G + col;
    const int64_t qh = (int64_t)i * h_q + hq;
    if (n_split == 1) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
        *reinterpret_cast<f32x4*>(out + qh * DV + dvb + nt * 16 + 4 * grp) = o[nt] * inv;
    } else {
      float* dst = ws_o + (qh * n_split + split) * DV + dvb;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) *reinterpret_cast<f32x4*>(dst + nt * 16 + 4 * grp) = o[nt];
      if (wave == 0 && grp == 0) {
        ws_ml[(qh * n_split + split) * 2 + 0] = m;
        ws_ml[(qh * n_split + split) * 2 + 1] = lsum;
      }
    }
  }
}

// ------------------------------------------------- MFMA, direct-to-LDS gathers (MLA)

// V aliasing K with DV = 512 (DKQ 512 or 576): the rows go from memory straight into
// LDS (fwd_lds.hpp), over the list that sparse_attn_select wrote.
template <typename T, int DKQ, bool QLDS>
__global__ void __launch_bounds__(256, QLDS ? 1 : 2)
fwd_lds_kernel(const T* __restrict__ q, const T* __restrict__ k, int64_t k_ld, int64_t k_hs,
               const int64_t* __restrict__ seq_row0, const int32_t* __restrict__ seq_len,
               const int32_t* __restrict__ q_seq, const int32_t* __restrict__ sel, int64_t sel_ld,
               const int32_t* __restrict__ n_sel, const float* __restrict__ sel_bias,
               const int32_t* __restrict__ q_pos, int window, int list_max, int h_q, int h_kv, float scale_log2, int n_split,
               int rows_per_split, float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  __shared__ FwdLdsSmem<T, DKQ, QLDS> sm;
  const int i = blockIdx.y / h_kv;
  const int64_t cap = min(sel_ld, (int64_t)list_max);
  const GlobalList ls{sel + (int64_t)i * sel_ld, sel_bias ? sel_bias + (int64_t)i * sel_ld : nullptr, (int)cap - 1,
                      n_sel + i, cap};
  fwd_lds_body<T, DKQ, QLDS>(sm, ls, q, k, k_ld, k_hs, seq_row0, seq_len, q_seq, q_pos, window, h_q, h_kv,
                             scale_log2, n_split, rows_per_split, out, ws_o, ws_ml);
}

// ------------------------------------------------------------------------- combine

// out[qh][dv] = sum_s 2^(m_s - M) o_s[dv] / sum_s 2^(m_s - M) l_s, M = max_s m_s.
// One thread per output element, kCombineThreads per workgroup (all of one (query,
// head), so the split statistics are wave-uniform), no LDS and no barriers.  Up to
// MAXS splits every partial value and statistic is loaded into registers before any
// is used (indices clamped, not guarded), so the combine costs one round trip;
// beyond that the splits stream in chunks.
constexpr int kCombineThreads = 64;

template <int MAXS>
__global__ void __launch_bounds__(kCombineThreads)
fwd_combine_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml, int n_split, int d_v,
                   int64_t n_out, float* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  if (e >= n_out) return;
  const int64_t qh = e / d_v;
  const int dv = (int)(e - qh * d_v);
  const float* ml = ws_ml + qh * n_split * 2;
  const float* src = ws_o + qh * n_split * d_v + dv;
  float acc = 0.f, L = 0.f;
  if (n_split <= MAXS) {
    float o[MAXS], m[MAXS], l[MAXS];
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      const int sc = min(s, n_split - 1);
      o[s] = src[(int64_t)sc * d_v];
      m[s] = s < n_split ? ml[2 * sc] : -INFINITY;
      l[s] = ml[2 * sc + 1];
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < MAXS; ++s) M = fmaxf(M, m[s]);
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      const float w = m[s] == -INFINITY ? 0.f : fast_exp2(m[s] - M);
      acc += w * o[s];
      L += w * l[s];
    }
  } else {
    float M = -INFINITY;
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, ml[2 * s]);
    for (int s = 0; s < n_split; ++s) {
      const float ms = ml[2 * s];
      const float w = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
      acc += w * src[(int64_t)s * d_v];
      L += w * ml[2 * s + 1];
    }
  }
  out[e] = L > 0.f ? acc / L : 0.f;
}

// Few splits (the batched decode's 8): two adjacent outputs per thread (d_v even), so
// each split's statistics are loaded and weighted once for both and the partials come
// as 8-byte pairs; the same arithmetic per output as above.  Measured against the
// one-output form: 38.3 against 40.3 us for the batched attention + combine, no gain
// at 33 splits.
template <int MAXS>
__global__ void __launch_bounds__(kCombineThreads)
fwd_combine2_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml, int n_split, int d_v,
                    int64_t n_out, float* __restrict__ out) {
  const int64_t e = ((int64_t)blockIdx.x * kCombineThreads + threadIdx.x) * 2;
  if (e >= n_out) return;
  const int64_t qh = e / d_v;
  const int dv = (int)(e - qh * d_v);
  const float* ml = ws_ml + qh * n_split * 2;
  const float* src = ws_o + qh * n_split * d_v + dv;
  asm volatile("" : "+v"(ml));                       // vector loads (scalar loads of the statistics are slower)
  float2 o[MAXS], st[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const int sc = min(s, n_split - 1);
    o[s] = *reinterpret_cast<const float2*>(src + (int64_t)sc * d_v);
    st[s] = *reinterpret_cast<const float2*>(ml + 2 * sc);
    if (s >= n_split) st[s].x = -INFINITY;
  }
  __builtin_amdgcn_sched_barrier(0);                 // every load issued before the first is used
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MAXS; ++s) M = fmaxf(M, st[s].x);
  float a0 = 0.f, a1 = 0.f, L = 0.f;
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const float w = st[s].x == -INFINITY ? 0.f : fast_exp2(st[s].x - M);
    a0 += w * o[s].x;
    a1 += w * o[s].y;
    L += w * st[s].y;
  }
  *reinterpret_cast<float2*>(out + e) = float2{L > 0.f ? a0 / L : 0.f, L > 0.f ? a1 / L : 0.f};
}

// ---------------------------------------------------------------------------- host

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int fwd_cap(const sa_dims& d) { return d.top_k + d.compress_ratio - 1; }

// Split plan for up to `rows` attended rows per query, for a kernel that `slots`
// workgroups fill (compute units x workgroups resident per unit).  The rows of whole
// blocks (all but the c - 1 rows a tail can add) go to splits of T 64-row tiles, T
// the smallest count for which the splits of all queries fit in one round of `slots`
// workgroups -- a second, partial round would leave most of the chip idle while it
// runs.  The tail rows get a split of their own when one more split per query still
// fits (so a list with a tail adds no tile to any split), else the last split takes
// them; kernels give the last split every remaining row.
static FwdPlan plan_rows(const sa_dims& d, int n_q, long long rows, long long slots) {
  FwdPlan p{};
  const long long units = (long long)n_q * d.h_kv;
  const long long tail = d.compress_ratio - 1;
  const long long bulk = rows - tail > 1 ? rows - tail : 1;
  const long long tiles = (bulk + kMfmaTile - 1) / kMfmaTile;
  if (slots > kPlanSlots) slots = kPlanSlots;
  if (slots < 1) slots = 1;
  long long per = tiles;                      // tiles per split
  if (units > 0 && units < slots && tiles > 1) per = (tiles * units + slots - 1) / slots;
  if (per < 1) per = 1;
  long long n = (tiles + per - 1) / per;
  if (tail > 0 && rows > bulk && units * (n + 1) <= slots) ++n;
  p.rows_per_split = (int)(per * kMfmaTile);
  p.list_max = fwd_cap(d);
  p.n_split = n > 1 ? (int)n : 1;
  p.ws_bytes = p.n_split > 1 ? (size_t)n_q * d.h_q * p.n_split * ((size_t)d.d_v + 2) * sizeof(float) : 0;
  return p;
}

FwdPlan plan_fwd(const sa_dims& d, int n_q) { return plan_rows(d, n_q, fwd_cap(d), kPlanSlots); }

static long long window_rows(const sa_dims& d, int window) { return (long long)fwd_cap(d) + (window > 0 ? window : 0); }

// With a dense window of `window` positions the rows per query grow by up to
// `window`.  When the workspace holds the partials of the plan for all those rows
// (workspace_bytes_window), that plan is used; otherwise the split count of the
// plain plan is kept -- its workspace always suffices -- and each split takes more rows.
// A plan for fewer slots than kPlanSlots never has more splits, so the workspace
// sizes below (taken at kPlanSlots) cover it.
FwdPlan plan_fwd_window(const sa_dims& d, int n_q, int window, size_t ws_avail, long long slots) {
  const long long total = window_rows(d, window);
  FwdPlan full = plan_rows(d, n_q, total, slots);
  if (full.ws_bytes <= ws_avail) return full;
  FwdPlan p = plan_rows(d, n_q, fwd_cap(d), slots);
  long long rps = (total + p.n_split - 1) / p.n_split;
  rps = (rps + kMfmaTile - 1) / kMfmaTile * kMfmaTile;
  if (rps > p.rows_per_split) p.rows_per_split = (int)rps;
  return p;
}

size_t workspace_bytes(const sa_dims& d, int n_q, int max_len) {
  const size_t f = plan_fwd(d, n_q).ws_bytes;
  const size_t s = select_scratch_bytes(d, n_q, max_len);
  const size_t l = cand_bytes(d, n_q, max_len);
  if (f == 0 && s == 0 && l == 0) return 0;
  // side by side: a fused launch reads one while it writes another; the candidate
  // list (read in 16-byte pieces) starts on a 256-byte boundary
  if (l == 0) return SA_WS_STATE_BYTES + s + f;
  return (SA_WS_STATE_BYTES + s + f + 255) / 256 * 256 + l;
}

size_t workspace_bytes_window(const sa_dims& d, int n_q, int max_len, int window) {
  const size_t base = workspace_bytes(d, n_q, max_len);
  const size_t f = plan_rows(d, n_q, window_rows(d, window), kPlanSlots).ws_bytes;
  const size_t w = f > 0 ? SA_WS_STATE_BYTES + f : 0;
  return w > base ? w : base;
}

bool fwd_uses_mfma(const sa_dims& d, const CacheArgs& c, const void* q) {
  if (d.dtype != SA_F16 && d.dtype != SA_BF16) return false;
  const int G = d.h_q / d.h_kv;
  if (G > 16) return false;
  const bool shape = (d.d_kq == 576 && d.d_v == 512) || (d.d_kq == 512 && d.d_v == 512) ||
                     (d.d_kq == 256 && d.d_v == 256) || (d.d_kq == 128 && d.d_v == 128);
  if (!shape) return false;
  const bool alias = c.v == c.k && c.v_ld == c.k_ld && c.v_hs == c.k_hs;
  if (c.k_ld % 8 || c.k_hs % 8 || !aligned16(c.k) || !aligned16(q)) return false;
  if (!alias && (c.v_ld % 8 || c.v_hs % 8 || !aligned16(c.v))) return false;
  return true;
}

// Workgroups the attention call's kernel fills the chip with: the register-path kernel
// with a separate V of 512+ dims holds a K and a V tile in LDS (135 KiB), one
// workgroup per compute unit; the other kernels fit two.
long long fwd_slots(const sa_dims& d, const CacheArgs& c, const void* q) {
  int cus = device_cus();
  if (cus <= 0) cus = 256;
  const bool alias = c.v == c.k && c.v_ld == c.k_ld && c.v_hs == c.k_hs;
  const bool one_per_cu = fwd_uses_mfma(d, c, q) && !alias && d.d_kq >= 512;
  return (long long)cus * (one_per_cu ? 1 : 2);
}

template <typename T, int DKQ, int DV, bool ALIAS>
static void launch_mfma_t(const sa_dims& d, const CacheArgs& c, const void* q, const int32_t* q_seq,
                          const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, const float* sel_bias, const int32_t* q_pos, int window, int n_q,
                          float scale_log2,
                          float* out, float* ws_o, float* ws_ml, const FwdPlan& plan, hipStream_t stream) {
  dim3 grid(plan.n_split, n_q * d.h_kv);
  hipLaunchKernelGGL((fwd_mfma_kernel<T, DKQ, DV, ALIAS>), grid, dim3(256), 0, stream, (const T*)q, (const T*)c.k,
                     c.k_ld, c.k_hs, (const T*)c.v, c.v_ld, c.v_hs, c.seq_row0, c.seq_len, q_seq, sel, sel_ld, n_sel,
                     sel_bias, q_pos, window, plan.list_max, d.h_q, d.h_kv, scale_log2, plan.n_split, plan.rows_per_split, out, ws_o, ws_ml);
}

// Compute units of the current device (cached per device; 0 if unknown).
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cus[dev] = n;
  }
  return cus[dev];
}

template <typename T, int DKQ>
static void launch_lds_t(const sa_dims& d, const CacheArgs& c, const void* q, const int32_t* q_seq,
                         const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, const float* sel_bias, const int32_t* q_pos, int window, int n_q,
                          float scale_log2,
                         float* out, float* ws_o, float* ws_ml, const FwdPlan& plan, hipStream_t stream) {
  dim3 grid(plan.n_split, n_q * d.h_kv);
  // at most one workgroup per CU: the query block goes through LDS
  const bool qlds = (long long)plan.n_split * n_q * d.h_kv <= device_cus();
#define SA_LDS_LAUNCH(QL)                                                                                        \
  hipLaunchKernelGGL((fwd_lds_kernel<T, DKQ, QL>), grid, dim3(256), 0, stream, (const T*)q, (const T*)c.k, c.k_ld,   \
                     c.k_hs, c.seq_row0, c.seq_len, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window, plan.list_max,   \
                     d.h_q, d.h_kv, scale_log2, plan.n_split, plan.rows_per_split, out, ws_o, ws_ml)
  if (qlds) SA_LDS_LAUNCH(true);
  else SA_LDS_LAUNCH(false);
#undef SA_LDS_LAUNCH
}

template <typename T>
static void dispatch_mfma(const sa_dims& d, const CacheArgs& c, const void* q, const int32_t* q_seq,
                          const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, const float* sel_bias, const int32_t* q_pos, int window, int n_q,
                          float scale_log2,
                          float* out, float* ws_o, float* ws_ml, const FwdPlan& plan, hipStream_t stream) {
  const bool alias = c.v == c.k && c.v_ld == c.k_ld && c.v_hs == c.k_hs;
  if (alias && d.d_v == 512 && (d.d_kq == 576 || d.d_kq == 512)) {   // MLA: gathers straight into LDS
    if (d.d_kq == 576) launch_lds_t<T, 576>(d, c, q, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window, n_q, scale_log2, out, ws_o, ws_ml, plan, stream);
    else launch_lds_t<T, 512>(d, c, q, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window, n_q, scale_log2, out, ws_o, ws_ml, plan, stream);
    return;
  }
#define SA_FWD_CASE(DKQ_, DV_)                                                                                  \
  if (d.d_kq == DKQ_ && d.d_v == DV_) {                                                                          \
    if (alias) launch_mfma_t<T, DKQ_, DV_, true>(d, c, q, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window, n_q, scale_log2, out, ws_o, \
                                                 ws_ml, plan, stream);                                           \
    else launch_mfma_t<T, DKQ_, DV_, false>(d, c, q, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window, n_q, scale_log2, out, ws_o,      \
                                            ws_ml, plan, stream);                                                \
    return;                                                                                                      \
  }
  // (V aliasing K at DV 512 went to the LDS kernel above)
  if (d.d_kq == 576 && d.d_v == 512) {
    launch_mfma_t<T, 576, 512, false>(d, c, q, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window, n_q, scale_log2, out, ws_o, ws_ml, plan, stream);
    return;
  }
  if (d.d_kq == 512 && d.d_v == 512) {
    launch_mfma_t<T, 512, 512, false>(d, c, q, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window, n_q, scale_log2, out, ws_o, ws_ml, plan, stream);
    return;
  }
  SA_FWD_CASE(256, 256)
  SA_FWD_CASE(128, 128)
#undef SA_FWD_CASE
}

template <typename T>
static void dispatch_valu(const sa_dims& d, const CacheArgs& c, const void* q, const int32_t* q_seq,
                          const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, const float* sel_bias, const int32_t* q_pos, int window, int n_q,
                          float scale_log2,
                          float* out, float* ws_o, float* ws_ml, const FwdPlan& plan, hipStream_t stream) {
  dim3 grid(plan.n_split, n_q * d.h_kv);
  const int per = (d.h_q / d.h_kv) * d.d_v;
  const KvPlain<T> kv{(const T*)c.k, c.k_ld, c.k_hs, (const T*)c.v, c.v_ld, c.v_hs};
#define SA_VALU_CASE(ACC_)                                                                                        \
  if (per <= 256 * ACC_) {                                                                                        \
    hipLaunchKernelGGL((fwd_valu_kernel<T, ACC_, KvPlain<T>>), grid, dim3(256), 0, stream, (const T*)q, kv,       \
                       c.seq_row0, c.seq_len, q_seq, sel, sel_ld, n_sel,                                          \
                       sel_bias, q_pos, window, plan.list_max, d.h_q, d.h_kv, d.d_kq, d.d_v, scale_log2, plan.n_split, plan.rows_per_split, out, ws_o,     \
                       ws_ml);                                                                                    \
    return;                                                                                                       \
  }
  SA_VALU_CASE(4)
  SA_VALU_CASE(16)
  SA_VALU_CASE(64)
#undef SA_VALU_CASE
}

hipError_t launch_fwd(const sa_dims& d, const CacheArgs& c, const void* q, const int32_t* q_seq, const int32_t* sel,
                      int64_t sel_ld, const int32_t* n_sel, const float* sel_bias, const int32_t* q_pos, int window,
                      int n_q, float scale, float* out, void* ws, const FwdPlan& plan, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  const float scale_log2 = scale * kLog2e;
  float* ws_o = (float*)ws;
  float* ws_ml = plan.n_split > 1 ? ws_o + (size_t)n_q * d.h_q * plan.n_split * d.d_v : nullptr;
  if (fwd_uses_mfma(d, c, q)) {
    if (d.dtype == SA_BF16) dispatch_mfma<bf16>(d, c, q, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window, n_q, scale_log2, out, ws_o, ws_ml, plan, stream);
    else dispatch_mfma<f16>(d, c, q, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window, n_q, scale_log2, out, ws_o, ws_ml, plan, stream);
  } else {
    switch (d.dtype) {
      case SA_F32: dispatch_valu<float>(d, c, q, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window, n_q, scale_log2, out, ws_o, ws_ml, plan, stream); break;
      case SA_F16: dispatch_valu<f16>(d, c, q, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window, n_q, scale_log2, out, ws_o, ws_ml, plan, stream); break;
      default: dispatch_valu<bf16>(d, c, q, q_seq, sel, sel_ld, n_sel, sel_bias, q_pos, window, n_q, scale_log2, out, ws_o, ws_ml, plan, stream); break;
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine(d, n_q, out, ws_o, ws_ml, plan, stream);
}

hipError_t launch_combine(const sa_dims& d, int n_q, float* out, const float* ws_o, const float* ws_ml,
                          const FwdPlan& plan, hipStream_t stream) {
  if (plan.n_split == 1 || n_q == 0) return hipSuccess;
  const int64_t n_out = (int64_t)n_q * d.h_q * d.d_v;
  const dim3 grid((unsigned)((n_out + kCombineThreads - 1) / kCombineThreads));
  if (plan.n_split <= 8 && d.d_v % 2 == 0 && ((uintptr_t)out & 7) == 0)
    hipLaunchKernelGGL(fwd_combine2_kernel<8>, dim3((unsigned)((n_out / 2 + kCombineThreads - 1) / kCombineThreads)),
                       dim3(kCombineThreads), 0, stream, ws_o, ws_ml, plan.n_split, d.d_v, n_out, out);
  else if (plan.n_split <= 40)
    hipLaunchKernelGGL(fwd_combine_kernel<40>, grid, dim3(kCombineThreads), 0, stream, ws_o, ws_ml, plan.n_split,
                       d.d_v, n_out, out);
  else
    hipLaunchKernelGGL(fwd_combine_kernel<8>, grid, dim3(kCombineThreads), 0, stream, ws_o, ws_ml, plan.n_split,
                       d.d_v, n_out, out);
  return hipGetLastError();
}

}  // namespace sa
