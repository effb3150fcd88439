// The MLA attention of one (query token, KV head, split) with rows gathered straight
// into LDS, as a device function over a source of list entries: the kernel of
// fwd.hip reads the list that sparse_attn_select wrote, the fused select + attention
// kernel of select_fwd.hip the list its own workgroup just selected into LDS.
//
// For V aliasing K with DV = 512 (DKQ 512 or 576, the MLA shapes) the rows go from
// memory straight into LDS (global_load_lds_dwordx4: each lane names its own 16
// source bytes, and a wave instruction fills 1 KiB of LDS contiguously).  One wave
// instruction therefore carries the first 512 dims of one row, with a wave-uniform
// row offset read from the lane that holds it; the 64 dims past 512 (DKQ 576) go 8
// rows to an instruction into a dense region whose 16-byte chunks are XOR-swizzled
// by row so that the MFMA operand reads spread over the LDS banks.  One tile buffer
// per workgroup keeps LDS at 78 KiB, so two workgroups share a CU and one's gathers
// overlap the other's compute.  There are no register buffers and no landing
// stores; the compute is that of the kernel above.
//
// QLDS (launches of at most one workgroup per CU, e.g. one decode token's splits):
// every wave needs the whole query block as its MFMA B operand, and four register
// copies of it cost a CU more load time than the tile's rows.  The block is then
// brought into LDS once, with the rows, and each wave reads its operands from there;
// the extra 19 KiB of LDS leave one workgroup per CU.
#pragma once

#include "fwd_common.hpp"

namespace sa {

// LDS of the kernel: one tile buffer (78 KiB with the score tile), so that two
// workgroups share a CU -- one computes while the other's gathers land -- and, with
// QLDS, the query block.
template <typename T, int DKQ, bool QLDS>
struct alignas(16) FwdLdsSmem {
  static_assert(DKQ == 512 || DKQ == 576, "MLA shapes only");
  static constexpr int RT = kMfmaTile;               // = 64: one list entry per lane
  static constexpr int MP = 512 + 16;                // pitch of the main region (elements): 8 dwords mod 64 banks
  static constexpr int REM = (DKQ - 512) / 8;        // 16-byte chunks per row past 512 dims (0 or 8)
  static constexpr int REMP = REM > 0 ? REM : 1;
  static constexpr int SP = RT + 4;                  // pitch of the transposed score tile (floats)
  // Query block in LDS (QLDS): 16-byte chunk p holds chunk p % QP of head p / QP; one
  // pad chunk per head spreads the heads over the banks.
  static constexpr int QCH = DKQ / 8;
  static constexpr int QP = QCH + 1;
  static constexpr int QINST = (16 * QP + kWave - 1) / kWave;   // wave instructions for 16 heads
  T kmain[RT * MP];
  T krem[RT * REMP * 8];
  float st[16 * SP];                                 // scaled scores, [head][row]
  T qs[QLDS ? QINST * kWave * 8 : 8];
};

// List entries as sparse_attn_select writes them: row i of sel (entries past the
// capacity are clamped, not guarded), with an optional bias per entry, and the count
// n_sel[i] clamped to the capacity.
struct GlobalList {
  const int32_t* list;
  const float* blist;                                // additive logit bias per entry, or null
  int lim;                                           // the last entry that may be read
  const int32_t* n_sel_i;
  int64_t cap;                                       // min(sel_ld, list capacity)
  __device__ __forceinline__ int at(int j) const { return list[min(j, lim)]; }
  __device__ __forceinline__ float bias(int j) const { return blist ? blist[min(j, lim)] : 0.f; }
  __device__ __forceinline__ bool has_bias() const { return blist != nullptr; }
  __device__ __forceinline__ int count() const { return max(0, (int)min((int64_t)*n_sel_i, cap)); }
  // the query's sequence (read here, with the first list entries in flight)
  __device__ __forceinline__ SeqMeta meta(const int32_t* q_seq, const int32_t* seq_len, const int64_t* seq_row0,
                                          int i) const {
    return seq_meta(q_seq, seq_len, seq_row0, nullptr, i);
  }
};

template <typename T, int DKQ, bool QLDS, typename ListSrc, bool QSTREAM = false>
__device__ __forceinline__ void fwd_lds_body(FwdLdsSmem<T, DKQ, QLDS>& lds, const ListSrc& ls,
                                             const T* __restrict__ q, const T* __restrict__ k, int64_t k_ld,
                                             int64_t k_hs, const int64_t* __restrict__ seq_row0,
                                             const int32_t* __restrict__ seq_len, const int32_t* __restrict__ q_seq,
                                             const int32_t* __restrict__ q_pos, int window, int h_q, int h_kv,
                                             float scale_log2, int n_split, int rows_per_split,
                                             float* __restrict__ out, float* __restrict__ ws_o,
                                             float* __restrict__ ws_ml) {
  static_assert(QLDS || !QSTREAM, "the query streams from LDS only when it is there");
  typedef FwdLdsSmem<T, DKQ, QLDS> S;
  typedef typename vec8<T>::type V8;
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int DV = 512;
  constexpr int RT = S::RT;
  constexpr int KST = DKQ / 32;       // QK^T MFMA steps
  constexpr int MP = S::MP;
  constexpr int REM = S::REM;
  constexpr int REMP = S::REMP;
  constexpr int DVW = DV / 4;         // output dims owned by one wave
  constexpr int NTW = DVW / 16;       // its 16-dim MFMA tiles
  constexpr int SP = S::SP;
  constexpr int QCH = S::QCH;
  constexpr int QP = S::QP;
  constexpr int QINST = S::QINST;
  T* const kmain0 = lds.kmain;
  T* const krem0 = lds.krem;
  float* const st = lds.st;
  T* const qs = lds.qs;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 15, grp = lane >> 4;
  const int split = blockIdx.x;
  const int i = blockIdx.y / h_kv, g = blockIdx.y % h_kv;
  const int G = h_q / h_kv;
  const int r_begin = split * rows_per_split;
  auto list_at = [&](int t) { return ls.at(r_begin + t * RT + lane); };
  auto bias_at = [&](int t) { return ls.bias(r_begin + t * RT + lane); };
  const int pre0 = list_at(0), pre1 = list_at(1), pre2 = list_at(2);
  const SeqMeta sm = ls.meta(q_seq, seq_len, seq_row0, i);
  const int L = sm.len;
  const int64_t row0 = sm.row0;
  const int cnt = ls.count();
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

  const T* qbase = q + ((int64_t)i * h_q + (int64_t)g * G) * DKQ;
  V8 qf[KST];
  if constexpr (QLDS) {
    // issued with the list reads; read into registers after the first tile's barrier.
    // Chunks past the G heads and the pad chunks repeat valid data.
    for (int u = wave; u < QINST; u += 256 / kWave) {
      const int p = u * kWave + lane;
      const int h = p / QP < G ? p / QP : 0;
      const int cc = p % QP < QCH ? p % QP : QCH - 1;
      __builtin_amdgcn_global_load_lds((const void*)(qbase + h * DKQ + cc * 8), (lds_void*)&qs[u * kWave * 8], 16, 0,
                                       0);
    }
  } else {
    const T* qh = qbase + (col < G ? col : 0) * DKQ + grp * 8;
#pragma unroll
    for (int st_ = 0; st_ < KST; ++st_) qf[st_] = *reinterpret_cast<const V8*>(qh + st_ * 32);
    if (col >= G) {
#pragma unroll
      for (int st_ = 0; st_ < KST; ++st_) qf[st_] = V8{};
    }
  }
  float m = -INFINITY, lsum = 0.f;
  f32x4 o[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A tile's rows: lane l has row l's element offset from kg (rows not selected
  // point at this query's own Q row: finite values, masked to -inf), and a mask
  // marks the selected rows.
  const int64_t safe_k = qbase - kg;
  auto row_off = [&](int pos, int t, uint64_t* valid) {
    const int j = r_begin + t * RT + lane;
    const int64_t row = tile_row(row_pos(pos, j, cnt, w0, wlen), j, r_end, L, row0);
    *valid = __ballot(row >= 0);
    return row >= 0 ? row * k_ld : safe_k;
  };
  // Issue tile t's gathers into LDS buffer b: wave w carries rows w*16 .. w*16+15
  // (one instruction each) and, for DKQ 576, rows w*16 .. w*16+15 of the dims past
  // 512 (two instructions of 8 rows).
  auto issue = [&](T* kmain, T* krem, int64_t ko) {
    const T* lanep = kg + lane * 8;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = wave * 16 + u;
      const int64_t off = readlane64(ko, r);
      __builtin_amdgcn_global_load_lds((const void*)(lanep + off), (lds_void*)&kmain[r * MP], 16, 0, 0);
    }
    if constexpr (REM > 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = wave * 16 + u * 8 + lane / REM;   // this lane's row
        const int p = lane % REM;                       // its LDS chunk within the row
        const int c = p ^ (r & 7);                      // the source chunk stored there
        const int lo = __shfl((int)(uint32_t)ko, r), hi = __shfl((int)(uint32_t)((uint64_t)ko >> 32), r);
        const int64_t off = (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
        __builtin_amdgcn_global_load_lds((const void*)(kg + off + 512 + c * 8),
                                         (lds_void*)&krem[(wave * 16 + u * 8) * REM * 8], 16, 0, 0);
      }
    }
  };

  const int wr = wave * 16;                          // this wave's 16 rows of S
  const int dvb = wave * DVW;                        // this wave's output dims
  auto compute = [&](const T* kmain, const T* krem, uint64_t valid, float bias) {
    {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      const int r = wr + col;
      const T* arow = &kmain[r * MP + grp * 8];
#pragma unroll
      for (int st_ = 0; st_ < KST; ++st_) {
        V8 a;
        if (st_ < 16) {
          a = *reinterpret_cast<const V8*>(arow + st_ * 32);
        } else {
          const int c = (st_ - 16) * 4 + grp;           // chunk past 512 dims
          a = *reinterpret_cast<const V8*>(&krem[(r * REMP + (c ^ (r & 7))) * 8]);
        }
        V8 qv;
        if constexpr (QSTREAM) {                        // the query operand read per step
          qv = reinterpret_cast<const V8*>(qs)[(col < G ? col : 0) * QP + grp + st_ * 4];
          if (col >= G) qv = V8{};
        } else {
          qv = qf[st_];
        }
        if (st_ & 1) s1 = mfma16x16x32<T>(a, qv, s1);
        else s0 = mfma16x16x32<T>(a, qv, s0);
      }
      if constexpr (!QSTREAM) {
        // four A reads ahead of the products (the compiler's own order keeps one or
        // two, and each product then waits on an LDS round trip)
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);           // 4 LDS reads
#pragma unroll
        for (int i = 0; i < KST - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // 1 MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // 1 LDS read
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      const f32x4 sacc = s0 + s1;
      f32x4 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float b = ls.has_bias() ? __shfl(bias, wr + 4 * grp + j) * kLog2e : 0.f;
        x[j] = ((valid >> (wr + 4 * grp + j)) & 1ull) ? sacc[j] * scale_log2 + b : -INFINITY;
      }
      *reinterpret_cast<f32x4*>(st + col * SP + wr + 4 * grp) = x;
    }
    lds_barrier();
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
    if (__ballot(alpha != 1.f) != 0ull) {            // the running max moved (else nothing to rescale)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) o[nt] *= alpha;
    }
    // V^T operand by transposing LDS reads: in each 16-lane group, lane r reads 4
    // dims at row 4*grp + r/4, dims 4*(r%4) .. +4 of the 16-dim tile, and lane i then
    // holds dim i of rows 4*grp .. 4*grp+3 -- the A-operand layout.  Two such reads,
    // rows 32*kk2 + 4*grp + [0, 4) and 16 rows further, make a lane group's 8 k-values
    // of one 16x16x32 product, with P's pieces pb[2*kk2] and pb[2*kk2 + 1].
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      const T* vrow0 = &kmain[(32 * kk2 + 4 * grp + (col >> 2)) * MP + dvb + 4 * (col & 3)];
      const T* vrow1 = vrow0 + 16 * MP;
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

  // Per tile: wait for its gathers, compute it, then gather the next one into the
  // same buffer (the other workgroup on the CU runs meanwhile); the list runs two
  // tiles ahead of the gathers.
  if (n_tiles > 0) {
    uint64_t v0, v1;
    float b0 = bias_at(0);
    issue(kmain0, krem0, row_off(pre0, 0, &v0));
    int raw1 = pre1, raw2 = pre2;                    // list entries of tiles t+1 and t+2
    for (int t = 0; t < n_tiles; ++t) {
      __builtin_amdgcn_s_waitcnt(0);                 // this wave's gathers of tile t
      __syncthreads();                               // everyone's
      if constexpr (QLDS && !QSTREAM) {
        if (t == 0) {                                // the query block landed with the first tile
          const V8* qrow = reinterpret_cast<const V8*>(qs) + (col < G ? col : 0) * QP + grp;
#pragma unroll
          for (int st_ = 0; st_ < KST; ++st_) qf[st_] = qrow[st_ * 4];
          if (col >= G) {
#pragma unroll
            for (int st_ = 0; st_ < KST; ++st_) qf[st_] = V8{};
          }
        }
      }
      const int raw_new = list_at(t + 3);
      const int64_t ko1 = row_off(raw1, t + 1, &v1);
      const float b1 = bias_at(t + 1);
      compute(kmain0, krem0, v0, b0);
      __syncthreads();                               // the buffer is free
      if (t + 1 < n_tiles) issue(kmain0, krem0, ko1);
      v0 = v1;
      b0 = b1;
      raw1 = raw2;
      raw2 = raw_new;
    }
  }
  if constexpr (QLDS) {
    if (n_tiles == 0) __builtin_amdgcn_s_waitcnt(0);   // the query block's loads land before the wave ends
  }

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

}  // namespace sa
