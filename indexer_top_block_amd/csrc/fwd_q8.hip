// Gather-fused attention over a q8_0 K/V cache.
//
// The pages put a quantized KV cache on the QSA attention path (qwen4exp commit
// series: support for a quantized KV cache there) and serve the sparse graph with K
// and V caches of type q8_0: blocks of 32 consecutive elements, each a float16
// scale d and 32 signed 8-bit codes c, element = d * c.  Here the codes and the
// scales are two planes of their own -- codes [rows][h_kv][d_kq] int8, scales
// [rows][h_kv][d_kq / 32] float16 -- so a row's codes are one 16-byte aligned run
// that gathers straight into LDS.
//
// MLA shapes (V = the first 512 elements of each K row, DKQ 512 or 576, up to 16
// query heads, f16/bf16 queries): `fwd_q8_lds_kernel`, 8 waves per workgroup.  Per
// 64-row tile each wave gathers 8 rows of codes into LDS (one instruction per row, 16
// bytes per lane) and those rows' scales (4 bytes per lane).  The scale never enters an MFMA operand
// rounded: S^T = K Q^T is taken one 32-element block at a time (one
// v_mfma_f32_16x16x32 per block, codes converted exactly to the query type) and
// each block's product is multiplied by that row's block scale in float32.  For
// O^T = V^T P^T the scale of (row, block) is folded into P before P is rounded to
// bf16 (P is rounded there in any case), and the codes of V^T come from LDS through
// ds_read_b64_tr_b8 (in each 16-lane group, lane i receives byte i % 8 of the eight
// bytes read by lanes i / 8, i / 8 + 2, ..., i / 8 + 14), which hands every lane one
// dimension of eight consecutive rows -- the A layout of the 16x16x32 product.
//
// Other shapes and dtypes: the generic VALU kernel with a q8_0 element reader.
#include "fwd_common.hpp"

namespace sa {

// Source of the gathers for tile rows that are not attended: zero codes, zero
// scales (a finite value that the -inf logit and the zero weight then discard).
__device__ __attribute__((aligned(16))) int8_t kQ8ZeroRow[1024] = {};

typedef int i32x2 __attribute__((ext_vector_type(2)));

// Eight signed codes (two dwords, lowest byte first) as eight exact values of T.
template <typename T>
__device__ __forceinline__ typename vec8<T>::type codes_to(uint32_t lo, uint32_t hi) {
  typename vec8<T>::type r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (T)(float)(int8_t)(lo >> (8 * e));
    r[4 + e] = (T)(float)(int8_t)(hi >> (8 * e));
  }
  return r;
}

__device__ __forceinline__ float half_lo(uint32_t w) { return (float)__builtin_bit_cast(f16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float half_hi(uint32_t w) { return (float)__builtin_bit_cast(f16, (uint16_t)(w >> 16)); }

__device__ __forceinline__ uint64_t shfl64(uint64_t x, int src) {
  const int lo = __shfl((int)(uint32_t)x, src), hi = __shfl((int)(uint32_t)(x >> 32), src);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// NW waves per workgroup (4 or 8).  With 8, two waves share each 16-row group of S
// (one takes the first half of the q8_0 blocks, the other the second, and the
// softmax sums the two partial tiles) and each wave owns 64 output dims, so a tile's
// conversion work -- the bulk of its VALU time -- is spread over twice the waves.
// QLDS: the query block is brought into LDS once and the waves read their operands
// from there, as in the bf16 kernel (launches of at most one workgroup per CU).
template <typename T, int DKQ, int NW, bool QLDS>
__global__ void __launch_bounds__(64 * NW, 8 / NW)
fwd_q8_lds_kernel(const T* __restrict__ q, const int8_t* __restrict__ kq, int64_t k_ld, int64_t k_hs,
                  const f16* __restrict__ ks, int64_t ks_ld, int64_t ks_hs, const int64_t* __restrict__ seq_row0,
                  const int32_t* __restrict__ seq_len, const int32_t* __restrict__ q_seq,
                  const int32_t* __restrict__ sel, int64_t sel_ld, const int32_t* __restrict__ n_sel, int list_max,
                  int h_q, int h_kv, float scale_log2, int n_split, int rows_per_split, float* __restrict__ out,
                  float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  typedef typename vec8<T>::type V8;
  typedef __attribute__((address_space(3))) void lds_void;
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  constexpr int DV = 512;
  constexpr int RT = kMfmaTile;                   // = 64: one list entry per lane
  constexpr int NBLK = DKQ / 32;                  // q8_0 blocks per K row = QK^T MFMA steps
  constexpr int KSPLIT = NW / 4;                  // waves sharing a 16-row group of S
  constexpr int KB = (NBLK / KSPLIT + 1) & ~1;    // blocks per such wave at most (even, so that
                                                  // every wave's first block starts a scale dword)
  constexpr int PITCH = DKQ + 16;                 // bytes per LDS code row: 4 or 20 dwords mod 64 banks
  constexpr int NCH = DKQ / 16;                   // 16-byte chunks per code row
  constexpr int SRCW = NBLK / 2;                  // scale dwords per cache row
  constexpr int SCW = (SRCW + 1) & ~1;            // scale dwords per LDS row (even: 8-byte aligned rows)
  constexpr int RPW = RT / NW;                    // rows gathered per wave
  constexpr int NSW = RPW * SCW;                  // scale dwords gathered per wave
  constexpr int DVW = DV / NW;                    // output dims owned by one wave
  constexpr int NTW = DVW / 16;                   // its 16-dim MFMA tiles
  constexpr int BPW = DVW / 32;                   // its q8_0 blocks of V
  constexpr int SP = RT + 4;                      // pitch of the transposed score tiles (floats)
  static_assert(DKQ == 512 || DKQ == 576, "MLA shapes only");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  __shared__ __attribute__((aligned(16))) int8_t kt[RT * PITCH];
  __shared__ __attribute__((aligned(16))) uint32_t sct[RT * SCW];
  __shared__ __attribute__((aligned(16))) float st[KSPLIT * 16 * SP];   // scaled partial scores, [part][head][row]
  // Query block in LDS (QLDS): 16-byte chunk p holds chunk p % QP of head p / QP; one
  // pad chunk per head spreads the heads over the banks.
  constexpr int QCH = DKQ / 8;
  constexpr int QP = QCH + 1;
  constexpr int QINST = (16 * QP + kWave - 1) / kWave;   // wave instructions for 16 heads
  __shared__ __attribute__((aligned(16))) T qs[QLDS ? QINST * kWave * 8 : 8];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 15, grp = lane >> 4;
  const int split = blockIdx.x;
  const int i = blockIdx.y / h_kv, g = blockIdx.y % h_kv;
  const int G = h_q / h_kv;
  const int32_t* list = sel + (int64_t)i * sel_ld;
  const int r_begin = split * rows_per_split;
  const int lim = (int)min(sel_ld, (int64_t)list_max) - 1;
  auto list_at = [&](int t) { return list[min(r_begin + t * RT + lane, lim)]; };
  const int pre0 = list_at(0), pre1 = list_at(1), pre2 = list_at(2);
  const SeqMeta sm = seq_meta(q_seq, seq_len, seq_row0, nullptr, i);
  const int L = sm.len;
  const int64_t row0 = sm.row0;
  const int cnt = max(0, (int)min((int64_t)n_sel[i], min(sel_ld, (int64_t)list_max)));
  // the last split takes every remaining row (the tail rows when they have no split of their own)
  const int r_end = split == n_split - 1 ? cnt : min(cnt, r_begin + rows_per_split);
  const int n_tiles = r_end > r_begin ? (r_end - r_begin + RT - 1) / RT : 0;
  const int8_t* kqg = kq + (int64_t)g * k_hs;
  const f16* ksg = ks + (int64_t)g * ks_hs;

  const int wr = (wave % 4) * 16;                 // this wave's 16 rows of S
  const int kb0 = (wave / 4) * KB;                // and its first q8_0 block
  const int nkb = min(KB, NBLK - kb0);            // and its block count (wave-uniform)
  const int dvb = wave * DVW;                     // its output dims
  const T* qbase = q + ((int64_t)i * h_q + (int64_t)g * G) * DKQ;
  V8 qf[KB];
  if constexpr (QLDS) {
    // issued with the list reads; read into registers after the first tile's barrier.
    // Chunks past the G heads and the pad chunks repeat valid data.
    for (int u = wave; u < QINST; u += NW) {
      const int p = u * kWave + lane;
      const int h = p / QP < G ? p / QP : 0;
      const int cc = p % QP < QCH ? p % QP : QCH - 1;
      __builtin_amdgcn_global_load_lds((const void*)(qbase + h * DKQ + cc * 8), (lds_void*)&qs[u * kWave * 8], 16, 0,
                                       0);
    }
  } else {
    const T* qh = qbase + (col < G ? col : 0) * DKQ + grp * 8 + kb0 * 32;
#pragma unroll
    for (int b = 0; b < KB; ++b) qf[b] = b < nkb ? *reinterpret_cast<const V8*>(qh + b * 32) : V8{};
    if (col >= G) {
#pragma unroll
      for (int b = 0; b < KB; ++b) qf[b] = V8{};
    }
  }
  float m = -INFINITY, lsum = 0.f;
  f32x4 o[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Lane l: the code and scale addresses of tile row l (rows not attended read the
  // zero row), and the mask of attended rows.
  auto row_src = [&](int pos, int t, uint64_t* valid, uint64_t* sp) {
    const int64_t row = tile_row(pos, r_begin + t * RT + lane, r_end, L, row0);
    *valid = __ballot(row >= 0);
    *sp = row >= 0 ? (uint64_t)(ksg + row * ks_ld) : (uint64_t)kQ8ZeroRow;
    return row >= 0 ? (uint64_t)(kqg + row * k_ld) : (uint64_t)kQ8ZeroRow;
  };
  // Wave w gathers the codes of rows RPW w .. RPW w + RPW - 1 (one instruction per
  // row, NCH lanes of 16 bytes) and their scales (SRCW dwords per row; the padding
  // dword of an LDS row repeats the last one).
  auto issue = [&](uint64_t kp, uint64_t sp) {
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int r = wave * RPW + u;
      const uint64_t base = (uint64_t)readlane64((int64_t)kp, r);
      if (lane < NCH)
        __builtin_amdgcn_global_load_lds((const void*)(base + lane * 16), (lds_void*)&kt[r * PITCH], 16, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < (NSW + 63) / 64; ++u) {
      const int f = u * 64 + lane;
      const int rl = min(f / SCW, RPW - 1);
      const int dw = min(f % SCW, SRCW - 1);
      const uint64_t sbase = shfl64(sp, wave * RPW + rl);
      if (f < NSW)
        __builtin_amdgcn_global_load_lds((const void*)(sbase + dw * 4), (lds_void*)&sct[wave * NSW + u * 64], 4, 0,
                                         0);
    }
  };

  auto compute = [&](uint64_t valid) {
    {
      // partial S^T over this wave's blocks: lane (col, grp) gets rows wr + 4 grp + j
      // every LDS read of the tile's part first (codes of the wave's blocks, scale
      // dwords of its 4 rows per lane), then the products
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      const int8_t* arow = &kt[(wr + col) * PITCH + grp * 8 + kb0 * 32];
      const uint32_t* srow = &sct[(wr + 4 * grp) * SCW + kb0 / 2];
      uint2 cw[KB];
      uint32_t sw[4][KB / 2];
#pragma unroll
      for (int b = 0; b < KB; ++b)
        if (b < nkb) cw[b] = *reinterpret_cast<const uint2*>(arow + b * 32);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int u = 0; u < KB / 2; ++u)
          if (2 * u < nkb) sw[j][u] = srow[j * SCW + u];
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        if (b < nkb) {
          const f32x4 part = mfma16x16x32<T>(codes_to<T>(cw[b].x, cw[b].y), qf[b], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t w = sw[j][b / 2];
            s[j] += ((b & 1) ? half_hi(w) : half_lo(w)) * part[j];
          }
        }
      }
      *reinterpret_cast<f32x4*>(st + ((wave / 4) * 16 + col) * SP + wr + 4 * grp) = s * scale_log2;
    }
    lds_barrier();
    // Lane (col, grp) takes head col's rows 32 kk + 8 grp + j, j < 8: the B layout of
    // the 16x16x32 product.
    float xs[2][8];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[kk][j] = 0.f;
#pragma unroll
      for (int part = 0; part < KSPLIT; ++part) {
        const float* src = st + (part * 16 + col) * SP + 32 * kk + 8 * grp;
        const f32x4 a = *reinterpret_cast<const f32x4*>(src);
        const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xs[kk][j] += a[j];
          xs[kk][4 + j] += b[j];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (!((valid >> (32 * kk + 8 * grp + j)) & 1ull)) xs[kk][j] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, xs[kk][j]);
    mx = max_xor32(max_xor16(mx));
    const float m_new = fmaxf(m, mx);
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m - m_new);
    float p[2][8];
    float psum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[kk][j] = (xs[kk][j] == -INFINITY) ? 0.f : fast_exp2(xs[kk][j] - m_new);
        psum += p[kk][j];
      }
    psum = sum_xor32(sum_xor16(psum));
    lsum = lsum * alpha + psum;
    m = m_new;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) o[nt] *= alpha;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // the scales of this lane's 8 rows for the wave's BPW blocks of V
      uint32_t sw[8][BPW / 2];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int u = 0; u < BPW / 2; ++u) sw[j][u] = sct[(32 * kk + 8 * grp + j) * SCW + dvb / 64 + u];
      // V^T codes: in each 16-lane group lane c reads row 32 kk + 8 grp + c / 2,
      // bytes 8 (c % 2) .. of the 16-dim tile; lane i then holds dim i of the 8 rows
      const int8_t* vrow = &kt[(32 * kk + 8 * grp + (col >> 1)) * PITCH + dvb + 8 * (col & 1)];
      i32x2 vc[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) vc[nt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vrow + nt * 16));
#pragma unroll
      for (int bb = 0; bb < BPW; ++bb) {
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t w = sw[j][bb / 2];
          const float d = (bb & 1) ? half_hi(w) : half_lo(w);
          pb[j] = (bf16)(p[kk][j] * d);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int nt = 2 * bb + h;
          o[nt] = mfma16x16x32<bf16>(codes_to<bf16>((uint32_t)vc[nt].x, (uint32_t)vc[nt].y), pb, o[nt]);
        }
      }
    }
  };

  if (n_tiles > 0) {
    uint64_t v0, v1, s0, s1;
    {
      const uint64_t k0 = row_src(pre0, 0, &v0, &s0);
      issue(k0, s0);
    }
    int raw1 = pre1, raw2 = pre2;
    for (int t = 0; t < n_tiles; ++t) {
      __builtin_amdgcn_s_waitcnt(0);              // this wave's gathers of tile t
      __syncthreads();                            // everyone's
      if constexpr (QLDS) {
        if (t == 0) {                             // the query block landed with the first tile
          const V8* qrow = reinterpret_cast<const V8*>(qs) + (col < G ? col : 0) * QP + grp + kb0 * 4;
#pragma unroll
          for (int b = 0; b < KB; ++b) qf[b] = b < nkb && col < G ? qrow[b * 4] : V8{};
        }
      }
      const int raw_new = list_at(t + 3);
      const uint64_t k1 = row_src(raw1, t + 1, &v1, &s1);
      compute(v0);
      __syncthreads();                            // the buffers are free
      if (t + 1 < n_tiles) issue(k1, s1);
      v0 = v1;
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

// ---------------------------------------------------------------------------- host

#ifndef SA_Q8_WAVES
#define SA_Q8_WAVES 8
#endif
constexpr int kQ8Waves = SA_Q8_WAVES;

static bool aligned_to(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool fwd_q8_uses_lds(const sa_dims& d, const Q8Args& kv, const void* q) {
  if (d.dtype != SA_F16 && d.dtype != SA_BF16) return false;
  if (d.h_q / d.h_kv > 16 || d.d_v != 512 || (d.d_kq != 512 && d.d_kq != 576)) return false;
  const bool alias = kv.v == kv.k && kv.v_ld == kv.k_ld && kv.v_hs == kv.k_hs && kv.vs == kv.ks &&
                     kv.vs_ld == kv.ks_ld && kv.vs_hs == kv.ks_hs;
  if (!alias) return false;
  if (!aligned_to(kv.k, 16) || kv.k_ld % 16 || kv.k_hs % 16) return false;
  if (!aligned_to(kv.ks, 4) || kv.ks_ld % 2 || kv.ks_hs % 2) return false;
  return aligned_to(q, 16);
}

template <typename T, int DKQ>
static void launch_q8_lds_t(const sa_dims& d, const CacheArgs& c, const Q8Args& kv, const void* q,
                            const int32_t* q_seq, const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, int n_q,
                            float scale_log2, float* out, float* ws_o, float* ws_ml, const FwdPlan& plan,
                            hipStream_t stream) {
  dim3 grid(plan.n_split, n_q * d.h_kv);
  // at most one workgroup per CU: the query block goes through LDS
  const bool qlds = (long long)plan.n_split * n_q * d.h_kv <= device_cus();
#define SA_Q8_LDS_LAUNCH(QL)                                                                                         \
  hipLaunchKernelGGL((fwd_q8_lds_kernel<T, DKQ, kQ8Waves, QL>), grid, dim3(64 * kQ8Waves), 0, stream, (const T*)q,   \
                     (const int8_t*)kv.k, kv.k_ld, kv.k_hs, (const f16*)kv.ks, kv.ks_ld, kv.ks_hs, c.seq_row0,      \
                     c.seq_len, q_seq, sel, sel_ld, n_sel, plan.list_max, d.h_q, d.h_kv, scale_log2, plan.n_split,  \
                     plan.rows_per_split, out, ws_o, ws_ml)
  if (qlds) SA_Q8_LDS_LAUNCH(true);
  else SA_Q8_LDS_LAUNCH(false);
#undef SA_Q8_LDS_LAUNCH
}

template <typename T>
static void dispatch_q8_valu(const sa_dims& d, const CacheArgs& c, const Q8Args& a, const void* q,
                             const int32_t* q_seq, const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, int n_q,
                             float scale_log2, float* out, float* ws_o, float* ws_ml, const FwdPlan& plan,
                             hipStream_t stream) {
  dim3 grid(plan.n_split, n_q * d.h_kv);
  const int per = (d.h_q / d.h_kv) * d.d_v;
  const KvQ8 kv{(const int8_t*)a.k, a.k_ld, a.k_hs, (const f16*)a.ks, a.ks_ld, a.ks_hs,
                (const int8_t*)a.v, a.v_ld, a.v_hs, (const f16*)a.vs, a.vs_ld, a.vs_hs};
#define SA_Q8_VALU_CASE(ACC_)                                                                                     \
  if (per <= 256 * ACC_) {                                                                                        \
    hipLaunchKernelGGL((fwd_valu_kernel<T, ACC_, KvQ8>), grid, dim3(256), 0, stream, (const T*)q, kv, c.seq_row0, \
                       c.seq_len, q_seq, sel, sel_ld, n_sel, nullptr, nullptr, 0, plan.list_max, d.h_q, d.h_kv,    \
                       d.d_kq, d.d_v, scale_log2, plan.n_split, plan.rows_per_split, out, ws_o, ws_ml);            \
    return;                                                                                                       \
  }
  SA_Q8_VALU_CASE(4)
  SA_Q8_VALU_CASE(16)
  SA_Q8_VALU_CASE(64)
#undef SA_Q8_VALU_CASE
}

hipError_t launch_fwd_q8(const sa_dims& d, const CacheArgs& c, const Q8Args& kv, const void* q, const int32_t* q_seq,
                         const int32_t* sel, int64_t sel_ld, const int32_t* n_sel, int n_q, float scale, float* out,
                         void* ws, const FwdPlan& plan, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  const float scale_log2 = scale * kLog2e;
  float* ws_o = (float*)ws;
  float* ws_ml = plan.n_split > 1 ? ws_o + (size_t)n_q * d.h_q * plan.n_split * d.d_v : nullptr;
  if (fwd_q8_uses_lds(d, kv, q)) {
    if (d.dtype == SA_BF16) {
      if (d.d_kq == 576) launch_q8_lds_t<bf16, 576>(d, c, kv, q, q_seq, sel, sel_ld, n_sel, n_q, scale_log2, out, ws_o, ws_ml, plan, stream);
      else launch_q8_lds_t<bf16, 512>(d, c, kv, q, q_seq, sel, sel_ld, n_sel, n_q, scale_log2, out, ws_o, ws_ml, plan, stream);
    } else {
      if (d.d_kq == 576) launch_q8_lds_t<f16, 576>(d, c, kv, q, q_seq, sel, sel_ld, n_sel, n_q, scale_log2, out, ws_o, ws_ml, plan, stream);
      else launch_q8_lds_t<f16, 512>(d, c, kv, q, q_seq, sel, sel_ld, n_sel, n_q, scale_log2, out, ws_o, ws_ml, plan, stream);
    }
  } else {
    switch (d.dtype) {
      case SA_F32: dispatch_q8_valu<float>(d, c, kv, q, q_seq, sel, sel_ld, n_sel, n_q, scale_log2, out, ws_o, ws_ml, plan, stream); break;
      case SA_F16: dispatch_q8_valu<f16>(d, c, kv, q, q_seq, sel, sel_ld, n_sel, n_q, scale_log2, out, ws_o, ws_ml, plan, stream); break;
      default: dispatch_q8_valu<bf16>(d, c, kv, q, q_seq, sel, sel_ld, n_sel, n_q, scale_log2, out, ws_o, ws_ml, plan, stream); break;
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine(d, n_q, out, ws_o, ws_ml, plan, stream);
}

}  // namespace sa
