// Indexer block scores: s[i][b] = sum_h max(0, qidx[i][h] . kpool[b]).
//
// The rectification is applied per head before the head sum (llama.cpp commit
// "llama: QSA sparse attention for qwen4exp", the paragraph on the direct index
// comparison against the reference implementation), and each query meets only its
// own sequence's blocks ("qwen4exp: support a non-unified KV cache in QSA").
//
// MFMA path (f16 / bf16, h_idx a multiple of 32, d_idx in {64, 128, 256}): a wave
// holds one query's indexer heads as the M operand of v_mfma_f32_32x32x16 in
// registers (staged once per workgroup through LDS) and streams 32 pooled keys per
// tile as the N operand from HBM straight into LDS (global_load_lds, four whole keys
// per wave instruction).  The contraction index is permuted identically in both operands (lane half
// hf, step s, slot j <-> dim hf*D/2 + s*8 + j), which leaves the dot products
// unchanged.  The epilogue rectifies the 32x32 fp32 tile, sums the 16 rows a lane
// holds, and adds the partner lane (lane ^ 32) that holds the other 16 rows of the
// same block column.
//
// VALU path (any dtype or shape): the query's heads are staged in LDS as float and
// each thread computes the rectified dot products of one block for a quarter of
// the heads.
#include "sa_common.hpp"
#include "sa_launch.hpp"
#include "select_wide.hpp"

namespace sa {

// ----------------------------------------------------------------------------- MFMA

template <typename T>
__device__ __forceinline__ f32x16 mfma32x32x16(const typename vec8<T>::type& a, const typename vec8<T>::type& b,
                                               const f32x16& c);
template <>
__device__ __forceinline__ f32x16 mfma32x32x16<bf16>(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32x32x16<f16>(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// max(x, 0) as one integer max on the bit pattern: every float with the sign bit set
// (negatives and -0) reads as a negative integer and becomes +0; the rest keep their
// value.  fmaxf takes a second instruction per element (it quiets a possible
// signalling NaN first) and gives the same result for every non-NaN x.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

constexpr int kScoreWaves = 4;        // waves per workgroup
constexpr int kScoreTile = 32;        // blocks per wave tile (MFMA N)
static_assert(kScoreTile == kCandTile, "one candidate tile per wave");

// grid = (ceil(max_blocks / (4 * 32)), n_q); wave w of workgroup x scores blocks
// [(x*4 + w) * 32, +32) of query blockIdx.y (with pooling, the grid is one-dimensional
// and x, y come from the workgroup index).
// With pooling (POOL), the launch also does sparse_attn_pool's work: rows y >= n_q
// of the grid pool sequence y - n_q's new blocks into the cache exactly as the pool
// kernel does, and a scoring wave takes the pooled keys of new blocks in its range
// -- blocks [n_pooled_in[s], end_s), which the cache does not hold yet -- from the
// raw keys itself, with the same arithmetic (float sum in index order, divided by c,
// rounded to the cache type), instead of from the cache.  The two kinds of
// workgroups share nothing, so the result is that of pool followed by score.
template <typename T>
struct PoolArgs {
  const T* kidx;
  int64_t kidx_ld;
  T* kpool;                           // written by the pooling workgroups only
  const int64_t* seq_row0;
  const int32_t* n_in;
  int32_t* n_out;                     // not n_in (the host checks)
  int max_new;
  int pool_wgs, n_seq;                // pooling workgroups per sequence; sequences
  int gx;                             // scoring workgroups per query
  // Optional (null: none): the candidate list of the selection, `cand_ld` words per
  // query token: for each wave's kCandTile blocks (tile g) its cand_keep best keys,
  // then their block indices, a record of cand_keep / 2 16-byte pieces laid out for
  // the select's loads (cand_offset in select_wide.hpp: the workgroup's thread t reads
  // its pieces q at q * kCandThreads + t).  A wave past the row's blocks writes nothing.
  uint32_t* cand;
  int64_t cand_ld;
  int cand_keep, cand_tpt;
};

template <typename T, int MT, int D, bool POOL>
__global__ void __launch_bounds__(256)
score_mfma_kernel(const T* __restrict__ qidx, const T* __restrict__ kpool, int64_t kpool_ld,
                  const int64_t* __restrict__ seq_blk0, const int32_t* __restrict__ seq_len,
                  const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c,
                  float* __restrict__ scores, int64_t scores_ld, PoolArgs<T> pa) {
  int wx = blockIdx.x, wy = blockIdx.y;             // this workgroup's block range and query
  if constexpr (POOL) {
    // one-dimensional grid, the pooling workgroups first (so that they start first)
    const int id = blockIdx.x, n_pool = pa.pool_wgs * pa.n_seq;
    if (id < n_pool) {                               // a pooling workgroup
      const int s = id / pa.pool_wgs, px = id % pa.pool_wgs;
      const int start = max(pa.n_in[s], 0);
      const int end = (int)min((long long)(max(seq_len[s], 0) / c), (long long)start + pa.max_new);
      const long long total = (long long)max(end - start, 0) * D;
      const int64_t row0 = pa.seq_row0[s], blk0 = seq_blk0[s];
      for (long long e = (long long)px * 256 + threadIdx.x; e < total; e += (long long)pa.pool_wgs * 256) {
        const int64_t b = start + e / D;
        const int d = (int)(e % D);
        const T* src = pa.kidx + (row0 + b * c) * pa.kidx_ld + d;
        pa.kpool[(blk0 + b) * kpool_ld + d] = (T)(pool_sum(src, pa.kidx_ld, c) / (float)c);
      }
      if (px == 0 && threadIdx.x == 0) pa.n_out[s] = end;
      return;
    }
    wx = (id - n_pool) % pa.gx;
    wy = (id - n_pool) / pa.gx;
  }
  typedef typename vec8<T>::type V8;
  constexpr int KS = D / 16;          // MFMA steps over the indexer dim (8 per lane half)
  constexpr int QP = D + 8;           // LDS pitch of a staged head row (elements)
  constexpr int QCH = MT * 32 * D / 8;                // 16-byte chunks of the query's heads
  constexpr int QLD = (QCH + 255) / 256;              // per thread
  __shared__ __attribute__((aligned(16))) T qs[MT * 32 * QP];
  __shared__ __attribute__((aligned(16))) T ks[kScoreWaves * kScoreTile * D];
  const int i = wy;
  const int tid = threadIdx.x;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int n = lane & 31;
  const int hf = lane >> 5;
  // The query's indexer heads are staged once per workgroup in LDS (the four waves
  // share them); they are read alongside the query's metadata, which the key
  // addresses depend on.
  const T* qrow = qidx + (int64_t)i * (MT * 32) * D;
  V8 qreg[QLD];
#pragma unroll
  for (int j = 0; j < QLD; ++j) {
    const int e = min(tid + 256 * j, QCH - 1);
    qreg[j] = *reinterpret_cast<const V8*>(qrow + (int64_t)e * 8);
  }
  const SeqMeta sm = seq_meta(q_seq, seq_len, POOL ? pa.seq_row0 : nullptr, seq_blk0, i);
  const int nb = visible_tokens(sm.len, q_pos[i]) / c;
  const int b_base = (wx * kScoreWaves + wave) * kScoreTile;
  // POOL: the sequence's pooled count, read with its metadata (sequence 0's at once,
  // like the rest of the metadata); used only after the gathers are issued
  int n_in_s = 0;
  if constexpr (POOL) n_in_s = sm.s == 0 ? pa.n_in[0] : pa.n_in[sm.s];

  // Pooled keys: each wave gathers its 32 keys straight into its own LDS region,
  // four whole keys per instruction (fully coalesced), clamped into the visible
  // blocks (scores past them are not written).  Chunk c of key k sits at position
  // c ^ (k % CH) of the key's row, so that the operand reads below, 32 keys at one
  // chunk, spread over the LDS banks.
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int CH = D / 8;                          // 16-byte chunks per key
  constexpr int KPI = kWave / CH;                    // keys per instruction
  const int b = b_base + n;
  const bool valid = b < nb;
  T* kw = ks + wave * kScoreTile * D;
  if (b_base < nb) {
    const int last = nb - 1;
#pragma unroll
    for (int j = 0; j < kScoreTile / KPI; ++j) {
      const int kk = j * KPI + lane / CH, p = lane % CH, c = p ^ (kk & (CH - 1));
      const T* src = kpool + (sm.blk0 + min(b_base + kk, last)) * kpool_ld + c * 8;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(kw + j * kWave * 8), 16, 0, 0);
    }
  }
  // POOL: the first KPI new blocks' raw rows, chunk lane % CH of block p_lo + lane / CH
  // (more new blocks in the range are pooled in further rounds below)
  // (issued now, summed after the barrier, so that the workgroup does not wait for
  // them before it stages the query)
  int p_lo = 0, p_hi = 0;                            // new blocks of this wave's range
  V8 raw[8];
  if constexpr (POOL) {
    const int start = max(n_in_s, 0);
    const int end = (int)min((long long)(max(sm.len, 0) / c), (long long)start + pa.max_new);
    p_lo = max(b_base, start);
    p_hi = min(min(b_base + kScoreTile, end), nb);
    if (p_lo < p_hi) {
      const int pb = min(p_lo + lane / CH, p_hi - 1);
      const T* src = pa.kidx + (sm.row0 + (int64_t)pb * c) * pa.kidx_ld + (lane % CH) * 8;
#pragma unroll
      for (int u = 0; u < 8; ++u) raw[u] = *reinterpret_cast<const V8*>(src + (int64_t)min(u, c - 1) * pa.kidx_ld);
    }
  }
#pragma unroll
  for (int j = 0; j < QLD; ++j) {
    const int e = tid + 256 * j;
    if (e < QCH) {
      const int r = e / (D / 8), cc = e % (D / 8);
      *reinterpret_cast<V8*>(qs + r * QP + cc * 8) = qreg[j];
    }
  }
  __syncthreads();
  if (b_base >= nb) return;

  // B operand: lane (n, hf) takes key n, dims hf*D/2 + st*8 .. +8 (chunk hf*CH/2 + st).
  __builtin_amdgcn_s_waitcnt(0);                     // this wave's keys are in LDS
  if constexpr (POOL) {
    // new blocks: their pooled keys replace the cache rows just gathered, KPI per round
    for (int g0 = p_lo; g0 < p_hi; g0 += KPI) {
      const int pb = g0 + lane / CH;
      float pacc[8];
      if (g0 > p_lo || c > 8) {
        pool_sum8<T>(pa.kidx + (sm.row0 + (int64_t)min(pb, p_hi - 1) * c) * pa.kidx_ld + (lane % CH) * 8,
                     pa.kidx_ld, c, pacc);
      } else {                                       // the first round's rows, loaded above
#pragma unroll
        for (int e = 0; e < 8; ++e) pacc[e] = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (u < c) {
#pragma unroll
            for (int e = 0; e < 8; ++e) pacc[e] += (float)raw[u][e];
          }
      }
      if (pb < p_hi) {
        V8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = (T)(pacc[e] / (float)c);
        const int kk = pb - b_base, q = lane % CH;
        *reinterpret_cast<V8*>(kw + kk * D + ((q ^ (kk & (CH - 1))) * 8)) = pv;
      }
    }
  }
  V8 kb[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st)
    kb[st] = *reinterpret_cast<const V8*>(kw + n * D + (((hf * (CH / 2) + st) ^ (n & (CH - 1))) * 8));

  // A operand, read from LDS per step: lane (n, hf) takes head mt*32 + n, dims
  // hf*D/2 + st*8 .. +8.
  float sum = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const T* qa = qs + (mt * 32 + n) * QP + hf * (D / 2);
    f32x16 acc = {};
#pragma unroll
    for (int st = 0; st < KS; ++st) acc = mfma32x32x16<T>(*reinterpret_cast<const V8*>(qa + st * 8), kb[st], acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += relu(acc[r]);
  }
  sum += __shfl_xor(sum, 32);
  if (hf == 0 && valid) scores[(int64_t)i * scores_ld + b] = sum + 0.0f;  // +0.0 turns -0.0 into +0.0
  if constexpr (POOL) {
    if (pa.cand != nullptr && b_base / kCandTile < kCandThreads * pa.cand_tpt) {   // the tile's best blocks
      // lanes n and n + 32 both hold block n's sum; the keep best of the tile's 32, ties
      // to the lower block, as a mask of lanes 0..31 (uniform)
      const uint32_t key = valid ? score_key(sum + 0.0f) : 0u;   // the selection's key of the stored score
      const int keep = pa.cand_keep;
      uint32_t taken = 0u;
      if (keep <= 4) {
        // the largest key not yet taken, keep times (the lowest lane holding it), each
        // over the 32 lanes of a half: fewer dependent steps than the bit search below
        // for 4, more for 8
        for (int r = 0; r < keep; ++r) {
          const bool alive = ((taken >> n) & 1u) == 0u;
          const uint32_t x = alive ? key : 0u;
          const uint32_t m = wave_extreme_u32<true, true>(x);
          const uint32_t hit = (uint32_t)__ballot(alive && x == m);
          taken |= hit & (0u - hit);
        }
      } else {
        // the keep-th largest key v, bit by bit; then the keys above v and the first of
        // those equal to it.  The search stops once exactly keep keys reach v: those are
        // the keep best (the first bit where the keep-th and the next largest differ)
        const uint64_t lo = 0xFFFFFFFFull;
        uint32_t v = 0u;
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t tv = v | (1u << bit);
          const int n_ge = __popcll(__ballot(key >= tv) & lo);
          if (n_ge >= keep) v = tv;
          if (n_ge == keep) break;
        }
        const uint64_t below_me = (1ull << lane) - 1ull;
        const int n_above = __popcll(__ballot(key > v) & lo);
        const int eq_rank = __popcll(__ballot(key == v) & lo & below_me);
        taken = (uint32_t)__ballot(key > v || (key == v && eq_rank < keep - n_above));
      }
      const bool take = hf == 0 && ((taken >> n) & 1u) != 0u;
      const int slot = __popc(taken & ((1u << n) - 1u));
      uint32_t* cw = pa.cand + (int64_t)i * pa.cand_ld;
      const int g = b_base / kCandTile;
      if (take) {                                    // exactly keep lanes (blocks past the row: key 0)
        cw[cand_offset(g, slot, keep, pa.cand_tpt)] = key;
        cw[cand_offset(g, keep + slot, keep, pa.cand_tpt)] = (uint32_t)b;
      }
    }
  }
}

// ------------------------------------------------------------- MFMA, many queries

// Prefill chunks (many query tokens of one sequence): a workgroup of kGemmQ waves
// takes kGemmQ consecutive query tokens -- wave w holds token w's indexer heads as
// the M operand in registers for the whole launch -- and walks a range of blocks in
// tiles of kGemmBN pooled keys that all its waves share.  Each tile is gathered once
// straight into LDS (global_load_lds, chunks XOR-swizzled by key so that the lanes'
// 16-byte reads spread over the banks) while the previous one is being multiplied, so
// the pooled keys are read from L2 once per kGemmQ queries instead of once per query,
// and each query's heads once per block range.  Scores above a token's own visible blocks are not
// written.  When the group's tokens belong to different sequences every wave reads
// its own sequence's keys straight from memory instead.
constexpr int kGemmQ = 8;             // query tokens (waves) per workgroup
constexpr int kGemmBN = 128;          // pooled keys per LDS tile

template <typename T, int MT, int D>
__global__ void __launch_bounds__(kGemmQ * 64, 2)
score_gemm_kernel(const T* __restrict__ qidx, const T* __restrict__ kpool, int64_t kpool_ld,
                  const int64_t* __restrict__ seq_blk0, const int32_t* __restrict__ seq_len,
                  const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int n_q,
                  int tiles_per_range, float* __restrict__ scores, int64_t scores_ld) {
  typedef typename vec8<T>::type V8;
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int KS = D / 16;
  constexpr int CH = D / 8;                          // 16-byte chunks per key row
  constexpr int KPI = kWave / CH;                    // keys per wave instruction
  constexpr int NI = kGemmBN / (KPI * kGemmQ);       // instructions per wave per tile
  static_assert(NI * KPI * kGemmQ == kGemmBN, "tile must split evenly");
  // two tile buffers as separate objects, so that reading one never waits on the
  // gathers into the other
  __shared__ __attribute__((aligned(16))) T ks0[kGemmBN * D];
  __shared__ __attribute__((aligned(16))) T ks1[kGemmBN * D];
  __shared__ int g_seq[kGemmQ], g_nb[kGemmQ];
  __shared__ int64_t g_blk0[kGemmQ];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int n = lane & 31, hf = lane >> 5;
  const int i = blockIdx.y * kGemmQ + wave;
  const bool has_q = i < n_q;
  const int ic = has_q ? i : n_q - 1;
  const T* qrow = qidx + (int64_t)ic * (MT * 32) * D + (int64_t)n * D + hf * (D / 2);
  V8 qa[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int st = 0; st < KS; ++st) qa[mt][st] = *reinterpret_cast<const V8*>(qrow + (int64_t)mt * 32 * D + st * 8);
  const SeqMeta sm = seq_meta(q_seq, seq_len, nullptr, seq_blk0, ic);
  const int nb = has_q ? visible_tokens(sm.len, q_pos[ic]) / c : 0;
  if (lane == 0) {
    g_seq[wave] = has_q ? sm.s : -1;
    g_nb[wave] = nb;
    g_blk0[wave] = sm.blk0;
  }
  __syncthreads();
  int nb_max = 0;
  bool shared = true;
  const int s0 = g_seq[0];
#pragma unroll
  for (int w = 0; w < kGemmQ; ++w) {
    nb_max = max(nb_max, g_nb[w]);
    shared = shared && (g_seq[w] == s0 || g_seq[w] < 0);
  }
  const int t_begin = blockIdx.x * tiles_per_range;
  const int t_end = min(t_begin + tiles_per_range, (nb_max + kGemmBN - 1) / kGemmBN);
  if (t_begin >= t_end) return;                      // uniform over the workgroup
  float* srow = scores + (int64_t)ic * scores_ld;

  // one 32-block product of this wave's query: ReLU, head sum, write
  auto finish = [&](const V8 (&kb)[KS], int b) {
    float sum = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x16 acc = {};
#pragma unroll
      for (int st = 0; st < KS; ++st) acc = mfma32x32x16<T>(qa[mt][st], kb[st], acc);
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += relu(acc[r]);
    }
    sum += __shfl_xor(sum, 32);
    if (hf == 0 && b < nb) srow[b] = sum + 0.0f;     // +0.0 turns -0.0 into +0.0
  };

  if (!shared) {                                     // tokens of different sequences
    const T* kseq = kpool + sm.blk0 * kpool_ld + hf * (D / 2);
    for (int t = t_begin; t < t_end; ++t) {
      for (int nt = 0; nt < kGemmBN / 32; ++nt) {
        const int b0 = t * kGemmBN + nt * 32;
        if (b0 >= nb) break;
        const int b = b0 + n;
        const T* krow = kseq + (int64_t)(b < nb ? b : nb - 1) * kpool_ld;
        V8 kb[KS];
#pragma unroll
        for (int st = 0; st < KS; ++st) kb[st] = *reinterpret_cast<const V8*>(krow + st * 8);
        finish(kb, b);
      }
    }
    return;
  }

  // Shared tiles: rows [t*BN, t*BN + BN), clamped into the sequence, gathered straight
  // into LDS (each wave NI instructions of KPI whole keys).  Chunk c of key k sits at
  // position c ^ (k % CH) of its row, so that the B reads below (32 keys at one chunk)
  // spread over the banks.  Tile t+1 is gathered into the other buffer while tile t is
  // multiplied.
  const T* kseq = kpool + g_blk0[0] * kpool_ld;
  const int last = nb_max - 1;
  auto issue = [&](int t, T* buf) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int k0 = (wave * NI + j) * KPI;          // first key of the instruction
      const int kk = k0 + lane / CH, p = lane % CH, cc = p ^ (kk & (CH - 1));
      const int b = min(t * kGemmBN + kk, last);
      __builtin_amdgcn_global_load_lds((const void*)(kseq + (int64_t)b * kpool_ld + cc * 8),
                                       (lds_void*)(buf + k0 * D), 16, 0, 0);
    }
  };
  // the products of one 32-block step of a tile: acc[mt] = heads mt*32.. x blocks
  // (B read once per step from LDS and shared by the M tiles)
  auto products = [&](const T* buf, int nt, f32x16 (&acc)[MT]) {
    const int key = nt * 32 + n;
    const T* krow = buf + key * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const V8 kb = *reinterpret_cast<const V8*>(krow + (((hf * (CH / 2) + st) ^ (key & (CH - 1))) * 8));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma32x32x16<T>(qa[mt][st], kb, acc[mt]);
    }
  };
  // ReLU and head sum of one step: lane (n, hf) holds 16 heads of block n per M tile,
  // the partner lane n ^ 32 the other 16
  auto reduce = [&](const f32x16 (&acc)[MT]) {
    float sum = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += relu(acc[mt][r]);
    return sum + __shfl_xor(sum, 32);
  };
  // A tile's four steps.  Pipelined (PIPE): over two accumulator sets, step nt+1's
  // products issued before step nt's epilogue, so the matrix pipe works while the
  // epilogue runs, the scores stored after the last step (a store per step is a
  // branch the scheduler does not cross; the last tile's steps past nb multiply
  // clamped keys and store nothing).  That takes ~60 more registers, so it is used
  // where the held heads take 64-96 registers and the kernel runs one workgroup per
  // CU either way (64 heads of 128 dims: ~220 registers against ~170; a 128-register
  // build, two workgroups per CU, spills and is no faster); smaller shapes keep two
  // or more workgroups per CU with one step at a time, and 128 heads of 128 dims
  // would spill.
  constexpr bool PIPE = MT * D >= 256 && MT * D <= 384;
  auto multiply = [&](int t, const T* buf) {
    if (t * kGemmBN >= nb) return;                   // uniform per wave
    constexpr int NT = kGemmBN / 32;
    if constexpr (PIPE) {
      float sums[NT];
      f32x16 acc0[MT], acc1[MT];
      products(buf, 0, acc0);
#pragma unroll
      for (int nt = 0; nt < NT; nt += 2) {
        products(buf, nt + 1, acc1);
        sums[nt] = reduce(acc0);
        if (nt + 2 < NT) products(buf, nt + 2, acc0);
        sums[nt + 1] = reduce(acc1);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int b = t * kGemmBN + nt * 32 + n;
        if (hf == 0 && b < nb) srow[b] = sums[nt] + 0.0f;   // +0.0 turns -0.0 into +0.0
      }
    } else {
      for (int nt = 0; nt < NT; ++nt) {
        const int b = t * kGemmBN + nt * 32 + n;
        if (b - n >= nb) break;                      // uniform per wave
        f32x16 acc[MT];
        products(buf, nt, acc);
        const float sum = reduce(acc);
        if (hf == 0 && b < nb) srow[b] = sum + 0.0f;   // +0.0 turns -0.0 into +0.0
      }
    }
  };
  issue(t_begin, ks0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = t_begin; t < t_end; t += 2) {
    if (t + 1 < t_end) issue(t + 1, ks1);
    multiply(t, ks0);
    __builtin_amdgcn_s_waitcnt(0);                   // this wave's gathers into ks1
    __syncthreads();                                 // everyone's; ks0 is free
    if (t + 1 >= t_end) break;
    if (t + 2 < t_end) issue(t + 2, ks0);
    multiply(t + 1, ks1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------- VALU

constexpr int kValuBlocks = 64;       // blocks per workgroup
constexpr int kValuQFloats = 8192;    // query floats staged in LDS per pass

template <typename T>
__global__ void __launch_bounds__(256)
score_valu_kernel(const T* __restrict__ qidx, const T* __restrict__ kpool, int64_t kpool_ld,
                  const int64_t* __restrict__ seq_blk0, const int32_t* __restrict__ seq_len,
                  const int32_t* __restrict__ q_seq, const int32_t* __restrict__ q_pos, int c, int h_idx, int d_idx,
                  float* __restrict__ scores, int64_t scores_ld) {
  __shared__ float sq[kValuQFloats];
  __shared__ float part[4][kValuBlocks];
  const int i = blockIdx.y;
  const SeqMeta sm = seq_meta(q_seq, seq_len, nullptr, seq_blk0, i);
  const int nb = visible_tokens(sm.len, q_pos[i]) / c;
  const int b0 = blockIdx.x * kValuBlocks;
  if (b0 >= nb) return;
  const int lb = threadIdx.x % kValuBlocks;
  const int hg = threadIdx.x / kValuBlocks;
  const int b = b0 + lb;
  const T* krow = kpool + (sm.blk0 + (b < nb ? b : 0)) * kpool_ld;
  const T* q = qidx + (int64_t)i * h_idx * d_idx;
  const int heads_per_pass = kValuQFloats / d_idx;
  float sum = 0.f;
  for (int h0 = 0; h0 < h_idx; h0 += heads_per_pass) {
    const int hn = min(heads_per_pass, h_idx - h0);
    __syncthreads();
    for (int e = threadIdx.x; e < hn * d_idx; e += blockDim.x) sq[e] = (float)q[(int64_t)h0 * d_idx + e];
    __syncthreads();
    if (b < nb) {
      for (int h = hg; h < hn; h += 4) {
        float dot = 0.f;
        for (int d = 0; d < d_idx; ++d) dot += sq[h * d_idx + d] * (float)krow[d];
        sum += fmaxf(dot, 0.f);
      }
    }
  }
  part[hg][lb] = sum;
  __syncthreads();
  if (hg == 0 && b < nb) {
    scores[(int64_t)i * scores_ld + b] = part[0][lb] + part[1][lb] + part[2][lb] + part[3][lb] + 0.0f;
  }
}

// ----------------------------------------------------------------------------- host

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool score_uses_mfma(const sa_dims& d, const CacheArgs& c, const void* qidx) {
  if (d.dtype != SA_F16 && d.dtype != SA_BF16) return false;
  if (d.h_idx % 32 != 0 || d.h_idx > 128) return false;
  if (d.d_idx != 64 && d.d_idx != 128 && d.d_idx != 256) return false;
  return c.kpool_ld % 8 == 0 && aligned16(c.kpool) && aligned16(qidx);
}

// Query tokens from which the shared-tile kernel is used (a prefill chunk).
constexpr int kGemmMinQueries = 64;

template <typename T, int MT, int D>
static void launch_mfma(const sa_dims& d, const CacheArgs& c, const void* qidx, const int32_t* q_seq,
                        const int32_t* q_pos, int n_q, float* scores, int64_t scores_ld, hipStream_t stream) {
  const long long max_blocks = (long long)c.max_len / d.compress_ratio;
  // (the 256-wide indexer with more than 32 heads would spill the held heads)
  if (n_q >= kGemmMinQueries && (D <= 128 || MT == 1)) {
    // block ranges per query group: enough workgroups for ~4 per CU, each range
    // long enough that the query heads are loaded once per many tiles
    const long long tiles = (max_blocks + kGemmBN - 1) / kGemmBN;
    const long long groups = (n_q + kGemmQ - 1) / kGemmQ;
    long long ranges = (1024 + groups - 1) / groups;
    ranges = ranges < 1 ? 1 : (ranges > tiles ? tiles : ranges);
    const int per_range = (int)((tiles + ranges - 1) / ranges);
    ranges = (tiles + per_range - 1) / per_range;
    if (tiles == 0) return;
    hipLaunchKernelGGL((score_gemm_kernel<T, MT, D>), dim3((unsigned)ranges, (unsigned)groups), dim3(kGemmQ * 64), 0,
                       stream, (const T*)qidx, (const T*)c.kpool, c.kpool_ld, c.seq_blk0, c.seq_len, q_seq, q_pos,
                       d.compress_ratio, n_q, per_range, scores, scores_ld);
    return;
  }
  const long long per_wg = kScoreWaves * kScoreTile;
  dim3 grid((unsigned)((max_blocks + per_wg - 1) / per_wg), (unsigned)n_q);
  if (grid.x == 0) return;
  hipLaunchKernelGGL((score_mfma_kernel<T, MT, D, false>), grid, dim3(256), 0, stream, (const T*)qidx,
                     (const T*)c.kpool, c.kpool_ld, c.seq_blk0, c.seq_len, q_seq, q_pos, d.compress_ratio, scores,
                     scores_ld, PoolArgs<T>{});
}

template <typename T, int MT, int D>
static void launch_pool_score_t(const sa_dims& d, const CacheArgs& c, const int32_t* n_in, int32_t* n_out,
                                int max_new, const void* qidx, const int32_t* q_seq, const int32_t* q_pos, int n_q,
                                float* scores, int64_t scores_ld, uint32_t* cand, int64_t cand_ld,
                                int cand_keep, int cand_tpt, hipStream_t stream) {
  const long long max_blocks = (long long)c.max_len / d.compress_ratio;
  const long long per_wg = kScoreWaves * kScoreTile;
  const long long gx = (max_blocks + per_wg - 1) / per_wg;
  const long long blocks = max_new < max_blocks ? max_new : max_blocks;
  long long pool_wgs = (blocks * d.d_idx + 255) / 256;
  pool_wgs = pool_wgs < 1 ? 1 : (pool_wgs > 2048 ? 2048 : pool_wgs);
  const dim3 grid((unsigned)(pool_wgs * c.n_seq + gx * n_q));
  const PoolArgs<T> pa{(const T*)c.kidx, c.kidx_ld, (T*)c.kpool, c.seq_row0, n_in, n_out, max_new,
                       (int)pool_wgs, c.n_seq, (int)gx, cand, cand_ld, cand_keep, cand_tpt};
  hipLaunchKernelGGL((score_mfma_kernel<T, MT, D, true>), grid, dim3(256), 0, stream, (const T*)qidx,
                     (const T*)c.kpool, c.kpool_ld, c.seq_blk0, c.seq_len, q_seq, q_pos, d.compress_ratio, scores,
                     scores_ld, pa);
}

template <typename T, int MT>
static void dispatch_mfma_d(const sa_dims& d, const CacheArgs& c, const void* qidx, const int32_t* q_seq,
                            const int32_t* q_pos, int n_q, float* scores, int64_t scores_ld, hipStream_t stream) {
  switch (d.d_idx) {
    case 64: launch_mfma<T, MT, 64>(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream); break;
    case 128: launch_mfma<T, MT, 128>(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream); break;
    default: launch_mfma<T, MT, 256>(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream); break;
  }
}

template <typename T>
static void dispatch_mfma(const sa_dims& d, const CacheArgs& c, const void* qidx, const int32_t* q_seq,
                          const int32_t* q_pos, int n_q, float* scores, int64_t scores_ld, hipStream_t stream) {
  switch (d.h_idx / 32) {
    case 1: dispatch_mfma_d<T, 1>(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream); break;
    case 2: dispatch_mfma_d<T, 2>(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream); break;
    case 3: dispatch_mfma_d<T, 3>(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream); break;
    default: dispatch_mfma_d<T, 4>(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream); break;
  }
}

template <typename T>
static void launch_valu(const sa_dims& d, const CacheArgs& c, const void* qidx, const int32_t* q_seq,
                        const int32_t* q_pos, int n_q, float* scores, int64_t scores_ld, hipStream_t stream) {
  const long long max_blocks = (long long)c.max_len / d.compress_ratio;
  dim3 grid((unsigned)((max_blocks + kValuBlocks - 1) / kValuBlocks), (unsigned)n_q);
  if (grid.x == 0) return;
  hipLaunchKernelGGL(score_valu_kernel<T>, grid, dim3(256), 0, stream, (const T*)qidx, (const T*)c.kpool,
                     c.kpool_ld, c.seq_blk0, c.seq_len, q_seq, q_pos, d.compress_ratio, d.h_idx, d.d_idx, scores,
                     scores_ld);
}

bool pool_score_fused(const sa_dims& d, const CacheArgs& c, const void* qidx, int n_q, const int32_t* n_in,
                      const int32_t* n_out) {
  if (!score_uses_mfma(d, c, qidx) || n_q <= 0 || n_q >= kGemmMinQueries) return false;
  if ((const void*)n_in == (const void*)n_out) return false;   // in-place counts: pool first
  const long long gx = ((long long)c.max_len / d.compress_ratio + kScoreWaves * kScoreTile - 1) / (kScoreWaves * kScoreTile);
  if ((long long)c.n_seq * 2048 + gx * n_q >= (1LL << 31)) return false;   // one-dimensional grid
  return c.kidx_ld % 8 == 0 && aligned16(c.kidx);
}

template <typename T>
static void dispatch_pool_score(const sa_dims& d, const CacheArgs& c, const int32_t* n_in, int32_t* n_out,
                                int max_new, const void* qidx, const int32_t* q_seq, const int32_t* q_pos, int n_q,
                                float* scores, int64_t scores_ld, uint32_t* cand, int64_t cand_ld,
                                int cand_keep, int cand_tpt, hipStream_t stream) {
#define SA_PS_CASE(MT_, D_)                                                                                        \
  if (d.h_idx / 32 == MT_ && d.d_idx == D_) {                                                                      \
    launch_pool_score_t<T, MT_, D_>(d, c, n_in, n_out, max_new, qidx, q_seq, q_pos, n_q, scores, scores_ld, cand, \
                                    cand_ld, cand_keep, cand_tpt, stream);                                         \
    return;                                                                                                        \
  }
  SA_PS_CASE(1, 64) SA_PS_CASE(1, 128) SA_PS_CASE(1, 256)
  SA_PS_CASE(2, 64) SA_PS_CASE(2, 128) SA_PS_CASE(2, 256)
  SA_PS_CASE(3, 64) SA_PS_CASE(3, 128) SA_PS_CASE(3, 256)
  SA_PS_CASE(4, 64) SA_PS_CASE(4, 128) SA_PS_CASE(4, 256)
#undef SA_PS_CASE
}

hipError_t launch_pool_score(const sa_dims& d, const CacheArgs& c, const int32_t* n_in, int32_t* n_out, int max_new,
                             const void* qidx, const int32_t* q_seq, const int32_t* q_pos, int n_q, float* scores,
                             int64_t scores_ld, hipStream_t stream, uint32_t* cand, int64_t cand_ld, int cand_keep,
                             int cand_tpt) {
  if (cand && (cand_keep % 4 != 0 || cand_keep > kCandKeep || cand_tpt < 1 ||
               cand_ld < (int64_t)kCandThreads * cand_tpt * 2 * cand_keep))
    return hipErrorInvalidValue;
  if (!pool_score_fused(d, c, qidx, n_q, n_in, n_out)) {
    if (cand) return hipErrorInvalidValue;           // candidates come only from the pooling scoring launch
    hipError_t err = launch_pool(d, c, n_in, n_out, max_new, stream);
    if (err != hipSuccess) return err;
    return launch_score(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream);
  }
  if (d.dtype == SA_BF16)
    dispatch_pool_score<bf16>(d, c, n_in, n_out, max_new, qidx, q_seq, q_pos, n_q, scores, scores_ld, cand, cand_ld,
                              cand_keep, cand_tpt, stream);
  else
    dispatch_pool_score<f16>(d, c, n_in, n_out, max_new, qidx, q_seq, q_pos, n_q, scores, scores_ld, cand, cand_ld,
                             cand_keep, cand_tpt, stream);
  return hipGetLastError();
}

hipError_t launch_score(const sa_dims& d, const CacheArgs& c, const void* qidx, const int32_t* q_seq,
                        const int32_t* q_pos, int n_q, float* scores, int64_t scores_ld, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  if (score_uses_mfma(d, c, qidx)) {
    if (d.dtype == SA_BF16) dispatch_mfma<bf16>(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream);
    else dispatch_mfma<f16>(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream);
  } else {
    switch (d.dtype) {
      case SA_F32: launch_valu<float>(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream); break;
      case SA_F16: launch_valu<f16>(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream); break;
      default: launch_valu<bf16>(d, c, qidx, q_seq, q_pos, n_q, scores, scores_ld, stream); break;
    }
  }
  return hipGetLastError();
}

}  // namespace sa
