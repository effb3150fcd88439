"""Seeded synthetic inputs for indexer-selected block-sparse attention.

This module only draws numbers and lays them out. It holds none of the method's
arithmetic (no pooling, scoring, selection or attention), so both the HIP path and
the CPU oracle may take their inputs from it.

Recipe (the same for every case):
  * generator: numpy PCG64.  Every tensor is cut into chunks of 2**22 elements and
    chunk i of tensor t is drawn from ``np.random.default_rng([seed, case_id, t, i])``
    (so chunks can be drawn on several host threads and the result does not depend
    on the thread count).  Tensor ids: 1 = q, 2 = indexer queries, 3 = sequence
    lengths, 4 = planted block ids, 1000+4s / 1001+4s / 1002+4s = K / V / raw
    indexer keys of sequence s;
  * values are standard normal float32 draws times the stated standard deviation;
  * each array is rounded to its storage dtype with round-to-nearest-even (torch's
    cast) and handed out as float32 holding exactly the stored values.

The workloads stand in for one attention layer of the models the pages benchmark:
a DeepSeek-V4-style MLA layer (one latent KV head, DKQ=576 / DV=512, 16 query heads)
and a 512/512 GQA layer with 8 query heads per KV head, indexer with 64 (or 32)
heads of size 128, compress_ratio 4 and an indexer_top_k budget of 2048 tokens
("CUDA + ggml: add sparse-fa for DSV4/GLM", the supported (DKQ, DV, heads per KV
head) pairs in the kernel-selection review comment; "llama: QSA sparse attention
for qwen4exp", the block budget).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Optional

import numpy as np
import torch

DTYPES = ("f32", "f16", "bf16")
_TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Dims:
    h_q: int
    h_kv: int
    d_kq: int
    d_v: int
    h_idx: int
    d_idx: int
    compress_ratio: int
    top_k: int
    dtype: str

    @property
    def n_kv_max(self) -> int:
        """Capacity of one query's selection list: top_k tokens of whole blocks + a tail."""
        return self.top_k + self.compress_ratio - 1


@dataclasses.dataclass
class Case:
    """One layer's caches and one batch of query tokens.

    Caches of all sequences are packed row-wise; sequence s owns rows
    [row0[s], row0[s] + cap[s]) and row row0[s] + t holds position t.
    """
    name: str
    dims: Dims
    seq_len: np.ndarray          # int32 [n_seq]   cached tokens L_s
    seq_cap: np.ndarray          # int32 [n_seq]   row capacity (multiple of c)
    row0: np.ndarray             # int64 [n_seq]
    blk0: np.ndarray             # int64 [n_seq]   = row0 / c
    k: np.ndarray                # f32 [rows, h_kv, d_kq]
    v: Optional[np.ndarray]      # f32 [rows, h_kv, d_v]; None -> V is the first d_v of each K row
    kidx: np.ndarray             # f32 [rows, d_idx]  raw indexer keys
    q: np.ndarray                # f32 [n_q, h_q, d_kq]
    qidx: np.ndarray             # f32 [n_q, h_idx, d_idx]
    q_seq: np.ndarray            # int32 [n_q]
    q_pos: np.ndarray            # int32 [n_q]
    scale: float
    planted_blocks: Optional[np.ndarray] = None

    @property
    def n_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_seq(self) -> int:
        return int(self.seq_len.shape[0])

    @property
    def rows(self) -> int:
        return int(self.kidx.shape[0])

    @property
    def v_aliases_k(self) -> bool:
        return self.v is None

    def v_rows(self) -> np.ndarray:
        """V as stored: a view of K's first d_v elements when V aliases K."""
        if self.v is None:
            return self.k[:, :, : self.dims.d_v]
        return self.v


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (RNE) and return them as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    t = torch.from_numpy(x).to(_TORCH_DT[dtype])
    return t.to(torch.float32).numpy()


_CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _normal(key, shape, std: float, dtype: str) -> np.ndarray:
    """Standard normal float32 draws for tensor ``key = (seed, case_id, tensor_id)``."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    n_chunks = (n + _CHUNK - 1) // _CHUNK

    def fill(i: int) -> None:
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.default_rng(list(key) + [i])
        g.standard_normal(size=hi - lo, dtype=np.float32, out=out[lo:hi])

    if n_chunks <= 1:
        for i in range(n_chunks):
            fill(i)
    else:
        with concurrent.futures.ThreadPoolExecutor(min(_THREADS, n_chunks)) as ex:
            list(ex.map(fill, range(n_chunks)))
    if std != 1.0:
        out *= np.float32(std)
    return round_to_dtype(out.reshape(shape), dtype)


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def make_case(name: str, dims: Dims, seq_lens, q_seq, q_pos, *, seed: int, case_id: int,
              std: str | float = 1.0, v_separate: bool = True, scale: Optional[float] = None,
              plant_fraction: float = 0.0, plant_sigmas: float = 3.0, q_std: Optional[float] = None) -> Case:
    """Draw a case with the given shapes.

    ``std`` is a number, or ``"inv_sqrt_dim"`` for N(0,1)/sqrt(last dim) per tensor.
    ``q_std`` (optional) replaces it for the attention queries alone, so that a test
    can widen the spread of the attention logits while K and V keep theirs.
    ``plant_fraction`` > 0 adds ``plant_sigmas`` standard deviations of the raw
    indexer keys to every element of every token of that fraction of the blocks of
    sequence 0 (blocks drawn without replacement).
    """
    c = dims.compress_ratio
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    n_seq = len(seq_lens)
    align = c * 64 // math.gcd(c, 64)          # rows per sequence: a multiple of c and of 64
    caps = np.array([_round_up(max(int(L), 1), align) for L in seq_lens], dtype=np.int64)
    row0 = np.zeros(n_seq, dtype=np.int64)
    if n_seq > 1:
        row0[1:] = np.cumsum(caps)[:-1]
    rows = int(caps.sum())

    def sd(last_dim: int) -> float:
        if std == "inv_sqrt_dim":
            return 1.0 / math.sqrt(last_dim)
        return float(std)

    k = np.zeros((rows, dims.h_kv, dims.d_kq), dtype=np.float32)
    v = np.zeros((rows, dims.h_kv, dims.d_v), dtype=np.float32) if v_separate else None
    kidx = np.zeros((rows, dims.d_idx), dtype=np.float32)
    for s in range(n_seq):
        L = int(seq_lens[s])
        r = slice(int(row0[s]), int(row0[s]) + L)
        k[r] = _normal((seed, case_id, 1000 + 4 * s), (L, dims.h_kv, dims.d_kq), sd(dims.d_kq), dims.dtype)
        if v_separate:
            v[r] = _normal((seed, case_id, 1001 + 4 * s), (L, dims.h_kv, dims.d_v), sd(dims.d_v), dims.dtype)
        kidx[r] = _normal((seed, case_id, 1002 + 4 * s), (L, dims.d_idx), sd(dims.d_idx), dims.dtype)
    n_q = len(q_seq)
    q = _normal((seed, case_id, 1), (n_q, dims.h_q, dims.d_kq), sd(dims.d_kq) if q_std is None else float(q_std),
                dims.dtype)
    qidx = _normal((seed, case_id, 2), (n_q, dims.h_idx, dims.d_idx), sd(dims.d_idx), dims.dtype)

    planted = None
    if plant_fraction > 0.0:
        L0 = int(seq_lens[0])
        nb = L0 // c
        n_plant = int(math.floor(plant_fraction * nb))
        prng = np.random.default_rng([seed, case_id, 4])
        planted = np.sort(prng.choice(nb, size=n_plant, replace=False)).astype(np.int64)
        offset = np.float32(plant_sigmas * sd(dims.d_idx))
        tok = (planted[:, None] * c + np.arange(c)[None, :]).reshape(-1) + int(row0[0])
        # add in float32, then store in the cache dtype
        kidx[tok] = round_to_dtype(kidx[tok] + offset, dims.dtype)

    if scale is None:
        scale = 1.0 / math.sqrt(dims.d_kq)
    return Case(name=name, dims=dims, seq_len=seq_lens.astype(np.int32), seq_cap=caps.astype(np.int32),
                row0=row0, blk0=row0 // c, k=k, v=v, kidx=kidx, q=q, qidx=qidx,
                q_seq=np.asarray(q_seq, dtype=np.int32), q_pos=np.asarray(q_pos, dtype=np.int32),
                scale=float(scale), planted_blocks=planted)


# ---------------------------------------------------------------------------
# The workloads.  Sizes follow the configurations the library is measured on;
# workload 6 is workload 2 with token-level selection (every token its own block).
# ---------------------------------------------------------------------------

WORKLOADS = {
    1: "tiny decode fp32: 1 seq x 1024 cached, q at 1024, 8:1 heads, D=128, idx 4x64, c=4, top_k=256",
    2: "DSV4-shaped decode bf16: 1 seq x 131072 cached, 16 heads on 1 latent KV head, DKQ/DV=576/512, idx 64x128, c=4, top_k=2048",
    3: "batched decode f16: 32 seqs, L~U[4096,65536], 8:1 heads, 512/512, idx 32x128, c=4, top_k=2048",
    4: "prefill chunk bf16: 2048 queries at 32768..34815, 16 heads, 576/512, idx 64x128, c=4, top_k=2048",
    5: "long decode bf16: 1 seq x 1048576 cached, 16 heads, 576/512, idx 64x128, c=4, top_k=2048, 1% planted blocks",
    6: "token-level decode bf16: 1 seq x 131072 cached, 16 heads on 1 latent KV head, 576/512, idx 64x128, c=1, top_k=2048",
}


def workload_dims(cfg: int) -> Dims:
    if cfg == 1:
        return Dims(h_q=8, h_kv=1, d_kq=128, d_v=128, h_idx=4, d_idx=64, compress_ratio=4, top_k=256, dtype="f32")
    if cfg in (2, 4, 5):
        return Dims(h_q=16, h_kv=1, d_kq=576, d_v=512, h_idx=64, d_idx=128, compress_ratio=4, top_k=2048,
                    dtype="bf16")
    if cfg == 3:
        return Dims(h_q=8, h_kv=1, d_kq=512, d_v=512, h_idx=32, d_idx=128, compress_ratio=4, top_k=2048,
                    dtype="f16")
    if cfg == 6:
        return Dims(h_q=16, h_kv=1, d_kq=576, d_v=512, h_idx=64, d_idx=128, compress_ratio=1, top_k=2048,
                    dtype="bf16")
    raise ValueError(f"unknown workload {cfg}")


def make_workload(cfg: int, seed: int = 0, ctx: Optional[int] = None, q_std: Optional[float] = None) -> Case:
    """Build workload ``cfg`` (1..6).  ``ctx`` overrides the cached length of the
    single-sequence decode workloads (used for reduced-size test variants); ``q_std``
    overrides the attention queries' standard deviation (see make_case)."""
    dims = workload_dims(cfg)
    if cfg == 1:
        L = ctx or 1024
        return make_case("tiny_decode_f32", dims, [L], [0], [L], seed=seed, case_id=cfg, std=1.0,
                         v_separate=True, scale=1.0 / math.sqrt(128), q_std=q_std)
    if cfg == 2:
        L = ctx or 131072
        return make_case("dsv4_decode_128k_bf16", dims, [L], [0], [L], seed=seed, case_id=cfg,
                         std="inv_sqrt_dim", v_separate=False, scale=1.0 / math.sqrt(576), q_std=q_std)
    if cfg == 3:
        lens = np.random.default_rng([seed, cfg, 3]).integers(4096, 65536, size=32, endpoint=True)
        return make_case("batched_decode_f16", dims, lens, list(range(32)), [int(x) for x in lens], seed=seed,
                         case_id=cfg, std=0.5, v_separate=True, scale=1.0 / math.sqrt(512), q_std=q_std)
    if cfg == 4:
        depth = ctx or 32768
        n_q = 2048
        L = depth + n_q
        return make_case("prefill_chunk_bf16", dims, [L], [0] * n_q, list(range(depth, depth + n_q)), seed=seed,
                         case_id=cfg, std="inv_sqrt_dim", v_separate=False, scale=1.0 / math.sqrt(576), q_std=q_std)
    if cfg == 5:
        L = ctx or 1048576
        return make_case("long_decode_1m_bf16", dims, [L], [0], [L], seed=seed, case_id=cfg, std="inv_sqrt_dim",
                         v_separate=False, scale=1.0 / math.sqrt(576), plant_fraction=0.01, plant_sigmas=3.0,
                         q_std=q_std)
    if cfg == 6:
        L = ctx or 131072
        return make_case("token_level_decode_128k_bf16", dims, [L], [0], [L], seed=seed, case_id=cfg,
                         std="inv_sqrt_dim", v_separate=False, scale=1.0 / math.sqrt(576), q_std=q_std)
    raise ValueError(f"unknown workload {cfg}")


# ---------------------------------------------------------------------------
# Additive masks in the form of the pages' sparse flash-attention tests.
# ---------------------------------------------------------------------------

def sparse_mask(n_rows: int, n_kv: int, n_kv_max: int, *, seed: int, case_id: int,
                count_spread: int = 17, single_entry_stride: int = 32, dtype: str = "f16") -> np.ndarray:
    """[n_rows, n_kv] float32 mask holding exactly the storage values of ``dtype``.

    Row r keeps 1 entry when r is a multiple of ``single_entry_stride`` and otherwise
    n_kv_max - r mod min(n_kv_max, count_spread) entries, at positions drawn without
    replacement from the seed; the i-th kept position (ascending) carries the value
    -(1 + (i + r) mod 7) / 32 and every other entry is -inf ("CUDA + ggml: add
    sparse-fa for DSV4/GLM", the test-backend-ops mask initialisation).
    """
    rng = np.random.default_rng([seed, case_id, 5])
    m = np.full((n_rows, n_kv), -np.inf, dtype=np.float32)
    for r in range(n_rows):
        cnt = 1 if r % single_entry_stride == 0 else n_kv_max - r % min(n_kv_max, count_spread)
        cnt = min(cnt, n_kv)
        pos = np.sort(rng.choice(n_kv, size=cnt, replace=False))
        m[r, pos] = -(1.0 + (np.arange(cnt) + r) % 7) / 32.0
    return round_to_dtype(m, dtype)


# ---------------------------------------------------------------------------
# Score rows that stress a block selection directly (not produced by scoring).
# ---------------------------------------------------------------------------

SCORE_ROW_KINDS = ("normal", "small_ints", "all_equal", "signed_zeros", "binade_gap", "lognormal_dups")


def score_row(kind: str, nb: int, k_blk: int, *, seed: int, case_id: int) -> np.ndarray:
    """[nb] float32 scores of one query's blocks, of a shape a selection must handle.

    normal          standard normal, so about half the scores are negative;
    small_ints      integers -3..4: few distinct values, the cut falls inside a run of
                    exact ties;
    all_equal       every score 1.5;
    signed_zeros    a few hundred positive scores, the rest +0.0 and -0.0 at random;
    binade_gap      k_blk scores of 4.0 at random blocks over uniform draws in [1, 2);
    lognormal_dups  positive lognormal draws, then the draws ranked k_blk - 40 ..
                    k_blk + 40 all set to the one ranked k_blk (ties across the cut).
    """
    rng = np.random.default_rng([seed, case_id, 6, SCORE_ROW_KINDS.index(kind)])
    if kind == "normal":
        s = rng.standard_normal(nb)
    elif kind == "small_ints":
        s = rng.integers(-3, 5, size=nb).astype(np.float64)
    elif kind == "all_equal":
        s = np.full(nb, 1.5)
    elif kind == "signed_zeros":
        s = np.where(rng.random(nb) < 0.5, 0.0, -0.0)
        hot = rng.choice(nb, size=min(nb, 300), replace=False)
        s[hot] = rng.random(hot.size) + 0.5
    elif kind == "binade_gap":
        s = rng.random(nb) + 1.0
        s[rng.choice(nb, size=min(nb, k_blk), replace=False)] = 4.0
    elif kind == "lognormal_dups":
        s = rng.lognormal(0.0, 0.5, size=nb)
        order = np.argsort(-s, kind="stable")
        lo, hi = max(0, k_blk - 41), min(nb, k_blk + 40)
        s[order[lo:hi]] = s[order[min(k_blk - 1, nb - 1)]]
    else:
        raise ValueError(f"unknown score row kind {kind}")
    return s.astype(np.float32)
