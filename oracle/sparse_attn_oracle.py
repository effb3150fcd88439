"""CPU oracle for indexer-selected block-sparse attention (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  The tests, the package smoke check and the CPU-baseline
leg of the benchmark use this module; the library's compute path never imports,
calls or links it, and it imports nothing from the library.

What it computes follows the pages' description of the method:

* "llama: QSA sparse attention for qwen4exp" (llama.cpp commit series for
  Qwen3.8-Flash-Next / qwen4exp, #27742) -- the indexer scores one mean-pooled key
  per block of ``compress_ratio`` tokens, keeps a budget of the best blocks plus
  the tail of tokens that do not yet form a complete block, and is exactly dense
  below ``indexer_top_k + compress_ratio - 1`` cached tokens; each head's dot
  product is rectified before the sum over heads; the indexer cache holds raw keys
  because pooling comes before the norm and rotation; blocks are cuts of the
  position line; block scores are expanded to tokens and cut on block boundaries
  because a block's members tie exactly.
* "qwen4exp: support a non-unified KV cache in QSA" (same series) -- each
  sequence's queries are scored only against that sequence's blocks.
* "CUDA + ggml: add sparse-fa for DSV4/GLM" (llama.cpp PR #27970) -- attention
  runs over only the KV rows named by an ascending int32 index list, with many
  query heads per KV head; V may be a view of K (its first DV elements).

Every floating-point step runs in float64 on the exact stored (dtype-rounded)
inputs.  The one place where a floating value decides an integer -- the block
selection -- takes that decision on the scores rounded to float32, the precision
the pages' graph produces them in (a float32 matrix product) and the precision the
GPU kernel writes them in.

Readings where the pages leave a step open are listed at each function.
"""
from __future__ import annotations

import numpy as np

_FORMATS = {
    # significand bits (incl. the implicit one), minimum normal exponent
    "f32": (24, -126),
    "f16": (11, -14),
    "bf16": (8, -126),
}


def round_to_storage(x, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest value of the storage format, ties to even.

    A value with binary exponent e (x = m * 2**e, 0.5 <= |m| < 1) has an ulp of
    2**(e - p) for p significand bits; below the smallest normal the ulp stays at the
    subnormal spacing.  Overflow is not handled (the workloads stay far from it).
    """
    p, emin = _FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    ulp_exp = np.maximum(e, emin + 1) - p
    return np.ldexp(np.rint(np.ldexp(x, -ulp_exp)), ulp_exp)


# --------------------------------------------------------------------------- pool

def pool_blocks(kidx: np.ndarray, c: int, dtype: str) -> np.ndarray:
    """Mean-pooled indexer key of every complete block of ``c`` consecutive positions.

    ``kidx`` holds the raw indexer keys of one sequence, row t = position t.  Block b
    covers positions [b*c, (b+1)*c).  The mean is taken in float64 and stored in the
    cache dtype (reading: the pages pool in the graph and do not say how the pooled
    key is stored; this library keeps it in the key cache's dtype).
    """
    kidx = np.asarray(kidx, dtype=np.float64)
    n_blocks = kidx.shape[0] // c
    blocks = kidx[: n_blocks * c].reshape(n_blocks, c, kidx.shape[1])
    return round_to_storage(blocks.sum(axis=1) / c, dtype)


# -------------------------------------------------------------------------- score

def block_scores(qidx: np.ndarray, pooled: np.ndarray) -> np.ndarray:
    """Indexer score of each block for one query token.

    s_b = sum over indexer heads h of max(0, q_h . kbar_b).  The rectification is
    applied to each head's dot product before the head sum.  The heads are summed
    without weights; a caller folds any per-head weight or scale into q_h (reading:
    the pages name no weights).  Returns float64 (+0.0 where every head is <= 0).
    """
    qidx = np.asarray(qidx, dtype=np.float64)          # [H_idx, D_idx]
    pooled = np.asarray(pooled, dtype=np.float64)      # [NB, D_idx]
    dots = pooled @ qidx.T                             # [NB, H_idx]
    return np.maximum(dots, 0.0).sum(axis=1) + 0.0


# ------------------------------------------------------------------------- select

def visible_tokens(seq_len: int, q_pos: int) -> int:
    """Cached positions a query at ``q_pos`` may attend: t <= q_pos and t < seq_len."""
    return int(max(0, min(int(seq_len), int(q_pos) + 1)))


def select_blocks(scores: np.ndarray, k_blk: int) -> np.ndarray:
    """Indices of the kept blocks, ascending.

    All blocks when there are at most ``k_blk`` of them; otherwise the first k_blk
    blocks in the order (score descending, block index ascending) -- reading: the
    pages do not state a tie rule; ties go to the lower block index.
    """
    scores = np.asarray(scores)
    nb = scores.shape[0]
    if nb <= k_blk:
        return np.arange(nb, dtype=np.int64)
    order = np.lexsort((np.arange(nb), -scores.astype(np.float64)))
    return np.sort(order[:k_blk]).astype(np.int64)


def select_positions(scores: np.ndarray, n_vis: int, c: int, top_k: int) -> np.ndarray:
    """Ascending positions one query attends to.

    The kept blocks' c positions each, then the tail [NB*c, n_vis) -- the positions
    that do not yet form a complete block, always kept and not charged to the
    budget (reading: the pages keep "a budget of the best blocks, plus the tail").
    With NB = n_vis // c <= top_k / c this is every visible position, i.e. exactly
    dense attention below top_k + c - 1 visible tokens.
    """
    nb = n_vis // c
    assert scores.shape[0] == nb
    kept = select_blocks(scores, top_k // c)
    body = (kept[:, None] * c + np.arange(c)[None, :]).reshape(-1)
    tail = np.arange(nb * c, n_vis, dtype=np.int64)
    return np.concatenate([body, tail]).astype(np.int64)


def select_positions_token_expanded(scores: np.ndarray, n_vis: int, c: int, top_k: int) -> np.ndarray:
    """The pages' graph formulation of the same selection, used as a cross-check.

    Every token of a complete block gets its block's score, a token-level top-k of
    ``top_k`` tokens is taken (ties to the lower position) and the tail tokens are
    added.  Because a block's tokens tie exactly and the budget is a whole number of
    blocks, the cut lands on a block boundary and the set equals select_positions.
    """
    nb = n_vis // c
    tok = np.repeat(np.asarray(scores, dtype=np.float64), c)
    n_tok = nb * c
    keep = min(top_k, n_tok)
    order = np.lexsort((np.arange(n_tok), -tok))
    body = np.sort(order[:keep])
    tail = np.arange(n_tok, n_vis, dtype=np.int64)
    return np.concatenate([body, tail]).astype(np.int64)


# ------------------------------------------------------------------------- attend

def attend(q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float,
           bias: np.ndarray | None = None) -> np.ndarray:
    """softmax(scale * q K^T + bias) V over the given rows, per query head.

    ``q`` is [H_q, DKQ]; ``k_rows`` [n, H_kv, DKQ]; ``v_rows`` [n, H_kv, DV].  Query
    head h reads KV head h // (H_q / H_kv).  ``bias`` (optional, [n]) is added to
    every head's logit of a row: the additive-mask form of the pages' sparse flash
    attention, where a row's mask value is its bias ("CUDA + ggml: add sparse-fa for
    DSV4/GLM", the mask-driven sparse mode).  With no rows the output is zero
    (reading: the pages define no value for an empty set).
    """
    q = np.asarray(q, dtype=np.float64)
    k_rows = np.asarray(k_rows, dtype=np.float64)
    v_rows = np.asarray(v_rows, dtype=np.float64)
    h_q = q.shape[0]
    n, h_kv, _ = k_rows.shape
    d_v = v_rows.shape[2]
    group = h_q // h_kv
    out = np.zeros((h_q, d_v), dtype=np.float64)
    if n == 0:
        return out
    b = np.zeros(n) if bias is None else np.asarray(bias, dtype=np.float64)
    for h in range(h_q):
        g = h // group
        logits = scale * (k_rows[:, g, :] @ q[h]) + b
        w = np.exp(logits - logits.max())
        out[h] = (w / w.sum()) @ v_rows[:, g, :]
    return out


# ------------------------------------------------------------ additive-mask form

def mask_positions(mask_row: np.ndarray) -> np.ndarray:
    """The positions of a mask row that form the K/V set: its finite entries, in
    ascending order.  In the pages' sparse flash attention the finite entries of each
    mask row are the keys attended (their values added to the logits) and the rest
    (-inf) are skipped; a bound on the finite count per row sizes the index list
    ("CUDA + ggml: add sparse-fa for DSV4/GLM", ggml_flash_attn_ext_set_sparse and
    the mask-to-indices kernel).  NaN entries are not finite and are skipped."""
    m = np.asarray(mask_row, dtype=np.float64)
    return np.flatnonzero(np.isfinite(m)).astype(np.int64)


# ------------------------------------------------------------- dense window form

def window_union(selected: np.ndarray, n_vis: int, window: int) -> np.ndarray:
    """The selected positions together with the ``window`` most recent visible ones,
    ascending and each once.  A dense attention over the contiguous block of recent
    keys, a sparse one over the selected keys, and a merge of the two is the
    optimisation the pages report from a Vulkan fork ("CUDA + ggml: add sparse-fa for
    DSV4/GLM", review thread); reading: the contiguous block is the most recent
    ``window`` visible positions, and the result is attention over the union."""
    w0 = max(0, n_vis - max(window, 0))
    return np.union1d(np.asarray(selected, dtype=np.int64), np.arange(w0, n_vis, dtype=np.int64))


def merge_partials(parts) -> np.ndarray:
    """Exact merge of attention results over disjoint row sets: ``parts`` holds
    (out, m, l) per set, out the normalised [H, DV] result, m and l the per-head max
    logit and the sum of exp(logit - m)."""
    M = np.max([p[1] for p in parts], axis=0)
    num = sum(p[0] * (p[2] * np.exp(p[1] - M))[:, None] for p in parts)
    den = sum(p[2] * np.exp(p[1] - M) for p in parts)
    return num / den[:, None]


# ------------------------------------------------------------ quantized KV cache

Q8_0_BLOCK = 32


def quantize_q8_0(x) -> tuple[np.ndarray, np.ndarray]:
    """Quantize rows to the q8_0 KV-cache type: per block of 32 consecutive values one
    scale d and 32 signed 8-bit codes, value ~ d * code.

    The pages put a quantized KV cache on the QSA attention path ("qwen4exp: support
    a quantized KV cache in the QSA attention path", in the qwen4exp commit series)
    and run the sparse graph with K and V cache types q8_0 (the commit there on
    reserving the sparse graph).  Reading: q8_0 is ggml's published block format --
    d = max|x| / 127 over the block, codes = x / d rounded half away from zero (0 for
    an all-zero block), d stored as float16.  The codes are integers decided by
    floating point, so that decision is taken in float32, the precision of the format's
    reference quantizer and of the GPU kernel: max|x| exact, one correctly rounded
    division for d and one for 1/d, one float32 product per value, then the rounding.

    ``x``: float values [..., n], n % 32 == 0.  Returns (codes int8 [..., n],
    scales float64 [..., n / 32] holding float16 values).

    Pinned to that definition (a hand-worked block, invariants); agreement with ggml's
    own quantizer is parity unpinned: the pages hold no q8_0 value to compare with.
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    assert n % Q8_0_BLOCK == 0, "row length must be a multiple of 32"
    blocks = x.reshape(x.shape[:-1] + (n // Q8_0_BLOCK, Q8_0_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    d = (amax / np.float32(127.0)).astype(np.float32)
    inv = np.zeros_like(d)
    nz = d != 0
    inv[nz] = np.float32(1.0) / d[nz]
    y = (blocks * inv[..., None]).astype(np.float32).astype(np.float64)
    codes = np.sign(y) * np.floor(np.abs(y) + 0.5)          # exact in float64: half away from zero
    return codes.astype(np.int8).reshape(x.shape), round_to_storage(d.astype(np.float64), "f16")


def dequantize_q8_0(codes, scales) -> np.ndarray:
    """The values a q8_0 cache holds: scale of the block times the code, in float64
    (exact: an 8-bit code times an 11-bit scale)."""
    codes = np.asarray(codes, dtype=np.float64)
    scales = np.asarray(scales, dtype=np.float64)
    return codes * np.repeat(scales, Q8_0_BLOCK, axis=-1)


# ----------------------------------------------------------------------- pipeline

class SequencePools:
    """Pooled indexer keys per sequence, computed once and reused by all queries."""

    def __init__(self, case):
        self.case = case
        self._pooled = {}

    def __call__(self, s: int) -> np.ndarray:
        if s not in self._pooled:
            case = self.case
            r0, L = int(case.row0[s]), int(case.seq_len[s])
            self._pooled[s] = pool_blocks(case.kidx[r0:r0 + L], case.dims.compress_ratio, case.dims.dtype)
        return self._pooled[s]


def run_query(case, qi: int, pools: SequencePools | None = None, positions: np.ndarray | None = None) -> dict:
    """Pool -> score -> select -> attend for query token ``qi`` of a case.

    ``positions`` overrides the selection (to run the attention on another set).
    Returns the float64 scores, the float32-rounded scores the selection used,
    the ascending positions and the [H_q, DV] output.
    """
    d = case.dims
    if pools is None:
        pools = SequencePools(case)
    s = int(case.q_seq[qi])
    n_vis = visible_tokens(case.seq_len[s], case.q_pos[qi])
    nb = n_vis // d.compress_ratio
    pooled = pools(s)[:nb]
    scores = block_scores(case.qidx[qi], pooled)
    scores32 = scores.astype(np.float32)
    if positions is None:
        positions = select_positions(scores32, n_vis, d.compress_ratio, d.top_k)
    rows = int(case.row0[s]) + np.asarray(positions, dtype=np.int64)
    k_rows = case.k[rows]
    v_rows = case.v_rows()[rows]
    out = attend(case.q[qi], k_rows, v_rows, case.scale)
    return {"n_vis": n_vis, "scores": scores, "scores32": scores32, "positions": positions, "out": out}


def run_case(case, queries=None) -> list[dict]:
    """run_query for each listed query (all by default), sharing the pooled keys."""
    pools = SequencePools(case)
    if queries is None:
        queries = range(case.n_q)
    return [run_query(case, int(qi), pools) for qi in queries]
