"""Comparison helpers for the GPU parity tests (HIP library vs the CPU oracle).

Tolerances
  * pooled keys: the library sums the c keys of a block in float32 (c - 1 roundings,
    each at most half an ulp of a partial sum, so at most (c-1) * 2**-24 * sum|x|
    in all), divides by c (one more float32 rounding) and rounds once to the cache
    dtype; the oracle rounds the exact mean once.  Tolerance: one ulp of the dtype
    at the mean plus c * 2**-24 * mean|x| -- with 8- or 11-bit inputs the float32
    sum is nearly always exact and the first term is all there is.
  * scores: |gpu - oracle| <= 1.5 * n * 2**-24 * sum_h sum_d |q_hd * kbar_d| with
    n = d_idx + h_idx, the standard bound for a float32 sum of n products (any
    order), plus the rectification (which never increases the error).
  * selection: the spec rule -- exact, except that blocks whose oracle score
    lies within 1e-3 (relative) of the K_blk-th oracle score may be exchanged.  When
    both sides see the same float32 scores (the select kernel fed the oracle's
    scores) the selection must be exact.
  * attention output: max-abs 2e-3 for f16/bf16 caches, 1e-5 for float32 caches.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

OUT_TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
NEAR_TIE_REL = 1e-3
ULP_BITS = {"f32": 24, "f16": 11, "bf16": 8}


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the dtype at |x| (normal range)."""
    _, e = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    emin = {"f32": -126, "f16": -14, "bf16": -126}[dtype]
    return np.ldexp(1.0, np.maximum(e, emin + 1) - ULP_BITS[dtype])


def check_pool(layer, case, pools: oracle.SequencePools) -> int:
    """Every complete block of every sequence; returns the number of elements that
    are not bit-identical to the oracle's (all within the tolerance)."""
    kpool = layer.kpool.float().cpu().numpy().astype(np.float64)
    c = case.dims.compress_ratio
    n_off = 0
    for s in range(case.n_seq):
        want = pools(s)
        nb = want.shape[0]
        b0, r0 = int(case.blk0[s]), int(case.row0[s])
        got = kpool[b0:b0 + nb]
        raw = np.abs(case.kidx[r0:r0 + nb * c].astype(np.float64)).reshape(nb, c, case.dims.d_idx).mean(axis=1)
        tol = ulp(want, case.dims.dtype) + c * 2.0 ** -24 * raw
        diff = np.abs(got - want)
        assert np.all(diff <= tol), (f"pooled keys of sequence {s} differ: worst "
                                     f"{float((diff / tol).max()) if diff.size else 0:.3g} x tolerance")
        n_off += int(np.count_nonzero(diff))
    return n_off


def score_tolerance(qidx: np.ndarray, pooled: np.ndarray) -> np.ndarray:
    q = np.abs(qidx.astype(np.float64))
    k = np.abs(pooled.astype(np.float64))
    mag = (k @ q.T).sum(axis=1)
    n = qidx.shape[1] + qidx.shape[0]
    return 1.5 * n * 2.0 ** -24 * mag + 1e-30


def check_scores(gpu_scores: np.ndarray, case, qi: int, res: dict, pools: oracle.SequencePools) -> float:
    s = int(case.q_seq[qi])
    nb = res["n_vis"] // case.dims.compress_ratio
    got = gpu_scores[:nb].astype(np.float64)
    want = res["scores"]
    tol = score_tolerance(case.qidx[qi], pools(s)[:nb])
    err = np.abs(got - want)
    assert np.all(err <= tol), f"query {qi}: score error {float((err / tol).max()):.3g} x tolerance"
    assert not np.any(np.signbit(gpu_scores[:nb])), "negative zero or negative score"
    return float((err / tol).max()) if nb else 0.0


def kept_blocks(positions: np.ndarray, nb: int, c: int) -> np.ndarray:
    p = np.asarray(positions, dtype=np.int64)
    return np.unique(p[p < nb * c] // c)


def check_list_form(positions: np.ndarray, n_vis: int, c: int, top_k: int) -> None:
    """Ascending, within the visible range, whole blocks, tail present, right size."""
    p = np.asarray(positions, dtype=np.int64)
    nb = n_vis // c
    assert np.all(np.diff(p) > 0), "positions not strictly ascending"
    assert p.size == 0 or (p[0] >= 0 and p[-1] < n_vis)
    want_len = min(nb, top_k // c) * c + (n_vis - nb * c)
    assert p.size == want_len, f"{p.size} positions, expected {want_len}"
    assert set(range(nb * c, n_vis)) <= set(p.tolist()), "tail missing"
    body = p[p < nb * c]
    assert body.size % c == 0 and np.all(body.reshape(-1, c) == (body.reshape(-1, c)[:, :1] + np.arange(c)))


def compare_selection(gpu_pos: np.ndarray, res: dict, case) -> str:
    """'exact' or 'near-tie' (allowed by the rule); raises otherwise."""
    d = case.dims
    c = d.compress_ratio
    check_list_form(gpu_pos, res["n_vis"], c, d.top_k)
    if np.array_equal(gpu_pos, res["positions"]):
        return "exact"
    nb = res["n_vis"] // c
    k_blk = d.top_k // c
    g = set(kept_blocks(gpu_pos, nb, c).tolist())
    o = set(kept_blocks(res["positions"], nb, c).tolist())
    assert len(g) == len(o)
    scores = res["scores"]
    s_k = np.sort(scores)[::-1][k_blk - 1]
    floor = 1e-6 * float(scores.max()) if scores.size else 0.0
    for b in g ^ o:
        assert abs(scores[b] - s_k) <= NEAR_TIE_REL * abs(s_k) + floor, (
            f"block {b} (score {scores[b]!r}) differs from the oracle's set; k-th score {s_k!r}")
    return "near-tie"


def check_out(got: np.ndarray, want: np.ndarray, dtype: str, what: str) -> float:
    err = float(np.max(np.abs(got.astype(np.float64) - want))) if want.size else 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= OUT_TOL[dtype], f"{what}: max-abs error {err:.3g} > {OUT_TOL[dtype]}"
    return err


def upload_selection(layer, positions_per_query) -> tuple[torch.Tensor, torch.Tensor]:
    sel = np.full((layer.n_q, layer.sel_ld), -1, dtype=np.int32)
    n_sel = np.zeros(layer.n_q, dtype=np.int32)
    for i, p in enumerate(positions_per_query):
        sel[i, : len(p)] = p
        n_sel[i] = len(p)
    return torch.from_numpy(sel).to(layer.device), torch.from_numpy(n_sel).to(layer.device)


def upload_scores(layer, scores_per_query) -> torch.Tensor:
    sc = np.zeros((layer.n_q, layer.scores_ld), dtype=np.float32)
    for i, s in enumerate(scores_per_query):
        sc[i, : len(s)] = s
    return torch.from_numpy(sc).to(layer.device)
