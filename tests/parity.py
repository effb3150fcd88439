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
  * attention output: max-abs 2e-3 for f16/bf16 caches, 1e-5 for float32 caches
    (the stated tolerances), and in addition a per-element bound derived from the
    kernels' arithmetic (out_bound), which scales with the output and so also holds
    where the outputs are much smaller than 2e-3.  The kernels compute the logits
    in float32 from the stored operands (exact products), take exp2 in float32, round
    each weight p once to the cache's 16-bit type for the P.V product (the q8_0
    kernel: p times the block scale, rounded once to bfloat16 whatever the query
    type) while the weight sum l uses the unrounded p, and
    accumulate everything else in float32.  With oracle weights p_t, output o and
    relative weight errors |eta_t| <= e_t (logits) and |rho_t| <= u (the one
    rounding of p), the result sum p_t(1+eta_t)(1+rho_t) v_t / sum p_t(1+eta_t)
    differs from o by at most
        sum_t p_t (u + e_t + c0) (|v_t| + |o|) + gamma_n sum_t p_t |v_t|   (+ f16 underflow)
    where e_t = gamma_DKQ * (scale * sum_d |q_d k_td| + |bias_t|) bounds a float32
    dot product of DKQ terms (2 * n * 2**-24, which also covers truncating
    accumulation), gamma_n the float32 accumulation over the rows, c0 = 2**-16 the
    exp2, rescale and combine roundings, and an f16 weight below the smallest
    normal is off by at most 2**-25 in absolute terms (the largest weight is 1).
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


def exact_fp32_sums(raw: np.ndarray) -> np.ndarray:
    """[nb, d] mask of the blocks' elements whose float32 sum, taken in position
    order, has no rounding: every partial sum equals the exact (float64) one.  raw is
    [nb, c, d] of stored values (at most 24 significant bits each)."""
    acc32 = raw[:, 0, :].astype(np.float32)
    acc64 = raw[:, 0, :].astype(np.float64)
    ok = np.ones(acc64.shape, dtype=bool)
    for i in range(1, raw.shape[1]):
        acc32 = (acc32 + raw[:, i, :].astype(np.float32)).astype(np.float32)
        acc64 = acc64 + raw[:, i, :].astype(np.float64)
        ok &= acc32.astype(np.float64) == acc64
    return ok


def check_pool(layer, case, pools: oracle.SequencePools, kpool: torch.Tensor | None = None) -> int:
    """Every complete block of every sequence; returns the number of elements that
    are not bit-identical to the oracle's (all within the tolerance).  Where the
    float32 sum of a block is exact and c is a power of two (so the division is
    exact too), the one remaining rounding is the oracle's, and the element must be
    bit-identical."""
    kp = (layer.kpool if kpool is None else kpool).float().cpu().numpy().astype(np.float64)
    c = case.dims.compress_ratio
    pow2 = c & (c - 1) == 0
    n_off = 0
    for s in range(case.n_seq):
        want = pools(s)
        nb = want.shape[0]
        b0, r0 = int(case.blk0[s]), int(case.row0[s])
        got = kp[b0:b0 + nb]
        raw_v = case.kidx[r0:r0 + nb * c].reshape(nb, c, case.dims.d_idx)
        raw = np.abs(raw_v.astype(np.float64)).mean(axis=1)
        tol = ulp(want, case.dims.dtype) + c * 2.0 ** -24 * raw
        diff = np.abs(got - want)
        assert np.all(diff <= tol), (f"pooled keys of sequence {s} differ: worst "
                                     f"{float((diff / tol).max()) if diff.size else 0:.3g} x tolerance")
        if pow2 and nb:
            exact = exact_fp32_sums(raw_v)
            bad = exact & (diff != 0)
            assert not bad.any(), (f"sequence {s}: {int(bad.sum())} pooled elements with an exact float32 sum "
                                   f"differ from the oracle")
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


P_ROUND = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}   # one rounding of a weight


def out_bound(q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float, dtype: str,
              bias: np.ndarray | None = None, p_dtype: str | None = None) -> np.ndarray:
    """[H_q, DV] bound on |gpu - oracle| of an attention output (derivation above).
    q [H_q, DKQ], k_rows [n, H_kv, DKQ], v_rows [n, H_kv, DV] as stored; p_dtype is
    the type the weights are rounded to for P.V (default: dtype)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k_rows, dtype=np.float64)
    v = np.asarray(v_rows, dtype=np.float64)
    h_q, d_kq = q.shape
    n, h_kv, _ = k.shape
    d_v = v.shape[2]
    bound = np.zeros((h_q, d_v))
    if n == 0:
        return bound
    u = P_ROUND[p_dtype or dtype]
    g_k = 2.0 * (d_kq + 2) * 2.0 ** -24 + 2.0 ** -22
    g_n = 2.0 * (n + 16) * 2.0 ** -24
    c0 = 2.0 ** -16
    b = np.zeros(n) if bias is None else np.asarray(bias, dtype=np.float64)
    group = h_q // h_kv
    for h in range(h_q):
        g = h // group
        x = scale * (k[:, g, :] @ q[h]) + b
        w = np.exp(x - x.max())
        l = w.sum()
        p = w / l
        av = np.abs(v[:, g, :])
        o = p @ v[:, g, :]
        e = g_k * (abs(scale) * (np.abs(k[:, g, :]) @ np.abs(q[h])) + np.abs(b)) + c0 + u
        t = (p * e) @ av + (p * e).sum() * np.abs(o) + g_n * (p @ av)
        if (p_dtype or dtype) == "f16":
            t += 2.0 ** -25 * av.sum(axis=0) / l
        bound[h] = t * (1.0 + 2.0 ** -10)
    return bound


WORST = {"ratio": 0.0}   # largest bound ratio met since the last reset (for the test logs)


def take_worst_ratio() -> float:
    r = WORST["ratio"]
    WORST["ratio"] = 0.0
    return r


def check_out(got: np.ndarray, want: np.ndarray, dtype: str, what: str, bound: np.ndarray | None = None) -> float:
    """The stated max-abs tolerance and, when given, the derived per-element bound.
    Returns the max-abs error."""
    got = np.asarray(got, dtype=np.float64)
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= OUT_TOL[dtype], f"{what}: max-abs error {err:.3g} > {OUT_TOL[dtype]}"
    if bound is not None and want.size:
        ratio = np.abs(got - want) / (bound + 1e-30)
        worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        WORST["ratio"] = max(WORST["ratio"], float(ratio[worst]))
        assert float(ratio[worst]) <= 1.0, (f"{what}: element {tuple(int(x) for x in worst)} off by "
                                            f"{float(np.abs(got - want)[worst]):.3g}, {float(ratio[worst]):.3g} x "
                                            f"its derived bound {float(bound[worst]):.3g}")
    return err


def check_attention(got: np.ndarray, q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float,
                    dtype: str, what: str, bias: np.ndarray | None = None, p_dtype: str | None = None) -> float:
    """An attention output against the oracle's attention over the same rows, under
    both tolerances; returns the max-abs error."""
    want = oracle.attend(q, k_rows, v_rows, scale, bias=bias)
    return check_out(got, want, dtype, what, out_bound(q, k_rows, v_rows, scale, dtype, bias, p_dtype))


def bound_ratio(got: np.ndarray, want: np.ndarray, bound: np.ndarray) -> float:
    """max |got - want| / bound (how close an output comes to its derived bound)."""
    if not want.size:
        return 0.0
    return float(np.max(np.abs(np.asarray(got, np.float64) - want) / (bound + 1e-30)))


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
