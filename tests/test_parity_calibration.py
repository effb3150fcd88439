"""Calibration of the attention-output comparison (CPU only).

The GPU parity tests accept an attention output when it meets the stated max-abs
tolerance and the per-element bound derived from the kernels' arithmetic
(tests/parity.py).  This file shows, at the shapes and inputs of the wide-logit GPU
cases (tests/attn_cases.py), that the comparison

  * accepts a correct computation with the kernels' roundings: a float32 emulation
    (float32 logits, exp2, each weight rounded once to the cache's 16-bit type for
    P.V, float32 sums) stays inside the bound, and
  * rejects wrong ones: each mistake below, planted in the oracle's inputs on the
    CPU, exceeds the bound on at least one checked query --
      uniform weights (Q.K^T ignored), the softmax scale dropped, the last 64 dims
      of K dropped from Q.K^T (the rope dims 512..575 of the 576-wide rows),
      head 0's query used for every head, any one 64-row tile of the list dropped,
      a dense window one row too short or too long, the bias dropped, scaled by the
      softmax scale or negated, and (q8_0) the block scales ignored.

The pages validate the same way: a scaled-down model with an init scale large
enough to give non-uniform logits, and a comparison shown to catch deliberately
seeded bugs ("model: add Qwen3.8-Flash-Next (qwen4exp)", the validation paragraph
of the CUDA-graph commit).
"""
import numpy as np
import pytest
import torch

import attn_cases
import oracle
import parity

TILE = 64


def emulate_kernel(q, k_rows, v_rows, scale, dtype, bias=None):
    """A correct attention with the kernels' roundings, in float32 (numpy/torch)."""
    q = np.asarray(q, np.float32)
    k = np.asarray(k_rows, np.float32)
    v = np.asarray(v_rows, np.float32)
    h_q = q.shape[0]
    n, h_kv, _ = k.shape
    out = np.zeros((h_q, v.shape[2]), np.float32)
    if n == 0:
        return out
    log2e = np.float32(1.4426950408889634)
    sl2 = np.float32(scale) * log2e
    b = np.zeros(n, np.float32) if bias is None else np.asarray(bias, np.float32) * log2e
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    g_of = h_q // h_kv
    for h in range(h_q):
        g = h // g_of
        x = (k[:, g, :] @ q[h]).astype(np.float32) * sl2 + b
        p = np.exp2(x - x.max()).astype(np.float32)
        pr = torch.from_numpy(p).to(tdt).to(torch.float32).numpy()
        out[h] = (pr @ v[:, g, :]).astype(np.float32) / np.float32(p.sum(dtype=np.float32))
    return out


class Checked:
    """The attention checks of one GPU case: per (query, window) the rows, bias and
    inputs, the oracle's output and its bound."""

    def __init__(self, spec: attn_cases.AttnCase):
        self.spec = spec
        case = spec.make()
        self.case = case
        d = case.dims
        self.dtype = d.dtype
        self.p_dtype = "bf16" if spec.q8 else d.dtype    # the q8_0 kernel rounds P times the scale to bf16
        k_all, v_all = case.k, case.v_rows()
        if spec.q8:
            kc, ks = oracle.quantize_q8_0(case.k)
            k_all = oracle.dequantize_q8_0(kc, ks)
            v_all = k_all[:, :, : d.d_v] if case.v is None else oracle.dequantize_q8_0(*oracle.quantize_q8_0(case.v))
        queries = range(case.n_q) if spec.queries is None else spec.queries
        mask = attn_cases.bias_mask(case) if spec.name == "bias_mla" else None
        pools = oracle.SequencePools(case)
        self.items = []
        for qi in queries:
            s = int(case.q_seq[qi])
            r0 = int(case.row0[s])
            bias = None
            if mask is not None:
                pos = oracle.mask_positions(mask[qi])
                bias = mask[qi, pos].astype(np.float64)
            else:
                pos = oracle.run_query(case, qi, pools)["positions"]
            n_vis = oracle.visible_tokens(case.seq_len[s], case.q_pos[qi])
            for w in spec.windows or (None,):
                p = pos if w is None else oracle.window_union(pos, n_vis, w)
                self.items.append(dict(qi=qi, w=w, n_vis=n_vis, sel=pos, pos=p, r0=r0, bias=bias,
                                       k=k_all[r0 + p], v=v_all[r0 + p]))
        for it in self.items:
            it["want"] = oracle.attend(case.q[it["qi"]], it["k"], it["v"], case.scale, bias=it["bias"])
            it["bound"] = parity.out_bound(case.q[it["qi"]], it["k"], it["v"], case.scale, self.dtype, it["bias"],
                                           self.p_dtype)

    def worst(self, mutant) -> float:
        """How far a mutant's output lies outside the comparison, over the checked
        items: the larger of its derived-bound ratio and its max-abs error over the
        stated tolerance (> 1: rejected)."""
        r = 0.0
        for it in self.items:
            got = mutant(it)
            if got is None:
                continue
            r = max(r, parity.bound_ratio(got, it["want"], it["bound"]),
                    float(np.abs(got - it["want"]).max()) / parity.OUT_TOL[self.dtype])
        return r


_CACHE = {}


def checked(name) -> Checked:
    if name not in _CACHE:
        _CACHE[name] = Checked(attn_cases.CASES[name])
    return _CACHE[name]


@pytest.mark.parametrize("name", list(attn_cases.CASES))
def test_correct_arithmetic_passes(name):
    c = checked(name)
    case = c.case
    worst = 0.0
    for it in c.items:
        got = emulate_kernel(case.q[it["qi"]], it["k"], it["v"], case.scale, c.p_dtype, it["bias"])
        parity.check_out(got, it["want"], c.dtype, f"{name} q{it['qi']} emulated", it["bound"])
        worst = max(worst, parity.bound_ratio(got, it["want"], it["bound"]))
    print(f"{name}: float32 emulation at {worst:.3f} of the derived bound")
    # the logits really are spread: the weights are far from uniform
    it = c.items[0]
    q = case.q[it["qi"]]
    x = case.scale * (np.asarray(it["k"], np.float64)[:, 0, :] @ np.asarray(q, np.float64)[0])
    if x.size > 16:
        assert np.std(x) > 0.5 * attn_cases.LOGIT_STD


def _planted(c: Checked):
    case = c.case
    d = case.dims
    sc = case.scale

    keep = object()

    def att(it, q=None, k=None, v=None, scale=None, bias=keep):
        return oracle.attend(case.q[it["qi"]] if q is None else q, it["k"] if k is None else k,
                             it["v"] if v is None else v, sc if scale is None else scale,
                             bias=it["bias"] if bias is keep else bias)

    def drop_dims(it):
        k = np.array(it["k"], copy=True)
        k[:, :, d.d_kq - 64:] = 0.0
        return att(it, k=k)

    def head0(it):
        q = case.q[it["qi"]]
        return att(it, q=np.repeat(q[:1], q.shape[0], axis=0))

    m = {"uniform weights": lambda it: att(it, scale=0.0, bias=None),
         "no softmax scale": lambda it: att(it, scale=1.0),
         "last 64 K dims dropped": drop_dims,
         "head 0 for every head": head0}
    if c.spec.windows:
        def window_off(delta):
            def f(it):
                w = it["w"] + delta
                if w < 0:
                    return None
                p = oracle.window_union(it["sel"], it["n_vis"], w)
                rows = it["r0"] + p
                kk, vv = case.k[rows], case.v_rows()[rows]
                return att(it, k=kk, v=vv)
            return f
        m["window one row short"] = window_off(-1)
        m["window one row long"] = window_off(+1)
    if c.spec.name == "bias_mla":
        m["bias dropped"] = lambda it: att(it, bias=None)
        m["bias times the softmax scale"] = lambda it: att(it, bias=it["bias"] * sc)
        m["bias negated"] = lambda it: att(it, bias=-it["bias"])
    if c.spec.q8:
        kc, ks = oracle.quantize_q8_0(case.k)
        codes_only = kc.astype(np.float64)

        def no_scales(it):
            rows = it["r0"] + it["pos"]
            k = codes_only[rows] * 0.01
            return att(it, k=k, v=k[:, :, : d.d_v])
        m["block scales ignored"] = no_scales
    return m


@pytest.mark.parametrize("name", list(attn_cases.CASES))
def test_planted_mistakes_are_rejected(name):
    c = checked(name)
    report = {}
    for label, mutant in _planted(c).items():
        r = c.worst(mutant)
        report[label] = r
        assert r > 1.0, f"{name}: the comparison accepts the mistake '{label}' (worst {r:.3g} x bound)"
    # any one 64-row tile of the list dropped (a split or tile the kernel skips)
    n_tiles = max((len(it["pos"]) + TILE - 1) // TILE for it in c.items)
    tile_worst = np.inf
    for j in range(n_tiles):
        def drop(it, j=j):
            n = len(it["pos"])
            if j * TILE >= n:
                return None
            keep = np.ones(n, bool)
            keep[j * TILE:(j + 1) * TILE] = False
            b = None if it["bias"] is None else it["bias"][keep]
            return oracle.attend(c.case.q[it["qi"]], it["k"][keep], it["v"][keep], c.case.scale, bias=b)
        r = c.worst(drop)
        assert r > 1.0, f"{name}: the comparison accepts dropping tile {j} (worst {r:.3g} x bound)"
        tile_worst = min(tile_worst, r)
    report["weakest dropped tile"] = tile_worst
    print(f"{name}: " + ", ".join(f"{k} {v:.3g}" for k, v in report.items()))
