"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one oracle function to a library routine on a special case, a
closed form worked by hand, brute force on tiny inputs, an invariant the pages
state, or the pages' own alternative formulation -- chosen so that a dropped term,
a wrong sign, an off-by-one block or tail, a wrong tie rule or a transposed
operand fails at least one of them.  The mutant tests at the end check that.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from indexer_top_block_amd import datagen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ rounding

def _fp32_ties(rng, n):
    """float64 values exactly halfway between two adjacent float32 values."""
    a = rng.standard_normal(n).astype(np.float32)
    b = np.nextafter(a, np.float32(np.inf))
    return (a.astype(np.float64) + b.astype(np.float64)) / 2


def test_round_f32_matches_hardware_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        _fp32_ties(rng, 5000), [0.0, -0.0, 1e-45, 3e-39, -2.5e-40]])
    got = oracle.round_to_storage(x, "f32")
    want = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(got, want)


def test_round_f16_matches_numpy_half():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 4, 20000)
    halves = rng.standard_normal(5000).astype(np.float16)
    ties = (halves.astype(np.float64) + np.nextafter(halves, np.float16(np.inf)).astype(np.float64)) / 2
    x = np.concatenate([x, ties, [6.0e-8, 3.0e-8, 1.0e-5, -4.5e-6]])
    x = x[np.abs(x) < 60000]
    got = oracle.round_to_storage(x, "f16")
    want = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, want)


def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(3)
    f = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0)
    bits = f.view(np.uint32)
    ties = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)       # exactly half a bf16 ulp
    x = np.concatenate([f, ties, np.array([1e-39, -2e-40], np.float32)])
    got = oracle.round_to_storage(x.astype(np.float64), "bf16")
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------- pool

def test_pool_identical_keys_pool_to_the_key():
    rng = np.random.default_rng(4)
    keys = datagen.round_to_dtype(rng.standard_normal((5, 16)).astype(np.float32), "bf16")
    kidx = np.repeat(keys, 4, axis=0)                               # 5 blocks of 4 equal rows
    assert np.array_equal(oracle.pool_blocks(kidx, 4, "bf16"), keys.astype(np.float64))


def test_pool_arithmetic_progression_closed_form():
    # row t holds the value t in every column; block b's mean is b*c + (c-1)/2
    for c in (1, 2, 3, 4, 8):
        L = 7 * c + (c - 1)                                         # 7 complete blocks + a partial one
        kidx = np.repeat(np.arange(L, dtype=np.float64)[:, None], 3, axis=1)
        got = oracle.pool_blocks(kidx, c, "f32")
        want = (np.arange(7) * c + (c - 1) / 2.0)[:, None].repeat(3, axis=1)
        assert got.shape == (7, 3)
        assert np.array_equal(got, want)


def test_pool_rounds_mean_to_nearest_even():
    # bf16 ulp at 1.0 is 2**-7.  Mean 1 + 2**-9 rounds down; 1 + 2**-8 is a tie -> even (1.0);
    # 1 + 3 * 2**-8 is a tie between 1 + 2**-7 (odd) and 1 + 2**-6 (even) -> 1 + 2**-6.
    u = 2.0 ** -7
    kidx = np.array([[1, 1], [1, 1], [1, 1], [1 + u, 1 + u],
                     [1, 1], [1, 1], [1 + u, 1 + u], [1 + u, 1 + u],
                     [1 + u, 1 + u], [1 + u, 1 + u], [1 + u, 1 + u], [1 + 2 * u, 1 + 2 * u]], dtype=np.float64)
    # block 2: mean = 1 + (3u + 2u)/4 = 1 + 1.25u -> nearest is 1 + u
    got = oracle.pool_blocks(kidx, 4, "bf16")[:, 0]
    assert list(got) == [1.0, 1.0, 1.0 + u]
    kidx2 = np.array([[1 + u], [1 + u], [1 + 2 * u], [1 + 2 * u]], dtype=np.float64)   # mean 1 + 1.5u: tie
    assert oracle.pool_blocks(kidx2, 4, "bf16")[0, 0] == 1.0 + 2 * u


# --------------------------------------------------------------------- score

# Worked by hand: heads q0 = (1, -2), q1 = (3, 1);
#   kbar0 = ( 1,  1): dots (-1, 4)  -> relu-sum 4   (sum-then-relu would give 3)
#   kbar1 = ( 2, -1): dots ( 4, 5)  -> 9
#   kbar2 = (-1, -1): dots ( 1, -4) -> 1            (sum-then-relu would give 0)
#   kbar3 = (-1,  0): dots (-1, -3) -> 0
HAND_Q = np.array([[1.0, -2.0], [3.0, 1.0]])
HAND_K = np.array([[1.0, 1.0], [2.0, -1.0], [-1.0, -1.0], [-1.0, 0.0]])
HAND_S = np.array([4.0, 9.0, 1.0, 0.0])


def test_score_hand_example():
    assert np.array_equal(oracle.block_scores(HAND_Q, HAND_K), HAND_S)


def test_score_single_head_is_relu_of_dot():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 32))
    k = rng.standard_normal((50, 32))
    want = np.array([max(0.0, float(np.dot(q[0], kk))) for kk in k])
    assert np.allclose(oracle.block_scores(q, k), want, rtol=1e-14, atol=1e-14)


def test_score_all_negative_is_positive_zero():
    q = np.array([[1.0, 1.0], [2.0, 0.5]])
    k = np.array([[-1.0, -1.0], [-3.0, -0.1]])
    s = oracle.block_scores(q, k)
    assert np.all(s == 0.0) and not np.any(np.signbit(s))


def test_score_positive_homogeneity_and_head_permutation():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((8, 16))
    k = rng.standard_normal((40, 16))
    s = oracle.block_scores(q, k)
    assert np.allclose(oracle.block_scores(4.0 * q, k), 4.0 * s, rtol=1e-14)
    assert np.allclose(oracle.block_scores(q[::-1], k), s, rtol=1e-13)
    # blocks are independent: scoring a subset gives the matching entries
    assert np.array_equal(oracle.block_scores(q, k[7:19]), s[7:19])


# -------------------------------------------------------------------- select

def _brute_force_blocks(scores, k_blk):
    """The unique k_blk-subset S with every member ahead of every non-member in
    (score desc, index asc) order, found by enumerating all subsets."""
    nb = len(scores)
    if nb <= k_blk:
        return list(range(nb))
    found = []
    for sub in itertools.combinations(range(nb), k_blk):
        inside = set(sub)
        ok = all((scores[i] > scores[j]) or (scores[i] == scores[j] and i < j)
                 for i in inside for j in range(nb) if j not in inside)
        if ok:
            found.append(list(sub))
    assert len(found) == 1
    return found[0]


def test_select_brute_force_tiny_with_ties():
    rng = np.random.default_rng(7)
    for _ in range(150):
        nb = int(rng.integers(1, 10))
        k_blk = int(rng.integers(1, 6))
        scores = rng.integers(0, 4, nb).astype(np.float32)          # many exact ties
        want = _brute_force_blocks(list(scores), k_blk)
        assert list(oracle.select_blocks(scores, k_blk)) == want


def test_select_matches_token_expanded_formulation():
    rng = np.random.default_rng(8)
    for _ in range(200):
        c = int(rng.integers(1, 6))
        k_blk = int(rng.integers(1, 12))
        n_vis = int(rng.integers(0, 120))
        nb = n_vis // c
        scores = rng.integers(0, 5, nb).astype(np.float32) * np.float32(0.25)
        a = oracle.select_positions(scores, n_vis, c, k_blk * c)
        b = oracle.select_positions_token_expanded(scores, n_vis, c, k_blk * c)
        assert np.array_equal(a, b)


def test_select_tail_size_order_and_dense_below_budget():
    rng = np.random.default_rng(9)
    for _ in range(300):
        c = int(rng.integers(1, 9))
        k_blk = int(rng.integers(1, 20))
        top_k = k_blk * c
        n_vis = int(rng.integers(0, 300))
        nb = n_vis // c
        tail = n_vis - nb * c
        scores = rng.random(nb).astype(np.float32)
        pos = oracle.select_positions(scores, n_vis, c, top_k)
        assert np.all(np.diff(pos) > 0)                              # ascending, distinct
        assert len(pos) == min(nb, k_blk) * c + tail <= top_k + c - 1
        assert set(range(nb * c, n_vis)) <= set(pos.tolist())       # the tail is always kept
        if n_vis <= top_k + c - 1:
            assert np.array_equal(pos, np.arange(n_vis))             # exactly dense
        else:
            assert len(pos) == top_k + tail
        blocks = set((p // c) for p in pos if p < nb * c)
        for b in blocks:                                            # whole blocks only
            assert all((b * c + i) in set(pos.tolist()) for i in range(c))


def test_select_page_budget_facts():
    facts = json.load(open(os.path.join(GOLDEN, "qsa_page_facts.json")))
    ex = facts["budget_example"]
    assert ex["tokens"] // ex["times_budget"] == ex["indexer_top_k"]
    d = facts["dense_below_budget"]
    top_k, c = d["indexer_top_k"], d["compress_ratio"]
    rng = np.random.default_rng(10)
    for n_vis in (d["fixture_tokens"], d["dense_through_n_vis"] - 1, d["dense_through_n_vis"]):
        scores = rng.random(n_vis // c).astype(np.float32)
        assert np.array_equal(oracle.select_positions(scores, n_vis, c, top_k), np.arange(n_vis))
    n_vis = d["first_sparse_n_vis"]
    scores = rng.random(n_vis // c).astype(np.float32)
    pos = oracle.select_positions(scores, n_vis, c, top_k)
    assert len(pos) == top_k and len(pos) < n_vis
    assert np.argmin(scores) * c not in set(pos.tolist())             # the one dropped block is the worst


def test_visible_tokens():
    assert oracle.visible_tokens(1024, 1024) == 1024                  # decode: query after the cache
    assert oracle.visible_tokens(34816, 32768) == 32769               # prefill: causal, itself included
    assert oracle.visible_tokens(10, -1) == 0
    assert oracle.visible_tokens(0, 5) == 0


# -------------------------------------------------------------------- attend

def _sdpa(q, k, v, scale, mask=None):
    """torch's scaled_dot_product_attention in float64 on the CPU, GQA by repeating KV."""
    h_q = q.shape[0]
    n, h_kv, _ = k.shape
    g = h_q // h_kv
    kk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).repeat_interleave(g, 0)
    vv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).repeat_interleave(g, 0)
    qq = torch.from_numpy(q)[:, None, :]
    m = None if mask is None else torch.from_numpy(mask)[None, None, :].expand(h_q, 1, n)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m, scale=scale)
    return o[:, 0, :].numpy()


def test_attend_matches_library_attention():
    rng = np.random.default_rng(11)
    for h_q, h_kv, dkq, dv, n in ((8, 1, 64, 64, 37), (16, 2, 96, 80, 100), (4, 4, 32, 16, 1)):
        q = rng.standard_normal((h_q, dkq))
        k = rng.standard_normal((n, h_kv, dkq))
        v = rng.standard_normal((n, h_kv, dv))
        scale = 1.0 / math.sqrt(dkq)
        assert np.allclose(oracle.attend(q, k, v, scale), _sdpa(q, k, v, scale), rtol=1e-12, atol=1e-12)


def test_attend_over_selection_equals_masked_dense_attention():
    # the pages' mechanism: attention over all rows with -inf on the unselected ones
    rng = np.random.default_rng(12)
    n, h_q, dkq, dv = 64, 8, 32, 24
    q = rng.standard_normal((h_q, dkq))
    k = rng.standard_normal((n, 1, dkq))
    v = rng.standard_normal((n, 1, dv))
    sel = np.sort(rng.choice(n, 20, replace=False))
    mask = np.full(n, -np.inf)
    mask[sel] = 0.0
    got = oracle.attend(q, k[sel], v[sel], 0.3)
    assert np.allclose(got, _sdpa(q, k, v, 0.3, mask), rtol=1e-12, atol=1e-12)


def test_attend_closed_forms():
    rng = np.random.default_rng(13)
    v = rng.standard_normal((9, 1, 5))
    q = rng.standard_normal((4, 6))
    # K == 0: uniform weights, the plain mean of the V rows
    assert np.allclose(oracle.attend(q, np.zeros((9, 1, 6)), v, 1.0), np.tile(v[:, 0].mean(0), (4, 1)))
    # equal V rows: the output is that row whatever the weights
    same = np.repeat(v[:1], 9, axis=0)
    k = rng.standard_normal((9, 1, 6))
    assert np.allclose(oracle.attend(q, k, same, 1.0), np.tile(v[0, 0], (4, 1)), rtol=1e-14)
    # no rows: zero output
    assert np.array_equal(oracle.attend(q, np.zeros((0, 1, 6)), np.zeros((0, 1, 5)), 1.0), np.zeros((4, 5)))
    # one row: that row's V
    assert np.allclose(oracle.attend(q, k[:1], v[:1], 1.0), np.tile(v[0, 0], (4, 1)))


# ------------------------------------------------------------ additive-mask form

def test_mask_positions_follow_the_pages_mask_pattern():
    """The pages' test masks: 1 finite entry on every 32nd row, otherwise
    n_kv_max - row mod min(n_kv_max, 17); mask_positions lists exactly the finite
    entries, ascending, and skips -inf, +inf and NaN."""
    facts = json.load(open(os.path.join(GOLDEN, "qsa_page_facts.json")))["sparse_mask_pattern"]
    spread, stride = facts["count_spread"], facts["single_entry_stride"]
    n_kv, n_kv_max = 4096, 512
    mask = datagen.sparse_mask(70, n_kv, n_kv_max, seed=0, case_id=900, count_spread=spread,
                               single_entry_stride=stride)
    for r in range(70):
        pos = oracle.mask_positions(mask[r])
        want = 1 if r % stride == 0 else n_kv_max - r % min(n_kv_max, spread)
        assert len(pos) == want and np.all(np.diff(pos) > 0)
        assert np.isfinite(mask[r, pos]).all() and np.isneginf(np.delete(mask[r], pos)).all()
    row = np.array([0.0, -np.inf, 1.5, np.nan, np.inf, -2.0])
    assert list(oracle.mask_positions(row)) == [0, 2, 5]


def test_attend_bias_matches_library_attention_with_a_float_mask():
    rng = np.random.default_rng(21)
    n, h_q, dkq, dv = 50, 8, 32, 24
    q = rng.standard_normal((h_q, dkq))
    k = rng.standard_normal((n, 2, dkq))
    v = rng.standard_normal((n, 2, dv))
    mask = np.full(n, -np.inf)
    sel = np.sort(rng.choice(n, 17, replace=False))
    mask[sel] = rng.uniform(-1.0, 0.5, size=17)
    got = oracle.attend(q, k[sel], v[sel], 0.2, bias=mask[sel])
    assert np.allclose(got, _sdpa(q, k, v, 0.2, mask), rtol=1e-12, atol=1e-12)


def test_attend_bias_closed_forms():
    rng = np.random.default_rng(22)
    q, k, v = rng.standard_normal((4, 8)), rng.standard_normal((10, 1, 8)), rng.standard_normal((10, 1, 6))
    b = rng.standard_normal(10)
    # a constant added to every bias leaves the softmax unchanged
    assert np.allclose(oracle.attend(q, k, v, 0.5, bias=b + 3.25), oracle.attend(q, k, v, 0.5, bias=b),
                       rtol=1e-13, atol=1e-13)
    # zero bias is no bias
    assert np.array_equal(oracle.attend(q, k, v, 0.5, bias=np.zeros(10)), oracle.attend(q, k, v, 0.5))
    # one row far above the rest takes all the weight
    dom = np.full(10, -1e4)
    dom[6] = 0.0
    assert np.allclose(oracle.attend(q, k, v, 0.5, bias=dom), np.tile(v[6, 0], (4, 1)), rtol=1e-13)


# ------------------------------------------------------------- dense window form

def _stats(q, k, v, scale):
    """(out, m, l) of one row set: the normalised output, per-head max logit and sum."""
    logits = scale * np.einsum("nd,hd->hn", k[:, 0], q)
    m = logits.max(axis=1)
    l = np.exp(logits - m[:, None]).sum(axis=1)
    return oracle.attend(q, k, v, scale), m, l


def test_window_union_definition_and_limits():
    sel = np.array([0, 1, 2, 3, 40, 41, 42, 43, 96, 97, 98, 99])
    assert np.array_equal(oracle.window_union(sel, 100, 0), sel)                 # no window: the selection
    assert np.array_equal(oracle.window_union(sel, 100, 10),
                          np.concatenate([sel[:8], np.arange(90, 100)]))          # overlap counted once
    assert np.array_equal(oracle.window_union(sel, 100, 500), np.arange(100))    # window past the start: dense
    assert np.array_equal(oracle.window_union(np.array([], np.int64), 5, 3), np.arange(2, 5))


def test_window_union_attention_is_the_merge_of_window_and_sparse_parts():
    # the dense-window + sparse + combine form computes attention over the union
    rng = np.random.default_rng(23)
    n, h_q, d = 300, 8, 32
    q = rng.standard_normal((h_q, d))
    k = rng.standard_normal((n, 1, d))
    v = rng.standard_normal((n, 1, 24))
    sel = np.sort(rng.choice(n, 60, replace=False))
    u = oracle.window_union(sel, n, 50)
    win = np.arange(n - 50, n)
    rest = np.setdiff1d(sel, win)
    parts = [_stats(q, k[win], v[win], 0.2), _stats(q, k[rest], v[rest], 0.2)]
    assert np.allclose(oracle.merge_partials(parts), oracle.attend(q, k[u], v[u], 0.2), rtol=1e-12, atol=1e-12)
    # counting the overlap twice is a different (wrong) answer
    dup = np.concatenate([sel, win])
    assert not np.allclose(oracle.attend(q, k[dup], v[dup], 0.2), oracle.attend(q, k[u], v[u], 0.2))


# ------------------------------------------------------------ quantized KV cache

def _f16(v: float) -> float:
    """float16 rounding by Python's own half-precision packing (ties to even)."""
    import struct
    return struct.unpack("<e", struct.pack("<e", v))[0]


def _round_half_away(fr):
    """Round a Fraction half away from zero."""
    from fractions import Fraction
    a = abs(fr)
    r = math.floor(a + Fraction(1, 2))
    return r if fr >= 0 else -r


def test_q8_0_hand_block():
    # codes = round(x * 127 / max|x|) in exact rational arithmetic (the block has no
    # value near a rounding tie, so float32 cannot change a code); scale = the float16
    # of max|x| / 127
    from fractions import Fraction
    x = (np.arange(32) - 16) * 3 + 1                              # -47 .. 46 step 3
    amax = int(np.abs(x).max())
    exact = [Fraction(int(v) * 127, amax) for v in x]
    assert all(abs(abs(e - math.floor(e)) - Fraction(1, 2)) > Fraction(1, 1000) for e in exact)
    want = [_round_half_away(e) for e in exact]
    codes, scales = oracle.quantize_q8_0(x.astype(np.float32))
    assert codes.tolist() == want
    assert codes[0] == -127
    assert scales.shape == (1,) and scales[0] == _f16(float(np.float32(amax) / np.float32(127)))


def test_q8_0_ties_round_half_away_from_zero():
    # max|x| = 127 makes d = 1 and 1/d = 1 exactly, so x * (1/d) = x: halves are ties
    x = np.zeros(32, np.float32)
    x[:8] = [127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5]
    codes, scales = oracle.quantize_q8_0(x)
    assert codes[:8].tolist() == [127, 3, -3, 1, -1, 2, -2, 127]
    assert scales[0] == 1.0


def test_q8_0_invariants():
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((40, 96)) * np.exp(rng.uniform(-6, 3, (40, 1)))).astype(np.float32)
    x[3, 32:64] = 0.0                                            # an all-zero block
    codes, scales = oracle.quantize_q8_0(x)
    assert codes.shape == x.shape and scales.shape == (40, 3)
    assert np.abs(codes.astype(int)).max() <= 127
    blk = x.reshape(40, 3, 32)
    cb = codes.reshape(40, 3, 32).astype(int)
    arg = np.abs(blk).argmax(axis=-1)
    top = np.take_along_axis(cb, arg[..., None], axis=-1)[..., 0]
    top_x = np.take_along_axis(blk, arg[..., None], axis=-1)[..., 0]
    nz = np.abs(top_x) > 0
    assert (np.abs(top[nz]) == 127).all() and (np.sign(top[nz]) == np.sign(top_x[nz])).all()
    assert (cb[3, 1] == 0).all() and scales[3, 1] == 0.0
    assert (np.sign(cb) * np.sign(blk) >= 0).all()                # signs kept (or zero)
    # reconstruction error: half a step, plus the scale's float16 rounding
    d32 = np.abs(blk).max(axis=-1).astype(np.float64) / 127.0
    err = np.abs(oracle.dequantize_q8_0(codes, scales) - x.astype(np.float64)).reshape(40, 3, 32).max(axis=-1)
    assert (err <= d32 / 2 * (1 + 1e-6) + 127 * np.abs(scales - d32) + 1e-30).all()
    # a power-of-two scaling of a block scales d and leaves the codes
    c2, s2 = oracle.quantize_q8_0(x[:, :32] * np.float32(4.0))
    ok = (scales[:, 0] * 4 < 65504) & (scales[:, 0] >= 2.0 ** -14)      # normal float16 both ways
    assert np.array_equal(c2[ok], codes[ok, :32]) and np.array_equal(s2[ok, 0], scales[ok, 0] * 4)


def test_q8_0_blocks_are_independent_and_round_trip_exactly():
    rng = np.random.default_rng(32)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    c0, s0 = oracle.quantize_q8_0(x)
    y = x.copy()
    y[:, 40] *= 50.0                                             # only the second block changes
    c1, s1 = oracle.quantize_q8_0(y)
    assert np.array_equal(c0[:, :32], c1[:, :32]) and np.array_equal(s0[:, 0], s1[:, 0])
    assert not np.array_equal(s0[:, 1], s1[:, 1])
    # values already of the form d * code (d a float16 power of two, one code of +-127)
    # quantize and dequantize back exactly
    codes = rng.integers(-127, 128, size=(6, 64))
    codes[:, ::32] = 127
    d = np.float64(2.0) ** rng.integers(-12, 2, size=(6, 2))
    vals = (codes * np.repeat(d, 32, axis=1)).astype(np.float32)
    c2, s2 = oracle.quantize_q8_0(vals)
    assert np.array_equal(c2, codes) and np.array_equal(s2, d)
    assert np.array_equal(oracle.dequantize_q8_0(c2, s2), vals.astype(np.float64))


def test_attention_on_a_q8_0_cache_is_attention_on_its_values():
    # rows exactly representable in q8_0 round-trip unchanged, so the attention over
    # the quantized cache equals torch's attention over the original values
    rng = np.random.default_rng(33)
    n, h_q, dkq, dv = 40, 8, 64, 64
    codes = rng.integers(-127, 128, size=(n, dkq))
    codes[:, ::32] = -127
    d = np.float64(2.0) ** rng.integers(-9, -5, size=(n, dkq // 32))
    k = codes * np.repeat(d, 32, axis=1)
    kc, ks = oracle.quantize_q8_0(k.astype(np.float32))
    kq = oracle.dequantize_q8_0(kc, ks)
    assert np.array_equal(kq, k)
    q = rng.standard_normal((h_q, dkq))
    got = oracle.attend(q, kq[:, None, :], kq[:, None, :dv], 0.125)
    assert np.allclose(got, _sdpa(q, k[:, None, :], k[:, None, :dv], 0.125), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ pipeline

def _small_dims(**kw):
    base = dict(h_q=8, h_kv=1, d_kq=32, d_v=32, h_idx=4, d_idx=16, compress_ratio=4, top_k=16, dtype="f32")
    base.update(kw)
    return datagen.Dims(**base)


def test_pipeline_below_budget_is_dense_causal_attention():
    dims = _small_dims(top_k=64)
    L = 40
    case = datagen.make_case("t", dims, [L], [0, 0, 0], [10, 39, 55], seed=0, case_id=100)
    for qi, r in enumerate(oracle.run_case(case)):
        n_vis = min(L, int(case.q_pos[qi]) + 1)
        assert np.array_equal(r["positions"], np.arange(n_vis))
        want = _sdpa(case.q[qi].astype(np.float64), case.k[:n_vis].astype(np.float64),
                     case.v[:n_vis].astype(np.float64), case.scale)
        assert np.allclose(r["out"], want, rtol=1e-12, atol=1e-12)


def test_pipeline_sequences_are_isolated():
    # the second sequence's query selects from its own rows only, whatever the first holds
    dims = _small_dims()
    case = datagen.make_case("t", dims, [50, 70], [0, 1], [50, 70], seed=1, case_id=101)
    r1 = oracle.run_query(case, 1)
    case.kidx[: case.seq_cap[0]] *= 100.0                               # perturb sequence 0 only
    case.k[: case.seq_cap[0]] = 0.0
    r1b = oracle.run_query(case, 1)
    assert np.array_equal(r1["positions"], r1b["positions"])
    assert np.array_equal(r1["out"], r1b["out"])


def test_pipeline_planted_blocks_are_preferred():
    dims = _small_dims(h_idx=16, d_idx=32, top_k=64, dtype="bf16")
    case = datagen.make_case("t", dims, [4096], [0], [4096], seed=2, case_id=102, std="inv_sqrt_dim",
                             v_separate=False, plant_fraction=0.01, plant_sigmas=3.0)
    r = oracle.run_query(case, 0)
    kept = set((r["positions"] // 4).tolist())
    planted = set(case.planted_blocks.tolist())
    assert len(planted) == 10
    assert len(kept & planted) >= 8                                     # planted blocks dominate
    assert r["n_vis"] == 4096 and len(r["positions"]) == 64


def test_pipeline_v_alias_reads_k_prefix():
    dims = _small_dims(d_kq=48, d_v=32, dtype="bf16")
    case = datagen.make_case("t", dims, [30], [0], [30], seed=3, case_id=103, v_separate=False)
    r = oracle.run_query(case, 0)
    pos = r["positions"]
    want = oracle.attend(case.q[0], case.k[pos], case.k[pos][:, :, :32], case.scale)
    assert np.array_equal(r["out"], want)


# -------------------------------------------------------------------- mutants

def test_mutants_are_caught():
    """Plausible mistakes, planted in copies of the oracle's steps, fail the pins."""
    # 1. sum over heads before the rectification
    def score_sum_then_relu(q, k):
        return np.maximum((k @ q.T).sum(axis=1), 0.0)
    assert not np.array_equal(score_sum_then_relu(HAND_Q, HAND_K), HAND_S)

    # 2. transposed operand: rows of the pooled keys scored against query dims swapped
    def score_transposed(q, k):
        return np.maximum(k @ q, 0.0).sum(axis=1)
    assert not np.array_equal(score_transposed(HAND_Q, HAND_K), HAND_S)

    # 3. ties to the higher block index
    def select_ties_high(scores, k_blk):
        nb = len(scores)
        order = np.lexsort((-np.arange(nb), -np.asarray(scores, np.float64)))
        return np.sort(order[:k_blk])
    scores = np.array([1, 2, 2, 2, 0], np.float32)
    assert list(select_ties_high(scores, 2)) != _brute_force_blocks(list(scores), 2)

    # 4. the tail charged to the budget (dropping a block when a tail exists)
    def select_tail_charged(scores, n_vis, c, top_k):
        nb = n_vis // c
        tail = n_vis - nb * c
        k_blk = (top_k - tail) // c
        kept = oracle.select_blocks(scores, k_blk)
        body = (kept[:, None] * c + np.arange(c)).reshape(-1)
        return np.concatenate([body, np.arange(nb * c, n_vis)])
    s = np.arange(10, dtype=np.float32)
    assert len(select_tail_charged(s, 43, 4, 16)) != len(oracle.select_positions(s, 43, 4, 16))

    # 5. pooling off by one position
    def pool_shifted(kidx, c):
        return np.asarray(kidx[1:1 + (kidx.shape[0] - 1) // c * c]).reshape(-1, c, kidx.shape[1]).mean(1)
    kidx = np.repeat(np.arange(12, dtype=np.float64)[:, None], 2, axis=1)
    assert not np.array_equal(pool_shifted(kidx, 4)[:2], oracle.pool_blocks(kidx, 4, "f32")[:2])

    # 6. softmax without the scale
    rng = np.random.default_rng(14)
    q, k, v = rng.standard_normal((2, 8)), rng.standard_normal((6, 1, 8)), rng.standard_normal((6, 1, 3))
    assert not np.allclose(oracle.attend(q, k, v, 1.0), _sdpa(q, k, v, 0.25))

    # 7. the mask bias scaled with the logits, or subtracted
    b = rng.uniform(-1.0, 0.0, size=6)
    want = _sdpa(q, k, v, 0.25, b)
    assert not np.allclose(oracle.attend(q, k, v, 0.25, bias=0.25 * b), want)
    assert not np.allclose(oracle.attend(q, k, v, 0.25, bias=-b), want)

    # 8. q8_0 with 128 levels, with ties to even, or with one scale per row
    x = np.zeros(32, np.float32)
    x[:8] = [127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5]
    def q8_levels128(x):
        d = np.abs(x).max() / np.float32(128.0)
        return np.rint(x / d).astype(int)
    assert q8_levels128(x)[:8].tolist() != [127, 3, -3, 1, -1, 2, -2, 127]
    assert np.rint(x[:8]).astype(int).tolist() != [127, 3, -3, 1, -1, 2, -2, 127]
    r = np.random.default_rng(15).standard_normal(64).astype(np.float32)
    r[40] *= 50.0
    def q8_per_row(x):
        d = np.abs(x).max() / np.float32(127.0)
        return np.sign(x / d) * np.floor(np.abs(x / d) + 0.5)
    assert not np.array_equal(q8_per_row(r)[:32], oracle.quantize_q8_0(r)[0][:32])
