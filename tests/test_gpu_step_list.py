"""sparse_attn_pool_score_select_fwd -- pool + score, then the selection from the
scoring launch's candidate list inside the attention's launch -- against
sparse_attn_pool_score followed by sparse_attn_select_fwd on the same inputs, through
the C ABI: pooled keys, counts, scores, lists and outputs bit for bit.  The candidate
list the scoring launch leaves in the workspace is checked against the per-group best
blocks of the scores, and the per-token flag saying whether the list decided the
selection against the decision rule applied to those scores here: the list's cut
decides when every block it leaves out scores below that cut."""
import math

import numpy as np
import pytest
import torch

import oracle
import parity
from indexer_top_block_amd import datagen
from indexer_top_block_amd import sparse_attn as sa
from indexer_top_block_amd.device import DeviceLayer

pytestmark = pytest.mark.gpu

GROUP = 32                    # blocks per group of the list
LIST_CAP = 32768              # listed keys one workgroup holds
READERS = 1024                # threads of the workgroup that reads the list


def record_word(g: int, r: int, keep: int, tpt: int) -> int:
    """Where word r of group g's record lies in a token's list: the reading thread t
    holds groups [tpt t, tpt t + tpt), and its 16-byte piece q (group j of its own,
    word r: q = j keep / 2 + r / 4) sits at q * READERS + t."""
    t, q = g // tpt, (g % tpt) * (keep // 2) + r // 4
    return (q * READERS + t) * 4 + r % 4


def poisson_tail(lam: float, k: int) -> float:
    """P(X >= k) for X ~ Poisson(lam)."""
    return float(1.0 - sum(math.exp(-lam) * lam ** j / math.factorial(j) for j in range(k)))


def keep_of(max_blocks: int, k_blk: int) -> int:
    """The best blocks the list keeps per group: the larger of 8 and 4 for which the
    list holds at most 32768 keys and a row of independent scores would fall back to
    its row select less than once in 10 (some group holding more kept blocks than
    that); else none (and none for rows that are always dense)."""
    groups = -(-max_blocks // GROUP)
    if max_blocks <= k_blk:
        return 0
    for keep in (8, 4):
        if groups * keep <= LIST_CAP and groups * poisson_tail(k_blk / groups, keep + 1) < 0.1:
            return keep
    return 0


def say(msg):
    print(msg, flush=True)


def _dims(**kw):
    base = dict(h_q=16, h_kv=1, d_kq=576, d_v=512, h_idx=64, d_idx=128, compress_ratio=4, top_k=2048, dtype="bf16")
    base.update(kw)
    return datagen.Dims(**base)


def _case(name, d, lens, q_seq, q_pos, case_id):
    return datagen.make_case(name, d, lens, q_seq, q_pos, seed=0, case_id=case_id, std="inv_sqrt_dim",
                             v_separate=False, q_std=2.0 * math.sqrt(d.d_kq))


def order_keys(scores: np.ndarray) -> np.ndarray:
    """The selection's order-preserving keys of float32 scores (+0 and -0 alike)."""
    u = (scores.astype(np.float32) + np.float32(0.0)).view(np.uint32)
    return np.where(u >> 31 == 1, ~u, u | np.uint32(0x80000000)).astype(np.uint32)


def expected_lists(keys: np.ndarray, nb: int, keep: int):
    """Per group g with 32 g < nb: its `keep` best blocks by (key descending, index
    ascending), their keys then their indices, listed by index (blocks past nb count
    as key 0)."""
    out = {}
    for g in range((nb + GROUP - 1) // GROUP):
        b = np.arange(g * GROUP, g * GROUP + GROUP)
        k = np.where(b < nb, keys[np.minimum(b, nb - 1)], 0).astype(np.int64)
        best = np.lexsort((b, -k))[:keep]
        take = np.sort(best)
        out[g] = np.concatenate([k[take], b[take]]).astype(np.uint32)
    return out


def radix_bound(listed: np.ndarray, k: int) -> int:
    """The cut of the radix select over 10/11/11-bit digits among the listed keys: the
    bin start when a pass's bin is taken whole, else the k-th largest key itself."""
    active = listed.astype(np.int64)
    prefix, k_rem = 0, k
    for shift, width in ((22, 10), (11, 11), (0, 11)):
        digits = (active >> shift) & ((1 << width) - 1)
        counts = np.bincount(digits, minlength=1 << width)
        above = np.concatenate([np.cumsum(counts[::-1])[::-1][1:], [0]])   # keys in higher digits
        d = int(np.nonzero((above < k_rem) & (above + counts >= k_rem))[0][0])
        prefix = (prefix << width) | d
        k_rem -= int(above[d])
        if counts[d] == k_rem and prefix != 0:
            return prefix << shift
        active = active[digits == d]
    return prefix


def min_groups(k_blk: int, keep: int) -> int:
    """The fewest whole groups a token's row needs for the list to be tried: the
    smallest g >= 2 k_blk / keep with g P(Poisson(k_blk / g) > keep) < 0.1 (the same
    rule as keep_of's, for the token's own row)."""
    cap = LIST_CAP // keep
    g = max(1, -(-2 * k_blk // keep))
    while g <= cap and g * poisson_tail(k_blk / g, keep + 1) >= 0.1:
        g += 1
    return g


def expected_decided(keys: np.ndarray, nb: int, k_blk: int, keep: int, max_over: int) -> int:
    """1 where the list decides the selection: its cut bound above every group's smallest
    listed key; else the groups whose smallest listed key reached the bound (at most
    max_over of them) are read whole and the cut is taken again over them and the other
    groups' listed keys, which decides when the new bound is above the other groups'
    smallest listed keys."""
    if nb <= k_blk or nb // GROUP < min_groups(k_blk, keep):
        return 0
    lists = expected_lists(keys, nb, keep)
    least = {g: int(v[:keep].min()) for g, v in lists.items()}
    listed = np.concatenate([v[:keep] for v in lists.values()])
    listed = listed[listed != 0]
    bound = radix_bound(listed, k_blk)
    if all(x < bound for x in least.values()):
        return 1
    over = {g for g, x in least.items() if x >= bound}
    if len(over) > max_over:
        return 0
    parts = []
    for g, v in lists.items():
        if g in over:
            parts.append(keys[g * GROUP: min(nb, g * GROUP + GROUP)].astype(np.int64))
        else:
            parts.append(v[:keep].astype(np.int64))
    merged = np.concatenate(parts)
    merged = merged[merged != 0]
    bound2 = radix_bound(merged, k_blk)
    return int(all(x < bound2 for g, x in least.items() if g not in over))


def _run(layer, fused_step: bool):
    """Fresh caches and outputs, then either the step call or the two calls; returns
    (kpool, n_out, scores, sel, n_sel, out) on the host."""
    layer.kpool.zero_()
    n_in = torch.zeros_like(layer.n_pooled)
    n_out = torch.full_like(layer.n_pooled, -7)
    layer.scores.fill_(-1.0)
    layer.sel.fill_(-7)
    layer.n_sel.fill_(-7)
    layer.out.fill_(float("nan"))
    if fused_step:
        layer.pool_score_select_fwd(n_in=n_in, n_out=n_out)
    else:
        sa.sparse_attn_pool_score(layer.dims, layer.cache, n_in, n_out, 2 ** 31 - 1, layer.qidx, layer.q_seq,
                                  layer.q_pos, layer.n_q, layer.scores, layer.scores_ld)
        layer.select_fwd()
    torch.cuda.synchronize()
    return tuple(t.clone() for t in (layer.kpool, n_out, layer.scores, layer.sel, layer.n_sel, layer.out))


def _check(case, expect_list, expect_decided=None, oracle_queries=()):
    d = case.dims
    c, k_blk = d.compress_ratio, d.top_k // d.compress_ratio
    say(f"[step_list] {case.name}: n_q={case.n_q} q_pos={list(case.q_pos)[:8]}")
    layer = DeviceLayer(case)
    n_probe = torch.zeros_like(layer.n_pooled) + 1
    assert layer.pool_score_select_fwd_uses_list(n_in=layer.n_pooled, n_out=n_probe) == expect_list, case.name
    two = _run(layer, fused_step=False)
    one = _run(layer, fused_step=True)
    names = ("kpool", "n_pooled_out", "scores", "sel", "n_sel", "out")
    for name, a, b in zip(names, two, one):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{case.name}: {name} differs"
    if expect_list:
        ws = layer.ws.cpu().numpy()
        keep = keep_of(layer.max_len // c, k_blk)
        tpt = 1 if layer.max_len // c <= LIST_CAP else 32 // keep      # groups per reading thread
        words = READERS * tpt * 2 * keep
        end = layer.ws_bytes
        flags = ws[end - 4 * case.n_q: end].view(np.int32)
        lists = ws[end - 4 * case.n_q * (words + 1): end - 4 * case.n_q].view(np.uint32).reshape(case.n_q, words)
        scores = one[2].cpu().numpy()
        got_decided = []
        for i in range(case.n_q):
            n_vis = oracle.visible_tokens(int(case.seq_len[case.q_seq[i]]), int(case.q_pos[i]))
            nb = n_vis // c
            keys = order_keys(scores[i, :nb])
            want = expected_decided(keys, nb, k_blk, keep, max_over=32 if tpt == 1 else 64)
            if nb > k_blk and nb // GROUP >= min_groups(k_blk, keep):
                for g, v in expected_lists(keys, nb, keep).items():
                    rec = lists[i, [record_word(g, r, keep, tpt) for r in range(2 * keep)]]
                    assert np.array_equal(rec, v), f"{case.name} q{i} group {g}"
            assert int(flags[i]) == want, f"{case.name} q{i}: decided {flags[i]}, expected {want}"
            got_decided.append(int(flags[i]))
        if expect_decided is not None:
            assert got_decided == list(expect_decided), f"{case.name}: decided {got_decided}"
        say(f"[step_list] {case.name}: decided by the list {got_decided}")
    if oracle_queries:
        pools = oracle.SequencePools(case)
        sel = layer.selections()
        out = layer.out.cpu().numpy()
        for qi in oracle_queries:
            res = oracle.run_query(case, qi, pools)
            parity.compare_selection(sel[qi], res, case)
            rows = int(case.row0[case.q_seq[qi]]) + np.asarray(sel[qi], dtype=np.int64)
            parity.check_attention(out[qi], case.q[qi], case.k[rows], case.v_rows()[rows], case.scale, d.dtype,
                                   f"{case.name} q{qi}")
    say(f"[step_list] {case.name}: list={expect_list}, bit for bit equal to the two calls")


def test_step_list_decode_128k(gpu_lib):
    # the 128K decode workload: 32768 blocks, 1024 groups, 8192 listed blocks for a cut of 512
    case = datagen.make_workload(2, q_std=2.0 * math.sqrt(576))
    _check(case, expect_list=True, expect_decided=[1], oracle_queries=[0])


def test_step_list_mixed_tokens(gpu_lib):
    # six tokens of one 40000-token sequence (10000 blocks: a last group of 16 blocks):
    # long rows the list decides (one with a 2-position tail), a row of too few groups
    # for the list to be tried (2000 blocks: its row select), the dense case at the
    # threshold, one visible position and none
    d = _dims()
    assert min_groups(512, 8) == 237
    q_pos = [39999, 35001, 8000, 2050, 0, -1]
    case = _case("step_list_mixed", d, [40000], [0] * len(q_pos), q_pos, 980)
    _check(case, expect_list=True, expect_decided=[1, 1, 0, 0, 0, 0], oracle_queries=[0, 1, 2, 3])


def test_step_list_shapes(gpu_lib):
    # 512/512 f16 with a 1024-token budget over two sequences; two KV heads of 8 query
    # heads each; c = 1 over rows of fewer than 32768 blocks
    d = _dims(d_kq=512, dtype="f16", top_k=1024)
    _check(_case("step_list_512_f16", d, [30000, 20000], [0, 1], [29999, 17001], 981), expect_list=True,
           oracle_queries=[0, 1])
    d = _dims(d_kq=512, h_kv=2, top_k=256)
    _check(_case("step_list_two_kv_heads", d, [24001], [0, 0], [24000, 15000], 982), expect_list=True,
           oracle_queries=[1])
    d = _dims(compress_ratio=1, top_k=512)
    _check(_case("step_list_token_level", d, [30000], [0], [29999], 983), expect_list=True, expect_decided=[1],
           oracle_queries=[0])


def test_step_list_completes_crowded_groups(gpu_lib):
    # groups of 32 blocks scaled up eight times (exact in bf16): all 32 are among the
    # best, so each such group's 8th best is above the list's cut; those groups are read
    # whole from the row and the cut taken again (one group; the last three groups, the
    # most recent positions); then 600 copies of one block scaled up four times, at most
    # 3 per group: the cut falls inside their common score (ties go to the lower blocks)
    # and the list decides it
    d = _dims()
    case = _case("step_list_crowded_group", d, [131072], [0], [131071], 984)
    tok = slice(int(case.row0[0]) + 64 * 4, int(case.row0[0]) + 96 * 4)
    case.kidx[tok] = case.kidx[tok] * np.float32(8.0)
    _check(case, expect_list=True, expect_decided=[1], oracle_queries=[0])
    case = _case("step_list_recent_groups", d, [131072], [0], [131071], 989)
    tok = slice(int(case.row0[0]) + (32768 - 96) * 4, int(case.row0[0]) + 32768 * 4)
    case.kidx[tok] = case.kidx[tok] * np.float32(8.0)
    _check(case, expect_list=True, expect_decided=[1], oracle_queries=[0])

    case = _case("step_list_tied_copies", d, [131072], [0], [131071], 985)
    rng = np.random.default_rng([985, 1])
    groups = rng.choice(1024, size=200, replace=False)
    blocks = np.sort((groups[:, None] * GROUP + rng.choice(GROUP, size=(200, 3), replace=True)).reshape(-1))
    blocks = np.unique(blocks)
    src = int(case.row0[0]) + 7 * 4
    base = case.kidx[src: src + 4] * np.float32(4.0)
    for b in blocks:
        r = int(case.row0[0]) + int(b) * 4
        case.kidx[r: r + 4] = base
    _check(case, expect_list=True, expect_decided=[1], oracle_queries=[0])


def test_step_list_long_rows(gpu_lib):
    # rows longer than one workgroup's registers (list_fwd_kernel): token level over
    # 40 000 positions (1250 groups, 8 listed each: 10 000 keys) with whole, ragged and
    # dense-at-the-threshold rows; and a crowded group in a 40 000-position row, read
    # whole from the row (4 listed per group: the 1M decode below)
    d = _dims(compress_ratio=1)
    assert keep_of(40000, 2048) == 8 and keep_of(262144, 512) == 4
    q_pos = [39999, 31234, 2047]              # 1250 groups; 976 (fewer than the 1178 the list needs); dense
    _check(_case("step_list_token_level_long", d, [40000], [0] * 3, q_pos, 990), expect_list=True,
           expect_decided=[1, 0, 0], oracle_queries=[0, 1, 2])
    case = _case("step_list_long_crowded", d, [40000], [0], [39999], 992)
    tok = slice(int(case.row0[0]) + 64, int(case.row0[0]) + 96)
    case.kidx[tok] = case.kidx[tok] * np.float32(8.0)
    _check(case, expect_list=True, expect_decided=[1], oracle_queries=[0])
    # ties at the cut inside crowded groups: 60 whole groups of copies of one key (scaled
    # up eight times) and up to 600 more copies, at most 3 per group, in lower groups:
    # some 2500 copies for the 2048 kept, the lower ones first; the 60 groups are read
    # whole and their kept and tied blocks placed by the threads that read them
    case = _case("step_list_long_tied_crowded", d, [40000], [0], [39999], 998)
    rng = np.random.default_rng([998, 1])
    r0 = int(case.row0[0])
    groups = rng.choice(600, size=200, replace=False)
    sparse = np.unique((groups[:, None] * GROUP + rng.choice(GROUP, size=(200, 3), replace=True)).reshape(-1))
    blocks = np.concatenate([sparse, np.arange(700 * GROUP, 760 * GROUP)])
    case.kidx[r0 + blocks] = case.kidx[r0 + 7] * np.float32(8.0)
    _check(case, expect_list=True, expect_decided=[1], oracle_queries=[0])
    # 70 crowded groups (2240 blocks scaled up, more than the 2048 kept): more than the
    # 64 the launch reads whole, so the streamed per-query select over the row runs
    case = _case("step_list_long_very_crowded", d, [40000], [0], [39999], 997)
    tok = slice(int(case.row0[0]) + 3200, int(case.row0[0]) + 3200 + 70 * 32)
    case.kidx[tok] = case.kidx[tok] * np.float32(8.0)
    _check(case, expect_list=True, expect_decided=[0], oracle_queries=[0])


def test_step_list_other_block_sizes(gpu_lib):
    # blocks of 8 and of 2 tokens (the list's positions written c at a time, not as
    # four-wide stores): c = 8 over 120 000 positions (15 000 blocks, with a 7-position
    # tail on the second token); c = 2 over 60 000 (one workgroup's registers) and over
    # 100 000 positions (50 000 blocks: list_fwd_kernel)
    d = _dims(compress_ratio=8, top_k=1024)
    _check(_case("step_list_c8", d, [120000], [0, 0], [119999, 90006], 994), expect_list=True,
           expect_decided=[1, 1], oracle_queries=[0, 1])
    d = _dims(compress_ratio=2)
    _check(_case("step_list_c2_wide", d, [60000], [0], [59999], 995), expect_list=True, expect_decided=[1],
           oracle_queries=[0])
    _check(_case("step_list_c2_long", d, [100000], [0, 0], [99999, 70000], 996), expect_list=True,
           expect_decided=[1, 1], oracle_queries=[0, 1])


def test_step_list_decode_1m(gpu_lib):
    # the 1M-context decode workload (262 144 blocks, 1% planted): 8192 groups, 4 listed each
    case = datagen.make_workload(5, q_std=2.0 * math.sqrt(576))
    _check(case, expect_list=True, expect_decided=[1], oracle_queries=[0])
    # the same row with its three most recent groups (384 positions) scaled up eight
    # times: 96 kept blocks in groups that list 4 each, read whole from the row
    case = datagen.make_workload(5, q_std=2.0 * math.sqrt(576))
    end = int(case.row0[0]) + int(case.seq_len[0]) // (4 * GROUP) * (4 * GROUP)
    case.kidx[end - 3 * 4 * GROUP: end] = case.kidx[end - 3 * 4 * GROUP: end] * np.float32(8.0)
    _check(case, expect_list=True, expect_decided=[1], oracle_queries=[0])


def test_step_list_not_used(gpu_lib):
    # token level over 140 000 positions (4375 groups: 8 listed each would exceed 32768
    # keys, and with 4 a row of independent scores would fall back about every other
    # time), a row of 5000 blocks for a cut of 512 (too few groups for the list), eight
    # tokens of 33 splits (more workgroups than compute units), and the batched decode
    # workload (a separate V: no fused form; 16 384 tiles in all): the two calls
    d = _dims(compress_ratio=1)
    assert keep_of(140032, 2048) == 0 and keep_of(5000, 512) == 0
    _check(_case("step_list_chunked_row", d, [140000], [0], [139999], 986), expect_list=False)
    d = _dims()
    q_pos = [19999 - 997 * j for j in range(8)]
    _check(_case("step_list_eight_tokens", d, [20000], [0] * 8, q_pos, 987), expect_list=False,
           oracle_queries=[0, 7])
    _check(datagen.make_workload(3), expect_list=False, oracle_queries=[0, 31])
