"""sparse_attn_select_fwd -- the selection inside the attention's launch -- against
sparse_attn_select followed by sparse_attn_fwd on the same inputs, through the C ABI:
lists, counts and outputs bit for bit, and the fused call's lists and outputs against
the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import parity
from indexer_top_block_amd import datagen
from indexer_top_block_amd.device import DeviceLayer

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _dims(**kw):
    base = dict(h_q=16, h_kv=1, d_kq=576, d_v=512, h_idx=64, d_idx=128, compress_ratio=4, top_k=2048, dtype="bf16")
    base.update(kw)
    return datagen.Dims(**base)


def _case(name, d, lens, q_seq, q_pos, case_id):
    # wide logits (standard deviation 2), so that the outputs depend on Q.K^T
    return datagen.make_case(name, d, lens, q_seq, q_pos, seed=0, case_id=case_id, std="inv_sqrt_dim",
                             v_separate=False, q_std=2.0 * math.sqrt(d.d_kq))


def _both(case):
    """(layer, two-call results, fused results): each a (sel, n_sel, out) on the host."""
    layer = DeviceLayer(case)
    layer.pool()
    layer.score()
    layer.select()
    layer.fwd()
    torch.cuda.synchronize()
    two = (layer.sel.clone(), layer.n_sel.clone(), layer.out.clone())
    layer.sel.fill_(-7)
    layer.n_sel.fill_(-7)
    layer.out.fill_(float("nan"))
    layer.select_fwd()
    torch.cuda.synchronize()
    fused = (layer.sel.clone(), layer.n_sel.clone(), layer.out.clone())
    return layer, two, fused


def _check(case, expect_fused, oracle_queries=None):
    say(f"[select_fwd] {case.name}: n_q={case.n_q} dims={case.dims}")
    layer, two, fused = _both(case)
    assert layer.select_fwd_is_fused() == expect_fused, case.name
    assert torch.equal(two[0], fused[0]), f"{case.name}: lists differ"
    assert torch.equal(two[1], fused[1]), f"{case.name}: counts differ"
    assert torch.equal(two[2].view(torch.int32), fused[2].view(torch.int32)), f"{case.name}: outputs differ"
    # the fused call's own results against the oracle
    queries = range(case.n_q) if oracle_queries is None else oracle_queries
    pools = oracle.SequencePools(case) if len(queries) else None
    sel = layer.selections()
    out = layer.out.cpu().numpy()
    for qi in queries:
        res = oracle.run_query(case, qi, pools)
        parity.compare_selection(sel[qi], res, case)
        rows = int(case.row0[case.q_seq[qi]]) + np.asarray(sel[qi], dtype=np.int64)
        parity.check_attention(out[qi], case.q[qi], case.k[rows], case.v_rows()[rows], case.scale,
                               case.dims.dtype, f"{case.name} q{qi} fused")
    say(f"[select_fwd] {case.name}: fused={expect_fused}, bit for bit equal to the two calls, "
        f"oracle bound-ratio={parity.take_worst_ratio():.3g}")


def test_select_fwd_decode_128k(gpu_lib):
    # the 128K decode workload: one token, 33 splits, the select of 32768 blocks in every workgroup
    case = datagen.make_workload(2, q_std=2.0 * math.sqrt(576))
    _check(case, expect_fused=True)


def test_select_fwd_mixed_tokens(gpu_lib):
    # five tokens of one sequence: whole blocks only, a 3-row tail, the dense case at
    # the threshold (n_vis = top_k + c - 1), one visible position, none visible
    d = _dims()
    q_pos = [19999, 10002, 2050, 0, -1]
    _check(_case("select_fwd_mixed", d, [20000], [0] * len(q_pos), q_pos, 960), expect_fused=True)


def test_select_fwd_shapes(gpu_lib):
    # 512/512 f16 with a 1024-token budget; two KV heads of 8 query heads each (the
    # workgroups of KV head 1 select too, and only head 0's write the list)
    d = _dims(d_kq=512, dtype="f16", top_k=1024)
    _check(_case("select_fwd_512_f16", d, [9000, 5000], [0, 1], [8999, 4001], 961), expect_fused=True)
    d = _dims(d_kq=512, h_kv=2, top_k=256)
    _check(_case("select_fwd_two_kv_heads", d, [3001], [0, 0], [3000, 1500], 962), expect_fused=True)


def _check_rows(case, kinds, expect_fused, case_id):
    """The fused call against the two calls on score rows of the given kinds (one per
    query token), uploaded in place of the indexer's scores; its lists against the
    oracle's selection of those rows and its outputs against the oracle's attention
    over the rows it selected."""
    say(f"[select_fwd] {case.name}: score rows {kinds}")
    d = case.dims
    layer = DeviceLayer(case)
    layer.pool()
    rows = []
    for i, kind in enumerate(kinds):
        n_vis = oracle.visible_tokens(int(case.seq_len[case.q_seq[i]]), int(case.q_pos[i]))
        rows.append(datagen.score_row(kind, n_vis // d.compress_ratio, d.top_k // d.compress_ratio, seed=0,
                                      case_id=case_id + i))
    scores = parity.upload_scores(layer, rows)
    layer.select(scores=scores)
    layer.fwd()
    torch.cuda.synchronize()
    two = (layer.sel.clone(), layer.n_sel.clone(), layer.out.clone())
    layer.sel.fill_(-7)
    layer.n_sel.fill_(-7)
    layer.out.fill_(float("nan"))
    layer.select_fwd(scores=scores)
    torch.cuda.synchronize()
    assert layer.select_fwd_is_fused() == expect_fused, case.name
    assert torch.equal(two[0], layer.sel) and torch.equal(two[1], layer.n_sel), f"{case.name}: lists differ"
    assert torch.equal(two[2].view(torch.int32), layer.out.view(torch.int32)), f"{case.name}: outputs differ"
    sel = layer.selections()
    out = layer.out.cpu().numpy()
    for i, kind in enumerate(kinds):
        n_vis = oracle.visible_tokens(int(case.seq_len[case.q_seq[i]]), int(case.q_pos[i]))
        want = oracle.select_positions(rows[i], n_vis, d.compress_ratio, d.top_k)
        assert np.array_equal(sel[i], want), f"{case.name} row {i} ({kind}): selection differs"
        r = int(case.row0[case.q_seq[i]]) + np.asarray(sel[i], dtype=np.int64)
        parity.check_attention(out[i], case.q[i], case.k[r], case.v_rows()[r], case.scale, d.dtype,
                               f"{case.name} q{i} {kind}")
    say(f"[select_fwd] {case.name}: fused={expect_fused}, bit for bit equal to the two calls, "
        f"oracle bound-ratio={parity.take_worst_ratio():.3g}")


def test_select_fwd_chunked_rows(gpu_lib):
    # rows longer than one workgroup holds: the chunked selection's histogram and
    # candidate launches, then its finishing pass inside every attention workgroup.
    # 35000 blocks of 4 tokens (18 chunks); token level (c = 1) over 40000 positions
    # with whole rows, a ragged row, the dense case at the threshold, one visible
    # position and none; two KV heads of 512/512 f16
    d = _dims()
    _check(_case("select_fwd_chunked_long_row", d, [140000], [0], [139999], 965), expect_fused=True)
    d = _dims(compress_ratio=1)
    q_pos = [39999, 31234, 2047, 0, -1]
    _check(_case("select_fwd_chunked_token_level", d, [40000], [0] * len(q_pos), q_pos, 966), expect_fused=True)
    d = _dims(d_kq=512, h_kv=2, compress_ratio=1, top_k=1024, dtype="f16")
    _check(_case("select_fwd_chunked_two_kv_heads", d, [36000], [0, 0], [35999, 20000], 967), expect_fused=True)


def test_select_fwd_chunked_adversarial_rows(gpu_lib):
    # score rows that the finishing pass must cut exactly: ties across the cut, a cut
    # inside a run of equal integers, and rows whose candidates overflow its LDS
    # (every score equal; a few hundred positive among signed zeros), which take the
    # per-query select inside the workgroup instead
    d = _dims(compress_ratio=1)
    kinds = ("lognormal_dups", "small_ints", "all_equal", "signed_zeros", "normal")
    q_pos = [39999, 39000, 38000, 37000, 36000]
    case = _case("select_fwd_chunked_rows", d, [40000], [0] * len(kinds), q_pos, 968)
    _check_rows(case, kinds, expect_fused=True, case_id=969)


def test_select_fwd_takes_two_calls_when_it_does_not_fit(gpu_lib):
    # eight tokens of 33 splits want more workgroups than compute units; a token-level
    # row of 600001 positions has more chunks (293) than the finishing pass reads at once
    d = _dims()
    q_pos = [19999 - 997 * j for j in range(8)]
    _check(_case("select_fwd_eight_tokens", d, [20000], [0] * 8, q_pos, 963), expect_fused=False,
           oracle_queries=[0, 7])
    d = _dims(compress_ratio=1)
    _check(_case("select_fwd_many_chunks", d, [600001], [0], [600000], 964), expect_fused=False,
           oracle_queries=[])
