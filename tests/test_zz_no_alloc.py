"""sparse_attn_fwd_noalloc (the attention without a workspace argument, its split
partials in the library's static scratch) against sparse_attn_fwd on the same
inputs, through the C ABI: two calls in a row, the second with a smaller input, so
the second runs on scratch the first left behind."""
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


def _case(name, lens, q_seq, q_pos, top_k, case_id):
    dims = datagen.Dims(h_q=16, h_kv=1, d_kq=576, d_v=512, h_idx=64, d_idx=128, compress_ratio=4, top_k=top_k,
                        dtype="bf16")
    # wide logits (standard deviation 2), so that the outputs depend on Q.K^T
    return datagen.make_case(name, dims, lens, q_seq, q_pos, seed=0, case_id=case_id, std="inv_sqrt_dim",
                             v_separate=False, q_std=2.0 * math.sqrt(576))


def _fwd_both(case):
    """(layer, output of sparse_attn_fwd, output of sparse_attn_fwd_noalloc)."""
    layer = DeviceLayer(case)
    layer.step()                       # pool, score, select, and the attention with a workspace
    torch.cuda.synchronize()
    with_ws = layer.out.clone()
    layer.out.fill_(-3.0)
    sa.sparse_attn_fwd_noalloc(layer.dims, layer.cache, layer.q, layer.q_seq, layer.sel, layer.sel_ld, layer.n_sel,
                               layer.n_q, layer.scale, layer.out)
    torch.cuda.synchronize()
    return layer, with_ws, layer.out.clone()


def test_noalloc_fwd_matches_fwd_on_two_calls(gpu_lib):
    # first call: 8 decode tokens of one long sequence, 33 splits each (8.7 MB of
    # partials); second call: one token with a 256-token budget (5 splits)
    big = _case("noalloc_big", [20000], [0] * 8, [19999 - 1111 * j for j in range(8)], 2048, 950)
    small = _case("noalloc_small", [3000], [0], [2999], 256, 951)
    for case in (big, small):
        need = sa.sparse_attn_workspace_bytes(sa.make_dims(16, 1, 576, 512, 64, 128, 4, case.dims.top_k, "bf16"),
                                              case.n_q, int(case.seq_cap.max())) - sa.WS_STATE_BYTES
        print(f"[no-alloc] {case.name}: n_q={case.n_q}, partials {need} B of {sa.STATIC_SCRATCH_BYTES}", flush=True)
        layer, with_ws, no_alloc = _fwd_both(case)
        assert torch.equal(with_ws.view(torch.int32), no_alloc.view(torch.int32)), \
            f"{case.name}: the no-alloc call differs from sparse_attn_fwd"
        sel = layer.selections()
        for qi in range(case.n_q):
            rows = np.asarray(sel[qi], dtype=np.int64)
            parity.check_attention(no_alloc[qi].cpu().numpy(), case.q[qi], case.k[rows], case.v_rows()[rows],
                                   case.scale, "bf16", f"{case.name} q{qi} no-alloc")
        print(f"[no-alloc] {case.name}: bit for bit equal to sparse_attn_fwd, within the oracle's bound", flush=True)


def test_noalloc_fwd_refuses_oversize(gpu_lib):
    # 16 decode tokens of 16 heads with 1024-wide K and V need more partials than the
    # static scratch holds: refused before any launch, and the output is untouched
    dims = datagen.Dims(h_q=16, h_kv=1, d_kq=1024, d_v=1024, h_idx=64, d_idx=128, compress_ratio=4, top_k=2048,
                        dtype="bf16")
    case = datagen.make_case("noalloc_oversize", dims, [3000], [0] * 16, [2999 - 100 * j for j in range(16)], seed=0,
                             case_id=952, std="inv_sqrt_dim", v_separate=True)
    layer = DeviceLayer(case)
    layer.out.fill_(-3.0)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_fwd_noalloc(layer.dims, layer.cache, layer.q, layer.q_seq, layer.sel, layer.sel_ld,
                                   layer.n_sel, layer.n_q, layer.scale, layer.out)
    assert e.value.code == sa.SA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((layer.out == -3.0).all())
