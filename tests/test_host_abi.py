"""The C ABI on the host (CPU only): the library loads, exports every function the
header declares, and rejects bad arguments before making any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

from indexer_top_block_amd import sparse_attn as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

# Any non-zero value: validation never dereferences device pointers on the host.
FAKE = 0x10000
FAKE2 = 0x20000               # a second distinct non-null address


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = sa.load()
    declared = _declared_functions()
    assert set(declared) == set(sa.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", sa.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT (sparse_attn_\w+)$", nm.stdout, flags=re.M))
    assert set(declared) <= exported


def test_version_and_strerror():
    assert "gfx950" in sa.sparse_attn_version()
    for code in (0, -1, -2, -3, -4, -5, -6, 7):
        assert isinstance(sa.sparse_attn_strerror(code), str) and sa.sparse_attn_strerror(code)


def _dims(**kw):
    base = dict(h_q=16, h_kv=1, d_kq=576, d_v=512, h_idx=64, d_idx=128, compress_ratio=4, top_k=2048, dtype="bf16")
    base.update(kw)
    return sa.make_dims(**base)


@pytest.mark.parametrize("kw", [
    dict(), dict(dtype="f32", h_q=8, d_kq=128, d_v=128, h_idx=4, d_idx=64, top_k=256),
    dict(dtype="f16", h_q=8, d_kq=512, h_idx=32), dict(compress_ratio=1, top_k=1),
    dict(h_q=32, h_kv=2), dict(compress_ratio=64, top_k=64 * 1024 - 64),
])
def test_check_dims_accepts(kw):
    assert sa.sparse_attn_check_dims(_dims(**kw)) == sa.SA_OK


@pytest.mark.parametrize("kw", [
    dict(top_k=2050), dict(compress_ratio=0), dict(compress_ratio=-4), dict(top_k=0), dict(h_q=17),
    dict(h_q=32, h_kv=1), dict(h_kv=0), dict(d_idx=100), dict(d_idx=0), dict(dtype=7), dict(h_idx=0),
    dict(h_idx=129), dict(d_kq=1025), dict(d_v=0), dict(compress_ratio=65, top_k=65),
    dict(compress_ratio=1, top_k=65537),
])
def test_check_dims_rejects(kw):
    assert sa.sparse_attn_check_dims(_dims(**kw)) == sa.SA_ERR_DIMS


def test_check_dims_null():
    lib = sa.load()
    assert lib.sparse_attn_check_dims(None) == sa.SA_ERR_NULL


def test_workspace_bytes():
    d = _dims()
    hdr = open(HEADER).read()
    assert f"#define SA_WS_STATE_BYTES ((size_t){sa.WS_STATE_BYTES})" in hdr
    partials_1 = 33 * 16 * (512 + 2) * 4            # one decode token: 33 splits of (o, m, l) for 16 heads
    # the candidate list of the pool + score + select call, after the partials on a
    # 256-byte boundary: room for 1024 records of 16 words (rows of up to 32768 blocks) or
    # 8192 of 8 (4 listed per group, longer rows) per token, then one flag per token
    def after(n):
        return (n + 255) // 256 * 256

    # short rows: state region + split-KV partials (no list: rows of at most k_blk = 512
    # blocks are always dense, and 32 groups of 1024 blocks are too few for a cut of 512)
    assert sa.sparse_attn_workspace_bytes(d, 1, 2048) == sa.WS_STATE_BYTES + partials_1
    assert sa.sparse_attn_workspace_bytes(d, 1, 4096) == sa.WS_STATE_BYTES + partials_1
    # 40 000 tokens (10 000 blocks: 8 listed per group, room for 1024 groups of 16 words)
    assert sa.sparse_attn_workspace_bytes(d, 1, 40000) == after(sa.WS_STATE_BYTES + partials_1) + (1024 * 16 + 1) * 4
    # a prefill chunk: unsplit attention and one selection workgroup per query token
    # (no list for 64 tokens or more)
    assert sa.sparse_attn_workspace_bytes(d, 2048, 34816) == 0
    # 128K rows: one workgroup holds a row of 32768 blocks, so selection adds nothing
    # but the list: 1024 groups
    assert sa.sparse_attn_workspace_bytes(d, 1, 131072) == after(sa.WS_STATE_BYTES + partials_1) + (1024 * 16 + 1) * 4
    # 1M rows: the chunked selection's 128 chunks of 2048 8-byte entries (after a
    # 768-byte head of counts), the partials, then the list (8192 groups of 4 listed, 8 words each)
    assert sa.sparse_attn_workspace_bytes(d, 1, 1048576) == (after(sa.WS_STATE_BYTES + 768 + 128 * 2048 * 8 + partials_1)
                                                             + (8192 * 8 + 1) * 4)
    assert sa.sparse_attn_workspace_bytes(_dims(top_k=2050), 1, 4096) == 0
    assert sa.sparse_attn_workspace_bytes(d, 1, -1) == 0


def _cache(**kw):
    base = dict(n_seq=1, max_len=4096, seq_row0=FAKE, seq_blk0=FAKE, seq_len=FAKE, k=FAKE, k_ld=576,
                k_head_stride=576, v=FAKE, v_ld=576, v_head_stride=576, kidx=FAKE, kidx_ld=128, kpool=FAKE,
                kpool_ld=128)
    base.update(kw)
    return sa.SaCache(**base)


def _call(name, *args):
    lib = sa.load()
    return getattr(lib, name)(*args)


def test_entry_points_reject_bad_arguments_before_any_launch():
    d = ctypes.byref(_dims())
    c = ctypes.byref(_cache())
    # pool
    assert _call("sparse_attn_pool", d, None, FAKE, FAKE, 1, None) == sa.SA_ERR_NULL
    assert _call("sparse_attn_pool", d, c, None, FAKE, 1, None) == sa.SA_ERR_NULL
    assert _call("sparse_attn_pool", d, c, FAKE, FAKE, -1, None) == sa.SA_ERR_ARG
    assert _call("sparse_attn_pool", d, ctypes.byref(_cache(kidx_ld=64)), FAKE, FAKE, 1, None) == sa.SA_ERR_ARG
    assert _call("sparse_attn_pool", d, ctypes.byref(_cache(n_seq=0)), FAKE, FAKE, 1, None) == sa.SA_ERR_ARG
    assert _call("sparse_attn_pool", ctypes.byref(_dims(top_k=3)), c, FAKE, FAKE, 1, None) == sa.SA_ERR_DIMS
    # score
    assert _call("sparse_attn_score", d, c, None, FAKE, FAKE, 1, FAKE, 1024, None) == sa.SA_ERR_NULL
    assert _call("sparse_attn_score", d, c, FAKE, FAKE, FAKE, -1, FAKE, 1024, None) == sa.SA_ERR_ARG
    assert _call("sparse_attn_score", d, c, FAKE, FAKE, FAKE, 1, FAKE, 1023, None) == sa.SA_ERR_ARG
    assert _call("sparse_attn_score", d, c, FAKE, FAKE, FAKE, 0, FAKE, 1024, None) == sa.SA_OK  # no-op
    # select
    assert _call("sparse_attn_select", d, c, FAKE, 1024, FAKE, FAKE, 1, FAKE, 2050, FAKE, None, 0, None) == sa.SA_ERR_ARG
    assert _call("sparse_attn_select", d, c, FAKE, 1023, FAKE, FAKE, 1, FAKE, 2051, FAKE, None, 0, None) == sa.SA_ERR_ARG
    assert _call("sparse_attn_select", d, c, FAKE, 1024, FAKE, FAKE, 1, FAKE, 2051, None, None, 0, None) == sa.SA_ERR_NULL
    assert _call("sparse_attn_select", d, ctypes.byref(_cache(seq_len=None)), FAKE, 1024, FAKE, FAKE, 1, FAKE,
                 2051, FAKE, None, 0, None) == sa.SA_ERR_NULL
    # a 1M row needs the chunked selection's workspace
    long_c = ctypes.byref(_cache(max_len=1048576))
    need = sa.sparse_attn_workspace_bytes(_dims(), 1, 1048576)
    assert _call("sparse_attn_select", d, long_c, FAKE, 262144, FAKE, FAKE, 1, FAKE, 2051, FAKE, None, 0,
                 None) == sa.SA_ERR_WORKSPACE
    assert need > 1000
    assert _call("sparse_attn_select", d, long_c, FAKE, 262144, FAKE, FAKE, 1, FAKE, 2051, FAKE, FAKE, 1000,
                 None) == sa.SA_ERR_WORKSPACE
    assert _call("sparse_attn_select", d, long_c, FAKE, 262144, FAKE, FAKE, 1, FAKE, 2051, FAKE, FAKE, need - 1,
                 None) == sa.SA_ERR_WORKSPACE
    # fwd
    ws = sa.sparse_attn_workspace_bytes(_dims(), 1, 4096)
    args = [d, c, FAKE, FAKE, FAKE, 2051, FAKE, 1, ctypes.c_float(0.04), FAKE]
    assert _call("sparse_attn_fwd", *args, None, 0, None) == sa.SA_ERR_WORKSPACE
    assert ws == sa.WS_STATE_BYTES + 33 * 16 * (512 + 2) * 4      # state + partials (no list at 4096 tokens)
    assert _call("sparse_attn_fwd", *args, FAKE, ws - 1, None) == sa.SA_ERR_WORKSPACE
    assert _call("sparse_attn_fwd", d, c, None, FAKE, FAKE, 2051, FAKE, 1, ctypes.c_float(0.04), FAKE, FAKE, ws,
                 None) == sa.SA_ERR_NULL
    assert _call("sparse_attn_fwd", d, c, FAKE, FAKE, FAKE, 2051, FAKE, 1, ctypes.c_float(float("nan")), FAKE, FAKE,
                 ws, None) == sa.SA_ERR_ARG
    # V aliasing K may not be wider than K
    bad = ctypes.byref(_dims(d_kq=512, d_v=576))
    assert _call("sparse_attn_fwd", bad, ctypes.byref(_cache(k_ld=512, v_ld=512)), FAKE, FAKE, FAKE, 2051, FAKE, 1,
                 ctypes.c_float(0.04), FAKE, FAKE, 1 << 30, None) == sa.SA_ERR_ARG
    assert _call("sparse_attn_fwd", d, c, FAKE, FAKE, FAKE, 2051, FAKE, 0, ctypes.c_float(0.04), FAKE, None, 0,
                 None) == sa.SA_OK  # no queries: nothing to do


def test_mask_form_entry_points_reject_bad_arguments():
    F16 = sa.SA_F16
    # bad dtype, negative sizes, too-short rows or lists
    assert _call("sparse_attn_mask_to_indices", FAKE, 7, 4096, 1, 4096, FAKE, 512, FAKE, None, None) == sa.SA_ERR_ARG
    assert _call("sparse_attn_mask_to_indices", FAKE, F16, 4096, -1, 4096, FAKE, 512, FAKE, None, None) == sa.SA_ERR_ARG
    assert _call("sparse_attn_mask_to_indices", FAKE, F16, 4095, 1, 4096, FAKE, 512, FAKE, None, None) == sa.SA_ERR_ARG
    assert _call("sparse_attn_mask_to_indices", FAKE, F16, 4096, 1, 4096, FAKE, 0, FAKE, None, None) == sa.SA_ERR_ARG
    # required pointers
    assert _call("sparse_attn_mask_to_indices", None, F16, 4096, 1, 4096, FAKE, 512, FAKE, None, None) == sa.SA_ERR_NULL
    assert _call("sparse_attn_mask_to_indices", FAKE, F16, 4096, 1, 4096, None, 512, FAKE, None, None) == sa.SA_ERR_NULL
    assert _call("sparse_attn_mask_to_indices", FAKE, F16, 4096, 1, 4096, FAKE, 512, None, None, None) == sa.SA_ERR_NULL
    # nothing to do
    assert _call("sparse_attn_mask_to_indices", None, F16, 4096, 0, 4096, None, 512, None, None, None) == sa.SA_OK
    # the biased attention validates like the plain one
    d = ctypes.byref(_dims())
    c = ctypes.byref(_cache())
    ws = sa.sparse_attn_workspace_bytes(_dims(), 1, 4096)
    assert _call("sparse_attn_fwd_bias", d, c, FAKE, FAKE, FAKE, 2051, FAKE, FAKE, 1, ctypes.c_float(0.04), FAKE, None,
                 0, None) == sa.SA_ERR_WORKSPACE
    assert _call("sparse_attn_fwd_bias", d, c, None, FAKE, FAKE, 2051, FAKE, FAKE, 1, ctypes.c_float(0.04), FAKE,
                 FAKE, ws, None) == sa.SA_ERR_NULL
    assert _call("sparse_attn_fwd_bias", d, c, FAKE, FAKE, FAKE, 2051, FAKE, None, 0, ctypes.c_float(0.04), FAKE,
                 None, 0, None) == sa.SA_OK


def test_window_entry_point_rejects_bad_arguments():
    d = ctypes.byref(_dims())
    c = ctypes.byref(_cache())
    ws = sa.sparse_attn_workspace_bytes(_dims(), 1, 4096)
    f = ctypes.c_float(0.04)
    # negative or oversized window
    assert _call("sparse_attn_fwd_window", d, c, FAKE, FAKE, FAKE, FAKE, 2051, FAKE, -1, 1, f, FAKE, FAKE, ws,
                 None) == sa.SA_ERR_ARG
    assert _call("sparse_attn_fwd_window", d, c, FAKE, FAKE, FAKE, FAKE, 2051, FAKE, (1 << 24) + 1, 1, f, FAKE, FAKE,
                 ws, None) == sa.SA_ERR_ARG
    # q_pos is required only with a window
    assert _call("sparse_attn_fwd_window", d, c, FAKE, FAKE, None, FAKE, 2051, FAKE, 128, 1, f, FAKE, FAKE, ws,
                 None) == sa.SA_ERR_NULL
    # same workspace as the plain attention, whatever the window
    assert _call("sparse_attn_fwd_window", d, c, FAKE, FAKE, FAKE, FAKE, 2051, FAKE, 4096, 1, f, FAKE, None, 0,
                 None) == sa.SA_ERR_WORKSPACE
    assert _call("sparse_attn_fwd_window", d, c, FAKE, FAKE, None, FAKE, 2051, FAKE, 0, 0, f, FAKE, None, 0,
                 None) == sa.SA_OK


def test_window_workspace_size():
    d = _dims()
    base = sa.sparse_attn_workspace_bytes(d, 1, 4096)
    assert sa.sparse_attn_workspace_bytes_window(d, 1, 4096, 0) == base
    assert sa.sparse_attn_workspace_bytes_window(d, 1, 4096, 128) >= base
    assert sa.sparse_attn_workspace_bytes_window(d, 1, 4096, 100000) > base
    assert sa.sparse_attn_workspace_bytes_window(d, 1, 4096, -1) == 0
    assert sa.sparse_attn_workspace_bytes_window(d, -1, 4096, 8) == 0


def test_q8_entry_points_reject_bad_arguments():
    F16 = sa.SA_F16
    q = "sparse_attn_quantize_q8_0"
    assert _call(q, FAKE, 9, 4, 64, 64, FAKE, 64, FAKE, 2, None) == sa.SA_ERR_ARG        # dtype
    assert _call(q, FAKE, F16, 4, 48, 48, FAKE, 48, FAKE, 2, None) == sa.SA_ERR_ARG      # n_cols % 32
    assert _call(q, FAKE, F16, -1, 64, 64, FAKE, 64, FAKE, 2, None) == sa.SA_ERR_ARG
    assert _call(q, FAKE, F16, 4, 64, 63, FAKE, 64, FAKE, 2, None) == sa.SA_ERR_ARG      # x_ld
    assert _call(q, FAKE, F16, 4, 64, 64, FAKE, 62, FAKE, 2, None) == sa.SA_ERR_ARG      # codes_ld
    assert _call(q, FAKE, F16, 4, 64, 64, FAKE, 64, FAKE, 1, None) == sa.SA_ERR_ARG      # scales_ld
    assert _call(q, FAKE, F16, 4, 64, 64, FAKE + 2, 64, FAKE, 2, None) == sa.SA_ERR_ARG  # codes alignment
    assert _call(q, FAKE, F16, 4, 64, 64, FAKE, 66, FAKE, 2, None) == sa.SA_ERR_ARG      # codes_ld alignment
    assert _call(q, None, F16, 4, 64, 64, FAKE, 64, FAKE, 2, None) == sa.SA_ERR_NULL
    assert _call(q, None, F16, 0, 64, 64, None, 64, None, 2, None) == sa.SA_OK
    d = _dims()
    kv = sa.SaKvQ8(FAKE, 576, 576, FAKE, 18, 18, FAKE, 576, 576, FAKE, 18, 18)
    f = ctypes.c_float(0.04)
    ws = sa.sparse_attn_workspace_bytes(d, 1, 4096)
    fq = "sparse_attn_fwd_q8_0"
    c = ctypes.byref(_cache())
    args = lambda kv_, dd=d, ws_=FAKE, wsb=ws: (ctypes.byref(dd), c, ctypes.byref(kv_) if kv_ is not None else None,
                                               FAKE, FAKE, FAKE, 2051, FAKE, 1, f, FAKE, ws_, wsb, None)
    assert _call(fq, *args(None)) == sa.SA_ERR_NULL
    assert _call(fq, *args(kv, ws_=None, wsb=0)) == sa.SA_ERR_WORKSPACE
    bad = sa.SaKvQ8(FAKE, 575, 576, FAKE, 18, 18, FAKE, 576, 576, FAKE, 18, 18)         # k_ld too small
    assert _call(fq, *args(bad)) == sa.SA_ERR_ARG
    bad = sa.SaKvQ8(FAKE, 576, 576, FAKE, 17, 18, FAKE, 576, 576, FAKE, 18, 18)         # scale ld too small
    assert _call(fq, *args(bad)) == sa.SA_ERR_ARG
    bad = sa.SaKvQ8(FAKE, 576, 576, None, 18, 18, FAKE, 576, 576, FAKE, 18, 18)
    assert _call(fq, *args(bad)) == sa.SA_ERR_NULL
    odd = _dims()
    odd.d_kq = 520
    assert _call(fq, *args(kv, dd=odd)) == sa.SA_ERR_ARG                                # d_kq % 32


def test_pool_score_rejects_bad_arguments():
    d = ctypes.byref(_dims())
    c = ctypes.byref(_cache())
    f = "sparse_attn_pool_score"
    assert _call(f, d, c, None, FAKE, 1, FAKE, FAKE, FAKE, 1, FAKE, 32768, None) == sa.SA_ERR_NULL
    assert _call(f, d, c, FAKE, FAKE, -1, FAKE, FAKE, FAKE, 1, FAKE, 32768, None) == sa.SA_ERR_ARG
    assert _call(f, d, c, FAKE, FAKE, 1, FAKE, FAKE, FAKE, -1, FAKE, 32768, None) == sa.SA_ERR_ARG
    assert _call(f, d, c, FAKE, FAKE, 1, None, FAKE, FAKE, 1, FAKE, 32768, None) == sa.SA_ERR_NULL
    assert _call(f, d, c, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 1, FAKE, 1000, None) == sa.SA_ERR_ARG   # scores_ld
    bad = _cache(kidx_ld=64)
    assert _call(f, d, ctypes.byref(bad), FAKE, FAKE, 1, FAKE, FAKE, FAKE, 1, FAKE, 32768, None) == sa.SA_ERR_ARG


def test_noalloc_fwd_rejects_bad_arguments_and_oversize():
    # sparse_attn_fwd_noalloc: the checks of sparse_attn_fwd, and a call whose split
    # partials exceed the static scratch is refused before any HIP call
    hdr = open(HEADER).read()
    assert f"#define SA_STATIC_SCRATCH_BYTES ((size_t){sa.STATIC_SCRATCH_BYTES})" in hdr
    d = ctypes.byref(_dims())
    c = ctypes.byref(_cache())
    f = ctypes.c_float(0.04)
    fn = "sparse_attn_fwd_noalloc"
    assert _call(fn, d, c, None, FAKE, FAKE, 2051, FAKE, 1, f, FAKE, None) == sa.SA_ERR_NULL
    assert _call(fn, d, c, FAKE, FAKE, FAKE, 2051, FAKE, 1, ctypes.c_float(float("nan")), FAKE, None) == sa.SA_ERR_ARG
    assert _call(fn, d, c, FAKE, FAKE, FAKE, 0, FAKE, 1, f, FAKE, None) == sa.SA_ERR_ARG
    assert _call(fn, d, c, FAKE, FAKE, FAKE, 2051, FAKE, 0, f, FAKE, None) == sa.SA_OK   # nothing to do
    # scratch needed = the workspace's partials part (rows of 2048 tokens, 512 blocks:
    # always dense, so the workspace holds no selection scratch and no candidate list);
    # every shape with d_v <= 512 fits, e.g. any number of decode tokens of 16 heads 576/512
    for n_q in (1, 15, 16, 31, 32, 256, 511):
        need = sa.sparse_attn_workspace_bytes(_dims(), n_q, 2048)
        assert (need - sa.WS_STATE_BYTES if need else 0) <= sa.STATIC_SCRATCH_BYTES, n_q
    # wider V heads can exceed it: 16 tokens of 16 heads 1024/1024 (32 splits each)
    wide = _dims(d_kq=1024, d_v=1024)
    need = sa.sparse_attn_workspace_bytes(wide, 16, 2048) - sa.WS_STATE_BYTES
    assert need > sa.STATIC_SCRATCH_BYTES
    wc = ctypes.byref(_cache(k_ld=1024, v_ld=1024))
    assert _call(fn, ctypes.byref(wide), wc, FAKE, FAKE, FAKE, 2051, FAKE, 16, f, FAKE, None) == sa.SA_ERR_SCRATCH
    assert "static scratch" in sa.sparse_attn_strerror(sa.SA_ERR_SCRATCH)


def test_select_fwd_rejects_bad_arguments():
    # sparse_attn_select_fwd: the checks of sparse_attn_select and of sparse_attn_fwd,
    # all before any HIP call
    fn = "sparse_attn_select_fwd"
    ws = sa.sparse_attn_workspace_bytes(_dims(), 1, 4096)
    # dims, cache, scores, scores_ld, q_seq, q_pos, q, n_q, scale, sel, sel_ld, n_sel, out, ws, ws_bytes, stream
    good = [ctypes.byref(_dims()), ctypes.byref(_cache()), FAKE, 1024, FAKE, FAKE, FAKE, 1, ctypes.c_float(0.04),
            FAKE, 2051, FAKE, FAKE, FAKE, ws, None]

    def call(**changes):
        args = list(good)
        for k, v in changes.items():
            args[int(k[1:])] = v
        return _call(fn, *args)

    assert call(a0=None) == sa.SA_ERR_NULL
    assert call(a0=ctypes.byref(_dims(top_k=2050))) == sa.SA_ERR_DIMS
    assert call(a1=ctypes.byref(_cache(seq_len=None))) == sa.SA_ERR_NULL
    assert call(a2=None) == sa.SA_ERR_NULL                            # scores
    assert call(a3=1023) == sa.SA_ERR_ARG                             # scores_ld < max_len / c
    assert call(a5=None) == sa.SA_ERR_NULL                            # q_pos
    assert call(a6=None) == sa.SA_ERR_NULL                            # q
    assert call(a7=-1) == sa.SA_ERR_ARG
    assert call(a7=0) == sa.SA_OK                                     # nothing to do
    assert call(a8=ctypes.c_float(float("nan"))) == sa.SA_ERR_ARG
    assert call(a10=2050) == sa.SA_ERR_ARG                            # sel_ld < top_k + c - 1
    assert call(a11=None) == sa.SA_ERR_NULL                           # n_sel
    assert call(a12=None) == sa.SA_ERR_NULL                           # out
    assert call(a13=None, a14=0) == sa.SA_ERR_WORKSPACE               # the split partials
    assert call(a14=sa.WS_STATE_BYTES + 33 * 16 * (512 + 2) * 4 - 1) == sa.SA_ERR_WORKSPACE
    # a 1M row needs the chunked selection's workspace
    long_c = ctypes.byref(_cache(max_len=1048576))
    need = sa.sparse_attn_workspace_bytes(_dims(), 1, 1048576)
    assert call(a1=long_c, a3=262144, a14=ws) == sa.SA_ERR_WORKSPACE
    assert call(a1=long_c, a3=262144, a14=need - 1) == sa.SA_ERR_WORKSPACE
    # the form query
    q = "sparse_attn_select_fwd_is_fused"
    assert _call(q, ctypes.byref(_dims()), ctypes.byref(_cache()), FAKE, 0) == sa.SA_ERR_ARG
    assert _call(q, ctypes.byref(_dims()), ctypes.byref(_cache()), None, 1) == sa.SA_ERR_NULL
    assert _call(q, ctypes.byref(_dims(top_k=2050)), ctypes.byref(_cache()), FAKE, 1) == sa.SA_ERR_DIMS


def test_pool_score_select_fwd_rejects_bad_arguments():
    # sparse_attn_pool_score_select_fwd: the checks of sparse_attn_pool_score and of
    # sparse_attn_select_fwd, all before any HIP call
    fn = "sparse_attn_pool_score_select_fwd"
    ws = sa.sparse_attn_workspace_bytes(_dims(), 1, 4096)
    # dims, cache, n_in, n_out, max_new, qidx, q_seq, q_pos, n_q, scores, scores_ld, q, scale, sel, sel_ld,
    # n_sel, out, ws, ws_bytes, stream
    good = [ctypes.byref(_dims()), ctypes.byref(_cache()), FAKE, FAKE2, 1, FAKE, FAKE, FAKE, 1, FAKE, 1024, FAKE,
            ctypes.c_float(0.04), FAKE, 2051, FAKE, FAKE, FAKE, ws, None]

    def call(**changes):
        args = list(good)
        for k, v in changes.items():
            args[int(k[1:])] = v
        return _call(fn, *args)

    assert call(a0=None) == sa.SA_ERR_NULL
    assert call(a0=ctypes.byref(_dims(top_k=2050))) == sa.SA_ERR_DIMS
    assert call(a1=ctypes.byref(_cache(seq_len=None))) == sa.SA_ERR_NULL
    assert call(a1=ctypes.byref(_cache(kidx_ld=64))) == sa.SA_ERR_ARG
    assert call(a2=None) == sa.SA_ERR_NULL                            # n_pooled_in
    assert call(a3=None) == sa.SA_ERR_NULL                            # n_pooled_out
    assert call(a4=-1) == sa.SA_ERR_ARG                               # max_new_blocks
    assert call(a5=None) == sa.SA_ERR_NULL                            # qidx
    assert call(a7=None) == sa.SA_ERR_NULL                            # q_pos
    assert call(a8=-1) == sa.SA_ERR_ARG
    assert call(a9=None) == sa.SA_ERR_NULL                            # scores
    assert call(a10=1023) == sa.SA_ERR_ARG                            # scores_ld < max_len / c
    assert call(a11=None) == sa.SA_ERR_NULL                           # q
    assert call(a12=ctypes.c_float(float("nan"))) == sa.SA_ERR_ARG
    assert call(a13=None) == sa.SA_ERR_NULL                           # sel
    assert call(a14=2050) == sa.SA_ERR_ARG                            # sel_ld < top_k + c - 1
    assert call(a15=None) == sa.SA_ERR_NULL                           # n_sel
    assert call(a16=None) == sa.SA_ERR_NULL                           # out
    assert call(a17=None, a18=0) == sa.SA_ERR_WORKSPACE               # the split partials
    assert call(a18=sa.WS_STATE_BYTES + 33 * 16 * (512 + 2) * 4 - 1) == sa.SA_ERR_WORKSPACE
    long_c = ctypes.byref(_cache(max_len=1048576))
    need = sa.sparse_attn_workspace_bytes(_dims(), 1, 1048576)
    assert call(a1=long_c, a10=262144, a18=need - 1) == sa.SA_ERR_WORKSPACE
    # the form query
    q = "sparse_attn_pool_score_select_fwd_uses_list"
    cc = ctypes.byref(_cache())
    assert _call(q, ctypes.byref(_dims()), cc, FAKE, FAKE2, FAKE, FAKE, 0) == sa.SA_ERR_ARG
    assert _call(q, ctypes.byref(_dims()), cc, None, FAKE2, FAKE, FAKE, 1) == sa.SA_ERR_NULL
    assert _call(q, ctypes.byref(_dims()), cc, FAKE, FAKE2, None, FAKE, 1) == sa.SA_ERR_NULL
    assert _call(q, ctypes.byref(_dims(top_k=2050)), cc, FAKE, FAKE2, FAKE, FAKE, 1) == sa.SA_ERR_DIMS
