"""ctypes binding of libsparse_attn.so (argument marshalling only).

Every function here has the name and argument order of the C entry point in
``include/sparse_attn.h``; tensors are passed as their device pointers, the stream
defaults to torch's current stream.  All computation happens in the HIP library:
there is no Python or CPU fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparse_attn.so")

SA_F32, SA_F16, SA_BF16 = 0, 1, 2
DTYPE_CODE = {"f32": SA_F32, "f16": SA_F16, "bf16": SA_BF16}
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

SA_OK, SA_ERR_NULL, SA_ERR_DIMS, SA_ERR_ARG, SA_ERR_WORKSPACE, SA_ERR_HIP, SA_ERR_SCRATCH = 0, -1, -2, -3, -4, -5, -6

# Leading bytes of a workspace that hold state between calls (zero-filled once by the
# caller, kept at zero by the library); SA_WS_STATE_BYTES in the header.
WS_STATE_BYTES = 1056768
STATIC_SCRATCH_BYTES = 16842752   # SA_STATIC_SCRATCH_BYTES

EXPORTS = (
    "sparse_attn_check_dims",
    "sparse_attn_workspace_bytes",
    "sparse_attn_pool",
    "sparse_attn_score",
    "sparse_attn_pool_score",
    "sparse_attn_select",
    "sparse_attn_fwd",
    "sparse_attn_fwd_noalloc",
    "sparse_attn_select_fwd",
    "sparse_attn_select_fwd_is_fused",
    "sparse_attn_pool_score_select_fwd",
    "sparse_attn_pool_score_select_fwd_uses_list",
    "sparse_attn_mask_to_indices",
    "sparse_attn_fwd_bias",
    "sparse_attn_workspace_bytes_window",
    "sparse_attn_fwd_window",
    "sparse_attn_quantize_q8_0",
    "sparse_attn_fwd_q8_0",
    "sparse_attn_strerror",
    "sparse_attn_version",
)


class SaDims(ctypes.Structure):
    _fields_ = [("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("d_kq", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("h_idx", ctypes.c_int32), ("d_idx", ctypes.c_int32),
                ("compress_ratio", ctypes.c_int32), ("top_k", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class SaCache(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("max_len", ctypes.c_int32),
                ("seq_row0", ctypes.c_void_p), ("seq_blk0", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
                ("k", ctypes.c_void_p), ("k_ld", ctypes.c_int64), ("k_head_stride", ctypes.c_int64),
                ("v", ctypes.c_void_p), ("v_ld", ctypes.c_int64), ("v_head_stride", ctypes.c_int64),
                ("kidx", ctypes.c_void_p), ("kidx_ld", ctypes.c_int64),
                ("kpool", ctypes.c_void_p), ("kpool_ld", ctypes.c_int64)]


class SaKvQ8(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("k_ld", ctypes.c_int64), ("k_head_stride", ctypes.c_int64),
                ("k_scale", ctypes.c_void_p), ("k_scale_ld", ctypes.c_int64), ("k_scale_head_stride", ctypes.c_int64),
                ("v", ctypes.c_void_p), ("v_ld", ctypes.c_int64), ("v_head_stride", ctypes.c_int64),
                ("v_scale", ctypes.c_void_p), ("v_scale_ld", ctypes.c_int64), ("v_scale_head_stride", ctypes.c_int64)]


class SparseAttnError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({code})")
        self.code = code


_lib: Optional[ctypes.CDLL] = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the library once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m indexer_top_block_amd.build` "
                           "(the compute path has no fallback)")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    dp, cp = ctypes.POINTER(SaDims), ctypes.POINTER(SaCache)
    lib.sparse_attn_check_dims.argtypes = [dp]
    lib.sparse_attn_check_dims.restype = ctypes.c_int
    lib.sparse_attn_workspace_bytes.argtypes = [dp, I32, I32]
    lib.sparse_attn_workspace_bytes.restype = SZ
    lib.sparse_attn_pool.argtypes = [dp, cp, P, P, I32, P]
    lib.sparse_attn_pool.restype = ctypes.c_int
    lib.sparse_attn_score.argtypes = [dp, cp, P, P, P, I32, P, I64, P]
    lib.sparse_attn_score.restype = ctypes.c_int
    lib.sparse_attn_pool_score.argtypes = [dp, cp, P, P, I32, P, P, P, I32, P, I64, P]
    lib.sparse_attn_pool_score.restype = ctypes.c_int
    lib.sparse_attn_select.argtypes = [dp, cp, P, I64, P, P, I32, P, I64, P, P, SZ, P]
    lib.sparse_attn_select.restype = ctypes.c_int
    lib.sparse_attn_fwd.argtypes = [dp, cp, P, P, P, I64, P, I32, ctypes.c_float, P, P, SZ, P]
    lib.sparse_attn_fwd.restype = ctypes.c_int
    lib.sparse_attn_fwd_noalloc.argtypes = [dp, cp, P, P, P, I64, P, I32, ctypes.c_float, P, P]
    lib.sparse_attn_fwd_noalloc.restype = ctypes.c_int
    lib.sparse_attn_select_fwd.argtypes = [dp, cp, P, I64, P, P, P, I32, ctypes.c_float, P, I64, P, P, P, SZ, P]
    lib.sparse_attn_select_fwd.restype = ctypes.c_int
    lib.sparse_attn_select_fwd_is_fused.argtypes = [dp, cp, P, I32]
    lib.sparse_attn_select_fwd_is_fused.restype = ctypes.c_int
    lib.sparse_attn_pool_score_select_fwd.argtypes = [dp, cp, P, P, I32, P, P, P, I32, P, I64, P, ctypes.c_float,
                                                      P, I64, P, P, P, SZ, P]
    lib.sparse_attn_pool_score_select_fwd.restype = ctypes.c_int
    lib.sparse_attn_pool_score_select_fwd_uses_list.argtypes = [dp, cp, P, P, P, P, I32]
    lib.sparse_attn_pool_score_select_fwd_uses_list.restype = ctypes.c_int
    lib.sparse_attn_mask_to_indices.argtypes = [P, I32, I64, I32, I32, P, I64, P, P, P]
    lib.sparse_attn_mask_to_indices.restype = ctypes.c_int
    lib.sparse_attn_fwd_bias.argtypes = [dp, cp, P, P, P, I64, P, P, I32, ctypes.c_float, P, P, SZ, P]
    lib.sparse_attn_fwd_bias.restype = ctypes.c_int
    lib.sparse_attn_workspace_bytes_window.argtypes = [dp, I32, I32, I32]
    lib.sparse_attn_workspace_bytes_window.restype = SZ
    lib.sparse_attn_fwd_window.argtypes = [dp, cp, P, P, P, P, I64, P, I32, I32, ctypes.c_float, P, P, SZ, P]
    lib.sparse_attn_fwd_window.restype = ctypes.c_int
    kp = ctypes.POINTER(SaKvQ8)
    lib.sparse_attn_quantize_q8_0.argtypes = [P, I32, I64, I32, I64, P, I64, P, I64, P]
    lib.sparse_attn_quantize_q8_0.restype = ctypes.c_int
    lib.sparse_attn_fwd_q8_0.argtypes = [dp, cp, kp, P, P, P, I64, P, I32, ctypes.c_float, P, P, SZ, P]
    lib.sparse_attn_fwd_q8_0.restype = ctypes.c_int
    lib.sparse_attn_strerror.argtypes = [ctypes.c_int]
    lib.sparse_attn_strerror.restype = ctypes.c_char_p
    lib.sparse_attn_version.argtypes = []
    lib.sparse_attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


# --------------------------------------------------------------------- marshalling

def make_dims(h_q, h_kv, d_kq, d_v, h_idx, d_idx, compress_ratio, top_k, dtype) -> SaDims:
    code = DTYPE_CODE[dtype] if isinstance(dtype, str) else int(dtype)
    return SaDims(h_q, h_kv, d_kq, d_v, h_idx, d_idx, compress_ratio, top_k, code)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Cache:
    """Owns the ctypes sa_cache struct and references to the tensors it points at."""

    def __init__(self, *, seq_row0, seq_blk0, seq_len, max_len, k, k_ld, k_head_stride, v, v_ld, v_head_stride,
                 kidx, kidx_ld, kpool, kpool_ld):
        self._keep = (seq_row0, seq_blk0, seq_len, k, v, kidx, kpool)
        self.struct = SaCache(int(seq_len.numel()), int(max_len), _ptr(seq_row0), _ptr(seq_blk0), _ptr(seq_len),
                              _ptr(k), int(k_ld), int(k_head_stride), _ptr(v), int(v_ld), int(v_head_stride),
                              _ptr(kidx), int(kidx_ld), _ptr(kpool), int(kpool_ld))


class KvQ8:
    """Owns the ctypes sa_kv_q8_0 struct and references to the planes it points at
    (codes int8, scales float16 -- passed as int16/float16 tensors)."""

    def __init__(self, *, k, k_ld, k_head_stride, k_scale, k_scale_ld, k_scale_head_stride, v, v_ld, v_head_stride,
                 v_scale, v_scale_ld, v_scale_head_stride):
        self._keep = (k, k_scale, v, v_scale)
        self.struct = SaKvQ8(_ptr(k), int(k_ld), int(k_head_stride), _ptr(k_scale), int(k_scale_ld),
                             int(k_scale_head_stride), _ptr(v), int(v_ld), int(v_head_stride), _ptr(v_scale),
                             int(v_scale_ld), int(v_scale_head_stride))


def _check(fn: str, rc: int) -> None:
    if rc != SA_OK:
        raise SparseAttnError(fn, rc, load().sparse_attn_strerror(rc).decode())


def sparse_attn_check_dims(dims: SaDims) -> int:
    return load().sparse_attn_check_dims(ctypes.byref(dims))


def sparse_attn_workspace_bytes(dims: SaDims, n_q: int, max_len: int) -> int:
    return int(load().sparse_attn_workspace_bytes(ctypes.byref(dims), int(n_q), int(max_len)))


def sparse_attn_workspace_bytes_window(dims: SaDims, n_q: int, max_len: int, window: int) -> int:
    return int(load().sparse_attn_workspace_bytes_window(ctypes.byref(dims), int(n_q), int(max_len), int(window)))


def sparse_attn_pool(dims: SaDims, cache: Cache, n_pooled_in, n_pooled_out, max_new_blocks: int,
                     stream=None) -> None:
    _check("sparse_attn_pool", load().sparse_attn_pool(ctypes.byref(dims), ctypes.byref(cache.struct),
                                                       _ptr(n_pooled_in), _ptr(n_pooled_out), int(max_new_blocks),
                                                       _stream(stream)))


def sparse_attn_score(dims: SaDims, cache: Cache, qidx, q_seq, q_pos, n_q: int, scores, scores_ld: int,
                      stream=None) -> None:
    _check("sparse_attn_score", load().sparse_attn_score(ctypes.byref(dims), ctypes.byref(cache.struct), _ptr(qidx),
                                                         _ptr(q_seq), _ptr(q_pos), int(n_q), _ptr(scores),
                                                         int(scores_ld), _stream(stream)))


def sparse_attn_pool_score(dims: SaDims, cache: Cache, n_pooled_in, n_pooled_out, max_new_blocks: int, qidx, q_seq,
                           q_pos, n_q: int, scores, scores_ld: int, stream=None) -> None:
    _check("sparse_attn_pool_score",
           load().sparse_attn_pool_score(ctypes.byref(dims), ctypes.byref(cache.struct), _ptr(n_pooled_in),
                                         _ptr(n_pooled_out), int(max_new_blocks), _ptr(qidx), _ptr(q_seq),
                                         _ptr(q_pos), int(n_q), _ptr(scores), int(scores_ld), _stream(stream)))


def sparse_attn_select(dims: SaDims, cache: Cache, scores, scores_ld: int, q_seq, q_pos, n_q: int, sel, sel_ld: int,
                       n_sel, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check("sparse_attn_select", load().sparse_attn_select(ctypes.byref(dims), ctypes.byref(cache.struct),
                                                           _ptr(scores), int(scores_ld), _ptr(q_seq), _ptr(q_pos),
                                                           int(n_q), _ptr(sel), int(sel_ld), _ptr(n_sel), _ptr(ws),
                                                           int(ws_bytes), _stream(stream)))


def sparse_attn_fwd(dims: SaDims, cache: Cache, q, q_seq, sel, sel_ld: int, n_sel, n_q: int, scale: float, out,
                    ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check("sparse_attn_fwd", load().sparse_attn_fwd(ctypes.byref(dims), ctypes.byref(cache.struct), _ptr(q),
                                                     _ptr(q_seq), _ptr(sel), int(sel_ld), _ptr(n_sel), int(n_q),
                                                     float(scale), _ptr(out), _ptr(ws), int(ws_bytes),
                                                     _stream(stream)))


def sparse_attn_fwd_noalloc(dims: SaDims, cache: Cache, q, q_seq, sel, sel_ld: int, n_sel, n_q: int, scale: float,
                            out, stream=None) -> None:
    _check("sparse_attn_fwd_noalloc",
           load().sparse_attn_fwd_noalloc(ctypes.byref(dims), ctypes.byref(cache.struct), _ptr(q), _ptr(q_seq),
                                          _ptr(sel), int(sel_ld), _ptr(n_sel), int(n_q), float(scale), _ptr(out),
                                          _stream(stream)))


def sparse_attn_select_fwd(dims: SaDims, cache: Cache, scores, scores_ld: int, q_seq, q_pos, q, n_q: int,
                           scale: float, sel, sel_ld: int, n_sel, out, ws=None, ws_bytes: int = 0,
                           stream=None) -> None:
    _check("sparse_attn_select_fwd",
           load().sparse_attn_select_fwd(ctypes.byref(dims), ctypes.byref(cache.struct), _ptr(scores), int(scores_ld),
                                         _ptr(q_seq), _ptr(q_pos), _ptr(q), int(n_q), float(scale), _ptr(sel),
                                         int(sel_ld), _ptr(n_sel), _ptr(out), _ptr(ws), int(ws_bytes),
                                         _stream(stream)))


def sparse_attn_select_fwd_is_fused(dims: SaDims, cache: Cache, q, n_q: int) -> bool:
    rc = load().sparse_attn_select_fwd_is_fused(ctypes.byref(dims), ctypes.byref(cache.struct), _ptr(q), int(n_q))
    if rc < 0:
        _check("sparse_attn_select_fwd_is_fused", rc)
    return rc == 1


def sparse_attn_pool_score_select_fwd(dims: SaDims, cache: Cache, n_pooled_in, n_pooled_out, max_new_blocks: int,
                                      qidx, q_seq, q_pos, n_q: int, scores, scores_ld: int, q, scale: float, sel,
                                      sel_ld: int, n_sel, out, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check("sparse_attn_pool_score_select_fwd",
           load().sparse_attn_pool_score_select_fwd(ctypes.byref(dims), ctypes.byref(cache.struct), _ptr(n_pooled_in),
                                                    _ptr(n_pooled_out), int(max_new_blocks), _ptr(qidx), _ptr(q_seq),
                                                    _ptr(q_pos), int(n_q), _ptr(scores), int(scores_ld), _ptr(q),
                                                    float(scale), _ptr(sel), int(sel_ld), _ptr(n_sel), _ptr(out),
                                                    _ptr(ws), int(ws_bytes), _stream(stream)))


def sparse_attn_pool_score_select_fwd_uses_list(dims: SaDims, cache: Cache, n_pooled_in, n_pooled_out, qidx, q,
                                                n_q: int) -> bool:
    rc = load().sparse_attn_pool_score_select_fwd_uses_list(ctypes.byref(dims), ctypes.byref(cache.struct),
                                                            _ptr(n_pooled_in), _ptr(n_pooled_out), _ptr(qidx),
                                                            _ptr(q), int(n_q))
    if rc < 0:
        _check("sparse_attn_pool_score_select_fwd_uses_list", rc)
    return rc == 1


def sparse_attn_mask_to_indices(mask, mask_dtype, mask_ld: int, n_q: int, n_kv: int, sel, sel_ld: int, n_sel,
                                sel_bias=None, stream=None) -> None:
    code = DTYPE_CODE[mask_dtype] if isinstance(mask_dtype, str) else int(mask_dtype)
    _check("sparse_attn_mask_to_indices",
           load().sparse_attn_mask_to_indices(_ptr(mask), code, int(mask_ld), int(n_q), int(n_kv), _ptr(sel),
                                              int(sel_ld), _ptr(n_sel), _ptr(sel_bias), _stream(stream)))


def sparse_attn_fwd_bias(dims: SaDims, cache: Cache, q, q_seq, sel, sel_ld: int, n_sel, sel_bias, n_q: int,
                         scale: float, out, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check("sparse_attn_fwd_bias",
           load().sparse_attn_fwd_bias(ctypes.byref(dims), ctypes.byref(cache.struct), _ptr(q), _ptr(q_seq),
                                       _ptr(sel), int(sel_ld), _ptr(n_sel), _ptr(sel_bias), int(n_q), float(scale),
                                       _ptr(out), _ptr(ws), int(ws_bytes), _stream(stream)))


def sparse_attn_fwd_window(dims: SaDims, cache: Cache, q, q_seq, q_pos, sel, sel_ld: int, n_sel, window: int,
                           n_q: int, scale: float, out, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check("sparse_attn_fwd_window",
           load().sparse_attn_fwd_window(ctypes.byref(dims), ctypes.byref(cache.struct), _ptr(q), _ptr(q_seq),
                                         _ptr(q_pos), _ptr(sel), int(sel_ld), _ptr(n_sel), int(window), int(n_q),
                                         float(scale), _ptr(out), _ptr(ws), int(ws_bytes), _stream(stream)))


def sparse_attn_strerror(code: int) -> str:
    return load().sparse_attn_strerror(int(code)).decode()


def sparse_attn_version() -> str:
    return load().sparse_attn_version().decode()


def sparse_attn_quantize_q8_0(x, x_dtype, n_rows: int, n_cols: int, x_ld: int, codes, codes_ld: int, scales,
                              scales_ld: int, stream=None) -> None:
    code = DTYPE_CODE[x_dtype] if isinstance(x_dtype, str) else int(x_dtype)
    _check("sparse_attn_quantize_q8_0",
           load().sparse_attn_quantize_q8_0(_ptr(x), code, int(n_rows), int(n_cols), int(x_ld), _ptr(codes),
                                            int(codes_ld), _ptr(scales), int(scales_ld), _stream(stream)))


def sparse_attn_fwd_q8_0(dims: SaDims, cache: Cache, kv: KvQ8, q, q_seq, sel, sel_ld: int, n_sel, n_q: int,
                         scale: float, out, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check("sparse_attn_fwd_q8_0",
           load().sparse_attn_fwd_q8_0(ctypes.byref(dims), ctypes.byref(cache.struct), ctypes.byref(kv.struct),
                                       _ptr(q), _ptr(q_seq), _ptr(sel), int(sel_ld), _ptr(n_sel), int(n_q),
                                       float(scale), _ptr(out), _ptr(ws), int(ws_bytes), _stream(stream)))
