"""Device-side buffers for one layer, and the library's calls on them.

Plumbing for tests, the smoke check and the benchmark: torch allocates the device
memory and supplies the stream; every step runs in libsparse_attn through the
ctypes binding.  Nothing here computes any part of the method.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import sparse_attn as sa
from .datagen import Case


def _dev(x: np.ndarray, dtype: torch.dtype, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).to(device)


class DeviceLayer:
    """One layer's caches and a batch of query tokens on the GPU."""

    def __init__(self, case: Case, device="cuda", max_len: Optional[int] = None):
        d = case.dims
        self.case = case
        self.device = torch.device(device)
        self.dims = sa.make_dims(d.h_q, d.h_kv, d.d_kq, d.d_v, d.h_idx, d.d_idx, d.compress_ratio, d.top_k, d.dtype)
        dt = sa.TORCH_DTYPE[d.dtype]
        c = d.compress_ratio
        self.k = _dev(case.k, dt, device)                                     # [rows, h_kv, d_kq]
        self.alias = case.v is None
        self.v = self.k if self.alias else _dev(case.v, dt, device)          # [rows, h_kv, d_v]
        self.kidx = _dev(case.kidx, dt, device)                               # [rows, d_idx]
        self.kpool = torch.zeros((case.rows // c, d.d_idx), dtype=dt, device=device)
        self.seq_row0 = torch.from_numpy(case.row0.astype(np.int64)).to(device)
        self.seq_blk0 = torch.from_numpy(case.blk0.astype(np.int64)).to(device)
        self.seq_len = torch.from_numpy(case.seq_len.astype(np.int32)).to(device)
        self.q = _dev(case.q, dt, device)
        self.qidx = _dev(case.qidx, dt, device)
        self.q_seq = torch.from_numpy(case.q_seq.astype(np.int32)).to(device)
        self.q_pos = torch.from_numpy(case.q_pos.astype(np.int32)).to(device)
        self.n_q = case.n_q
        self.max_len = int(max_len if max_len is not None else max(int(case.seq_cap.max()), 1))
        self.scores_ld = max(1, self.max_len // c)
        self.sel_ld = d.top_k + c - 1
        self.scores = torch.zeros((self.n_q, self.scores_ld), dtype=torch.float32, device=device)
        self.sel = torch.full((self.n_q, self.sel_ld), -7, dtype=torch.int32, device=device)
        self.n_sel = torch.zeros((self.n_q,), dtype=torch.int32, device=device)
        self.out = torch.zeros((self.n_q, d.h_q, d.d_v), dtype=torch.float32, device=device)
        self.ws_bytes = sa.sparse_attn_workspace_bytes(self.dims, self.n_q, self.max_len)
        # zero-filled once: the leading state region must start at zero (the library keeps it so)
        self.ws = torch.zeros((max(self.ws_bytes, 16),), dtype=torch.uint8, device=device)
        self.n_pooled = torch.zeros((case.n_seq,), dtype=torch.int32, device=device)
        self.scale = case.scale
        self.cache = self._make_cache(self.k, self.v, self.kidx, self.kpool)

    def _make_cache(self, k, v, kidx, kpool) -> sa.Cache:
        d = self.case.dims
        return sa.Cache(seq_row0=self.seq_row0, seq_blk0=self.seq_blk0, seq_len=self.seq_len, max_len=self.max_len,
                        k=k, k_ld=d.h_kv * d.d_kq, k_head_stride=d.d_kq,
                        v=v, v_ld=(d.h_kv * d.d_kq if self.alias else d.h_kv * d.d_v),
                        v_head_stride=(d.d_kq if self.alias else d.d_v),
                        kidx=kidx, kidx_ld=d.d_idx, kpool=kpool, kpool_ld=d.d_idx)

    # ------------------------------------------------------------------ the calls
    def pool(self, max_new_blocks: int = 2 ** 31 - 1, n_in=None, n_out=None, stream=None) -> None:
        n_in = self.n_pooled if n_in is None else n_in
        n_out = self.n_pooled if n_out is None else n_out
        sa.sparse_attn_pool(self.dims, self.cache, n_in, n_out, max_new_blocks, stream)

    def score(self, stream=None) -> None:
        sa.sparse_attn_score(self.dims, self.cache, self.qidx, self.q_seq, self.q_pos, self.n_q, self.scores,
                             self.scores_ld, stream)

    def select(self, scores: Optional[torch.Tensor] = None, stream=None) -> None:
        scores = self.scores if scores is None else scores
        sa.sparse_attn_select(self.dims, self.cache, scores, scores.shape[1], self.q_seq, self.q_pos, self.n_q,
                              self.sel, self.sel_ld, self.n_sel, self.ws, self.ws_bytes, stream)

    def fwd(self, sel: Optional[torch.Tensor] = None, n_sel: Optional[torch.Tensor] = None, stream=None) -> None:
        sel = self.sel if sel is None else sel
        n_sel = self.n_sel if n_sel is None else n_sel
        sa.sparse_attn_fwd(self.dims, self.cache, self.q, self.q_seq, sel, sel.shape[1], n_sel, self.n_q,
                           self.scale, self.out, self.ws, self.ws_bytes, stream)

    def select_fwd(self, scores: Optional[torch.Tensor] = None, stream=None) -> None:
        """select then fwd in one call (the selection inside the attention's launch
        where it fits)."""
        scores = self.scores if scores is None else scores
        sa.sparse_attn_select_fwd(self.dims, self.cache, scores, scores.shape[1], self.q_seq, self.q_pos, self.q,
                                  self.n_q, self.scale, self.sel, self.sel_ld, self.n_sel, self.out, self.ws,
                                  self.ws_bytes, stream)

    def select_fwd_is_fused(self) -> bool:
        return sa.sparse_attn_select_fwd_is_fused(self.dims, self.cache, self.q, self.n_q)

    def pool_score_select_fwd(self, max_new_blocks: int = 2 ** 31 - 1, n_in=None, n_out=None, stream=None) -> None:
        """pool + score, then select and attend (sparse_attn_pool_score_select_fwd): the
        selection from the scoring launch's candidate list where it applies."""
        n_in, n_out = self._counts(n_in, n_out)
        sa.sparse_attn_pool_score_select_fwd(self.dims, self.cache, n_in, n_out, max_new_blocks, self.qidx,
                                             self.q_seq, self.q_pos, self.n_q, self.scores, self.scores_ld, self.q,
                                             self.scale, self.sel, self.sel_ld, self.n_sel, self.out, self.ws,
                                             self.ws_bytes, stream)

    def pool_score_select_fwd_uses_list(self, n_in=None, n_out=None) -> bool:
        n_in, n_out = self._counts(n_in, n_out)
        return sa.sparse_attn_pool_score_select_fwd_uses_list(self.dims, self.cache, n_in, n_out, self.qidx, self.q,
                                                              self.n_q)

    def _counts(self, n_in, n_out):
        """Pooled-count arrays in and out: distinct by default (the pooling scoring
        launch needs them apart); the output becomes the layer's count."""
        if n_in is None:
            n_in = self.n_pooled
        if n_out is None:
            if not hasattr(self, "n_pooled_next"):
                self.n_pooled_next = torch.zeros_like(self.n_pooled)
            n_out = self.n_pooled_next
        return n_in, n_out

    def list_decided(self) -> np.ndarray:
        """The n_q int32 that end the workspace: 1 where sparse_attn_pool_score_select_fwd's
        candidate list decided the token's selection, 0 where the row did."""
        return self.ws[self.ws_bytes - 4 * self.n_q: self.ws_bytes].view(torch.int32).cpu().numpy()

    def fwd_window(self, window: int, sel: Optional[torch.Tensor] = None, n_sel: Optional[torch.Tensor] = None,
                   stream=None) -> None:
        sel = self.sel if sel is None else sel
        n_sel = self.n_sel if n_sel is None else n_sel
        sa.sparse_attn_fwd_window(self.dims, self.cache, self.q, self.q_seq, self.q_pos, sel, sel.shape[1], n_sel,
                                  window, self.n_q, self.scale, self.out, self.ws, self.ws_bytes, stream)

    # ------------------------------------------------------------ q8_0 K/V cache
    def quantize_kv(self, stream=None) -> None:
        """Quantize the layer's K (and a separate V) into q8_0 planes on the GPU:
        codes [rows][h_kv][d] int8, scales [rows][h_kv][d / 32] float16."""
        d = self.case.dims
        rows = self.case.rows
        self.kq = torch.zeros((rows, d.h_kv, d.d_kq), dtype=torch.int8, device=self.device)
        self.kqs = torch.zeros((rows, d.h_kv, d.d_kq // 32), dtype=torch.float16, device=self.device)
        sa.sparse_attn_quantize_q8_0(self.k, d.dtype, rows * d.h_kv, d.d_kq, d.d_kq, self.kq, d.d_kq, self.kqs,
                                     d.d_kq // 32, stream)
        if self.alias:
            self.vq, self.vqs = self.kq, self.kqs
            vd = d.d_kq
        else:
            self.vq = torch.zeros((rows, d.h_kv, d.d_v), dtype=torch.int8, device=self.device)
            self.vqs = torch.zeros((rows, d.h_kv, d.d_v // 32), dtype=torch.float16, device=self.device)
            sa.sparse_attn_quantize_q8_0(self.v, d.dtype, rows * d.h_kv, d.d_v, d.d_v, self.vq, d.d_v, self.vqs,
                                         d.d_v // 32, stream)
            vd = d.d_v
        self.kv_q8 = sa.KvQ8(k=self.kq, k_ld=d.h_kv * d.d_kq, k_head_stride=d.d_kq, k_scale=self.kqs,
                             k_scale_ld=d.h_kv * d.d_kq // 32, k_scale_head_stride=d.d_kq // 32,
                             v=self.vq, v_ld=d.h_kv * vd, v_head_stride=vd, v_scale=self.vqs,
                             v_scale_ld=d.h_kv * vd // 32, v_scale_head_stride=vd // 32)

    def fwd_q8(self, sel: Optional[torch.Tensor] = None, n_sel: Optional[torch.Tensor] = None, stream=None) -> None:
        sel = self.sel if sel is None else sel
        n_sel = self.n_sel if n_sel is None else n_sel
        sa.sparse_attn_fwd_q8_0(self.dims, self.cache, self.kv_q8, self.q, self.q_seq, sel, sel.shape[1], n_sel,
                                self.n_q, self.scale, self.out, self.ws, self.ws_bytes, stream)

    def step(self, stream=None) -> None:
        """One pass of the whole path in one call (sparse_attn_pool_score_select_fwd):
        pool what is new, score, select, attend.  The pooled counts go from n_pooled to
        a second array, and the two are swapped (the pooling scoring launch needs them
        apart)."""
        n_in, n_out = self._counts(None, None)
        self.pool_score_select_fwd(n_in=n_in, n_out=n_out, stream=stream)
        self.n_pooled, self.n_pooled_next = n_out, n_in

    # ------------------------------------------------------------------ readback
    def selections(self) -> list[np.ndarray]:
        sel = self.sel.cpu().numpy()
        n = self.n_sel.cpu().numpy()
        return [sel[i, : n[i]].astype(np.int64) for i in range(self.n_q)]
