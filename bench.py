"""Benchmark of the indexer-selected sparse-attention decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

A step is one pass of the whole path -- pool the newest block, score every block,
select, attend -- for one decode token of a DeepSeek-V4-shaped layer at 128K context
(16 query heads on one 576-wide latent KV head with V = its first 512 dims; indexer of
64 heads x 128, compress_ratio 4, top_k 2048; bf16 caches), made by one call,
sparse_attn_pool_score_select_fwd: the pooling scoring launch (which also writes each
32-block group's 8 best blocks), the selection from that list inside the attention's
launch, and the split combine.  The timed steps are replayed as one HIP graph (the
same kernel launches, without the host-side launch overhead of the Python binding).

Cold (the headline): `--layers` independent copies of the layer's caches are resident
(like a model's layers) and step k runs on copy k mod layers.  Between the untimed
and the timed replay a 1 GiB buffer is read, four times the 256 MB last-level cache,
so every step of the timed replay reads a copy that nothing has touched since; with
more steps than copies, a copy comes back only after all the others (more than twice
the cache) have streamed through.  This holds for any --steps.  Warm: every step on
the same copy, right after an untimed replay, so its ~10.7 MB stay cached.

Prints one JSON line.  `value` is algorithmic HBM bytes per step (pooled indexer keys
of the visible blocks + gathered K rows) divided by the cold step time, in GB/s.
Further sections: the prefill chunk (TFLOP/s against the dense bf16 MFMA peak, the
vendor figure and one measured with a plain MFMA loop), the 1M-context decode, the
batched 32-sequence decode, the token-level decode, the mask form, the dense window,
the q8_0 cache, and the CPU oracle's rate on the same decode step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from indexer_top_block_amd import datagen  # noqa: E402
from indexer_top_block_amd import sparse_attn as sa  # noqa: E402

METRIC = "sparse-attn decode µs/step + HBM GB/s @128K ctx; prefill TFLOP/s (% roofline)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------- layers

class RotatingLayers:
    """`n` copies of one layer's caches in HBM, and the calls of one decode step on copy r."""

    def __init__(self, case: datagen.Case, n: int, device="cuda"):
        d = case.dims
        self.case, self.n, self.device = case, n, torch.device(device)
        self.dims = sa.make_dims(d.h_q, d.h_kv, d.d_kq, d.d_v, d.h_idx, d.d_idx, d.compress_ratio, d.top_k, d.dtype)
        dt = sa.TORCH_DTYPE[d.dtype]
        c = d.compress_ratio
        rows = case.rows
        self.alias = case.v is None
        k1 = torch.from_numpy(case.k).to(dt).to(device)
        kidx1 = torch.from_numpy(case.kidx).to(dt).to(device)
        self.k = torch.empty((n, rows, d.h_kv, d.d_kq), dtype=dt, device=device)
        self.kidx = torch.empty((n, rows, d.d_idx), dtype=dt, device=device)
        self.kpool = torch.zeros((n, rows // c, d.d_idx), dtype=dt, device=device)
        for r in range(n):
            self.k[r].copy_(k1)
            self.kidx[r].copy_(kidx1)
        del k1, kidx1
        if not self.alias:
            v1 = torch.from_numpy(case.v).to(dt).to(device)
            self.v = torch.empty((n, rows, d.h_kv, d.d_v), dtype=dt, device=device)
            for r in range(n):
                self.v[r].copy_(v1)
            del v1
        else:
            self.v = self.k
        self.seq_row0 = torch.from_numpy(case.row0.astype(np.int64)).to(device)
        self.seq_blk0 = torch.from_numpy(case.blk0.astype(np.int64)).to(device)
        self.seq_len = torch.from_numpy(case.seq_len.astype(np.int32)).to(device)
        self.q = torch.from_numpy(case.q).to(dt).to(device)
        self.qidx = torch.from_numpy(case.qidx).to(dt).to(device)
        self.q_seq = torch.from_numpy(case.q_seq.astype(np.int32)).to(device)
        self.q_pos = torch.from_numpy(case.q_pos.astype(np.int32)).to(device)
        self.n_q = case.n_q
        self.max_len = int(case.seq_cap.max())
        self.scores_ld = self.max_len // c
        self.sel_ld = d.top_k + c - 1
        self.scores = torch.zeros((self.n_q, self.scores_ld), dtype=torch.float32, device=device)
        self.sel = torch.zeros((self.n_q, self.sel_ld), dtype=torch.int32, device=device)
        self.n_sel = torch.zeros((self.n_q,), dtype=torch.int32, device=device)
        self.out = torch.zeros((self.n_q, d.h_q, d.d_v), dtype=torch.float32, device=device)
        self.ws_bytes = sa.sparse_attn_workspace_bytes(self.dims, self.n_q, self.max_len)
        # zero-filled once: the leading state region must start at zero (the library keeps it so)
        self.ws = torch.zeros((max(self.ws_bytes, 16),), dtype=torch.uint8, device=device)
        nb_full = (case.seq_len.astype(np.int64) // c).astype(np.int32)
        # each step re-pools the newest complete block (what a decode step adds every c tokens)
        self.n_pooled_prev = torch.from_numpy(np.maximum(nb_full - 1, 0)).to(device)
        self.n_pooled_out = torch.zeros_like(self.n_pooled_prev)
        self.caches = []
        for r in range(n):
            self.caches.append(sa.Cache(
                seq_row0=self.seq_row0, seq_blk0=self.seq_blk0, seq_len=self.seq_len, max_len=self.max_len,
                k=self.k[r], k_ld=d.h_kv * d.d_kq, k_head_stride=d.d_kq,
                v=(self.k[r] if self.alias else self.v[r]),
                v_ld=(d.h_kv * d.d_kq if self.alias else d.h_kv * d.d_v),
                v_head_stride=(d.d_kq if self.alias else d.d_v),
                kidx=self.kidx[r], kidx_ld=d.d_idx, kpool=self.kpool[r], kpool_ld=d.d_idx))

    def fill_pools(self) -> None:
        zeros = torch.zeros_like(self.n_pooled_prev)
        for r in range(self.n):
            sa.sparse_attn_pool(self.dims, self.caches[r], zeros, self.n_pooled_out, 2 ** 31 - 1)

    # the calls of a step, on copy r
    def pool(self, r):
        sa.sparse_attn_pool(self.dims, self.caches[r], self.n_pooled_prev, self.n_pooled_out, 1)

    def score(self, r):
        sa.sparse_attn_score(self.dims, self.caches[r], self.qidx, self.q_seq, self.q_pos, self.n_q, self.scores,
                             self.scores_ld)

    def select(self, r):
        sa.sparse_attn_select(self.dims, self.caches[r], self.scores, self.scores_ld, self.q_seq, self.q_pos,
                              self.n_q, self.sel, self.sel_ld, self.n_sel, self.ws, self.ws_bytes)

    def fwd(self, r):
        sa.sparse_attn_fwd(self.dims, self.caches[r], self.q, self.q_seq, self.sel, self.sel_ld, self.n_sel,
                           self.n_q, self.case.scale, self.out, self.ws, self.ws_bytes)

    def pool_score(self, r):
        """pool + score in one call (one launch on the decode path)."""
        sa.sparse_attn_pool_score(self.dims, self.caches[r], self.n_pooled_prev, self.n_pooled_out, 1, self.qidx,
                                  self.q_seq, self.q_pos, self.n_q, self.scores, self.scores_ld)

    def select_fwd(self, r):
        """select + fwd in one call (the selection inside the attention's launch where it fits)."""
        sa.sparse_attn_select_fwd(self.dims, self.caches[r], self.scores, self.scores_ld, self.q_seq, self.q_pos,
                                  self.q, self.n_q, self.case.scale, self.sel, self.sel_ld, self.n_sel, self.out,
                                  self.ws, self.ws_bytes)

    def select_fwd_is_fused(self) -> bool:
        return sa.sparse_attn_select_fwd_is_fused(self.dims, self.caches[0], self.q, self.n_q)

    def pool_score_select_fwd(self, r):
        """pool + score, then select + fwd, in one call (the selection from the scoring
        launch's candidate list where it applies)."""
        sa.sparse_attn_pool_score_select_fwd(self.dims, self.caches[r], self.n_pooled_prev, self.n_pooled_out, 1,
                                             self.qidx, self.q_seq, self.q_pos, self.n_q, self.scores,
                                             self.scores_ld, self.q, self.case.scale, self.sel, self.sel_ld,
                                             self.n_sel, self.out, self.ws, self.ws_bytes)

    def uses_list(self) -> bool:
        return sa.sparse_attn_pool_score_select_fwd_uses_list(self.dims, self.caches[0], self.n_pooled_prev,
                                                              self.n_pooled_out, self.qidx, self.q, self.n_q)

    def list_decided(self) -> list:
        """Per token, 1 where the last call's candidate list decided the selection."""
        tail = self.ws[self.ws_bytes - 4 * self.n_q: self.ws_bytes].view(torch.int32)
        return [int(x) for x in tail.cpu()]

    def two_calls(self, r):
        self.pool_score(r)
        self.select_fwd(r)

    def step(self, r):
        self.pool_score_select_fwd(r)


def algorithmic_bytes(case: datagen.Case, kv: str = "cache") -> dict:
    """Bytes a step must read from HBM: pooled keys of every visible complete block of
    every query, and the selected K rows (plus V rows when V is stored separately).
    kv="q8_0": the rows are q8_0 codes (1 byte per element) plus a 2-byte scale per
    32 elements."""
    d = case.dims
    es = 4 if d.dtype == "f32" else 2
    row_bytes = (lambda n: n * es) if kv == "cache" else (lambda n: n + n // 32 * 2)
    c = d.compress_ratio
    pooled = 0
    gathered = 0
    for i in range(case.n_q):
        s = int(case.q_seq[i])
        n_vis = max(0, min(int(case.seq_len[s]), int(case.q_pos[i]) + 1))
        nb = n_vis // c
        n_sel = min(nb, d.top_k // c) * c + (n_vis - nb * c)
        pooled += nb * d.d_idx * es
        gathered += n_sel * row_bytes(d.h_kv * d.d_kq + (0 if case.v is None else d.h_kv * d.d_v))
    return {"pooled": pooled, "gathered": gathered, "total": pooled + gathered}


# ----------------------------------------------------------------------- timing

def score_source_digest() -> str:
    """sha256 over the score kernel's source and the device headers it includes (the
    launch header holds host declarations only)."""
    import hashlib
    h = hashlib.sha256()
    for f in ("score.hip", "sa_common.hpp", "select_wide.hpp"):
        h.update(open(os.path.join(ROOT, "indexer_top_block_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def traffic_from_counters(path: str):
    """HBM bytes per launch of the score kernel, as measured by the FETCH_SIZE and
    WRITE_SIZE counters (scaled by what they read for a copy of known size), if that
    measurement exists and was taken on the current kernel source.  The summary file
    holds `key: value` lines."""
    try:
        rec = dict(l.split(":", 1) for l in open(path).read().splitlines() if ":" in l and not l.startswith(" "))
    except OSError:
        return None
    rec = {k.strip(): v.strip() for k, v in rec.items()}
    if score_source_digest() != rec.get("score_source_sha256"):
        return None                  # the kernel changed since the counters were taken
    try:
        return int(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Flusher:
    """Reads a buffer of `mib` MiB (a reduction kernel): evicts the L2s and the
    last-level cache without leaving dirty lines to be written back later."""

    def __init__(self, mib: int):
        self.mib = mib
        self.buf = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device="cuda") if mib > 0 else None

    def __call__(self) -> None:
        if self.buf is not None:
            torch.sum(self.buf)


def time_graph(fn_per_step, n_steps: int, warmup: int, flush: "Flusher | None" = None) -> float:
    """Capture n_steps calls of fn_per_step(k) in one graph; return ms per step of a
    replay.  One untimed replay comes first; with `flush`, the cache-evicting read
    runs between it and the timed replay (outside the timed region)."""
    for k in range(max(warmup, 1)):
        fn_per_step(k)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(n_steps):
            fn_per_step(k)
    torch.cuda.synchronize()
    g.replay()                       # one untimed replay
    if flush is not None:
        flush()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    del g
    return start.elapsed_time(end) / n_steps


def time_eager(fn_per_step, n_steps: int, warmup: int) -> float:
    for k in range(warmup):
        fn_per_step(k)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(n_steps):
        fn_per_step(k)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n_steps


def gbs(nbytes: float, ms: float) -> float:
    return nbytes / (ms * 1e-3) / 1e9


def decode_section(lay: "RotatingLayers", ab: dict, steps: int, warmup: int, flush: Flusher,
                   kernels=("pool_score", "select_fwd", "two_calls", "select", "fwd"), warm: bool = True) -> dict:
    """Cold step time over the rotated copies (flush before the timed replay), each
    entry point alone under the same protocol (two_calls: sparse_attn_pool_score then
    sparse_attn_select_fwd, the step without the candidate list), and (optionally)
    the warm step time."""
    R = lay.n
    ms = time_graph(lambda k: lay.step(k % R), steps, warmup, flush)
    decided = lay.list_decided() if lay.uses_list() else None
    rec = {"us_per_step": round(ms * 1e3, 3), "value": round(gbs(ab["total"], ms), 2), "unit": "GB/s",
           "frac_of_hbm_peak": round(gbs(ab["total"], ms) / HBM_PEAK_GBS, 4), "bytes_per_step": ab,
           "timed_region": {"steps": steps, "distinct_layer_copies": min(steps, R),
                            "distinct_bytes": min(steps, R) * ab["total"],
                            "read_before_it_bytes": flush.mib << 20}}
    per = {}
    for name in kernels:
        fn = getattr(lay, name)
        per[name] = round(time_graph(lambda k, fn=fn: fn(k % R), steps, warmup, flush) * 1e3, 3)
    rec["kernel_avg_us"] = per
    rec["select_fwd_fused"] = lay.select_fwd_is_fused()
    # the step's form: the selection from the scoring launch's candidate list, and for
    # how many tokens of the last timed step the list decided it (else their rows did)
    rec["select_from_list"] = decided is not None
    if decided is not None:
        rec["tokens_decided_by_list"] = f"{sum(decided)} of {len(decided)}"
    if warm:
        wms = time_graph(lambda k: lay.step(0), steps, warmup)
        rec["warm"] = {"us_per_step": round(wms * 1e3, 3), "value": round(gbs(ab["total"], wms), 2),
                       "unit": "GB/s", "protocol": "every step on the same layer copy, after an untimed replay"}
    return rec


SCORE_KERNEL = ("score_mfma_kernel (pooling variant) as sparse_attn_pool_score launches it; in the step's "
                "sparse_attn_pool_score_select_fwd the same launch also writes the candidate list")


def roofline_block(ab: dict, sec: dict, score_kernel: str, traffic=None) -> dict:
    """Roofline of the scoring launch (the step's dominant byte stream), with the whole
    step's and the attention call's fractions beside it."""
    us = sec["kernel_avg_us"]["pool_score"]
    achieved = gbs(ab["pooled"], us * 1e-3)
    r = {"bound": "hbm", "kernel": score_kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
         "bytes_per_launch": ab["pooled"], "avg_launch_us": us,
         "step_share": round(us / sec["us_per_step"], 3),
         "step": {"achieved": sec["value"], "frac": sec["frac_of_hbm_peak"], "bytes": ab["total"],
                  "us": sec["us_per_step"]}}
    if "fwd" in sec["kernel_avg_us"]:
        fus = sec["kernel_avg_us"]["fwd"]
        fa = gbs(ab["gathered"], fus * 1e-3)
        r["attention"] = {"kernels": "attention + split combine (sparse_attn_fwd)", "bytes_per_call": ab["gathered"],
                          "avg_call_us": fus, "achieved": round(fa, 1), "frac": round(fa / HBM_PEAK_GBS, 4)}
    if "select_fwd" in sec["kernel_avg_us"]:
        sus = sec["kernel_avg_us"]["select_fwd"]
        sb = ab["gathered"]
        fa = gbs(sb, sus * 1e-3)
        r["select_attention"] = {
            "kernels": ("selection + attention in one launch, then the split combine (sparse_attn_select_fwd)"
                        if sec.get("select_fwd_fused") else "sparse_attn_select then sparse_attn_fwd "
                                                            "(sparse_attn_select_fwd, unfused form)"),
            "bytes_per_call": sb, "avg_call_us": sus, "achieved": round(fa, 1), "frac": round(fa / HBM_PEAK_GBS, 4)}
    return r


# ------------------------------------------------------------ MFMA peak (probe)

def measured_mfma_peak() -> dict:
    """The dense bf16 rate of a plain loop of v_mfma_f32_32x32x16_bf16 chains
    (libsa_probe.so), beside the vendor's figure."""
    import ctypes

    path = os.path.join(ROOT, "indexer_top_block_amd", "libsa_probe.so")
    lib = ctypes.CDLL(path)
    lib.sa_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.sa_probe_mfma_bf16.restype = ctypes.c_int
    lib.sa_probe_mfma_bf16_flop.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.sa_probe_mfma_bf16_flop.restype = ctypes.c_double
    n_wg, iters = 2048, 4096
    ab = (torch.randn(128 * 8, device="cuda") * 0.01).to(torch.bfloat16)
    out = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        assert lib.sa_probe_mfma_bf16(n_wg, iters, ab.data_ptr(), out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    start.record()
    for _ in range(reps):
        lib.sa_probe_mfma_bf16(n_wg, iters, ab.data_ptr(), out.data_ptr(), stream)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    tf = lib.sa_probe_mfma_bf16_flop(n_wg, iters) / (ms * 1e-3) / 1e12
    return {"vendor_tflops": MFMA_BF16_PEAK_TFLOPS, "measured_tflops": round(tf, 1),
            "measured_with": f"{n_wg} workgroups x 4 waves x {iters} rounds of 8 independent "
                             "v_mfma_f32_32x32x16_bf16, no memory traffic"}


# -------------------------------------------------------------------- CPU oracle

def cpu_baseline(case: datagen.Case, seconds: float, bytes_per_step: int) -> dict:
    """The oracle's decode step on the host: re-pool the newest block, score every
    block against the resident pooled keys, select, attend -- repeated for about
    `seconds` of wall time."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([int(x.get("num_threads", 1)) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    d = case.dims
    c = d.compress_ratio
    L = int(case.seq_len[0])
    n_vis = min(L, int(case.q_pos[0]) + 1)
    nb = n_vis // c
    pooled = oracle.pool_blocks(case.kidx[:L], c, d.dtype)           # resident state, untimed
    k_rows = case.k
    v_rows = case.v_rows()

    def one_step():
        newest = oracle.pool_blocks(case.kidx[(nb - 1) * c: nb * c], c, d.dtype)
        pooled[nb - 1] = newest[0]
        scores = oracle.block_scores(case.qidx[0], pooled[:nb])
        pos = oracle.select_positions(scores.astype(np.float32), n_vis, c, d.top_k)
        return oracle.attend(case.q[0], k_rows[pos], v_rows[pos], case.scale)

    one_step()
    n = 0
    t0 = time.perf_counter()
    while True:
        one_step()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 10000:
            break
    per = el / n
    return {"value": round(bytes_per_step / per / 1e9, 4), "unit": "GB/s", "cores": blas_threads,
            "kind": "oracle", "sample": f"{n} full decode steps of the same workload (1 query), "
                                        f"{per * 1e3:.1f} ms/step, numpy fp64",
            "ms_per_step": round(per * 1e3, 3)}


def measured_hbm_read() -> dict:
    """The read bandwidth a plain streaming kernel and a gather of random 1 KiB rows
    get from HBM on this chip (libsa_probe.so), beside the 8 TB/s peak: the ceilings
    the byte-bound kernels are compared with.  Each figure is the best of 5 cold runs
    (a 1 GiB read between them), timed with events around one eager launch."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "indexer_top_block_amd", "libsa_probe.so"))
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    lib.sa_probe_stream_read.argtypes = [P, I64, ctypes.c_int, P, P]
    lib.sa_probe_stream_read.restype = ctypes.c_int
    lib.sa_probe_gather_read.argtypes = [P, P, I64, ctypes.c_int, P, P]
    lib.sa_probe_gather_read.restype = ctypes.c_int
    stream = torch.cuda.current_stream().cuda_stream
    src_bytes = 2 << 30
    src = torch.ones(src_bytes // 4, dtype=torch.int32, device="cuda")
    out = torch.empty(8192 * 256, dtype=torch.int32, device="cuda")
    flush = Flusher(1024)

    def best(fn, nbytes):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(5):
            flush()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return round(nbytes / (min(ms) * 1e-3) / 1e9, 1)

    res = {"peak_gbs": HBM_PEAK_GBS}
    for mib in (64, 2048):
        nb = mib << 20
        res[f"stream_{mib}MiB_gbs"] = best(lambda nb=nb: lib.sa_probe_stream_read(src.data_ptr(), nb, 8192,
                                                                                  out.data_ptr(), stream), nb)
    rows = torch.from_numpy(np.random.default_rng(0).integers(0, src_bytes // 1024, 131072).astype(np.int32)).cuda()
    res["gather_1KiB_rows_128MiB_gbs"] = best(lambda: lib.sa_probe_gather_read(src.data_ptr(), rows.data_ptr(), 131072,
                                                                               1024, out.data_ptr(), stream),
                                              131072 * 1024)
    res["measured_with"] = ("a grid-stride kernel of 16-byte loads (8192 workgroups of 256 threads); one wave per "
                            "random 1 KiB row, 1024 workgroups")
    del src, out, flush
    torch.cuda.empty_cache()
    return res


def measured_latency() -> dict:
    """Floors of a chain of small kernels on this chip (libsa_probe.so), each a graph
    of 32 back-to-back launches replayed cold: an empty kernel, and one thread per
    workgroup following 1, 2 or 4 dependent loads through a 1 GiB table of random
    indices (each load a cache miss)."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "indexer_top_block_amd", "libsa_probe.so"))
    P = ctypes.c_void_p
    lib.sa_probe_empty.argtypes = [ctypes.c_int, P]
    lib.sa_probe_empty.restype = ctypes.c_int
    lib.sa_probe_chain.argtypes = [P, P, ctypes.c_int, ctypes.c_int, P, P]
    lib.sa_probe_chain.restype = ctypes.c_int
    n = 1 << 28                                   # 1 GiB of int32 indices
    rng = np.random.default_rng(1)
    nxt = torch.randint(0, n, (n,), dtype=torch.int32, device="cuda")
    starts = [torch.from_numpy(rng.integers(0, n, 256).astype(np.int32)).cuda() for _ in range(32)]
    out = torch.empty(256, dtype=torch.int32, device="cuda")
    flush = Flusher(1024)

    def per_launch_us(call):
        return round(time_graph(lambda k: call(k), 32, 2, flush) * 1e3, 3)

    res = {"empty_kernel_us": per_launch_us(lambda k: lib.sa_probe_empty(256, torch.cuda.current_stream().cuda_stream))}
    for hops in (1, 2, 4):
        res[f"dependent_loads_{hops}_us"] = per_launch_us(
            lambda k, h=hops: lib.sa_probe_chain(nxt.data_ptr(), starts[k % 32].data_ptr(), h, 256, out.data_ptr(),
                                                 torch.cuda.current_stream().cuda_stream))
    res["measured_with"] = ("graph replays of 32 launches after a 1 GiB read; 256 workgroups; chains through a "
                            "1 GiB table of random int32 indices")
    del nxt, out, flush
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------ prefill

def prefill_report(steps: int, mfma_peak: dict) -> dict:
    """Workload 4: 2048 query tokens at depth 32768 -- the chunk's pooling (its 512
    new blocks), scoring, selection and attention; TFLOP/s of the score and the
    attention stages and of the whole chunk, against the dense bf16 MFMA peak (the
    vendor figure and the measured one)."""
    from indexer_top_block_amd.device import DeviceLayer

    case = datagen.make_workload(4)
    lay = DeviceLayer(case)
    d = case.dims
    c = d.compress_ratio
    depth = int(case.q_pos[0])
    # the cache before the chunk holds depth / c pooled blocks; every step pools the
    # chunk's own blocks again from there
    n_before = torch.full_like(lay.n_pooled, depth // c)
    n_after = torch.zeros_like(lay.n_pooled)
    lay.pool()
    torch.cuda.synchronize()
    nb = np.array([min(int(case.seq_len[0]), int(p) + 1) // c for p in case.q_pos], dtype=np.int64)
    idx_flop = 2.0 * d.h_idx * d.d_idx * float(nb.sum())
    lay.score(); lay.select(); torch.cuda.synchronize()
    n_sel = lay.n_sel.cpu().numpy().astype(np.int64)
    att_flop = 2.0 * d.h_q * float(n_sel.sum()) * (d.d_kq + d.d_v)
    pool = lambda k: lay.pool(n_in=n_before, n_out=n_after)
    t_pool = time_eager(pool, steps, 2)
    t_score = time_eager(lambda k: lay.score(), steps, 2)
    t_select = time_eager(lambda k: lay.select(), steps, 2)
    t_fwd = time_eager(lambda k: lay.fwd(), steps, 2)
    t_all = time_eager(lambda k: (pool(k), lay.score(), lay.select(), lay.fwd()), steps, 2)
    tf = lambda flop, ms: flop / (ms * 1e-3) / 1e12
    total = tf(idx_flop + att_flop, t_all)
    return {
        "workload": datagen.WORKLOADS[4],
        "ms_per_step": round(t_all, 4),
        "tflops": round(total, 2),
        "frac_of_mfma_peak": round(total / MFMA_BF16_PEAK_TFLOPS, 4),
        "frac_of_measured_mfma_peak": round(total / mfma_peak["measured_tflops"], 4),
        "gflop": {"indexer": round(idx_flop / 1e9, 2), "attention": round(att_flop / 1e9, 2)},
        "stage_ms": {"pool": round(t_pool, 4), "score": round(t_score, 4), "select": round(t_select, 4),
                     "fwd": round(t_fwd, 4)},
        "stage_tflops": {"score": round(tf(idx_flop, t_score), 2), "fwd": round(tf(att_flop, t_fwd), 2)},
        "stage_frac_of_mfma_peak": {"score": round(tf(idx_flop, t_score) / MFMA_BF16_PEAK_TFLOPS, 4),
                                    "fwd": round(tf(att_flop, t_fwd) / MFMA_BF16_PEAK_TFLOPS, 4)},
        "timing": "eager launches, steps back to back; the chunk's pooling re-pools its 512 blocks each step",
    }


# ------------------------------------------------------------------ mask form

def mask_form_report(lay: "RotatingLayers", steps: int, warmup: int, flush: Flusher) -> dict:
    """The additive-mask form on the 128K decode layer: one f16 mask row of 131072
    columns whose finite entries are the step's selected positions (values -k/32)
    -> index list -> attention with the mask values as bias, per step (cold)."""
    R = lay.n
    lay.step(0)
    torch.cuda.synchronize()
    n_kv = lay.max_len
    n_fin = int(lay.n_sel[0].item())
    pos = lay.sel[0, :n_fin].cpu().numpy()
    mask = np.full((1, n_kv), -np.inf, dtype=np.float32)
    mask[0, pos] = -(1.0 + np.arange(len(pos)) % 7) / 32.0
    dev_mask = torch.from_numpy(mask).to(torch.float16).cuda()
    sel_bias = torch.zeros((1, lay.sel_ld), dtype=torch.float32, device="cuda")

    def m2i(k):
        sa.sparse_attn_mask_to_indices(dev_mask, "f16", n_kv, 1, n_kv, lay.sel, lay.sel_ld, lay.n_sel, sel_bias)

    def fwd_b(k):
        sa.sparse_attn_fwd_bias(lay.dims, lay.caches[k % R], lay.q, lay.q_seq, lay.sel, lay.sel_ld, lay.n_sel,
                                sel_bias, 1, lay.case.scale, lay.out, lay.ws, lay.ws_bytes)

    both = time_graph(lambda k: (m2i(k), fwd_b(k)), steps, warmup, flush)
    t_m2i = time_graph(m2i, steps, warmup, flush)
    t_fwd = time_graph(fwd_b, steps, warmup, flush)
    return {"workload": f"one 131072-column f16 mask row over the 128K decode layer, {n_fin} finite entries",
            "us_per_step": round(both * 1e3, 3),
            "kernel_avg_us": {"mask_to_indices": round(t_m2i * 1e3, 3), "fwd_bias": round(t_fwd * 1e3, 3)},
            "mask_bytes": n_kv * 2}


# ------------------------------------------------------------------ dense window

def window_report(lay: "RotatingLayers", steps: int, warmup: int, flush: Flusher, window: int = 128) -> dict:
    """The decode step with the attention taken over the selected rows together with
    the `window` most recent positions (dense window + selection, merged in one pass;
    the window size is not fixed by the method's description, 128 is an example)."""
    R = lay.n
    ws_bytes = sa.sparse_attn_workspace_bytes_window(lay.dims, lay.n_q, lay.max_len, window)
    ws = torch.zeros((max(ws_bytes, 16),), dtype=torch.uint8, device=lay.device)

    def fwd_w(k):
        sa.sparse_attn_fwd_window(lay.dims, lay.caches[k % R], lay.q, lay.q_seq, lay.q_pos, lay.sel, lay.sel_ld,
                                  lay.n_sel, window, lay.n_q, lay.case.scale, lay.out, ws, ws_bytes)

    def select_w(k):
        sa.sparse_attn_select(lay.dims, lay.caches[k % R], lay.scores, lay.scores_ld, lay.q_seq, lay.q_pos,
                              lay.n_q, lay.sel, lay.sel_ld, lay.n_sel, ws, ws_bytes)

    def step_w(k):
        lay.pool_score(k % R)
        select_w(k)
        fwd_w(k)

    ms = time_graph(step_w, steps, warmup, flush)
    t_fwd = time_graph(fwd_w, steps, warmup, flush)
    return {"workload": f"the 128K decode step with a dense window of the {window} most recent positions",
            "window": window, "us_per_step": round(ms * 1e3, 3), "kernel_avg_us": {"fwd_window": round(t_fwd * 1e3, 3)}}


# ------------------------------------------------------------------ q8_0 cache

def q8_report(lay: "RotatingLayers", steps: int, warmup: int, flush: Flusher) -> dict:
    """The 128K decode step over q8_0 copies of the layer's K/V cache (quantized once on
    the GPU from the bf16 copies): pool, score, select, attention over the q8_0 rows."""
    d = lay.case.dims
    R = lay.n
    rows = lay.case.rows
    nb = d.d_kq // 32
    codes = torch.empty((R, rows, d.d_kq), dtype=torch.int8, device=lay.device)
    scales = torch.empty((R, rows, nb), dtype=torch.float16, device=lay.device)
    for r in range(R):
        sa.sparse_attn_quantize_q8_0(lay.k[r], d.dtype, rows, d.d_kq, d.d_kq, codes[r], d.d_kq, scales[r], nb)
    kvs = [sa.KvQ8(k=codes[r], k_ld=d.d_kq, k_head_stride=d.d_kq, k_scale=scales[r], k_scale_ld=nb,
                   k_scale_head_stride=nb, v=codes[r], v_ld=d.d_kq, v_head_stride=d.d_kq, v_scale=scales[r],
                   v_scale_ld=nb, v_scale_head_stride=nb) for r in range(R)]
    torch.cuda.synchronize()

    def fwd_q(k):
        sa.sparse_attn_fwd_q8_0(lay.dims, lay.caches[k % R], kvs[k % R], lay.q, lay.q_seq, lay.sel, lay.sel_ld,
                                lay.n_sel, lay.n_q, lay.case.scale, lay.out, lay.ws, lay.ws_bytes)

    def step_q(k):
        lay.pool_score(k % R)
        lay.select(k % R)
        fwd_q(k)

    new_row = lay.k[0, rows - 1:rows]

    def write_row(k):                            # the cache write of one new token (18 blocks)
        sa.sparse_attn_quantize_q8_0(new_row, d.dtype, 1, d.d_kq, d.d_kq, codes[k % R, rows - 1:rows], d.d_kq,
                                     scales[k % R, rows - 1:rows], nb)

    ms = time_graph(step_q, steps, warmup, flush)
    t_fwd = time_graph(fwd_q, steps, warmup, flush)
    t_w = time_graph(write_row, steps, warmup, flush)
    ab = algorithmic_bytes(lay.case, kv="q8_0")
    del kvs, codes, scales
    torch.cuda.empty_cache()
    return {"workload": "the 128K decode step over a q8_0 K/V cache (V = K[:512])", "us_per_step": round(ms * 1e3, 3),
            "value": round(gbs(ab["total"], ms), 2), "unit": "GB/s", "bytes_per_step": ab,
            "kernel_avg_us": {"fwd_q8_0": round(t_fwd * 1e3, 3), "quantize_one_row": round(t_w * 1e3, 3)}}


# ------------------------------------------------- other decode workloads

def workload_decode_report(cfg: int, steps: int, warmup: int, layers: int, flush: Flusher) -> dict:
    """A whole decode step of workload `cfg` (the token-level, the 1M-context or the
    batched 32-sequence decode) under the cold protocol, its entry points alone, and
    the roofline of its scoring launch and its attention."""
    log(f"[bench] generating workload {cfg}")
    case = datagen.make_workload(cfg)
    ab = algorithmic_bytes(case)
    lay = RotatingLayers(case, layers)
    lay.fill_pools()
    torch.cuda.synchronize()
    log(f"[bench] workload {cfg}: {layers} copies resident; timing")
    sec = decode_section(lay, ab, steps, warmup, flush, warm=True)
    sec["workload"] = datagen.WORKLOADS[cfg]
    sec["layers_rotated"] = layers
    sec["roofline"] = roofline_block(ab, sec, SCORE_KERNEL)
    del lay
    torch.cuda.empty_cache()
    return sec


# --------------------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=64, help="copies of the layer's caches the steps cycle through")
    ap.add_argument("--flush-mib", type=int, default=1024, help="MiB read between the untimed and the timed replay")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-token-level", action="store_true")
    ap.add_argument("--no-long", action="store_true", help="skip the 1M-context decode")
    ap.add_argument("--no-batched", action="store_true", help="skip the batched 32-sequence decode")
    ap.add_argument("--no-forms", action="store_true", help="skip the mask, window and q8_0 sections")
    ap.add_argument("--eager", action="store_true", help="launch every step from the host (no graph)")
    ap.add_argument("--workload", type=int, choices=[2, 3, 5, 6], default=2,
                    help="decode workload of --only")
    ap.add_argument("--only", choices=["pool_score", "pool", "score", "select", "fwd", "select_fwd", "step",
                                       "two_calls", "prefill_score", "prefill_fwd"], default=None,
                    help="run just this call for --steps launches over the rotated copies of --workload, or one "
                         "stage of the prefill chunk (counter collection)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--traffic-file", default=os.path.join(ROOT, "profiles", "score_mfma_kernel_decode128k_traffic.txt"),
                    help="HBM bytes per launch of the score kernel from FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; the path runs on one MI355X and has no "
                                   "multi-GPU mode (a sequence- or query-sharded layout is described in the design "
                                   "notes)", "n_gpus": args.gpus}))
        return 2
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 2
    torch.cuda.set_device(0)
    sa.load()

    if args.copy_probe_mb:
        n = args.copy_probe_mb * 1024 * 1024 // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)             # one elementwise kernel: reads and writes the size once
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {args.copy_probe_mb} MiB read + written by one elementwise kernel")
        del src, dst

    if args.only in ("prefill_score", "prefill_fwd"):
        from indexer_top_block_amd.device import DeviceLayer

        log(f"[bench] --only {args.only}: generating workload 4")
        lay = DeviceLayer(datagen.make_workload(4))
        lay.pool(); lay.score(); lay.select()
        torch.cuda.synchronize()
        fn = lay.score if args.only == "prefill_score" else lay.fwd
        ms = time_eager(lambda k: fn(), args.steps, args.warmup)
        print(json.dumps({"only": args.only, "workload": 4, "launches": args.steps, "ms_per_launch": ms}))
        return 0
    if args.only:
        cfg = args.workload
        layers = args.layers if cfg in (2, 6) else {5: 8, 3: 4}[cfg]
        log(f"[bench] --only {args.only}: generating workload {cfg}")
        case = datagen.make_workload(cfg)
        lay = RotatingLayers(case, layers)
        lay.fill_pools()
        lay.step(0)                              # a real selection for select / fwd (same on every copy)
        torch.cuda.synchronize()
        fn = getattr(lay, args.only)
        ms = time_eager(lambda k: fn(k % layers), args.steps, args.warmup)
        print(json.dumps({"only": args.only, "workload": cfg, "launches": args.steps, "ms_per_launch": ms}))
        return 0

    flush = Flusher(args.flush_mib)
    log("[bench] generating workload 2")
    case = datagen.make_workload(2)
    ab = algorithmic_bytes(case)
    lay = RotatingLayers(case, args.layers)
    lay.fill_pools()
    torch.cuda.synchronize()
    R = args.layers
    log(f"[bench] {R} layer copies resident; algorithmic bytes/step {ab}")

    log("[bench] timing the 128K decode step (cold and warm)")
    if args.eager:
        ms = time_eager(lambda k: lay.step(k % R), args.steps, args.warmup)
        sec = {"us_per_step": round(ms * 1e3, 3), "value": round(gbs(ab["total"], ms), 2),
               "frac_of_hbm_peak": round(gbs(ab["total"], ms) / HBM_PEAK_GBS, 4),
               "kernel_avg_us": {n: round(time_eager(lambda k, fn=getattr(lay, n): fn(k % R), args.steps,
                                                     args.warmup) * 1e3, 3)
                                 for n in ("pool_score", "pool", "score", "select", "fwd", "select_fwd",
                                           "two_calls")}}
    else:
        sec = decode_section(lay, ab, args.steps, args.warmup, flush,
                             kernels=("pool_score", "pool", "score", "select_fwd", "two_calls", "select", "fwd"))
    ms = sec["us_per_step"] * 1e-3
    log(f"[bench] step {sec['us_per_step']:.2f} us (cold); per-call us {sec['kernel_avg_us']}; "
        f"warm {sec.get('warm', {}).get('us_per_step')}")
    # The roofline is taken on the scoring kernel with the newest block pooled inside,
    # timed as sparse_attn_pool_score launches it (one kernel launch streaming the
    # pooled indexer keys -- most of the step's algorithmic bytes).  Inside the step
    # (sparse_attn_pool_score_select_fwd) the same kernel also writes the candidate
    # list, which the per-call figure of the step's own launches includes.
    roofline = roofline_block(ab, sec, SCORE_KERNEL, traffic_from_counters(args.traffic_file))

    rec = {
        "metric": METRIC, "value": sec["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "us_per_step": sec["us_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "dsv4_decode_128k_bf16: 1 decode token, ctx 131072, 16 q heads on 1 latent KV "
                               "head (DKQ 576 / DV 512, V = K[:512]), indexer 64x128, compress_ratio 4, "
                               "top_k 2048",
                   "layers_rotated": R, "graph": not args.eager, "bytes_per_step": ab},
        "protocol": ("cold: step k on layer copy k mod layers; a 1 GiB read between the untimed and the timed "
                     "replay; the timed replay is exactly `steps` steps"),
        "timed_region": sec.get("timed_region"),
        "warm": sec.get("warm"),
        "kernel_avg_us": sec["kernel_avg_us"],
        "select_from_list": sec.get("select_from_list"),
        "tokens_decided_by_list": sec.get("tokens_decided_by_list"),
        "roofline": roofline,
    }
    if not args.no_forms:
        log("[bench] mask form")
        rec["mask_form"] = mask_form_report(lay, args.steps, args.warmup, flush)
        log("[bench] dense window + selection")
        rec["window"] = window_report(lay, args.steps, args.warmup, flush)
        log("[bench] q8_0 cache")
        rec["q8_0"] = q8_report(lay, args.steps, args.warmup, flush)
    del lay
    torch.cuda.empty_cache()
    log("[bench] MFMA peak and HBM read probes")
    peak = measured_mfma_peak()
    rec["mfma_bf16_peak"] = peak
    rec["hbm_read_measured"] = measured_hbm_read()
    rec["latency_measured"] = measured_latency()
    if not args.no_prefill:
        log("[bench] prefill workload")
        rec["prefill"] = prefill_report(max(5, min(args.steps, 20)), peak)
    if not args.no_token_level:
        rec["token_level"] = workload_decode_report(6, args.steps, args.warmup, min(args.layers, 32), flush)
    if not args.no_long:
        rec["long_decode_1m"] = workload_decode_report(5, args.steps, args.warmup, 8, flush)
    if not args.no_batched:
        rec["batched_decode"] = workload_decode_report(3, args.steps, args.warmup, 4, flush)
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        rec["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds, ab["total"])
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
