"""Attention cases with a wide spread of logits, shared by the GPU parity tests
(tests/test_gpu_parity.py) and the CPU calibration of the output comparison
(tests/test_parity_calibration.py).

With every tensor drawn N(0, 1/dim), as the workloads are, the logits of the MLA
shapes have a standard deviation of 1/576 and the softmax is uniform to 0.2%: an
attention kernel that ignored Q.K^T entirely would still match.  These cases draw
the attention queries wider, so that scale * q . k has a standard deviation of
LOGIT_STD while K and V keep their workload distributions, which makes the weights
peaked but spread over many rows.  The calibration test shows that the comparison
rejects wrong kernels (uniform weights, no scale, dropped dims, wrong head, a
dropped tile of rows, a window off by one, a dropped or rescaled bias) at exactly
these cases.

Each case names the kernel and launch form it is meant for.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Optional

import numpy as np

from indexer_top_block_amd import datagen

LOGIT_STD = 2.0


def q_std_for(dims: datagen.Dims, k_std: float, scale: float, logit_std: float = LOGIT_STD) -> float:
    """Query standard deviation giving scale * q . k a standard deviation of logit_std
    for K entries of standard deviation k_std (independent, zero-mean)."""
    return logit_std / (scale * math.sqrt(dims.d_kq) * k_std)


@dataclasses.dataclass
class AttnCase:
    name: str
    kernel: str                       # which kernel and launch form the case is for
    make: Callable[[], datagen.Case]
    queries: Optional[list] = None    # the queries checked (None: all)
    windows: tuple = ()               # dense-window sizes (window form)
    q8: bool = False                  # q8_0 K/V cache


def _mla(d_kq: int, dtype: str, top_k: int = 2048) -> datagen.Dims:
    return datagen.Dims(h_q=16, h_kv=1, d_kq=d_kq, d_v=512, h_idx=64, d_idx=128, compress_ratio=4, top_k=top_k,
                        dtype=dtype)


def _spread_case(name, dims, lens, q_seq, q_pos, case_id):
    scale = 1.0 / math.sqrt(dims.d_kq)
    k_std = 1.0 / math.sqrt(dims.d_kq)
    return datagen.make_case(name, dims, lens, q_seq, q_pos, seed=0, case_id=case_id, std="inv_sqrt_dim",
                             v_separate=False, scale=scale, q_std=q_std_for(dims, k_std, scale))


def decode_128k() -> datagen.Case:
    """Workload 2 (one decode token at 128K, 576/512, V = K[:512]) with wide logits:
    fwd_lds_kernel with the query block through LDS, 33 splits and the combine."""
    dims = datagen.workload_dims(2)
    scale = 1.0 / math.sqrt(576)
    return datagen.make_workload(2, q_std=q_std_for(dims, 1.0 / math.sqrt(576), scale))


def decode_512_alias() -> datagen.Case:
    """512/512 with V = K (f16): one decode token at 40000 plus a short one."""
    return _spread_case("spread_decode_512", _mla(512, "f16"), [40000, 3000], [0, 1], [40000, 2999], 701)


def prefill_576() -> datagen.Case:
    """520 query tokens of one sequence, 576/512 bf16: one workgroup per token (no
    split), 33 row tiles each, the register query operand."""
    n_q = 520
    pos = list(range(5999, 5999 - 7 * n_q, -7))
    return _spread_case("spread_prefill_576", _mla(576, "bf16"), [6000], [0] * n_q, pos, 702)


def prefill_512_alias() -> datagen.Case:
    n_q = 520
    pos = list(range(4999, 4999 - 5 * n_q, -5))
    return _spread_case("spread_prefill_512", _mla(512, "f16"), [5000], [0] * n_q, pos, 703)


def window_mla() -> datagen.Case:
    """Short contexts and a small budget, so that every attended row carries weight."""
    dims = _mla(576, "bf16", top_k=64)
    lens = [3000, 300]
    q_seq = [0, 0, 0, 1, 1]
    q_pos = [2999, 900, 70, 299, 40]
    return _spread_case("spread_window_mla", dims, lens, q_seq, q_pos, 704)


def bias_mla() -> datagen.Case:
    """The mask form's MLA shape (c = 1, the list is the mask's finite entries)."""
    dims = datagen.Dims(h_q=16, h_kv=1, d_kq=576, d_v=512, h_idx=32, d_idx=128, compress_ratio=1, top_k=2048,
                        dtype="bf16")
    n_kv, n_q = 4096, 6
    return _spread_case("spread_bias_mla", dims, [n_kv], [0] * n_q, [n_kv - 1] * n_q, 705)


def q8_decode_128k() -> datagen.Case:
    return decode_128k()


def q8_prefill_512() -> datagen.Case:
    n_q = 600
    pos = list(range(4999, 4999 - 6 * n_q, -6))
    return _spread_case("spread_q8_prefill_512", _mla(512, "f16"), [5000], [0] * n_q, pos, 706)


PREFILL_SAMPLE = [0, 1, 2, 63, 64, 200, 259, 260, 399, 519]

CASES = {
    "decode_128k": AttnCase("decode_128k", "fwd_lds_kernel<bf16,576,QLDS>, 33 splits + combine", decode_128k),
    "decode_512_alias": AttnCase("decode_512_alias", "fwd_lds_kernel<f16,512,QLDS>, split + combine",
                                 decode_512_alias),
    "prefill_576": AttnCase("prefill_576", "fwd_lds_kernel<bf16,576>, unsplit", prefill_576, PREFILL_SAMPLE),
    "prefill_512_alias": AttnCase("prefill_512_alias", "fwd_lds_kernel<f16,512>, unsplit", prefill_512_alias,
                                  PREFILL_SAMPLE),
    "window_mla": AttnCase("window_mla", "fwd_lds_kernel<bf16,576> with a dense window", window_mla,
                           windows=(1, 17, 64, 200)),
    "bias_mla": AttnCase("bias_mla", "fwd_lds_kernel<bf16,576> with a bias per entry (mask form)", bias_mla),
    "q8_decode_128k": AttnCase("q8_decode_128k", "fwd_q8_lds_kernel<bf16,576>, split + combine", q8_decode_128k,
                               q8=True),
    "q8_prefill_512": AttnCase("q8_prefill_512", "fwd_q8_lds_kernel<f16,512>, unsplit", q8_prefill_512,
                               [0, 1, 100, 333, 599], q8=True),
}


def bias_mask(case: datagen.Case) -> np.ndarray:
    """[n_q, L] float32 mask of the bias case, f16 values: each row keeps a seeded set
    of columns (different sizes, one with more than the list holds is avoided) with
    values spread over [-4, 1], so that the bias moves the weights as much as the
    logits do; -inf elsewhere."""
    L = int(case.seq_len[0])
    rng = np.random.default_rng([0, 705, 9])
    m = np.full((case.n_q, L), -np.inf, dtype=np.float32)
    for r in range(case.n_q):
        cnt = [2048, 2047, 1000, 300, 64, 1][r]
        cols = rng.choice(L, size=cnt, replace=False)
        m[r, cols] = rng.uniform(-4.0, 1.0, size=cnt)
    return datagen.round_to_dtype(m, "f16")
