"""Causal prefill attention at arbitrary query positions (CPU, fp64).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only tests, the
smoke check and the benchmark's CPU leg use it; the HIP library never does.

Pages: the write-up's core formula (核心公式) gives the attention each query
row computes, p = softmax(K q / sqrt(d)) and a = sum_j p_j v_j, with causal
visibility (代码映射与边界: causal tail alignment); the atlas summary
(Experimental setup) says the paper's scorer builds on FlashAttention-2, and
the paper's abstract (fugumt page) describes fused kernels that never
materialise the attention matrix. A prefill attention pass computes exactly
this output for every position of the sequence; its last `window` rows are
the observation window whose statistics (largest logit, rest mass, argmax,
output) the scorer needs, so such a pass can hand them over.

The reading used here: query row (h, pos) of head h at position pos sees keys
0..pos of KV head h // G (contiguous GQA groups), as for the window rows.
"""

from __future__ import annotations

import math
from typing import Iterable, Tuple

import numpy as np

from .dropkv_oracle import as_f64


def prefill_outputs(q_all, k, v, rows: Iterable[Tuple[int, int]], *, Hq: int, Hkv: int,
                    dtype: str = "f64") -> np.ndarray:
    """Attention outputs o(h, pos) = sum_{j <= pos} p_j v_j with p = softmax over keys 0..pos
    of q(h, pos) . k_j / sqrt(d), for each (h, pos) in `rows`; q_all [Hq][n][d], k/v [Hkv][n][d].
    Returns [len(rows)][d] float64."""
    G = Hq // Hkv
    qf, kf, vf = as_f64(q_all, dtype), as_f64(k, dtype), as_f64(v, dtype)
    d = qf.shape[2]
    rows = list(rows)
    out = np.empty((len(rows), d))
    for r, (h, pos) in enumerate(rows):
        g = h // G
        x = kf[g, : pos + 1] @ qf[h, pos] / math.sqrt(d)
        e = np.exp(x - np.max(x))
        out[r] = (e / e.sum()) @ vf[g, : pos + 1]
    return out
