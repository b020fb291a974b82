"""FP8 (E4M3) weights: the second weight format of the pages' checkpoints,
written as a plain definition in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed
----------------
The pages' checkpoints carry FP8 E4M3 next to NVFP4: NVIDIA's 27B export
keeps every linear-attention and self-attention projection in FP8
(dgx-spark-qwen38 README, the paragraph on NVIDIA's own 27B NVFP4 export),
and TandemLLM serves an FP8 (e4m3) output head (TandemLLM README, "The
parts").  A weight is then one E4M3 byte per element, W8[N][K], and

    Y[m, n] = sum_k  x[m, k] * w[n, k],     w[n, k] = g * r[n] * E4M3(W8[n, k])

with an fp32 tensor scale g and an optional fp32 scale r[n] per output row
(absent: r = 1).  Reading taken (the pages name the format, not its scale
layout): per-tensor and per-row scales, no block scales.

Exactness: E4M3 values have 4 significant bits and bf16 activations 8, so
x * E4M3 is exact; the scale product g * r[n] (each fp32) is formed in
fp64 and the whole product rounds at most once (relative 2**-53), far
below the acceptance bound; then only the K-summation rounds.
"""
from __future__ import annotations

import numpy as np

from .nvfp4 import bf16_bits_to_f64, e4m3_table, tolerance_bound

_E4M3 = e4m3_table()


def fp8_dequant(w8: np.ndarray, row_scale: np.ndarray | None, g: float) -> np.ndarray:
    """float64[N][K] weights g * r[n] * E4M3(w8[n, k])."""
    w8 = np.asarray(w8, dtype=np.uint8)
    s = np.float64(np.float32(g))
    if row_scale is None:
        return s * _E4M3[w8]
    r = np.asarray(row_scale, dtype=np.float32).astype(np.float64)
    if r.shape != (w8.shape[0],):
        raise ValueError("row_scale must have one entry per row")
    return (s * r)[:, None] * _E4M3[w8]


def fp8_gemm_ref(x_bits: np.ndarray, w8: np.ndarray, row_scale: np.ndarray | None, g: float,
                 *, row_chunk: int = 4096):
    """Y[M][N] = X . W^T in fp64 and the acceptance bound
    B = 1e-3 * sum_k |x w| + 1e-6."""
    x = bf16_bits_to_f64(x_bits)
    w8 = np.asarray(w8, dtype=np.uint8)
    n = w8.shape[0]
    y = np.empty((x.shape[0], n))
    b = np.empty((x.shape[0], n))
    ax = np.abs(x)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        w = fp8_dequant(w8[r0:r1], None if row_scale is None else np.asarray(row_scale)[r0:r1], g)
        y[:, r0:r1] = x @ w.T
        b[:, r0:r1] = tolerance_bound(ax @ np.abs(w).T)
    return y, b
