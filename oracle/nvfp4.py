"""NVFP4 format and the skinny GEMM, written as plain definitions in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed
----------------
A weight matrix W[N][K] is held block-scaled in 4 bits: an E2M1 code per
element, one E4M3 scale per 16 consecutive K-elements of a row, and one
fp32 tensor scale g.  The weight pass computes

    Y[m, n] = sum_k  x[m, k] * w[n, k],     w[n, k] = g * s[n, k // 16] * e[n, k]

for a skinny X (M = 1, 17, up to 68 rows).  The pages call this format
"NVFP4 group-16" (dgx-spark-qwen38 README, "The seven targets": the
quantisation map puts the 64 MLP triplets and the lm_head in NVFP4 with
group size 16); TandemLLM README ("Architecture: the parts") serves every
projection in NVFP4.  The pages do not spell out the bit formats; E2M1 and
E4M3 are the OCP microscaling FP4 and FP8 ("fn": no infinities) element
formats, decoded here from their published field layouts.

Readings taken where the pages are silent (each pinned by a test):
  * element 2j of a row is the LOW nibble of packed byte j;
  * scales are row-major [N][K/16], unswizzled;
  * E4M3 sign bits are honoured; 0x7F / 0xFF decode to NaN (out of contract);
  * g multiplies every dequantised weight.

Exactness: x (bf16, 8 significant bits) * s (E4M3, 4 bits) * e (E2M1,
2 bits) * g (fp32, 24 bits) has at most 38 significant bits, so every
product below is exact in fp64; only the K-summation rounds.
"""
from __future__ import annotations

import math

import numpy as np

# Acceptance bound constants: |y - y_ref| <= REL * sum_k |x_k w_k| + ABS.
BOUND_REL = 1e-3
BOUND_ABS = 1e-6


# --------------------------------------------------------------------------
# Element formats (closed forms from the field layouts)
# --------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    """Decode one 4-bit E2M1 code: 1 sign, 2 exponent (bias 1), 1 mantissa bit.

    exponent field 0 is subnormal: value = 0.5 * m; otherwise
    value = 2**(e - 1) * (1 + m / 2).
    """
    if not 0 <= code <= 15:
        raise ValueError("E2M1 code out of range")
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    mag = 0.5 * m if e == 0 else math.ldexp(1.0 + m / 2.0, e - 1)
    return sign * mag


def e2m1_table() -> np.ndarray:
    """All 16 E2M1 codes decoded, float64[16]."""
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e4m3_value(b: int) -> float:
    """Decode one E4M3 byte (OCP FP8 'fn' variant): 1 sign, 4 exponent
    (bias 7), 3 mantissa bits; no infinities; exponent 15 with mantissa 7
    is NaN; exponent 0 is subnormal (2**-6 * m / 8)."""
    if not 0 <= b <= 255:
        raise ValueError("E4M3 byte out of range")
    sign = -1.0 if (b >> 7) & 1 else 1.0
    e = (b >> 3) & 15
    m = b & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * math.ldexp(m / 8.0, -6)
    return sign * math.ldexp(1.0 + m / 8.0, e - 7)


def e4m3_table() -> np.ndarray:
    """All 256 E4M3 bytes decoded, float64[256] (NaN at 0x7F and 0xFF)."""
    return np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)


_E2M1 = e2m1_table()
_E4M3 = e4m3_table()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an IEEE binary32: widen the bit pattern to
    32 bits and reinterpret.  Exact."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):        # NaN patterns stay NaN
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Unpack and dequantise
# --------------------------------------------------------------------------
def unpack_codes(wq: np.ndarray) -> np.ndarray:
    """uint8[N][K/2] packed codes -> uint8[N][K] codes.

    Element 2j is the low nibble of byte j, element 2j+1 the high nibble."""
    wq = np.asarray(wq, dtype=np.uint8)
    n, kb = wq.shape
    codes = np.empty((n, 2 * kb), dtype=np.uint8)
    codes[:, 0::2] = wq & 0x0F
    codes[:, 1::2] = wq >> 4
    return codes


def dequant(wq: np.ndarray, ws: np.ndarray, g: float) -> np.ndarray:
    """float64[N][K] weights w[n,k] = g * E4M3(ws[n, k//16]) * E2M1(code(n,k))."""
    codes = unpack_codes(wq)
    n, k = codes.shape
    ws = np.asarray(ws, dtype=np.uint8)
    if ws.shape != (n, k // 16) or k % 16:
        raise ValueError(f"scale shape {ws.shape} does not match codes {codes.shape}")
    e = _E2M1[codes]                                   # [N][K]
    s = np.repeat(_E4M3[ws], 16, axis=1)               # [N][K], block k//16
    return np.float64(np.float32(g)) * s * e


def tolerance_bound(abs_sum: np.ndarray) -> np.ndarray:
    """The acceptance bound for an output whose sum_k |x_k w_k| is abs_sum."""
    return BOUND_REL * abs_sum + BOUND_ABS


# --------------------------------------------------------------------------
# The GEMM
# --------------------------------------------------------------------------
def nvfp4_gemm_ref(x_bits: np.ndarray, wq: np.ndarray, ws: np.ndarray, g: float,
                   *, with_bound: bool = True, row_chunk: int = 4096):
    """Y[M][N] = X . dequant(W)^T in fp64, and the acceptance bound B[M][N].

    x_bits: uint16[M][K] bf16 bit patterns.  wq: uint8[N][K/2].  ws: uint8[N][K/16].
    Returns (Y, B) as float64 arrays (B is None when with_bound is False).
    W is dequantised ``row_chunk`` rows at a time only to bound memory; the
    arithmetic per output is the plain K-sum.
    """
    x = bf16_bits_to_f64(x_bits)
    m, k = x.shape
    wq = np.asarray(wq, dtype=np.uint8)
    n = wq.shape[0]
    if wq.shape[1] * 2 != k:
        raise ValueError("K of X and W differ")
    y = np.empty((m, n), dtype=np.float64)
    b = np.empty((m, n), dtype=np.float64) if with_bound else None
    ax = np.abs(x) if with_bound else None
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        w = dequant(wq[r0:r1], np.asarray(ws)[r0:r1], g)
        y[:, r0:r1] = x @ w.T
        if with_bound:
            b[:, r0:r1] = tolerance_bound(ax @ np.abs(w).T)
    return y, b


def nvfp4_gemm_ref_entries(x_bits: np.ndarray, wq_rows: np.ndarray, ws_rows: np.ndarray,
                           g: float, pairs):
    """Single outputs Y[m, n] (and their bounds), one dot product each.

    Used where the full Y is too large for the host: the caller passes the
    W rows it needs (wq_rows[i], ws_rows[i] for pair i) and (m, n) pairs.
    Returns (y, b) float64 arrays of len(pairs)."""
    x = bf16_bits_to_f64(x_bits)
    out_y = np.empty(len(pairs), dtype=np.float64)
    out_b = np.empty(len(pairs), dtype=np.float64)
    for i, (mi, _n) in enumerate(pairs):
        w = dequant(wq_rows[i:i + 1], ws_rows[i:i + 1], g)[0]
        out_y[i] = float(np.dot(x[mi], w))
        out_b[i] = float(tolerance_bound(np.dot(np.abs(x[mi]), np.abs(w))))
    return out_y, out_b
