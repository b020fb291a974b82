"""Exact rational brute force for the NVFP4 GEMM (test helper).

A second, independent formulation used only to pin the fp64 oracle: every
element format is decoded by one generic minifloat rule with exact
``fractions.Fraction`` arithmetic, the nibble order is read bit by bit, and
the K-sum is carried out without rounding.  Every value involved is a dyadic
rational, so the result is the exact mathematical Y.
"""
from fractions import Fraction


def minifloat(bits: int, ebits: int, mbits: int, bias: int, nan_all_ones: bool):
    """Decode an IEEE-style minifloat with no infinities.  Returns a Fraction,
    or None for NaN (the all-ones exponent-and-mantissa pattern when
    nan_all_ones)."""
    sign = (bits >> (ebits + mbits)) & 1
    exp = (bits >> mbits) & ((1 << ebits) - 1)
    man = bits & ((1 << mbits) - 1)
    if nan_all_ones and exp == (1 << ebits) - 1 and man == (1 << mbits) - 1:
        return None
    if exp == 0:
        mag = Fraction(man, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        mag = (1 + Fraction(man, 1 << mbits)) * Fraction(2) ** (exp - bias)
    return -mag if sign else mag


def fp4(code):
    return minifloat(code, 2, 1, 1, False)


def fp8(byte):
    return minifloat(byte, 4, 3, 7, True)


def bf16(bits):
    return minifloat(bits, 8, 7, 127, False)


def code_at(row_bytes, k):
    byte = row_bytes[k >> 1]
    return (byte >> 4) & 15 if k & 1 else byte & 15


def exact_gemm(x_bits, wq, ws, g):
    """x_bits: list of lists of uint16; wq, ws: lists of byte rows; g: float.
    Returns (Y, abs_sum) as lists of lists of Fractions."""
    gf = Fraction(g)
    m = len(x_bits)
    n = len(wq)
    k = len(x_bits[0])
    ys, abss = [], []
    for i in range(m):
        yrow, arow = [], []
        for j in range(n):
            acc = Fraction(0)
            aacc = Fraction(0)
            for kk in range(k):
                xv = bf16(int(x_bits[i][kk]))
                wv = gf * fp8(int(ws[j][kk // 16])) * fp4(code_at(wq[j], kk))
                acc += xv * wv
                aacc += abs(xv * wv)
            yrow.append(acc)
            arow.append(aacc)
        ys.append(yrow)
        abss.append(arow)
    return ys, abss
