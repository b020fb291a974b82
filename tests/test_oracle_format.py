"""Pins for the oracle's element decoders (CPU only).

Each decoder is checked against something other than itself: the OCP
specification's enumerated value list, torch's own float8_e4m3fn and
bfloat16 decoders, and the exact-rational minifloat rule of exact_ref.
"""
import math

import numpy as np
import pytest
import torch

import exact_ref
import oracle
from verify_gemm_amd import synth

# The eight non-negative E2M1 magnitudes as listed by the OCP microscaling
# specification's FP4 value table, codes 0..7; codes 8..15 are their negatives.
OCP_E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_matches_spec_value_list():
    t = oracle.e2m1_table()
    assert t[:8].tolist() == OCP_E2M1_MAGNITUDES
    assert t[8:].tolist() == [-v for v in OCP_E2M1_MAGNITUDES]
    assert math.copysign(1.0, t[8]) == -1.0  # code 8 is -0


def test_e2m1_matches_rational_rule():
    for c in range(16):
        assert oracle.e2m1_value(c) == float(exact_ref.fp4(c))


def test_e2m1_embedded_in_e4m3_via_torch():
    """Every E2M1 value is exactly representable in E4M3; embed the code by
    moving its fields (exponent e -> e + 6, mantissa bit -> top mantissa bit)
    and let torch's float8_e4m3fn decoder produce the value."""
    emb = []
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0:
            byte = 0x30 if m else 0x00          # 0.5 = 2^-1 is a normal E4M3 number
        else:
            byte = ((e + 6) << 3) | (m << 2)
        emb.append(byte | (s << 7))
    via_torch = torch.tensor(emb, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(via_torch, oracle.e2m1_table())


def test_e4m3_matches_torch_all_codes():
    ours = oracle.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan_ours = np.isnan(ours)
    np.testing.assert_array_equal(nan_ours, np.isnan(ref))
    assert set(np.flatnonzero(nan_ours).tolist()) == {0x7F, 0xFF}
    np.testing.assert_array_equal(ours[~nan_ours], ref[~nan_ours])
    # signs of zero follow the sign bit
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_matches_rational_rule_and_landmarks():
    for b in range(256):
        r = exact_ref.fp8(b)
        v = oracle.e4m3_value(b)
        if r is None:
            assert math.isnan(v)
        else:
            assert v == float(r)
    assert oracle.e4m3_value(0x7E) == 448.0            # largest finite
    assert oracle.e4m3_value(0x01) == 2.0 ** -9        # smallest subnormal
    assert oracle.e4m3_value(0x08) == 2.0 ** -6        # smallest normal
    assert oracle.e4m3_value(0x3C) == 1.5


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(ours[finite], ref[finite])
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))


def test_unpack_low_nibble_first():
    wq = np.array([[0x21, 0x43, 0xF0]], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.unpack_codes(wq), [[1, 2, 3, 4, 0, 15]])


def test_synth_scale_bytes_are_powers_of_two():
    vals = [oracle.e4m3_value(int(b)) for b in synth.POW2_SCALE_BYTES]
    assert vals == [2.0 ** u for u in range(-4, 3)]
