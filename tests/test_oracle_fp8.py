"""Pins for the oracle's FP8 (E4M3) weight format (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
from verify_gemm_amd import synth


def _x(vals):
    return synth.f32_to_bf16_bits(np.array(vals, dtype=np.float32))


def test_fp8_hand_worked():
    # row 0: bytes 38 40 B8 30 00 44 C0 3C then 38 x 8 = 1, 2, -1, 0.5, 0, 3, -2, 1.5, 1 x 8;
    #   with x = 1..16: 1 + 4 - 3 + 2 + 0 + 18 - 14 + 12 + (9 + ... + 16 = 100) = 120,
    #   sum |x w| = 1 + 4 + 3 + 2 + 0 + 18 + 14 + 12 + 100 = 154; r = 0.5, g = 2 -> 120 and 154
    # row 1: 7E (448, the largest value) x 16, r = 0.25: 448 * 136 * 0.5 = 30464
    # row 2: 01 (2**-9, the smallest subnormal) x 16 with sign bits on the odd
    #   elements, r = 1: (1 - 2 + 3 - ... - 16) * 2**-9 * 2 = -8 * 2**-8 = -1/32
    w8 = np.array([[0x38, 0x40, 0xB8, 0x30, 0x00, 0x44, 0xC0, 0x3C] + [0x38] * 8,
                   [0x7E] * 16,
                   [0x01, 0x81] * 8], dtype=np.uint8)
    rs = np.array([0.5, 0.25, 1.0], dtype=np.float32)
    x = _x([list(range(1, 17))])
    y, b = oracle.fp8_gemm_ref(x, w8, rs, 2.0)
    assert y[0].tolist() == [120.0, 30464.0, -1.0 / 32]
    assert b[0, 0] == pytest.approx(1e-3 * 154 + 1e-6, rel=1e-15)


def test_fp8_matches_torch_decoder_and_matmul():
    rng = np.random.default_rng(7)
    w8 = rng.integers(0, 256, size=(37, 64), dtype=np.uint8)
    w8[(w8 & 0x7F) == 0x7F] = 0x38                    # no NaN codes
    x = synth.gen_x(rng, 5, 64)
    wt = torch.from_numpy(w8).view(torch.float8_e4m3fn).double().numpy()
    xf = oracle.bf16_bits_to_f64(x)
    y, _ = oracle.fp8_gemm_ref(x, w8, None, 1.0)
    assert np.allclose(y, xf @ wt.T, rtol=1e-12, atol=1e-12)
    rs = rng.uniform(0.5, 2.0, size=37).astype(np.float32)
    y2, _ = oracle.fp8_gemm_ref(x, w8, rs, 1.5)
    assert np.allclose(y2, 1.5 * (xf @ wt.T) * rs.astype(np.float64)[None, :], rtol=1e-12, atol=1e-12)


def test_fp8_sign_bit_negates_and_row_scale_is_linear():
    rng = np.random.default_rng(8)
    w8 = rng.integers(0, 127, size=(9, 48), dtype=np.uint8)
    x = synth.gen_x(rng, 3, 48)
    y, _ = oracle.fp8_gemm_ref(x, w8, None, 1.0)
    yn, _ = oracle.fp8_gemm_ref(x, w8 ^ 0x80, None, 1.0)
    assert np.array_equal(yn, -y)
    rs = np.ones(9, np.float32)
    rs[4] = 8.0
    ys, _ = oracle.fp8_gemm_ref(x, w8, rs, 1.0)
    assert np.array_equal(ys[:, 4], 8.0 * y[:, 4]) and np.array_equal(np.delete(ys, 4, 1), np.delete(y, 4, 1))


def test_fp8_lmhead_argmax_uses_row_scales():
    rng = np.random.default_rng(9)
    v, k = 50, 32
    w8 = rng.integers(0, 0x70, size=(v, k), dtype=np.uint8)
    x = synth.gen_x(rng, 4, k)
    rs = rng.uniform(0.5, 2.0, size=v).astype(np.float32)
    r = oracle.lmhead_ref(x, w8, rs, 1.0, T=1, fp8=True)
    y, _ = oracle.fp8_gemm_ref(x, w8, rs, 1.0)
    assert np.array_equal(r["argmax"], np.argmax(y, axis=1))
