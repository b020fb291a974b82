"""Pins for the oracle's GEMM and acceptance bound (CPU only).

Pinned against: the hand-worked cases in tests/golden/ (values derived by
hand, not by the oracle), exact rational brute force on random tiny shapes
(hypothesis), a special case that reduces to a plain float matmul of the
spec's value list, and invariants that hold exactly on dyadic inputs.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import exact_ref
import oracle
from verify_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_case(name):
    with open(os.path.join(GOLDEN, name)) as f:
        c = json.load(f)
    x = synth.f32_to_bf16_bits(np.array(c["x"], dtype=np.float32))
    wq = np.array([list(bytes.fromhex(h)) for h in c["wq_hex"]], dtype=np.uint8)
    ws = np.array([list(bytes.fromhex(h)) for h in c["ws_hex"]], dtype=np.uint8)
    return c, x, wq, ws


@pytest.mark.parametrize("name", ["case_a_1x16.json", "case_b_2x32.json"])
def test_hand_worked_cases(name):
    c, x, wq, ws = load_case(name)
    y, b = oracle.nvfp4_gemm_ref(x, wq, ws, c["g"])
    np.testing.assert_array_equal(y, np.array(c["y"]))
    np.testing.assert_array_equal(b, 1e-3 * np.array(c["abs_sum"]) + 1e-6)


@pytest.mark.parametrize("name", ["case_a_1x16.json", "case_b_2x32.json"])
def test_hand_worked_cases_match_exact_rationals(name):
    c, x, wq, ws = load_case(name)
    ys, abss = exact_ref.exact_gemm(x.tolist(), wq.tolist(), ws.tolist(), c["g"])
    assert [[float(v) for v in r] for r in ys] == c["y"]
    assert [[float(v) for v in r] for r in abss] == c["abs_sum"]


def _finite_scale_codes():
    return [b for b in range(256) if b not in (0x7F, 0xFF)]


@settings(max_examples=60, deadline=None)
@given(m=st.integers(1, 3), n=st.integers(1, 3), kb=st.integers(1, 3),
       seed=st.integers(0, 2**31 - 1), g=st.sampled_from([1.0, 0.5, 1.75, 0.3333333432674408]))
def test_matches_exact_rationals_random(m, n, kb, seed, g):
    rng = np.random.default_rng(seed)
    k = 16 * kb
    wq = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    ws = synth.gen_scale_bytes(rng, n, k, _finite_scale_codes())
    x = synth.f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32) * 3)
    y, b = oracle.nvfp4_gemm_ref(x, wq, ws, g)
    ys, abss = exact_ref.exact_gemm(x.tolist(), wq.tolist(), ws.tolist(), g)
    ye = np.array([[float(v) for v in r] for r in ys])
    ae = np.array([[float(v) for v in r] for r in abss])
    # only the fp64 K-sum rounds: error <= K * 2^-52 * sum|xw|
    assert np.all(np.abs(y - ye) <= k * 2.0 ** -52 * ae)
    np.testing.assert_allclose(b, 1e-3 * ae + 1e-6, rtol=1e-12, atol=0)


def test_unit_scales_reduce_to_float_matmul():
    """All scales 1.0 (byte 0x38) and g = 1: Y is a plain product with the
    spec's value list, built here element by element from the bytes."""
    rng = np.random.default_rng(7)
    m, n, k = 3, 5, 64
    wq = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    ws = np.full((n, k // 16), 0x38, np.uint8)
    xf = rng.standard_normal((m, k)).astype(np.float32)
    x = synth.f32_to_bf16_bits(xf)
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    w = np.zeros((n, k))
    for r in range(n):
        for kk in range(k):
            byte = int(wq[r, kk // 2])
            code = (byte >> 4) if kk % 2 else (byte & 15)
            w[r, kk] = (-1.0 if code & 8 else 1.0) * mags[code & 7]
    xd = np.array([[float(np.float32(np.uint32(int(v) << 16).view(np.float32))) for v in row] for row in x])
    y, _ = oracle.nvfp4_gemm_ref(x, wq, ws, 1.0)
    np.testing.assert_allclose(y, xd @ w.T, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ invariants
def _rand_case(seed, m=2, n=3, k=48, codes=None):
    rng = np.random.default_rng(seed)
    wq = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    codes = codes if codes is not None else synth.POW2_SCALE_BYTES
    ws = synth.gen_scale_bytes(rng, n, k, codes)
    # small integers: bf16-exact, so sums and scalings below stay exact
    xf = rng.integers(-8, 9, (m, k)).astype(np.float32)
    return xf, wq, ws


def test_linear_in_x():
    xf1, wq, ws = _rand_case(1)
    xf2 = np.random.default_rng(2).integers(-8, 9, xf1.shape).astype(np.float32)
    a, b = 3.0, -2.0
    f = lambda xf: oracle.nvfp4_gemm_ref(synth.f32_to_bf16_bits(xf), wq, ws, 1.25)[0]
    np.testing.assert_array_equal(f(a * xf1 + b * xf2), a * f(xf1) + b * f(xf2))


def test_linear_in_g():
    xf, wq, ws = _rand_case(3)
    x = synth.f32_to_bf16_bits(xf)
    y1 = oracle.nvfp4_gemm_ref(x, wq, ws, 1.0)[0]
    y2 = oracle.nvfp4_gemm_ref(x, wq, ws, 0.75)[0]
    np.testing.assert_array_equal(y2, 0.75 * y1)


def test_code_sign_flip_negates():
    xf, wq, ws = _rand_case(4)
    x = synth.f32_to_bf16_bits(xf)
    y = oracle.nvfp4_gemm_ref(x, wq, ws, 1.0)[0]
    yf = oracle.nvfp4_gemm_ref(x, wq ^ np.uint8(0x88), ws, 1.0)[0]
    np.testing.assert_array_equal(yf, -y)


def test_scale_exponent_bump_doubles():
    normal = [b for b in range(256) if 1 <= ((b >> 3) & 15) <= 13]
    xf, wq, ws = _rand_case(5, codes=normal)
    x = synth.f32_to_bf16_bits(xf)
    y = oracle.nvfp4_gemm_ref(x, wq, ws, 1.0)[0]
    y2 = oracle.nvfp4_gemm_ref(x, wq, (ws + 8).astype(np.uint8), 1.0)[0]
    np.testing.assert_array_equal(y2, 2 * y)


def test_kblock_permutation_invariant():
    xf, wq, ws = _rand_case(6, k=64)
    perm = [2, 0, 3, 1]
    xp = np.concatenate([xf[:, 16 * p:16 * p + 16] for p in perm], axis=1)
    wqp = np.concatenate([wq[:, 8 * p:8 * p + 8] for p in perm], axis=1)
    wsp = ws[:, perm]
    y = oracle.nvfp4_gemm_ref(synth.f32_to_bf16_bits(xf), wq, ws, 1.0)[0]
    yp = oracle.nvfp4_gemm_ref(synth.f32_to_bf16_bits(xp), wqp, wsp, 1.0)[0]
    np.testing.assert_array_equal(y, yp)


def test_row_n_depends_only_on_row_n():
    xf, wq, ws = _rand_case(8, n=4)
    x = synth.f32_to_bf16_bits(xf)
    y = oracle.nvfp4_gemm_ref(x, wq, ws, 1.0)[0]
    wq2 = wq.copy(); ws2 = ws.copy()
    wq2[1] ^= 0x5A; ws2[1] = 0x40
    y2 = oracle.nvfp4_gemm_ref(x, wq2, ws2, 1.0)[0]
    np.testing.assert_array_equal(y2[:, [0, 2, 3]], y[:, [0, 2, 3]])
    assert not np.array_equal(y2[:, 1], y[:, 1])


def test_row_chunking_does_not_change_results():
    xf, wq, ws = _rand_case(9, n=37)
    x = synth.f32_to_bf16_bits(xf)
    y1, b1 = oracle.nvfp4_gemm_ref(x, wq, ws, 1.5, row_chunk=5)
    y2, b2 = oracle.nvfp4_gemm_ref(x, wq, ws, 1.5, row_chunk=4096)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(b1, b2)


def test_entries_match_full():
    xf, wq, ws = _rand_case(10, m=3, n=6)
    x = synth.f32_to_bf16_bits(xf)
    y, b = oracle.nvfp4_gemm_ref(x, wq, ws, 0.5)
    pairs = [(0, 5), (2, 0), (1, 3)]
    ye, be = oracle.nvfp4_gemm_ref_entries(x, wq[[p[1] for p in pairs]], ws[[p[1] for p in pairs]], 0.5, pairs)
    np.testing.assert_allclose(ye, [y[p] for p in pairs], rtol=0, atol=1e-12)
    np.testing.assert_allclose(be, [b[p] for p in pairs], rtol=1e-15)
