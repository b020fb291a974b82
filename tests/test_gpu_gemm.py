"""GPU parity of nvfp4_gemm against the CPU oracle (needs an MI355X).

Every comparison is element by element against the oracle's fp64 result
with the acceptance bound |y - y_ref| <= 1e-3 * sum_k |x_k w_k| + 1e-6."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_bf16, dev_u8, guarded_output, guards_intact, within_bound
from verify_gemm_amd import binding, synth

pytestmark = pytest.mark.gpu


def run_gemm(x_bits, wq, ws, g, *, workspace=None):
    m, k = x_bits.shape
    n = wq.shape[0]
    y, buf, pad = guarded_output((m, n))
    ws_t = None
    if workspace:
        ws_t = binding.new_workspace(binding.gemm_workspace_bytes(m, n, k))
    binding.nvfp4_gemm(dev_bf16(x_bits), dev_u8(wq), dev_u8(ws), g, y, workspace=ws_t)
    torch.cuda.synchronize()
    assert guards_intact(buf, pad), "write outside Y"
    return y.cpu().numpy()


def check(x_bits, wq, ws, g, label, workspace=False):
    print(f"[case] {label} M={x_bits.shape[0]} N={wq.shape[0]} K={x_bits.shape[1]}", flush=True)
    y = run_gemm(x_bits, wq, ws, g, workspace=workspace)
    y_ref, bound = oracle.nvfp4_gemm_ref(x_bits, wq, ws, g)
    ok, worst, at = within_bound(y, y_ref, bound)
    assert ok, f"{label}: worst err/bound {worst:.3g} at {at}: gpu {y[at]} ref {y_ref[at]}"
    return y


def test_tiny_gemv_1024():
    c = synth.tiny_gemv()
    check(c["x"], c["wq"], c["ws"], c["g"], "tiny gemv")


@pytest.mark.parametrize("n,k", [(17408, 5120), (5120, 5120)])
def test_decode_gemv_shapes(n, k):
    c = synth.decode_gemv(n, k)
    check(c["x"], c["wq"], c["ws"], c["g"], "decode gemv")


@pytest.mark.parametrize("n,k", [(5120, 17408), (17408, 5120)])
def test_verify_gemm_shapes(n, k):
    c = synth.verify_gemm(n, k)
    check(c["x"], c["wq"], c["ws"], c["g"], "verify gemm")
    check(c["x"], c["wq"], c["ws"], c["g"], "verify gemm (caller workspace)", workspace=True)


def test_down_proj_m68():
    c = synth.verify_gemm(5120, 17408, m=68)
    check(c["x"], c["wq"], c["ws"], c["g"], "down M=68")


@pytest.mark.parametrize("m", list(range(1, 69)))
def test_every_m(m):
    rng = np.random.default_rng(5000 + m)
    n, k = 200, 2048                      # N not a multiple of any tile; several K windows
    wq, ws = synth.gen_weights(rng, n, k)
    x = synth.gen_x(rng, m, k)
    check(x, wq, ws, 1.25, "every M")


@pytest.mark.parametrize("m", [1, 2, 16, 17, 33, 68])
@pytest.mark.parametrize("n,k", [(1, 16), (7, 48), (65, 272), (130, 1040), (64, 1056), (3, 5136)])
def test_k_and_n_tails(m, n, k):
    rng = np.random.default_rng(7000 + m * 31 + n * 7 + k)
    wq, ws = synth.gen_weights(rng, n, k)
    x = synth.gen_x(rng, m, k)
    check(x, wq, ws, 0.75, "tails")


@pytest.mark.parametrize("m", [1, 17])
def test_all_finite_scale_codes_and_signs(m):
    rng = np.random.default_rng(8000 + m)
    n, k = 254, 4096
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    wq = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    ws = np.resize(finite, (n, k // 16)).astype(np.uint8)       # every code, negative and subnormal
    ws = ws[:, rng.permutation(k // 16)]
    x = synth.gen_x(rng, m, k)
    check(x, wq, ws, 1.5, "all scale codes")


@pytest.mark.parametrize("m", [1, 4, 17, 68])
def test_zero_blocks_and_zero_scales(m):
    rng = np.random.default_rng(9000 + m)
    n, k = 128, 1024
    wq, ws = synth.gen_weights(rng, n, k)
    wq[:, :64] = 0x00            # +0 codes
    wq[:, 64:128] = 0x88         # -0 codes
    ws[:, 20:30] = 0x00          # zero scale
    ws[:, 30:32] = 0x80          # -0 scale
    wq[5] = 0
    x = synth.gen_x(rng, m, k)
    y = check(x, wq, ws, 1.0, "zero blocks")
    assert np.all(y[:, 5] == 0)


@pytest.mark.parametrize("m", [1, 17, 68])
def test_wide_dynamic_range_x(m):
    rng = np.random.default_rng(9100 + m)
    n, k = 96, 2048
    wq, ws = synth.gen_weights(rng, n, k)
    mag = np.exp2(rng.integers(-60, 61, (m, k))).astype(np.float32)
    sign = np.where(rng.random((m, k)) < 0.5, -1.0, 1.0).astype(np.float32)
    x = synth.f32_to_bf16_bits(mag * sign * (1 + rng.integers(0, 128, (m, k)) / 128).astype(np.float32))
    check(x, wq, ws, 1.0, "wide range X")


@pytest.mark.parametrize("m,n,k", [(1, 17408, 5120), (17, 5120, 5120), (68, 5120, 17408)])
def test_bitwise_repeatable(m, n, k):
    rng = np.random.default_rng(9200 + m)
    wq, ws = synth.gen_weights(rng, n, k)
    x = synth.gen_x(rng, m, k)
    xd, wqd, wsd = dev_bf16(x), dev_u8(wq), dev_u8(ws)
    outs = []
    for _ in range(3):
        outs.append(binding.nvfp4_gemm(xd, wqd, wsd, 1.0).cpu().numpy())
    ws_t = binding.new_workspace(binding.gemm_workspace_bytes(m, n, k))
    outs.append(binding.nvfp4_gemm(xd, wqd, wsd, 1.0, workspace=ws_t).cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


@pytest.mark.parametrize("m,k", [(1, 5120), (1, 17408), (1, 2048), (17, 5120)])
def test_row_bits_independent_of_matrix_height(m, k):
    """A row's output bits do not depend on how many other rows the launch
    has: the first rows of a 5120-row matrix, launched alone as matrices of
    256, 300 and 1000 rows, give the same bits.  At M = 1 and K = 17408 or
    2048 (the step kernel) the row split then gives a workgroup 1-4 rows of
    a chunk instead of 20, so its waves lay out one row per half-wave
    instead of two (the summation must not change with the layout); at
    K = 5120 the single call takes the GEMV items, the last one partial."""
    print(f"[case] row bits vs matrix height M={m} K={k}", flush=True)
    rng = np.random.default_rng(9600 + m + k)
    wq, ws = synth.gen_weights(rng, 5120, k)
    x = synth.gen_x(rng, m, k)
    xd = dev_bf16(x)
    big = binding.nvfp4_gemm(xd, dev_u8(wq), dev_u8(ws), 1.25).cpu().numpy()
    for n in (256, 300, 1000):
        small = binding.nvfp4_gemm(xd, dev_u8(wq[:n].copy()), dev_u8(ws[:n].copy()), 1.25).cpu().numpy()
        assert np.array_equal(small.view(np.uint32), big[:, :n].view(np.uint32)), f"N={n}"
    y_ref, bound = oracle.nvfp4_gemm_ref(x, wq[:300], ws[:300], 1.25)
    ok, worst, at = within_bound(big[:, :300], y_ref, bound)
    assert ok, f"worst err/bound {worst:.3g} at {at}"


@pytest.mark.parametrize("m,n,k", [(2, 5120, 17408), (17, 333, 5120), (68, 1000, 2048), (17, 5120, 5120)])
def test_sliced_gemm_same_bits(m, n, k):
    """With a workspace, nvfp4_gemm_ex deals a narrow matrix's K slices to
    separate workgroups (the one completing a block adds the slice sums in
    slice order); the bits equal nvfp4_gemm's, where one workgroup runs
    every slice of a block, over three calls on one workspace (the counters
    reset themselves), and stay within the oracle's bound."""
    print(f"[case] sliced gemm M={m} N={n} K={k}", flush=True)
    need = binding.gemm_workspace_bytes(m, n, k)
    assert need > 0
    rng = np.random.default_rng(9400 + m + n)
    wq, ws = synth.gen_weights(rng, n, k)
    x = synth.gen_x(rng, m, k)
    xd, wqd, wsd = dev_bf16(x), dev_u8(wq), dev_u8(ws)
    plain = binding.nvfp4_gemm(xd, wqd, wsd, 0.75).cpu().numpy()
    ws_t = binding.new_workspace(need)
    for _ in range(3):
        y = binding.nvfp4_gemm(xd, wqd, wsd, 0.75, workspace=ws_t).cpu().numpy()
        assert np.array_equal(y.view(np.uint32), plain.view(np.uint32))
    assert int(ws_t[:1024].count_nonzero()) == 0
    y_ref, bound = oracle.nvfp4_gemm_ref(x, wq, ws, 0.75)
    ok, worst, at = within_bound(y, y_ref, bound)
    assert ok, f"worst err/bound {worst:.3g} at {at}"


def test_workspace_reused_across_shapes():
    """One caller workspace serves shapes with different tile counts in turn:
    the split-K counters of one shape must never sit under another shape's
    partial sums (regression: a 2-tile shape's partials used to overwrite
    the counters of tiles 64..79 of a 5120-row shape)."""
    rng = np.random.default_rng(9300)
    shapes = [(68, 96, 2048), (17, 5120, 5120), (68, 96, 2048), (17, 5120, 5120), (33, 1000, 4096)]
    need = max(binding.gemm_workspace_bytes(*s) for s in shapes)
    ws_t = binding.new_workspace(need)
    for m, n, k in shapes:
        wq, ws = synth.gen_weights(rng, n, k)
        x = synth.gen_x(rng, m, k)
        print(f"[case] shared workspace M={m} N={n} K={k}", flush=True)
        y = binding.nvfp4_gemm(dev_bf16(x), dev_u8(wq), dev_u8(ws), 1.0, workspace=ws_t).cpu().numpy()
        y_ref, bound = oracle.nvfp4_gemm_ref(x, wq, ws, 1.0)
        ok, worst, at = within_bound(y, y_ref, bound)
        assert ok, f"M={m} N={n} K={k}: worst err/bound {worst:.3g} at {at}"


def _random_shape(case):
    """Seeded shape of sweep case `case`: M over 1..68 (every fourth case in
    65..68, the five-tile range), N ragged, K a multiple of 128 (the
    shared-activation item) or only of 16 (the guarded item)."""
    rng = np.random.default_rng(9900 + case)
    m = int(rng.integers(65, 69)) if case % 4 == 0 else int(rng.integers(1, 69))
    n = int(rng.integers(1, 900))
    k = 128 * int(rng.integers(1, 41)) if case % 2 == 0 else 16 * int(rng.integers(1, 321))
    return rng, m, n, k


@pytest.mark.parametrize("case", range(24))
def test_random_shapes(case):
    """A seeded sweep of shapes off the tuned grid.  Each case: the oracle's
    bound, and, where a workspace applies (K slices dealt to separate
    workgroups), the same bits with and without it."""
    rng, m, n, k = _random_shape(case)
    wq, ws = synth.gen_weights(rng, n, k)
    x = synth.gen_x(rng, m, k)
    g = float(rng.uniform(0.25, 2.0))
    y = check(x, wq, ws, g, f"sweep case {case}")
    if binding.gemm_workspace_bytes(m, n, k) > 0:
        y_ws = run_gemm(x, wq, ws, g, workspace=True)
        assert np.array_equal(y_ws.view(np.uint32), y.view(np.uint32)), "sliced launch changed the bits"


@pytest.mark.parametrize("m", [1, 4, 17, 33, 68])
def test_half_window_scales_stay_in_their_row(m):
    """K = 1152 ends in half a 256-element window, whose scale fetch also
    covers the first bytes of the next row's scales.  Row 1's first scale
    byte is the E4M3 NaN pattern: row 1's outputs are NaN (as the oracle
    says), and rows 0 and 2 must be untouched by it."""
    rng = np.random.default_rng(9950 + m)
    n, k = 3, 1152
    wq, ws = synth.gen_weights(rng, n, k)
    ws[1, 0] = 0x7F
    x = synth.gen_x(rng, m, k)
    print(f"[case] half-window scales M={m} N={n} K={k}", flush=True)
    y = run_gemm(x, wq, ws, 1.0)
    y_ref, bound = oracle.nvfp4_gemm_ref(x, wq, ws, 1.0)
    assert np.isnan(y_ref[:, 1]).all() and np.isnan(y[:, 1]).all()
    keep = [0, 2]
    ok, worst, at = within_bound(y[:, keep], y_ref[:, keep], bound[:, keep])
    assert ok, f"worst err/bound {worst:.3g} at {at}"
