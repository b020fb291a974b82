"""The C-ABI library loads without a GPU, exports every symbol the header
declares, and rejects bad arguments before any HIP call (CPU only).

The pointers passed here are host addresses that are never dereferenced:
every call below fails validation, which happens before the library
touches the HIP runtime."""
import ctypes
import os
import re

import numpy as np
import pytest

from verify_gemm_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

VG_OK, VG_ERR_NULL, VG_ERR_SHAPE, VG_ERR_UNSUPPORTED = 0, -1, -2, -3
VG_ERR_HIP, VG_ERR_WORKSPACE, VG_ERR_ALIGN, VG_ERR_FLAGS = -4, -5, -6, -7
VG_ERR_SCRATCH = -8


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from verify_gemm_amd import build
        build.build()
    return binding.load()


@pytest.fixture(scope="module")
def buf():
    # 64-byte aligned host scratch used only as non-null pointer values
    raw = np.zeros(4096 + 64, dtype=np.uint8)
    base = raw.ctypes.data
    off = (-base) % 64
    return raw, base + off


def test_exports_every_header_symbol(lib):
    names = binding.header_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert lib.vg_abi_version() == int(re.search(r"#define VG_ABI_VERSION (\d+)",
                                                 open(binding.HEADER).read()).group(1))


def test_status_strings(lib):
    for code in (VG_OK, VG_ERR_NULL, VG_ERR_SHAPE, VG_ERR_UNSUPPORTED, VG_ERR_HIP, VG_ERR_WORKSPACE,
                 VG_ERR_ALIGN, VG_ERR_FLAGS, VG_ERR_SCRATCH):
        assert binding.status_string(code) != "unknown status"
    assert binding.status_string(12345) == "unknown status"


def test_gemm_null_pointers(lib, buf):
    _, p = buf
    for args in [(None, p, p, p), (p, None, p, p), (p, p, None, p), (p, p, p, None)]:
        x, wq, ws, y = args
        assert lib.nvfp4_gemm(x, wq, ws, 1.0, 1, 16, 16, y, None) == VG_ERR_NULL
        assert lib.nvfp4_gemm_ex(x, wq, ws, 1.0, 1, 16, 16, y, None, 0, None) == VG_ERR_NULL


@pytest.mark.parametrize("m,n,k,code", [
    (0, 16, 16, VG_ERR_SHAPE), (-1, 16, 16, VG_ERR_SHAPE), (1, 0, 16, VG_ERR_SHAPE),
    (1, 16, 0, VG_ERR_SHAPE), (1, 16, 8, VG_ERR_SHAPE), (1, 16, 24, VG_ERR_SHAPE),
    (1, 16, 17, VG_ERR_SHAPE), (69, 16, 16, VG_ERR_UNSUPPORTED), (1000, 16, 16, VG_ERR_UNSUPPORTED),
])
def test_gemm_bad_shapes(lib, buf, m, n, k, code):
    _, p = buf
    assert lib.nvfp4_gemm(p, p, p, 1.0, m, n, k, p, None) == code
    assert lib.nvfp4_gemm_ex(p, p, p, 1.0, m, n, k, p, p, 1 << 30, None) == code


def test_gemm_misaligned(lib, buf):
    _, p = buf
    for x, wq, ws in [(p + 2, p, p), (p, p + 4, p), (p, p, p + 1)]:
        assert lib.nvfp4_gemm(x, wq, ws, 1.0, 1, 16, 16, p, None) == VG_ERR_ALIGN


def test_gemm_ex_workspace_contract(lib, buf):
    """nvfp4_gemm_ex slices a narrow matrix's blocks over more workgroups
    when given the workspace vg_gemm_workspace_bytes asks for; a smaller
    one is an error and a NULL one means no slicing (checked on the host,
    before any launch)."""
    _, p = buf
    need = lib.vg_gemm_workspace_bytes(17, 5120, 17408)
    assert need > 0
    assert lib.nvfp4_gemm_ex(p, p, p, 1.0, 17, 5120, 17408, p, p, need - 1, None) == VG_ERR_WORKSPACE
    assert lib.nvfp4_gemm_ex(p, p, p, 1.0, 17, 5120, 17408, p, p + 4, need, None) == VG_ERR_ALIGN
    # validation still applies to the _ex form
    assert lib.nvfp4_gemm_ex(p, p, p, 1.0, 17, 5120, 24, p, None, 0, None) == VG_ERR_SHAPE


def test_noalloc_validation(lib, buf):
    """nvfp4_gemm_noalloc checks its arguments as nvfp4_gemm does, before any
    HIP call; the largest slice workspace any M <= 68 shape needs on a
    256-CU device fits its 16 MiB static scratch."""
    _, p = buf
    for x, wq, ws, y in [(None, p, p, p), (p, None, p, p), (p, p, None, p), (p, p, p, None)]:
        assert lib.nvfp4_gemm_noalloc(x, wq, ws, 1.0, 17, 5120, 5120, y, None) == VG_ERR_NULL
    for m, n, k, code in [(0, 16, 16, VG_ERR_SHAPE), (1, 0, 16, VG_ERR_SHAPE), (1, 16, 24, VG_ERR_SHAPE),
                          (69, 16, 16, VG_ERR_UNSUPPORTED)]:
        assert lib.nvfp4_gemm_noalloc(p, p, p, 1.0, m, n, k, p, None) == code
    for x, wq, ws in [(p + 2, p, p), (p, p + 4, p), (p, p, p + 1)]:
        assert lib.nvfp4_gemm_noalloc(x, wq, ws, 1.0, 17, 5120, 5120, p, None) == VG_ERR_ALIGN
    # the most slices a shape can have: fewer 64-row blocks than CUs, three
    # K slices each
    worst = max(lib.vg_gemm_workspace_bytes(68, 64 * nb, 17408) for nb in (1, 80, 255))
    assert 0 < worst <= 16 << 20


def test_workspace_sizes(lib):
    # M = 1 takes the GEMV kernel, K = 1024 is too short to slice, invalid shapes need nothing
    for m, n, k in [(1, 5120, 5120), (17, 5120, 1024), (0, 1, 16), (69, 5120, 5120), (17, 5120, 24)]:
        assert lib.vg_gemm_workspace_bytes(m, n, k) == 0
    # narrow matrices at M >= 2: 80 blocks of 64 rows, 3 K slices each; a
    # counter area of one size for every shape, then an M x 64 float block
    # per slice
    sizes = {}
    for m, n, k in [(17, 5120, 5120), (68, 5120, 17408), (2, 5120, 17408)]:
        sizes[m] = lib.vg_gemm_workspace_bytes(m, n, k)
        assert sizes[m] > 240 * m * 64 * 4
    counters = {b - 240 * m * 64 * 4 for m, b in sizes.items()}
    assert len(counters) == 1 and counters.pop() % 256 == 0
    assert lib.vg_lmhead_workspace_bytes(17) >= 8 * 68 * 16
    assert lib.vg_lmhead_workspace_bytes(0) == 0 and lib.vg_lmhead_workspace_bytes(69) == 0


def test_pass_create_validation(lib, buf):
    """vg_pass_create rejects bad job lists before touching the device."""
    _, p = buf
    J = binding.GemmJob
    L = binding.LmheadJob
    out = ctypes.c_void_p()

    def create(jobs, m, lm=None):
        arr = (J * max(len(jobs), 1))(*jobs)
        return lib.vg_pass_create(ctypes.cast(arr, ctypes.c_void_p), len(jobs), m,
                                  ctypes.byref(lm) if lm is not None else None, ctypes.byref(out))

    good = J(p, p, 1.0, 64, 128, p, p, 0)
    assert lib.vg_pass_create(None, 1, 1, None, ctypes.byref(out)) == VG_ERR_NULL
    assert lib.vg_pass_create(None, 0, 1, None, None) == VG_ERR_NULL
    assert create([], 1) == VG_ERR_SHAPE                                   # nothing to run
    assert create([good], 0) == VG_ERR_SHAPE
    assert create([good], 69) == VG_ERR_UNSUPPORTED
    assert create([J(p, p, 1.0, 64, 120, p, p, 0)], 1) == VG_ERR_SHAPE     # K % 16
    assert create([J(p, None, 1.0, 64, 128, p, p, 0)], 1) == VG_ERR_NULL
    assert create([J(p + 4, p, 1.0, 64, 128, p, p, 0)], 1) == VG_ERR_ALIGN
    assert create([good, J(p, p, 1.0, 64, 128, p, p, -1)], 1) == VG_ERR_SHAPE   # negative stage
    assert create([J(p, p, 1.0, 64, 128, p, p, 3), J(p, p, 1.0, 64, 128, p, p, 2)], 1) == VG_ERR_SHAPE
    bad_lm = L(p, p, 1.0, 100, 5120, p, 5, p, p, p)                        # M % T != 0
    assert create([good], 17, bad_lm) == VG_ERR_SHAPE
    assert create([good], 17, L(p, p, 1.0, 100, 5120, p, 17, None, p, p)) == VG_ERR_NULL
    assert out.value is None
    lib.vg_pass_destroy(None)                                              # no-op


def test_pass_handle_null_checks(lib):
    e = ctypes.c_int()
    assert lib.vg_pass_run(None, None) == VG_ERR_NULL
    assert lib.vg_pass_run_unfused(None, None) == VG_ERR_NULL
    assert lib.vg_pass_run_staged(None, None) == VG_ERR_NULL
    assert lib.vg_pass_check(None, ctypes.byref(e)) == VG_ERR_NULL
    assert lib.vg_pass_info(None, None, None, None) == VG_ERR_NULL
    assert lib.vg_pass_grid(None, None) == VG_ERR_NULL


def test_lmhead_validation(lib, buf):
    _, p = buf
    f = lib.lmhead_argmax_accept
    assert f(None, p, p, p, 17, 100, p, p, None) == VG_ERR_NULL
    assert f(p, p, p, None, 17, 100, p, p, None) == VG_ERR_NULL      # drafts needed when M > 1
    assert f(p, p, p, p, 17, 0, p, p, None) == VG_ERR_SHAPE
    assert f(p, p, p, p, 0, 100, p, p, None) == VG_ERR_SHAPE
    assert f(p, p, p, p, 69, 100, p, p, None) == VG_ERR_UNSUPPORTED
    assert f(p + 2, p, p, p, 17, 100, p, p, None) == VG_ERR_ALIGN
    g = lib.lmhead_argmax_accept_ex
    ws = lib.vg_lmhead_workspace_bytes(17)
    assert g(p, p, p, 1.0, p, 17, 5120, 100, 5, p, p, p, ws, None) == VG_ERR_SHAPE   # M % T
    assert g(p, p, p, 1.0, p, 17, 5120, 100, 18, p, p, p, ws, None) == VG_ERR_SHAPE  # T > M
    assert g(p, p, p, 1.0, p, 17, 5120, 100, 0, p, p, p, ws, None) == VG_ERR_SHAPE
    assert g(p, p, p, 1.0, p, 17, 40, 100, 17, p, p, p, ws, None) == VG_ERR_SHAPE    # K % 16
    assert g(p, p, p, 1.0, p, 17, 5120, 100, 17, p, p, None, ws, None) == VG_ERR_WORKSPACE
    assert g(p, p, p, 1.0, p, 17, 5120, 100, 17, p, p, p, ws - 1, None) == VG_ERR_WORKSPACE
    assert g(p, p, p, 1.0, None, 17, 5120, 100, 17, p, p, p, ws, None) == VG_ERR_NULL


def test_bwprobe_validation(lib, buf):
    _, p = buf
    assert lib.vg_bwprobe(None, 1024, p, None) == VG_ERR_NULL
    assert lib.vg_bwprobe(p, 1024, None, None) == VG_ERR_NULL
    assert lib.vg_bwprobe(p, 0, p, None) == VG_ERR_SHAPE
    assert lib.vg_bwprobe(p, 1000, p, None) == VG_ERR_ALIGN
    assert lib.vg_bwprobe(p + 8, 1024, p, None) == VG_ERR_ALIGN
    assert lib.vg_bwprobe_sink_floats() >= 256


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    saved = binding._lib
    try:
        binding._lib = None
        with pytest.raises(ImportError):
            binding.load(str(tmp_path / "missing.so"))
    finally:
        binding._lib = saved


def test_invariant_and_verify_validation(lib, buf):
    """The batch-invariant GEMM, lmhead_verify and vg_pass_create_ex validate
    like their plain forms, and reject unknown flag bits."""
    _, p = buf
    assert lib.nvfp4_gemm_invariant(None, p, p, 1.0, 1, 16, 16, p, None) == VG_ERR_NULL
    assert lib.nvfp4_gemm_invariant(p, p, p, 1.0, 1, 16, 24, p, None) == VG_ERR_SHAPE
    assert lib.nvfp4_gemm_invariant(p, p, p, 1.0, 69, 16, 16, p, None) == VG_ERR_UNSUPPORTED
    assert lib.nvfp4_gemm_invariant(p + 2, p, p, 1.0, 1, 16, 16, p, None) == VG_ERR_ALIGN
    f = lib.lmhead_verify
    ws = lib.vg_lmhead_workspace_bytes(17)
    # X, Wq, Ws, g, tokens, parents, map, M, K, V, T, flags, argmax, len, node, ws, bytes, stream
    assert f(p, p, p, 1.0, p, p, p, 17, 5120, 100, 17, 2, p, p, p, p, ws, None) == VG_ERR_FLAGS
    assert f(p, p, p, 1.0, p, None, None, 17, 5120, 100, 17, 0, p, p, None, None, ws, None) == VG_ERR_WORKSPACE
    assert f(p, p, p, 1.0, None, p, p, 17, 5120, 100, 17, 0, p, p, p, p, ws, None) == VG_ERR_NULL
    assert f(p, p, p, 1.0, p, p, p, 17, 5120, 100, 5, 0, p, p, p, p, ws, None) == VG_ERR_SHAPE
    assert f(p, p, p, 1.0, p, p, p, 17, 5120, 100, 17, 0, None, p, p, p, ws, None) == VG_ERR_NULL
    out = ctypes.c_void_p()
    J = binding.GemmJob
    arr = (J * 1)(J(p, p, 1.0, 64, 128, p, p, 0))
    assert lib.vg_pass_create_ex(ctypes.cast(arr, ctypes.c_void_p), 1, 1, None, None, None, None, 4,
                                 ctypes.byref(out)) == VG_ERR_FLAGS
    assert lib.vg_pass_create_ex(ctypes.cast(arr, ctypes.c_void_p), 1, 0, None, None, None, None, 1,
                                 ctypes.byref(out)) == VG_ERR_SHAPE
    assert out.value is None
    assert lib.vg_status_string(VG_ERR_FLAGS).decode() == "unknown flag bits"


def test_fp8_validation(lib, buf):
    _, p = buf
    assert lib.fp8_gemm(None, p, None, 1.0, 1, 16, 16, p, None) == VG_ERR_NULL
    assert lib.fp8_gemm(p, None, None, 1.0, 1, 16, 16, p, None) == VG_ERR_NULL
    assert lib.fp8_gemm(p, p, None, 1.0, 1, 16, 24, p, None) == VG_ERR_SHAPE
    assert lib.fp8_gemm(p, p, None, 1.0, 69, 16, 16, p, None) == VG_ERR_UNSUPPORTED
    assert lib.fp8_gemm(p, p + 8, None, 1.0, 1, 16, 16, p, None) == VG_ERR_ALIGN
    assert lib.fp8_gemm(p, p, p + 2, 1.0, 1, 16, 16, p, None) == VG_ERR_ALIGN      # row scales
    f = lib.lmhead_verify_fp8
    ws = lib.vg_lmhead_workspace_bytes(17)
    assert f(p, p, None, 1.0, p, None, None, 17, 5120, 100, 17, 4, p, p, None, p, ws, None) == VG_ERR_FLAGS
    assert f(p, p, None, 1.0, None, None, None, 17, 5120, 100, 17, 0, p, p, None, p, ws, None) == VG_ERR_NULL
    assert f(p, p, p + 1, 1.0, p, None, None, 17, 5120, 100, 17, 0, p, p, None, p, ws, None) == VG_ERR_ALIGN
    assert f(p, p, None, 1.0, p, None, None, 17, 5120, 100, 17, 0, p, p, None, None, ws, None) == VG_ERR_WORKSPACE
