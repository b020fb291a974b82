"""Thin ctypes binding of libvgemm.so: argument marshalling only.

Every function checks that its torch tensors have the layout the C ABI
expects (device, dtype, shape, contiguity), passes raw device pointers and
the current HIP stream, and raises on a non-zero status.  All arithmetic
happens in the HIP kernels; there is no fallback of any kind -- if the
library is not built, importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvgemm.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "vgemm.h")

VG_OK = 0
VG_MAX_M = 68
VG_LMHEAD_K = 5120
VG_BATCH_INVARIANT = 1

_lib = None


class VgemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libvgemm.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m verify_gemm_amd.build` "
                          "(the HIP library is required, there is no fallback)")
    # torch ships its own copy of the HIP runtime under the same soname
    # (libamdhip64.so.7).  Importing torch first makes the dynamic loader
    # bind this library to that copy, so the process has ONE runtime and
    # torch's device pointers and streams are valid here; loading this
    # library first would map /opt/rocm's copy as a second, separate runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    sigs = {
        "nvfp4_gemm": (i32, [vp, vp, vp, f32, i32, i32, i32, vp, vp]),
        "nvfp4_gemm_ex": (i32, [vp, vp, vp, f32, i32, i32, i32, vp, vp, sz, vp]),
        "vg_gemm_workspace_bytes": (sz, [i32, i32, i32]),
        "nvfp4_gemm_noalloc": (i32, [vp, vp, vp, f32, i32, i32, i32, vp, vp]),
        "lmhead_argmax_accept": (i32, [vp, vp, vp, vp, i32, i32, vp, vp, vp]),
        "lmhead_argmax_accept_ex": (i32, [vp, vp, vp, f32, vp, i32, i32, i32, i32, vp, vp, vp, sz, vp]),
        "vg_lmhead_workspace_bytes": (sz, [i32]),
        "vg_pass_create": (i32, [vp, i32, i32, vp, ctypes.POINTER(vp)]),
        "vg_pass_run": (i32, [vp, vp]),
        "vg_pass_run_unfused": (i32, [vp, vp]),
        "vg_pass_run_staged": (i32, [vp, vp]),
        "vg_pass_check": (i32, [vp, ctypes.POINTER(i32)]),
        "vg_pass_info": (i32, [vp, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]),
        "vg_pass_grid": (i32, [vp, ctypes.POINTER(i32)]),
        "vg_pass_run_persistent": (i32, [vp, vp]),
        "vg_pass_destroy": (None, [vp]),
        "nvfp4_gemm_invariant": (i32, [vp, vp, vp, f32, i32, i32, i32, vp, vp]),
        "lmhead_verify": (i32, [vp, vp, vp, f32, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                sz, vp]),
        "vg_pass_create_ex": (i32, [vp, i32, i32, vp, vp, vp, vp, i32, ctypes.POINTER(vp)]),
        "fp8_gemm": (i32, [vp, vp, vp, f32, i32, i32, i32, vp, vp]),
        "lmhead_verify_fp8": (i32, [vp, vp, vp, f32, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                    sz, vp]),
        "vg_bwprobe": (i32, [vp, sz, vp, vp]),
        "vg_bwprobe_sink_floats": (sz, []),
        "vg_status_string": (ctypes.c_char_p, [i32]),
        "vg_abi_version": (i32, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions(header: str = HEADER) -> list[str]:
    """Names of every function the public header declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char|void)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def status_string(status: int) -> str:
    return load().vg_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != VG_OK:
        raise VgemmError(status, where)


# --------------------------------------------------------------------------
# torch marshalling
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_ptr(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _need(t, dtype, ndim: int, name: str):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _check_weights(wq, ws, k: int):
    torch = _torch()
    _need(wq, torch.uint8, 2, "Wq")
    _need(ws, torch.uint8, 2, "Ws")
    n = wq.shape[0]
    if wq.shape[1] * 2 != k or tuple(ws.shape) != (n, k // 16):
        raise ValueError(f"weights {tuple(wq.shape)}/{tuple(ws.shape)} do not match K={k}")
    return n


def gemm_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(load().vg_gemm_workspace_bytes(m, n, k))


def lmhead_workspace_bytes(m: int) -> int:
    return int(load().vg_lmhead_workspace_bytes(m))


def new_workspace(nbytes: int, device=None):
    """A zeroed device buffer for the _ex entry points (None if nbytes == 0)."""
    torch = _torch()
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device or "cuda")


def nvfp4_gemm(x, wq, ws, gscale: float, y=None, *, workspace=None, invariant=False, stream=None):
    """Y[M][N] = gscale * X . dequant(Wq, Ws)^T (fp32).  x: bf16 [M][K];
    wq: uint8 [N][K/2]; ws: uint8 [N][K/16].  With ``workspace`` (a zeroed
    uint8 device tensor of gemm_workspace_bytes bytes) the _ex entry point
    is used, which slices narrow matrices over more workgroups (same bits).
    ``invariant`` selects
    nvfp4_gemm_invariant (rows bit-identical for any M)."""
    torch = _torch()
    lib = load()
    px = _need(x, torch.bfloat16, 2, "X")
    m, k = x.shape
    n = _check_weights(wq, ws, k)
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    py = _need(y, torch.float32, 2, "Y")
    if tuple(y.shape) != (m, n):
        raise ValueError("Y must be [M][N]")
    sp = _stream_ptr(stream)
    if invariant:
        st = lib.nvfp4_gemm_invariant(px, wq.data_ptr(), ws.data_ptr(), float(gscale), m, n, k, py, sp)
    elif workspace is None:
        st = lib.nvfp4_gemm(px, wq.data_ptr(), ws.data_ptr(), float(gscale), m, n, k, py, sp)
    else:
        pw = _need(workspace, torch.uint8, 1, "workspace")
        st = lib.nvfp4_gemm_ex(px, wq.data_ptr(), ws.data_ptr(), float(gscale), m, n, k, py,
                               pw, workspace.numel(), sp)
    _check(st, "nvfp4_gemm")
    return y


def nvfp4_gemm_noalloc(x, wq, ws, gscale: float, y, *, stream=None):
    """nvfp4_gemm_noalloc: the workspace form with the library's static
    per-GPU scratch (no allocation anywhere; ``y`` must be given)."""
    torch = _torch()
    lib = load()
    px = _need(x, torch.bfloat16, 2, "X")
    m, k = x.shape
    n = _check_weights(wq, ws, k)
    py = _need(y, torch.float32, 2, "Y")
    if tuple(y.shape) != (m, n):
        raise ValueError("Y must be [M][N]")
    st = lib.nvfp4_gemm_noalloc(px, wq.data_ptr(), ws.data_ptr(), float(gscale), m, n, k, py,
                                _stream_ptr(stream))
    _check(st, "nvfp4_gemm_noalloc")
    return y


def lmhead_argmax_accept(x, wq, ws, draft_ids=None, argmax=None, accept_len=None, *, stream=None):
    """Short form: one sequence of T = M rows, K = 5120, tensor scale 1."""
    torch = _torch()
    lib = load()
    px = _need(x, torch.bfloat16, 2, "X")
    m, k = x.shape
    if k != VG_LMHEAD_K:
        raise ValueError(f"the short lm_head form needs K = {VG_LMHEAD_K}")
    v = _check_weights(wq, ws, k)
    pd = None
    if draft_ids is not None:
        pd = _need(draft_ids, torch.int32, 1, "draft_ids")
        if draft_ids.numel() != m - 1:
            raise ValueError("draft_ids must have M-1 entries")
    argmax = argmax if argmax is not None else torch.empty(m, dtype=torch.int32, device=x.device)
    accept_len = accept_len if accept_len is not None else torch.empty(1, dtype=torch.int32, device=x.device)
    pa = _need(argmax, torch.int32, 1, "argmax")
    pl = _need(accept_len, torch.int32, 1, "accept_len")
    st = lib.lmhead_argmax_accept(px, wq.data_ptr(), ws.data_ptr(), pd, m, v, pa, pl, _stream_ptr(stream))
    _check(st, "lmhead_argmax_accept")
    return argmax, accept_len


def lmhead_argmax_accept_ex(x, wq, ws, gscale: float, draft_ids, T: int, workspace,
                            argmax=None, accept_len=None, *, stream=None):
    """General form: S = M/T sequences; draft_ids int32 [S][T-1] (None iff T == 1);
    workspace: zeroed uint8 device tensor of lmhead_workspace_bytes(M) bytes."""
    torch = _torch()
    lib = load()
    px = _need(x, torch.bfloat16, 2, "X")
    m, k = x.shape
    v = _check_weights(wq, ws, k)
    s = m // T if T > 0 else 0
    pd = None
    if draft_ids is not None:
        pd = _need(draft_ids, torch.int32, 2, "draft_ids")
        if tuple(draft_ids.shape) != (s, T - 1):
            raise ValueError("draft_ids must be [M/T][T-1]")
    argmax = argmax if argmax is not None else torch.empty(m, dtype=torch.int32, device=x.device)
    accept_len = accept_len if accept_len is not None else torch.empty(max(s, 1), dtype=torch.int32, device=x.device)
    pa = _need(argmax, torch.int32, 1, "argmax")
    pl = _need(accept_len, torch.int32, 1, "accept_len")
    pw = _need(workspace, torch.uint8, 1, "workspace")
    st = lib.lmhead_argmax_accept_ex(px, wq.data_ptr(), ws.data_ptr(), float(gscale), pd, m, k, v, T,
                                     pa, pl, pw, workspace.numel(), _stream_ptr(stream))
    _check(st, "lmhead_argmax_accept_ex")
    return argmax, accept_len


def lmhead_verify(x, wq, ws, gscale: float, tokens, T: int, workspace, *, parents=None, token_map=None,
                  flags: int = 0, argmax=None, accept_len=None, accept_node=None, stream=None):
    """lmhead_verify: S = M/T trees (or chains, parents None) of T nodes;
    tokens and parents int32 [S][T-1] (tokens None iff T == 1); token_map
    int32 [V] or None; flags 0 or VG_BATCH_INVARIANT.  Returns (argmax,
    accept_len, accept_node)."""
    torch = _torch()
    lib = load()
    px = _need(x, torch.bfloat16, 2, "X")
    m, k = x.shape
    v = _check_weights(wq, ws, k)
    s = m // T if T > 0 else 0
    pt = pp = pm = None
    if tokens is not None:
        pt = _need(tokens, torch.int32, 2, "tokens")
        if tuple(tokens.shape) != (s, T - 1):
            raise ValueError("tokens must be [M/T][T-1]")
    if parents is not None:
        pp = _need(parents, torch.int32, 2, "parents")
        if tuple(parents.shape) != (s, T - 1):
            raise ValueError("parents must be [M/T][T-1]")
    if token_map is not None:
        pm = _need(token_map, torch.int32, 1, "token_map")
        if token_map.numel() != v:
            raise ValueError("token_map must have V entries")
    dev = x.device
    argmax = argmax if argmax is not None else torch.empty(m, dtype=torch.int32, device=dev)
    accept_len = accept_len if accept_len is not None else torch.empty(max(s, 1), dtype=torch.int32, device=dev)
    accept_node = accept_node if accept_node is not None else torch.empty(max(s, 1), dtype=torch.int32, device=dev)
    pa = _need(argmax, torch.int32, 1, "argmax")
    pl = _need(accept_len, torch.int32, 1, "accept_len")
    pn = _need(accept_node, torch.int32, 1, "accept_node")
    pw = _need(workspace, torch.uint8, 1, "workspace")
    st = lib.lmhead_verify(px, wq.data_ptr(), ws.data_ptr(), float(gscale), pt, pp, pm, m, k, v, T,
                           int(flags), pa, pl, pn, pw, workspace.numel(), _stream_ptr(stream))
    _check(st, "lmhead_verify")
    return argmax, accept_len, accept_node


def fp8_gemm(x, w8, gscale: float, row_scale=None, y=None, *, stream=None):
    """Y[M][N] = X . W^T, w = gscale * row_scale[n] * E4M3(w8): x bf16 [M][K],
    w8 uint8 [N][K], row_scale float32 [N] or None."""
    torch = _torch()
    lib = load()
    px = _need(x, torch.bfloat16, 2, "X")
    m, k = x.shape
    pw = _need(w8, torch.uint8, 2, "W8")
    n = w8.shape[0]
    if w8.shape[1] != k:
        raise ValueError("W8 must be [N][K]")
    pr = None
    if row_scale is not None:
        pr = _need(row_scale, torch.float32, 1, "row_scale")
        if row_scale.numel() != n:
            raise ValueError("row_scale must have N entries")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    py = _need(y, torch.float32, 2, "Y")
    if tuple(y.shape) != (m, n):
        raise ValueError("Y must be [M][N]")
    _check(lib.fp8_gemm(px, pw, pr, float(gscale), m, n, k, py, _stream_ptr(stream)), "fp8_gemm")
    return y


def lmhead_verify_fp8(x, w8, gscale: float, tokens, T: int, workspace, *, row_scale=None, parents=None,
                      token_map=None, flags: int = 0, stream=None):
    """lmhead_verify with an FP8 head (w8 uint8 [V][K], row_scale float32 [V]
    or None).  Returns (argmax, accept_len, accept_node)."""
    torch = _torch()
    lib = load()
    px = _need(x, torch.bfloat16, 2, "X")
    m, k = x.shape
    pw = _need(w8, torch.uint8, 2, "W8")
    v = w8.shape[0]
    if w8.shape[1] != k:
        raise ValueError("W8 must be [V][K]")
    s = m // T if T > 0 else 0
    pt = _need(tokens, torch.int32, 2, "tokens") if tokens is not None else None
    pp = _need(parents, torch.int32, 2, "parents") if parents is not None else None
    pm = _need(token_map, torch.int32, 1, "token_map") if token_map is not None else None
    pr = _need(row_scale, torch.float32, 1, "row_scale") if row_scale is not None else None
    dev = x.device
    argmax = torch.empty(m, dtype=torch.int32, device=dev)
    accept_len = torch.empty(max(s, 1), dtype=torch.int32, device=dev)
    accept_node = torch.empty(max(s, 1), dtype=torch.int32, device=dev)
    pws = _need(workspace, torch.uint8, 1, "workspace")
    st = lib.lmhead_verify_fp8(px, pw, pr, float(gscale), pt, pp, pm, m, k, v, T, int(flags),
                               argmax.data_ptr(), accept_len.data_ptr(), accept_node.data_ptr(), pws,
                               workspace.numel(), _stream_ptr(stream))
    _check(st, "lmhead_verify_fp8")
    return argmax, accept_len, accept_node


class GemmJob(ctypes.Structure):
    """vg_gemm_job of include/vgemm.h."""
    _fields_ = [("Wq", ctypes.c_void_p), ("Ws", ctypes.c_void_p), ("gscale", ctypes.c_float),
                ("N", ctypes.c_int), ("K", ctypes.c_int), ("X", ctypes.c_void_p),
                ("Y", ctypes.c_void_p), ("stage", ctypes.c_int), ("row_scale", ctypes.c_void_p)]


class LmheadJob(ctypes.Structure):
    """vg_lmhead_job of include/vgemm.h."""
    _fields_ = [("Wq", ctypes.c_void_p), ("Ws", ctypes.c_void_p), ("gscale", ctypes.c_float),
                ("V", ctypes.c_int), ("K", ctypes.c_int), ("X", ctypes.c_void_p), ("T", ctypes.c_int),
                ("draft_ids", ctypes.c_void_p), ("argmax", ctypes.c_void_p),
                ("accept_len", ctypes.c_void_p)]


class Pass:
    """A whole step (vg_pass_*): GEMM jobs in dependency order plus an
    optional lm_head job.  ``run`` takes the faster schedule for M (one
    persistent launch at M = 1, one launch per stage above),
    ``run_persistent`` / ``run_staged`` / ``run_unfused`` (one launch per
    job) one of them explicitly.  ``gemms`` is a list
    of (x, wq, ws, gscale, y, stage[, row_scale]) with torch device tensors
    (row_scale: float32 [N] or None, see vg_gemm_job); ``lmhead`` is
    (x, wq, ws, gscale, T, drafts, argmax, accept_len) or None.  ``parents``,
    ``token_map``, ``accept_node`` and ``flags`` are the lm_head options of
    lmhead_verify (vg_pass_create_ex).  The tensors must outlive the Pass
    (it keeps references)."""

    def __init__(self, gemms, M: int, lmhead=None, *, parents=None, token_map=None, accept_node=None,
                 flags: int = 0):
        torch = _torch()
        lib = load()
        self._keep = []
        arr = (GemmJob * max(len(gemms), 1))()
        for i, job in enumerate(gemms):
            x, wq, ws, g, y, stage = job[:6]
            rs = job[6] if len(job) > 6 else None
            _need(x, torch.bfloat16, 2, "X")
            _need(y, torch.float32, 2, "Y")
            k = x.shape[1]
            n = _check_weights(wq, ws, k)
            if tuple(y.shape) != (M, n) or x.shape[0] != M:
                raise ValueError("X must be [M][K] and Y [M][N]")
            prs = None
            if rs is not None:
                prs = _need(rs, torch.float32, 1, "row_scale")
                if rs.numel() != n:
                    raise ValueError("row_scale must have N entries")
            arr[i] = GemmJob(wq.data_ptr(), ws.data_ptr(), float(g), n, k, x.data_ptr(), y.data_ptr(),
                             int(stage), prs)
            self._keep += [x, wq, ws, y, rs]
        lm = None
        if lmhead is not None:
            x, wq, ws, g, T, drafts, am, al = lmhead
            _need(x, torch.bfloat16, 2, "X")
            k = x.shape[1]
            v = _check_weights(wq, ws, k)
            _need(am, torch.int32, 1, "argmax")
            _need(al, torch.int32, 1, "accept_len")
            pd = None
            if T > 1:
                pd = _need(drafts, torch.int32, 2, "draft_ids")
            lm = LmheadJob(wq.data_ptr(), ws.data_ptr(), float(g), v, k, x.data_ptr(), int(T), pd,
                           am.data_ptr(), al.data_ptr())
            self._keep += [x, wq, ws, drafts, am, al]
        pp = _need(parents, torch.int32, 2, "parents") if parents is not None else None
        pm = _need(token_map, torch.int32, 1, "token_map") if token_map is not None else None
        pn = _need(accept_node, torch.int32, 1, "accept_node") if accept_node is not None else None
        self._keep += [parents, token_map, accept_node]
        h = ctypes.c_void_p()
        st = lib.vg_pass_create_ex(ctypes.cast(arr, ctypes.c_void_p), len(gemms), int(M),
                                   ctypes.byref(lm) if lm is not None else None, pp, pm, pn, int(flags),
                                   ctypes.byref(h))
        _check(st, "vg_pass_create_ex")
        self._lib = lib
        self.handle = h

    def run(self, stream=None):
        _check(self._lib.vg_pass_run(self.handle, _stream_ptr(stream)), "vg_pass_run")

    def run_unfused(self, stream=None):
        _check(self._lib.vg_pass_run_unfused(self.handle, _stream_ptr(stream)), "vg_pass_run_unfused")

    def run_staged(self, stream=None):
        _check(self._lib.vg_pass_run_staged(self.handle, _stream_ptr(stream)), "vg_pass_run_staged")

    def run_persistent(self, stream=None):
        _check(self._lib.vg_pass_run_persistent(self.handle, _stream_ptr(stream)), "vg_pass_run_persistent")

    def check(self) -> int:
        e = ctypes.c_int(0)
        _check(self._lib.vg_pass_check(self.handle, ctypes.byref(e)), "vg_pass_check")
        return int(e.value)

    def info(self):
        a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _check(self._lib.vg_pass_info(self.handle, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
               "vg_pass_info")
        g = ctypes.c_int()
        _check(self._lib.vg_pass_grid(self.handle, ctypes.byref(g)), "vg_pass_grid")
        return {"jobs": a.value, "stages": b.value, "items": c.value, "grid": g.value}

    def close(self):
        if getattr(self, "handle", None):
            self._lib.vg_pass_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def bwprobe(buf, sink, *, stream=None):
    """Stream-read every byte of ``buf`` (a 16-byte-aligned device tensor)."""
    lib = load()
    nbytes = buf.numel() * buf.element_size()
    st = lib.vg_bwprobe(buf.data_ptr(), nbytes, sink.data_ptr(), _stream_ptr(stream))
    _check(st, "vg_bwprobe")


def bwprobe_sink_floats() -> int:
    return int(load().vg_bwprobe_sink_floats())
