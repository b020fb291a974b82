"""Helpers shared by the GPU parity tests: moving seeded host inputs to the
device and comparing against the oracle's bound."""
import numpy as np
import torch


def dev_bf16(x_bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bf16 tensor (bit-exact)."""
    t = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16).copy())
    return t.cuda().view(torch.bfloat16)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def within_bound(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray):
    """(all within, worst |err|/bound, index of worst)."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    ratio = err / bound
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else ()
    ok = bool(np.all(err <= bound)) and bool(np.all(np.isfinite(y_gpu)))
    return ok, float(ratio.max()) if ratio.size else 0.0, worst


def guarded_output(shape, dtype=torch.float32, pad: int = 64, sentinel: float = 12345.5):
    """An output tensor with sentinel-filled guard regions on both sides.
    Returns (view, backing buffer, pad)."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * pad,), sentinel, dtype=dtype, device="cuda")
    return buf[pad:pad + n].view(*shape), buf, pad


def guards_intact(buf: torch.Tensor, pad: int, sentinel: float = 12345.5) -> bool:
    h = buf.cpu()
    return bool(torch.all(h[:pad] == sentinel)) and bool(torch.all(h[-pad:] == sentinel))
