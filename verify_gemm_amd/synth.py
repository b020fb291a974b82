"""Seeded synthetic inputs for the NVFP4 weight pass.

This module only draws random numbers in the shapes, value distributions and
layouts of the workloads; it holds none of the method's arithmetic.  Both the
HIP path and the CPU oracle consume what it produces (the oracle always as
host bytes), so neither needs the other.

Workload recipes (shapes of a ~27B hybrid: hidden 5120, MLP 17408, vocab
248,320 and its 65,536-row slice; 16 drafts + 1 committed token per verify;
up to 4 sequences per weight read):

  * packed codes: uniform bytes, i.e. both nibbles uniform over the 16 E2M1
    codes;
  * block scales: the E4M3 encodings of 2**u, u uniform in {-4, ..., 2};
  * tensor scale g: 1.0 for the tiny case, else uniform in [0.5, 2] (fp32);
  * X: bf16 of N(0, sigma**2) (sigma = 0.1 for the decode GEMV), rounded to
    nearest-even by torch;
  * drafts: position j equals the target argmax of row j with probability
    0.7, otherwise uniform over [0, V).

Host generation uses numpy PCG64 streams spawned from one SeedSequence per
workload; device generation (the 14 GB full pass) uses torch's device
generator seeded per matrix.
"""
from __future__ import annotations

import numpy as np

SEED_BASE = 1000

# E4M3 bytes of 2**u for u = -4 .. 2 (exponent field u + 7, mantissa 0).
POW2_SCALE_BYTES = np.array([0x18, 0x20, 0x28, 0x30, 0x38, 0x40, 0x48], dtype=np.uint8)

HIDDEN = 5120
MLP = 17408
VOCAB = 248320
VOCAB_SLICE = 65536
DRAFTS = 16
T_VERIFY = DRAFTS + 1

# The synthetic 64-layer pass: per layer q, k, v, o (5120x5120), gate, up
# (17408x5120) and down (5120x17408), then the lm_head.
LAYERS = 64
LAYER_MATS = (("q", HIDDEN, HIDDEN), ("k", HIDDEN, HIDDEN), ("v", HIDDEN, HIDDEN),
              ("o", HIDDEN, HIDDEN), ("gate", MLP, HIDDEN), ("up", MLP, HIDDEN),
              ("down", HIDDEN, MLP))


def streams(seed: int, n: int) -> list[np.random.Generator]:
    """n independent PCG64 generators derived from one seed."""
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def gen_weights(rng: np.random.Generator, n: int, k: int):
    """Packed codes uint8[n][k/2] and block-scale bytes uint8[n][k/16]."""
    if k % 16:
        raise ValueError("K must be a multiple of 16")
    wq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    ws = POW2_SCALE_BYTES[rng.integers(0, POW2_SCALE_BYTES.size, size=(n, k // 16))]
    return wq, ws


def gen_fp8_weights(rng: np.random.Generator, n: int, k: int, row_scales: bool = True):
    """FP8 weights: E4M3 bytes uint8[n][k] uniform over the 254 non-NaN
    codes (so every exponent, subnormals and +-448 included), and per-row
    scales float32[n] ~ U[0.5, 2] (None if not row_scales)."""
    w8 = rng.integers(0, 254, size=(n, k), dtype=np.uint16)
    w8 = (w8 + (w8 >= 0x7F)).astype(np.uint8)       # skip 0x7F; 254 -> 0xFF never drawn
    rs = rng.uniform(0.5, 2.0, size=n).astype(np.float32) if row_scales else None
    return w8, rs


def gen_scale_bytes(rng: np.random.Generator, n: int, k: int, codes: np.ndarray):
    """Block-scale bytes drawn uniformly from an explicit set of byte codes."""
    codes = np.asarray(codes, dtype=np.uint8)
    return codes[rng.integers(0, codes.size, size=(n, k // 16))]


def gen_gscale(rng: np.random.Generator, lo: float = 0.5, hi: float = 2.0) -> float:
    return float(np.float32(rng.uniform(lo, hi)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even, via torch) -> uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def gen_x(rng: np.random.Generator, m: int, k: int, sigma: float = 1.0) -> np.ndarray:
    """bf16 bits uint16[m][k] of sigma * N(0, 1)."""
    a = rng.standard_normal((m, k), dtype=np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(a)


def gen_drafts(rng: np.random.Generator, target_argmax: np.ndarray, v: int,
               p_match: float = 0.7) -> np.ndarray:
    """Drafts int32[S][T-1] from the target argmax int[S][T]: d[s][j] equals
    target_argmax[s][j] with probability p_match, otherwise uniform in [0, v)."""
    am = np.asarray(target_argmax).reshape(target_argmax.shape[0], -1)
    s, t = am.shape
    match = rng.random((s, t - 1)) < p_match
    rand = rng.integers(0, v, size=(s, t - 1))
    return np.where(match, am[:, :t - 1], rand).astype(np.int32)


# --------------------------------------------------------------------------
# Named workloads (host)
# --------------------------------------------------------------------------
def tiny_gemv(seed: int = SEED_BASE + 0):
    """M=1, N=K=1024, g = 1.0, X ~ N(0,1)."""
    rw, rx = streams(seed, 2)
    wq, ws = gen_weights(rw, 1024, 1024)
    return {"x": gen_x(rx, 1, 1024), "wq": wq, "ws": ws, "g": 1.0}


def decode_gemv(n: int, k: int, seed: int = SEED_BASE + 1):
    """M=1 at a projection shape, g ~ U[0.5, 2], X ~ 0.1 N(0,1)."""
    rw, rg, rx = streams(seed * 100003 + n * 7 + k, 3)
    wq, ws = gen_weights(rw, n, k)
    return {"x": gen_x(rx, 1, k, 0.1), "wq": wq, "ws": ws, "g": gen_gscale(rg)}


def verify_gemm(n: int, k: int, m: int = T_VERIFY, seed: int = SEED_BASE + 2):
    """M=17 (or m) speculative-verify GEMM, rows of X independent N(0,1)."""
    rw, rg, rx = streams(seed * 100003 + n * 7 + k + m * 13, 3)
    wq, ws = gen_weights(rw, n, k)
    return {"x": gen_x(rx, m, k), "wq": wq, "ws": ws, "g": gen_gscale(rg)}


def lmhead_weights(v: int, k: int = HIDDEN, seed: int = SEED_BASE + 3):
    """One lm_head weight set per vocabulary size, fixed over all steps."""
    rw, rg = streams(seed * 100003 + v, 2)
    wq, ws = gen_weights(rw, v, k)
    return wq, ws, gen_gscale(rg)


def lmhead_steps_x(steps: int, v: int, m: int = T_VERIFY, k: int = HIDDEN,
                   seed: int = SEED_BASE + 3) -> np.ndarray:
    """Fresh X per step: uint16[steps*m][k] (step s owns rows s*m .. s*m+m-1)."""
    (rx,) = streams(seed * 100003 + v + 1, 1)
    return gen_x(rx, steps * m, k)


def lmhead_steps_drafts(target_argmax: np.ndarray, v: int,
                        seed: int = SEED_BASE + 3) -> np.ndarray:
    """Drafts for every step from the oracle's argmax int[steps][T]."""
    (rd,) = streams(seed * 100003 + v + 2, 1)
    return gen_drafts(rd, target_argmax, v)


# --------------------------------------------------------------------------
# Device generation (the 14 GB pass does not fit a host round trip per run)
# --------------------------------------------------------------------------
def gen_weights_device(n: int, k: int, seed: int, device):
    """Packed codes and E4M3 2**u scale bytes generated on the device."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    wq = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device=device, generator=gen)
    table = torch.from_numpy(POW2_SCALE_BYTES).to(device)
    idx = torch.randint(0, POW2_SCALE_BYTES.size, (n, k // 16), device=device, generator=gen)
    return wq, table[idx]


def gen_x_device(m: int, k: int, seed: int, device, sigma: float = 1.0):
    """bf16 sigma*N(0,1) [m][k] generated on the device."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return (torch.randn((m, k), device=device, generator=gen) * sigma).to(torch.bfloat16)


def pass_matrix_seed(layer: int, mat: int, seed: int = SEED_BASE + 4) -> int:
    """Seed of matrix ``mat`` (0..6) of ``layer``; the lm_head is layer LAYERS, mat 0."""
    return seed * 1000 + layer * 8 + mat


def pass_gscale(layer: int, mat: int, seed: int = SEED_BASE + 4) -> float:
    (rg,) = streams(pass_matrix_seed(layer, mat, seed), 1)
    return gen_gscale(rg)
