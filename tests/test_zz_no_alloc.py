"""nvfp4_gemm_noalloc, the entry point that allocates nothing (needs an
MI355X): through the C ABI it gives the bits of the existing nvfp4_gemm_ex
with a caller-owned workspace, call after call on the shared static scratch
-- the second call with a smaller input than the first -- and its outputs
lie within the oracle's bound."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_bf16, dev_u8, within_bound
from verify_gemm_amd import binding, synth

pytestmark = pytest.mark.gpu

# (M, N, K): narrow matrices whose K slices run as separate workgroups
# (sliced, so the scratch holds slice sums and counters), largest first;
# then a shape that is not sliced (M = 1) and the largest again.
CASES = [(68, 5120, 17408), (17, 1280, 5120), (1, 1024, 5120), (68, 5120, 17408)]


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_noalloc_matches_workspace_form_call_after_call():
    rng = np.random.default_rng(47000)
    inputs = {}
    for i, (m, n, k) in enumerate(CASES):
        print(f"[case] noalloc call {i}: M={m} N={n} K={k}", flush=True)
        if (m, n, k) not in inputs:
            wq, ws = synth.gen_weights(rng, n, k)
            inputs[(m, n, k)] = (synth.gen_x(rng, m, k), wq, ws, synth.gen_gscale(rng))
        xh, wq, ws, g = inputs[(m, n, k)]
        x, wqd, wsd = dev_bf16(xh), dev_u8(wq), dev_u8(ws)
        need = binding.gemm_workspace_bytes(m, n, k)
        assert (need > 0) == (m > 1), f"slicing expected exactly at M > 1 for {(m, n, k)}"
        assert need <= 16 << 20, "the shape fits the static scratch"
        ws_buf = binding.new_workspace(need)
        y_ex = binding.nvfp4_gemm(x, wqd, wsd, g, workspace=ws_buf)
        y_na = torch.full((m, n), float("nan"), device="cuda")
        binding.nvfp4_gemm_noalloc(x, wqd, wsd, g, y_na)
        torch.cuda.synchronize()
        assert same_bits(y_na, y_ex), f"call {i}: nvfp4_gemm_noalloc differs from nvfp4_gemm_ex"
        # the oracle's bound: every entry of the smaller shapes, sampled
        # entries of the largest
        yh = y_na.cpu().numpy()
        if n * k <= 1280 * 5120:
            y_ref, bound = oracle.nvfp4_gemm_ref(xh, wq, ws, g)
            ok, worst, at = within_bound(yh, y_ref, bound)
            assert ok, f"call {i}: worst err/bound {worst:.3g} at {at}"
        else:
            rows = rng.integers(0, n, 48)
            ms = rng.integers(0, m, 48)
            pairs = list(zip(ms.tolist(), range(48)))
            ye, be = oracle.nvfp4_gemm_ref_entries(xh, wq[rows], ws[rows], g, pairs)
            got = np.array([yh[a, r] for a, r in zip(ms.tolist(), rows.tolist())], dtype=np.float64)
            assert np.all(np.abs(got - ye) <= be), f"call {i}: sampled entries outside the bound"
