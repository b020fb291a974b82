"""GPU parity of the FP8 (E4M3) weight variant against the oracle (needs an
MI355X): fp8_gemm at M = 1 / 4 / 17 / 68 on tuned and ragged shapes, with
and without per-row scales, and the FP8 lm_head (lmhead_verify_fp8) with
argmax, tree accept and the token map."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_bf16, dev_i32, dev_u8, guarded_output, guards_intact, within_bound
from verify_gemm_amd import binding, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,n,k", [(1, 1024, 5120), (1, 300, 1040), (1, 77, 48), (4, 100, 4096),
                                   (17, 512, 5120), (17, 96, 17408), (68, 256, 1024), (68, 33, 80),
                                   (65, 700, 2048), (67, 129, 4096)])
@pytest.mark.parametrize("with_rs", [True, False])
def test_fp8_gemm_matches_oracle(m, n, k, with_rs):
    print(f"[case] fp8_gemm M={m} N={n} K={k} row_scale={with_rs}", flush=True)
    rng = np.random.default_rng(45000 + m * 7 + n + k)
    w8, rs = synth.gen_fp8_weights(rng, n, k, row_scales=with_rs)
    g = synth.gen_gscale(rng)
    x = synth.gen_x(rng, m, k)
    y, buf, pad = guarded_output((m, n))
    binding.fp8_gemm(dev_bf16(x), dev_u8(w8), g, torch.from_numpy(rs).cuda() if with_rs else None, y)
    torch.cuda.synchronize()
    y_ref, bound = oracle.fp8_gemm_ref(x, w8, rs, g)
    ok, worst, at = within_bound(y.cpu().numpy(), y_ref, bound)
    assert ok, f"worst err/bound {worst:.3g} at {at}"
    assert guards_intact(buf, pad), "a write landed outside Y"


@pytest.mark.parametrize("M,T", [(1, 1), (17, 17), (68, 17), (66, 33)])
def test_fp8_lmhead_verify(M, T):
    print(f"[case] fp8 lm_head M={M} T={T}", flush=True)
    rng = np.random.default_rng(46000 + M)
    v, k = 12000, 5120
    w8, rs = synth.gen_fp8_weights(rng, v, k)
    g = synth.gen_gscale(rng)
    x = synth.gen_x(rng, M, k)
    token_map = (rng.permutation(v) + 5000).astype(np.int32)
    base = oracle.lmhead_ref(x, w8, rs, g, T=1, token_map=token_map, fp8=True)
    S = M // T
    tokens = parents = None
    if T > 1:
        parents = np.array([[rng.integers(0, i) for i in range(1, T)] for _ in range(S)], np.int32)
        tokens = np.empty((S, T - 1), np.int32)
        for q in range(S):
            for i in range(1, T):
                p = parents[q, i - 1]
                tokens[q, i - 1] = base["argmax"][q * T + p] if rng.random() < 0.7 else token_map[rng.integers(0, v)]
    ref = oracle.lmhead_ref(x, w8, rs, g, T=T, drafts=tokens, token_map=token_map, parents=parents, fp8=True)
    wsp = binding.new_workspace(binding.lmhead_workspace_bytes(M))
    am, al, an = binding.lmhead_verify_fp8(dev_bf16(x), dev_u8(w8), g,
                                           dev_i32(tokens) if tokens is not None else None, T, wsp,
                                           row_scale=torch.from_numpy(rs).cuda(),
                                           parents=dev_i32(parents) if parents is not None else None,
                                           token_map=dev_i32(token_map))
    torch.cuda.synchronize()
    assert int(wsp.count_nonzero()) == 0
    am = am.cpu().numpy()
    dec = ref["decisive"]
    assert np.array_equal(am[dec], ref["argmax"][dec])
    nd = ~dec
    assert np.all((am[nd] == ref["argmax"][nd]) | (am[nd] == token_map[ref["idx2"][nd]]))
    if T > 1:
        sd = ref["step_decisive"]
        assert np.array_equal(al.cpu().numpy()[:S][sd], ref["accept_len"][sd])
        assert np.array_equal(an.cpu().numpy()[:S][sd], ref["accept_node"][sd])
    else:
        assert int(al.cpu()[0]) == 0
