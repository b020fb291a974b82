"""GPU parity of the verify-pass extensions (needs an MI355X):

* batch-invariant rows -- nvfp4_gemm_invariant and the VG_BATCH_INVARIANT
  flag: a row's result is bit-identical whatever batch it is computed in,
  M = 1 included (TandemLLM README, "The parts");
* tree verify and the sliced head's row-to-token map -- lmhead_verify and
  vg_pass_create_ex, against the oracle's tree rule (TandemLLM README, flow
  diagram; dgx-spark-qwen38 README, opening section).

argmax must match the oracle on decisive rows, accept_len / accept_node on
decisive steps (every row the tree rule compares is decisive)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_bf16, dev_i32, dev_u8, within_bound
from verify_gemm_amd import binding, synth

pytestmark = pytest.mark.gpu

INV = binding.VG_BATCH_INVARIANT


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


@pytest.mark.parametrize("n,k", [(1024, 5120), (300, 1040), (96, 17408), (40, 48)])
def test_gemm_rows_are_batch_invariant(n, k):
    print(f"[case] invariant gemm N={n} K={k}", flush=True)
    rng = np.random.default_rng(40000 + n + k)
    wq, ws = synth.gen_weights(rng, n, k)
    g = synth.gen_gscale(rng)
    x = synth.gen_x(rng, 68, k)
    xd, wqd, wsd = dev_bf16(x), dev_u8(wq), dev_u8(ws)
    y68 = binding.nvfp4_gemm(xd, wqd, wsd, g, invariant=True)
    torch.cuda.synchronize()
    y_ref, bound = oracle.nvfp4_gemm_ref(x, wq, ws, g)
    ok, worst, at = within_bound(y68.cpu().numpy(), y_ref, bound)
    assert ok, f"worst err/bound {worst:.3g} at {at}"
    for m0, m1 in [(0, 1), (5, 6), (67, 68), (0, 17), (17, 21), (40, 41), (3, 35)]:
        ys = binding.nvfp4_gemm(xd[m0:m1].contiguous(), wqd, wsd, g, invariant=True)
        torch.cuda.synchronize()
        assert same_bits(ys, y68[m0:m1]), f"rows {m0}:{m1} differ from the 68-row batch"
    # the plain form at M >= 2 runs the same MFMA path, so it agrees too
    y17 = binding.nvfp4_gemm(xd[:17].contiguous(), wqd, wsd, g)
    torch.cuda.synchronize()
    assert same_bits(y17, y68[:17])


def make_tree(rng, argmax_ids, token_map, S, T, p_match=0.7):
    """Random trees: mostly valid parents (a few point at or past the node,
    or are negative), tokens equal to the parent row's argmax id with
    probability p_match, else a random token id of the head."""
    parents = np.empty((S, T - 1), np.int32)
    tokens = np.empty((S, T - 1), np.int32)
    v = token_map.shape[0]
    for q in range(S):
        for i in range(1, T):
            u = rng.random()
            if u < 0.9:
                p = int(rng.integers(0, i))
            elif u < 0.95:
                p = int(rng.integers(i, T + 3))
            else:
                p = -1 - int(rng.integers(0, 3))
            parents[q, i - 1] = p
            hit = 0 <= p < i and rng.random() < p_match
            tokens[q, i - 1] = argmax_ids[q * T + p] if hit else int(token_map[rng.integers(0, v)])
    return tokens, parents


def check_against_oracle(ref, am, al, an, token_map, label):
    dec = ref["decisive"]
    assert np.array_equal(am[dec], ref["argmax"][dec]), f"{label}: argmax differs on a decisive row"
    nd = ~dec
    assert np.all((am[nd] == ref["argmax"][nd]) | (am[nd] == token_map[ref["idx2"][nd]]))
    sd = ref["step_decisive"]
    assert np.array_equal(al[sd], ref["accept_len"][sd]), f"{label}: accept_len"
    assert np.array_equal(an[sd], ref["accept_node"][sd]), f"{label}: accept_node"
    return int(nd.sum()), int((~sd).sum())


@pytest.mark.parametrize("M,T", [(17, 17), (68, 17), (8, 4)])
def test_lmhead_verify_tree_and_map(M, T):
    print(f"[case] lmhead_verify tree+map M={M} T={T}", flush=True)
    rng = np.random.default_rng(41000 + 100 * M + T)
    v, k = 20000, 5120
    wq, ws = synth.gen_weights(rng, v, k)
    g = synth.gen_gscale(rng)
    x = synth.gen_x(rng, M, k)
    token_map = (rng.permutation(v) * 3 + 7).astype(np.int32)   # distinct ids, not row numbers
    base = oracle.lmhead_ref(x, wq, ws, g, T=1, token_map=token_map)
    S = M // T
    tokens, parents = make_tree(rng, base["argmax"], token_map, S, T)
    ref = oracle.lmhead_ref(x, wq, ws, g, T=T, drafts=tokens, token_map=token_map, parents=parents)
    assert ref["accept_len"].max() > 0, "the trees should accept something"
    xd, wqd, wsd = dev_bf16(x), dev_u8(wq), dev_u8(ws)
    td, pd, md = dev_i32(tokens), dev_i32(parents), dev_i32(token_map)
    wsp = binding.new_workspace(binding.lmhead_workspace_bytes(M))
    out = {}
    for flags in (0, INV):
        am, al, an = binding.lmhead_verify(xd, wqd, wsd, g, td, T, wsp, parents=pd, token_map=md,
                                           flags=flags)
        torch.cuda.synchronize()
        assert int(wsp.count_nonzero()) == 0          # left zeroed for the next call
        out[flags] = (am.cpu().numpy(), al.cpu().numpy()[:S], an.cpu().numpy()[:S])
        ties, nd_steps = check_against_oracle(ref, *out[flags], token_map, f"flags={flags}")
        print(f"[case]   flags={flags}: near-tie rows {ties}, near-tie steps {nd_steps}", flush=True)
    # M >= 2: the plain and the invariant form run the same kernel
    assert all(np.array_equal(a, b) for a, b in zip(out[0], out[INV]))
    # chain (no parents) is the greedy rule, with accept_node == accept_len
    am_c, al_c, an_c = binding.lmhead_verify(xd, wqd, wsd, g, td, T, wsp, token_map=md)
    ref_c = oracle.lmhead_ref(x, wq, ws, g, T=T, drafts=tokens, token_map=token_map)
    torch.cuda.synchronize()
    al_c, an_c = al_c.cpu().numpy()[:S], an_c.cpu().numpy()[:S]
    sd = ref_c["step_decisive"]
    assert np.array_equal(al_c[sd], ref_c["accept_len"][sd]) and np.array_equal(al_c, an_c)
    # every row alone, batch-invariant: the same argmax as inside the batch
    wsp1 = binding.new_workspace(binding.lmhead_workspace_bytes(1))
    for m in sorted({0, M // 2, M - 1}):
        am1, al1, an1 = binding.lmhead_verify(xd[m:m + 1].contiguous(), wqd, wsd, g, None, 1, wsp1,
                                              token_map=md, flags=INV)
        torch.cuda.synchronize()
        assert int(am1.cpu()[0]) == int(out[INV][0][m]), f"row {m} alone differs from the batch"
        assert int(al1.cpu()[0]) == 0 and int(an1.cpu()[0]) == 0


SHAPES = [(5120, 5120, 0), (5120, 5120, 1), (17408, 5120, 2), (5120, 17408, 3)]


def build_pass(M, T, x_rows, rng_w, lm_v, flags, tree=None, token_map=None):
    """One layer's o/gate/down-like jobs plus an lm_head on the given X rows
    (dict K -> host bf16 bits [M][K]); weights drawn from rng_w."""
    gemms, host, ys = [], [], []
    xd = {k: dev_bf16(v) for k, v in x_rows.items()}
    for n, k, stage in SHAPES:
        wq, ws = synth.gen_weights(rng_w, n, k)
        g = synth.gen_gscale(rng_w)
        y = torch.full((M, n), float("nan"), dtype=torch.float32, device="cuda")
        gemms.append((xd[k], dev_u8(wq), dev_u8(ws), g, y, stage))
        host.append((wq, ws, g))
        ys.append(y)
    wq, ws = synth.gen_weights(rng_w, lm_v, 5120)
    g = synth.gen_gscale(rng_w)
    S = M // T
    am = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    al = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    an = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    td = dev_i32(tree[0]) if tree is not None else torch.zeros((S, 0), dtype=torch.int32, device="cuda")
    lm = (xd[5120], dev_u8(wq), dev_u8(ws), g, T, td, am, al)
    p = binding.Pass(gemms, M, lm, parents=dev_i32(tree[1]) if tree is not None else None,
                     token_map=dev_i32(token_map) if token_map is not None else None, accept_node=an,
                     flags=flags)
    return p, ys, (am, al, an), host, (wq, ws, g)


def test_pass_batch_invariant_rows_and_tree():
    print("[case] pass: invariant M=17 vs M=1, tree + map", flush=True)
    rng = np.random.default_rng(42000)
    x17 = {k: synth.gen_x(rng, 17, k) for k in (5120, 17408)}
    v = 20000
    seed_w = 42001
    token_map = (np.random.default_rng(42002).permutation(v) + 100000).astype(np.int32)
    # the lm_head weights are the 5th draw of the weight stream: recompute them for the oracle
    rng_w = np.random.default_rng(seed_w)
    for n, k, _ in SHAPES:
        synth.gen_weights(rng_w, n, k)
        synth.gen_gscale(rng_w)
    lwq, lws = synth.gen_weights(rng_w, v, 5120)
    lg = synth.gen_gscale(rng_w)
    base = oracle.lmhead_ref(x17[5120], lwq, lws, lg, T=1, token_map=token_map)
    tokens, parents = make_tree(rng, base["argmax"], token_map, 1, 17)
    ref = oracle.lmhead_ref(x17[5120], lwq, lws, lg, T=17, drafts=tokens, token_map=token_map,
                            parents=parents)

    p17, ys17, lm17, host, _ = build_pass(17, 17, x17, np.random.default_rng(seed_w), v, INV,
                                          (tokens, parents), token_map)
    p17.run_persistent()
    torch.cuda.synchronize()
    assert p17.check() == 0
    am, al, an = (t.cpu().numpy() for t in lm17)
    check_against_oracle(ref, am, al, an, token_map, "pass M=17")
    for (wq, ws, g), y, (n, k, _) in zip(host, ys17, SHAPES):
        y_ref, bound = oracle.nvfp4_gemm_ref(x17[k], wq, ws, g)
        ok, worst, at = within_bound(y.cpu().numpy(), y_ref, bound)
        assert ok, f"N={n} K={k}: worst err/bound {worst:.3g} at {at}"
    # the unfused schedule of the same pass gives the same bits
    first = [y.clone() for y in ys17] + [t.clone() for t in lm17]
    for y in ys17:
        y.fill_(float("nan"))
    p17.run_unfused()
    torch.cuda.synchronize()
    assert all(same_bits(a, b) if a.dtype == torch.float32 else torch.equal(a, b)
               for a, b in zip(first, [y for y in ys17] + list(lm17)))
    # row 0 alone, as an M = 1 batch-invariant pass: the same bits as in the 17-row pass
    x1 = {k: v_[:1].copy() for k, v_ in x17.items()}
    p1, ys1, lm1, _, _ = build_pass(1, 1, x1, np.random.default_rng(seed_w), v, INV, None, token_map)
    p1.run_persistent()
    torch.cuda.synchronize()
    assert p1.check() == 0
    for y1, y17 in zip(ys1, ys17):
        assert same_bits(y1[0], y17[0])
    assert int(lm1[0].cpu()[0]) == int(am[0])
    p1.close()
    p17.close()


@pytest.mark.parametrize("M", [1, 4, 17, 33, 52, 68])
def test_row_scales_stack_matrices_bitwise(M):
    """Two matrices stacked by rows as one job with per-row scales (each
    member's own tensor scale) give the same bits as two jobs, in every
    schedule (one persistent launch, one launch per stage, one launch per
    job, and vg_pass_run's choice), and lie within the
    oracle's bound with each member's own g.  K = 5120 and 17408 (the step
    kernel at M = 1; the LDS-shared MFMA item with one to five M-tiles
    above, the five-tile compact ring at M = 68, K slices dealt as separate
    items in the step) and K = 48 (the stream kernel's guarded path).  304
    rows keep the second member's code and scale rows 16-byte aligned at
    every K."""
    print(f"[case] row scales M={M}", flush=True)
    rng = np.random.default_rng(44000 + M)
    for k in (5120, 17408, 48):
        parts = [synth.gen_weights(rng, n, k) for n in (304, 208)]
        gs = [synth.gen_gscale(rng), synth.gen_gscale(rng)]
        xh = synth.gen_x(rng, M, k)
        x = dev_bf16(xh)
        wq = dev_u8(np.concatenate([p[0] for p in parts]))
        ws = dev_u8(np.concatenate([p[1] for p in parts]))
        rs = torch.cat([torch.full((304,), gs[0]), torch.full((208,), gs[1])]).float().cuda()
        ya = torch.empty((M, 304), device="cuda")
        yb = torch.empty((M, 208), device="cuda")
        yf = torch.empty((M, 512), device="cuda")
        sep = binding.Pass([(x, wq[:304], ws[:304], gs[0], ya, 0), (x, wq[304:], ws[304:], gs[1], yb, 0)], M)
        fus = binding.Pass([(x, wq, ws, 123.0, yf, 0, rs)], M)   # gscale ignored with row scales
        for run in ("run", "run_persistent", "run_staged", "run_unfused"):
            yf.fill_(float("nan"))
            getattr(sep, run)()
            getattr(fus, run)()
            torch.cuda.synchronize()
            assert sep.check() == 0 and fus.check() == 0, f"K={k} {run}: a stage wait timed out"
            assert same_bits(yf, torch.cat([ya, yb], 1)), f"K={k} {run}"
        yh = yf.cpu().numpy()
        c0 = 0
        for (pq, ps), g in zip(parts, gs):
            y_ref, bound = oracle.nvfp4_gemm_ref(xh, pq, ps, g)
            ok, worst, at = within_bound(yh[:, c0:c0 + pq.shape[0]], y_ref, bound)
            assert ok, f"K={k} member at column {c0}: worst err/bound {worst:.3g} at {at}"
            c0 += pq.shape[0]
        sep.close()
        fus.close()
