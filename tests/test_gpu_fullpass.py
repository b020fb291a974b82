"""The full 64-layer step at its real size (449 NVFP4 matrices, 14.1 GB,
generated on the device), in the launch configuration the benchmark times,
checked against the oracle on sampled outputs and on the complete lm_head
argmax / accept (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
from verify_gemm_amd import synth, weightpass

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def weights():
    w = weightpass.PassWeights("cuda")
    torch.cuda.synchronize()
    yield w
    del w
    torch.cuda.empty_cache()


def host_bits(x):
    return x.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("M", [1, 4, 17, 68])
def test_full_step_sampled(weights, M):
    print(f"[case] full step M={M}", flush=True)
    run = weightpass.PassRun(weights, M)
    run.run_persistent()
    torch.cuda.synchronize()
    assert run.check() == 0
    rng = np.random.default_rng(40000 + M)
    xs = {k: host_bits(v) for k, v in run.x.items()}
    picks = [0, 3, 4, 6, 7 * 31 + 1, 7 * 31 + 5, 7 * 63 + 2, 7 * 63 + 6]
    for idx in picks:
        m = weights.mats[idx]
        y = run.y[idx].cpu().numpy()
        rows = rng.integers(0, m["n"], 24)
        ms = rng.integers(0, M, 24)
        wq = m["wq"][torch.from_numpy(rows).cuda()].cpu().numpy()
        ws = m["ws"][torch.from_numpy(rows).cuda()].cpu().numpy()
        pairs = list(zip(ms.tolist(), rows.tolist()))
        ye, be = oracle.nvfp4_gemm_ref_entries(xs[m["k"]], wq, ws, m["g"], pairs)
        got = np.array([y[a, b] for a, b in pairs], dtype=np.float64)
        assert np.all(np.abs(got - ye) <= be), f"matrix {idx} ({m['name']}, layer {m['layer']})"
    # the one-launch-per-matrix and one-launch-per-stage schedules give the
    # same bits on every output
    first = [y.clone() for y in run.y] + [run.argmax.clone(), run.accept_len.clone()]
    for sched in (run.run_unfused, run.run_staged):
        for y in run.y:
            y.fill_(float("nan"))
        sched()
        torch.cuda.synchronize()
        again = [y for y in run.y] + [run.argmax, run.accept_len]
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b), sched.__name__
    run.close()


def test_full_step_lmhead_argmax_accept(weights):
    """M = 17 (16 drafts + 1): the complete lm_head argmax over 248,320 rows
    against the oracle; drafts follow the oracle's argmax with p = 0.7."""
    M = 17
    run = weightpass.PassRun(weights, M)
    lm = weights.lmhead
    x = host_bits(run.x[synth.HIDDEN])
    wq, ws = lm["wq"].cpu().numpy(), lm["ws"].cpu().numpy()
    ref = oracle.lmhead_ref(x, wq, ws, lm["g"], T=M)
    drafts = synth.gen_drafts(np.random.default_rng(41000), ref["argmax"].reshape(1, M), synth.VOCAB)
    run.set_drafts(torch.from_numpy(drafts).cuda())
    ref = oracle.lmhead_ref(x, wq, ws, lm["g"], T=M, drafts=drafts)
    run.run_persistent()
    torch.cuda.synchronize()
    assert run.check() == 0
    am = run.argmax.cpu().numpy()
    al = int(run.accept_len.cpu()[0])
    dec = ref["decisive"]
    assert np.array_equal(am[dec], ref["argmax"][dec])
    if ref["step_decisive"][0]:
        assert al == int(ref["accept_len"][0])
    print(f"full-step lm_head: decisive rows {int(dec.sum())}/17, accept_len {al} "
          f"(oracle {int(ref['accept_len'][0])})", flush=True)
    run.close()


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


@pytest.mark.parametrize("M", [1, 4, 17, 68])
def test_fused_projections_full_size(weights, M):
    """{q, k, v} and {gate, up} as one job each (257 jobs, each member's
    tensor scale kept as per-row scales): the same bits as the separate
    jobs, in vg_pass_run's schedule, one launch per job and one launch per
    stage; sampled fused outputs against the oracle."""
    print(f"[case] fused projections M={M}", flush=True)
    sep = weightpass.PassRun(weights, M)
    fus = weightpass.PassRun(weights, M, fused=True)
    assert fus.step.info()["jobs"] == 4 * weights.layers + 1
    sep.run_persistent()
    fus.run_persistent()
    torch.cuda.synchronize()
    assert sep.check() == 0 and fus.check() == 0
    for layer in range(weights.layers):
        s = sep.y[7 * layer:7 * layer + 7]
        f = fus.y[4 * layer:4 * layer + 4]
        assert torch.equal(_bits(f[0]), _bits(torch.cat(s[0:3], 1))), f"layer {layer} qkv"
        assert torch.equal(_bits(f[1]), _bits(s[3])), f"layer {layer} o"
        assert torch.equal(_bits(f[2]), _bits(torch.cat(s[4:6], 1))), f"layer {layer} gate|up"
        assert torch.equal(_bits(f[3]), _bits(s[6])), f"layer {layer} down"
    assert torch.equal(sep.argmax, fus.argmax) and torch.equal(sep.accept_len, fus.accept_len)
    rng = np.random.default_rng(43000 + M)
    xs = {k: host_bits(v) for k, v in fus.x.items()}
    for layer, gname, yi in [(0, "qkv", 0), (63, "gateup", 4 * 63 + 2)]:
        grp = weights.fused[layer][gname]
        members = [m for m in weights.mats if m["layer"] == layer and m["name"] in grp["members"]]
        y = fus.y[yi].cpu().numpy()
        r0 = 0
        for mem in members:   # each member's rows with its own tensor scale
            rows = rng.integers(0, mem["n"], 16)
            ms = rng.integers(0, M, 16)
            idx = torch.from_numpy(rows).cuda()
            wq, ws = mem["wq"][idx].cpu().numpy(), mem["ws"][idx].cpu().numpy()
            pairs = list(zip(ms.tolist(), rows.tolist()))
            ye, be = oracle.nvfp4_gemm_ref_entries(xs[grp["k"]], wq, ws, mem["g"], pairs)
            got = np.array([y[a, r0 + b] for a, b in pairs], dtype=np.float64)
            assert np.all(np.abs(got - ye) <= be), f"fused {gname} of layer {layer}, {mem['name']}"
            r0 += mem["n"]
    # the schedule vg_pass_run takes for this M (the one the benchmark
    # times), and the other one, give the same bits
    first = [y.clone() for y in fus.y] + [fus.argmax.clone(), fus.accept_len.clone()]
    for run in (fus.run, fus.run_unfused, fus.run_staged):
        for y in fus.y:
            y.fill_(float("nan"))
        run()
        torch.cuda.synchronize()
        assert fus.check() == 0
        assert all(torch.equal(_bits(a), _bits(b))
                   for a, b in zip(first, list(fus.y) + [fus.argmax, fus.accept_len]))
    sep.close()
    fus.close()
