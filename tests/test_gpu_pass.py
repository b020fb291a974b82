"""GPU parity of the step executor (vg_pass_*): a whole step as one
persistent launch, checked job by job against the CPU oracle, against the
one-launch-per-matrix schedule (bitwise), across repeated launches and graph
replays (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_bf16, dev_i32, dev_u8, within_bound
from verify_gemm_amd import binding, synth

pytestmark = pytest.mark.gpu


def build(M, T, specs, lm_spec, seed):
    """specs: list of (N, K, stage); lm_spec: (V, K) or None."""
    rng = np.random.default_rng(seed)
    host, gemms, ys = [], [], []
    xs = {}
    for n, k, stage in specs:
        if k not in xs:
            xs[k] = synth.gen_x(rng, M, k)
        wq, ws = synth.gen_weights(rng, n, k)
        g = synth.gen_gscale(rng)
        y = torch.full((M, n), float("nan"), dtype=torch.float32, device="cuda")
        host.append((xs[k], wq, ws, g))
        ys.append(y)
        gemms.append((None, dev_u8(wq), dev_u8(ws), g, y, stage))
    xd = {k: dev_bf16(v) for k, v in xs.items()}
    gemms = [(xd[specs[i][1]],) + gemms[i][1:] for i in range(len(gemms))]
    lm = None
    lmhost = None
    if lm_spec is not None:
        v, k = lm_spec
        if k not in xs:
            xs[k] = synth.gen_x(rng, M, k)
            xd[k] = dev_bf16(xs[k])
        wq, ws = synth.gen_weights(rng, v, k)
        g = synth.gen_gscale(rng)
        ref = oracle.lmhead_ref(xs[k], wq, ws, g, T=T)
        drafts = ref["argmax"].reshape(M // T, T)[:, :T - 1].copy()
        for q in range(M // T):                       # a mismatch at a random position
            j = int(rng.integers(0, T))
            if j < T - 1:
                drafts[q, j] = (drafts[q, j] + 1) % v
        am = torch.full((M,), -7, dtype=torch.int32, device="cuda")
        al = torch.full((M // T,), -7, dtype=torch.int32, device="cuda")
        dd = dev_i32(drafts) if T > 1 else torch.zeros((M // T, 0), dtype=torch.int32, device="cuda")
        lm = (xd[k], dev_u8(wq), dev_u8(ws), g, T, dd, am, al)
        lmhost = (xs[k], wq, ws, g, drafts)
    p = binding.Pass(gemms, M, lm)
    return p, host, ys, lm, lmhost


def check_outputs(M, T, host, ys, lm, lmhost, label):
    for i, ((x, wq, ws, g), y) in enumerate(zip(host, ys)):
        y_ref, bound = oracle.nvfp4_gemm_ref(x, wq, ws, g)
        ok, worst, at = within_bound(y.cpu().numpy(), y_ref, bound)
        assert ok, f"{label} job {i} N={wq.shape[0]} K={x.shape[1]}: worst err/bound {worst:.3g} at {at}"
    if lm is not None:
        x, wq, ws, g, drafts = lmhost
        ref = oracle.lmhead_ref(x, wq, ws, g, T=T, drafts=drafts if T > 1 else None)
        am = lm[6].cpu().numpy()
        al = lm[7].cpu().numpy()
        dec = ref["decisive"]
        assert np.array_equal(am[dec], ref["argmax"][dec]), f"{label}: lm_head argmax"
        if T > 1:
            sd = ref["step_decisive"]
            assert np.array_equal(al[sd], ref["accept_len"][sd]), f"{label}: accept_len"
        else:
            assert np.all(al == 0)


def snapshot(ys, lm):
    out = [y.clone() for y in ys]
    if lm is not None:
        out += [lm[6].clone(), lm[7].clone()]
    return out


def same(a, b):
    return all(torch.equal(u.view(torch.int32) if u.dtype == torch.float32 else u,
                           v.view(torch.int32) if v.dtype == torch.float32 else v) for u, v in zip(a, b))


LAYER = [(5120, 5120, 0), (5120, 5120, 0), (5120, 5120, 0), (5120, 5120, 1),
         (17408, 5120, 2), (17408, 5120, 2), (5120, 17408, 3)]


@pytest.mark.parametrize("M,T", [(1, 1), (4, 1), (17, 17), (68, 17)])
def test_one_layer_step(M, T):
    print(f"[case] one-layer step M={M} T={T}", flush=True)
    p, host, ys, lm, lmhost = build(M, T, LAYER, (20000, 5120), 31000 + M)
    info = p.info()
    assert info["jobs"] == 8 and info["stages"] == 5
    p.run_persistent()
    torch.cuda.synchronize()
    assert p.check() == 0
    check_outputs(M, T, host, ys, lm, lmhost, f"M={M}")
    first = snapshot(ys, lm)
    # repeated launches: the control block resets itself
    for _ in range(3):
        p.run_persistent()
    torch.cuda.synchronize()
    assert p.check() == 0
    assert same(first, snapshot(ys, lm))
    # the one-launch-per-matrix schedule computes the same bits
    for y in ys:
        y.fill_(float("nan"))
    p.run_unfused()
    torch.cuda.synchronize()
    assert same(first, snapshot(ys, lm))
    # so does the one-launch-per-stage schedule (q, k, v in one launch)
    for y in ys:
        y.fill_(float("nan"))
    p.run_staged()
    torch.cuda.synchronize()
    assert same(first, snapshot(ys, lm))
    p.close()


@pytest.mark.parametrize("M,T", [(1, 1), (4, 1), (17, 17), (68, 17)])
def test_default_schedule_same_bits(M, T):
    """vg_pass_run takes the persistent launch at M = 1 and one launch per
    stage (narrow matrices sliced) above: the same bits as the persistent
    launch at every M."""
    print(f"[case] default schedule M={M}", flush=True)
    p, host, ys, lm, lmhost = build(M, T, LAYER, (20000, 5120), 36000 + M)
    p.run_persistent()
    torch.cuda.synchronize()
    assert p.check() == 0
    first = snapshot(ys, lm)
    for y in ys:
        y.fill_(float("nan"))
    p.run()
    torch.cuda.synchronize()
    assert p.check() == 0
    assert same(first, snapshot(ys, lm))
    p.close()


SPREAD = [(1280, 17408, 0), (333, 5120, 1), (4096, 1024, 2), (16640, 5120, 3)]


def sliced_items(blocks, k, grid):
    """Items of a one-job stage of `blocks` 64-row blocks under the step's
    slicing rule: S = clamp(W // 4, 1, 3) slices of the W = ceil(K/256)
    windows; all blocks sliced when fewer than the compute units (`grid`)
    and estimated faster, else the blocks past the last whole round."""
    w = -(-k // 256)
    s = min(3, max(1, w // 4))
    whole = -(-blocks // grid) * w
    slice_w = -(-w // s) + 1
    cut = 0
    if s > 1:
        if blocks < grid:
            cut = blocks if -(-(blocks * s) // grid) * slice_w * 5 < whole * 4 else 0
        elif blocks % grid:
            r = blocks % grid
            cut = r if blocks // grid * w + -(-(r * s) // grid) * slice_w < whole else 0
    return blocks + cut * (s - 1)


@pytest.mark.parametrize("M", [2, 17, 68])
def test_spread_slices(M):
    """The step deals blocks of the M >= 2 MFMA item as K slices, one item
    per slice, where that balances a stage better: every block of a narrow
    matrix (1280 x 17408, 333 x 5120; 4096 x 1024 has K too short to slice;
    the lm_head 1000 x 2048), or only the blocks past the last whole round
    of a wide one (16640 x 5120: 260 blocks).  The slice sums are added in
    slice order by the workgroup that completes a block.  The item count
    shows the schedule; the bits equal the one-launch-per-matrix schedule,
    where one workgroup runs every slice of a block; repeated launches (the
    per-block counts reset themselves) give the same bits; every output is
    within the oracle's bound."""
    print(f"[case] spread slices M={M}", flush=True)
    p, host, ys, lm, lmhost = build(M, 1, SPREAD, (1000, 2048), 33000 + M)
    info = p.info()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert info["grid"] >= cus
    want = sum(sliced_items(-(-n // 64), k, cus) for n, k, _ in SPREAD) + sliced_items(-(-1000 // 64), 2048, cus)
    assert info["items"] == want
    p.run_persistent()
    torch.cuda.synchronize()
    assert p.check() == 0
    check_outputs(M, 1, host, ys, lm, lmhost, f"spread M={M}")
    first = snapshot(ys, lm)
    for _ in range(3):
        p.run_persistent()
    torch.cuda.synchronize()
    assert p.check() == 0
    assert same(first, snapshot(ys, lm))
    for y in ys:
        y.fill_(float("nan"))
    p.run_unfused()
    torch.cuda.synchronize()
    assert same(first, snapshot(ys, lm))
    # one launch per stage: the step's slices, the per-block counts reset
    for _ in range(2):
        for y in ys:
            y.fill_(float("nan"))
        p.run_staged()
        torch.cuda.synchronize()
        assert same(first, snapshot(ys, lm))
    p.close()


ODD = [(77, 48, 0), (300, 1040, 0), (1, 2048, 1), (129, 272, 2), (64, 1024, 2), (200, 5120, 3)]


@pytest.mark.parametrize("M,T", [(1, 1), (2, 2), (17, 17), (34, 17), (68, 4)])
def test_odd_shapes_step(M, T):
    print(f"[case] odd-shape step M={M} T={T}", flush=True)
    p, host, ys, lm, lmhost = build(M, T, ODD, (1000, 2048), 32000 + M)
    p.run_persistent()
    torch.cuda.synchronize()
    assert p.check() == 0
    check_outputs(M, T, host, ys, lm, lmhost, f"odd M={M}")
    first = snapshot(ys, lm)
    p.run_unfused()
    torch.cuda.synchronize()
    assert same(first, snapshot(ys, lm))
    # one launch per stage: stages of jobs with different K (and K not a
    # multiple of 128) in one launch
    for y in ys:
        y.fill_(float("nan"))
    p.run_staged()
    torch.cuda.synchronize()
    assert same(first, snapshot(ys, lm))
    p.close()


# A stage whose matrices stay spread over the whole grid at M = 1: giving
# them their own runs of workgroups would leave the largest share above
# 33/32 of the even split's (on 256 workgroups).  The first matrix's 235
# extra rows end at workgroup 235, where the 300-row matrix's extra rows
# start, wrapping past the last workgroup to the first ones.
EVEN_ROTATED = [(491, 1024, 0), (768, 1024, 0), (300, 64, 0), (129, 1024, 1)]


def test_step_stage_spread_over_grid():
    print("[case] rotated even split M=1", flush=True)
    p, host, ys, lm, lmhost = build(1, 1, EVEN_ROTATED, (500, 1024), 38000)
    p.run_persistent()
    torch.cuda.synchronize()
    assert p.check() == 0
    check_outputs(1, 1, host, ys, lm, lmhost, "rotated even split M=1")
    first = snapshot(ys, lm)
    for sched in (p.run_unfused, p.run):
        for y in ys:
            y.fill_(float("nan"))
        sched()
        torch.cuda.synchronize()
        assert same(first, snapshot(ys, lm)), sched.__name__
    p.close()


def _selection_weights(n, k, rng):
    """NVFP4 weights [n][k] whose row r is 1.0 at one column col[r] (E2M1
    code 2; every E4M3 block scale 1.0, 0x38) and 0 elsewhere: with gscale
    1, Y[m][r] = X[m][col[r]] exactly."""
    col = rng.permutation(k)[:n]
    wq = np.zeros((n, k // 2), np.uint8)
    for r, c in enumerate(col):
        wq[r, c // 2] = 2 if c % 2 == 0 else 2 << 4   # element 2j: the low nibble of byte j
    ws = np.full((n, k // 16), 0x38, np.uint8)
    return wq, ws, col


def _as_activations(x_bits, col):
    """The bf16 row that Y[m][r] = x[m][col[r]] (fp32, little-endian) reads
    as: each float's low half (zero: x is bf16) then its high half."""
    out = np.zeros((x_bits.shape[0], 2 * len(col)), np.uint16)
    out[:, 1::2] = x_bits[:, col]
    return out


@pytest.mark.parametrize("M", [1, 17])
def test_stage_reads_what_an_earlier_stage_wrote(M):
    """The stage contract with aliasing: stage 0 writes a buffer whose bytes
    stage 1 reads as its activations; stage 2 writes the same buffer again
    from other inputs and stage 3 reads it -- in one launch at M = 1, and
    in every schedule.  A stage that read a stale copy of the buffer (what
    stage 0 wrote, still cached from stage 1) would give stage 3 stage 1's
    results."""
    print(f"[case] chained stages through one buffer M={M}", flush=True)
    rng = np.random.default_rng(39000 + M)
    k0, k1, n1 = 1024, 2048, 300
    wsel, ssel, col = _selection_weights(k1 // 2, k0, rng)
    xs = []
    for _ in range(2):
        x = synth.gen_x(rng, M, k0)
        x[(x & 0x7FFF) == 0] = 0x3F80                 # no signed zeros: 0 + (-0) would read back as +0
        xs.append(x)
    w1, s1 = synth.gen_weights(rng, n1, k1)
    g1 = 0.75
    buf = torch.full((M, k1 // 2), float("nan"), dtype=torch.float32, device="cuda")
    xbuf = buf.view(torch.bfloat16)                   # [M][k1]: the same bytes
    y1 = torch.empty((M, n1), dtype=torch.float32, device="cuda")
    y2 = torch.empty((M, n1), dtype=torch.float32, device="cuda")
    sel_q, sel_s, q1, sc1 = dev_u8(wsel), dev_u8(ssel), dev_u8(w1), dev_u8(s1)
    gemms = [(dev_bf16(xs[0]), sel_q, sel_s, 1.0, buf, 0), (xbuf, q1, sc1, g1, y1, 1),
             (dev_bf16(xs[1]), sel_q, sel_s, 1.0, buf, 2), (xbuf, q1, sc1, g1, y2, 3)]
    p = binding.Pass(gemms, M, None)
    refs = [oracle.nvfp4_gemm_ref(_as_activations(x, col), w1, s1, g1) for x in xs]
    for sched in (p.run, p.run_persistent, p.run_staged, p.run_unfused):
        for y in (y1, y2):
            y.fill_(float("nan"))
        sched()
        torch.cuda.synchronize()
        assert p.check() == 0
        assert np.array_equal(xbuf.cpu().view(torch.int16).numpy().view(np.uint16), _as_activations(xs[1], col))
        for y, (y_ref, bound), name in ((y1, refs[0], "stage 1"), (y2, refs[1], "stage 3")):
            ok, worst, at = within_bound(y.cpu().numpy(), y_ref, bound)
            assert ok, f"{sched.__name__} {name}: worst err/bound {worst:.3g} at {at}"
    p.close()


WIDE = [(640, 1024, 0), (64, 1024, 0), (1000, 1024, 0), (1, 1024, 0), (300, 1024, 0), (128, 2048, 1),
        (2049, 1024, 2)]


@pytest.mark.parametrize("M", [1, 2, 17, 33])
def test_many_jobs_in_one_stage(M):
    """A stage of five matrices of different heights (one of a single row):
    at M >= 2 the per-stage schedule launches them together, their blocks in
    list order; at M = 1 the step kernel gives each matrix its own run of
    workgroups (the one-row matrix a single workgroup).  The bits equal the
    other schedules', and every output is within the oracle's bound."""
    print(f"[case] five-job stage M={M}", flush=True)
    p, host, ys, lm, lmhost = build(M, 1, WIDE, (700, 1024), 37000 + M)
    p.run_persistent()
    torch.cuda.synchronize()
    assert p.check() == 0
    check_outputs(M, 1, host, ys, lm, lmhost, f"five-job stage M={M}")
    first = snapshot(ys, lm)
    for sched in (p.run_staged, p.run_unfused, p.run):
        for y in ys:
            y.fill_(float("nan"))
        sched()
        torch.cuda.synchronize()
        assert same(first, snapshot(ys, lm)), sched.__name__
    p.close()


@pytest.mark.parametrize("M", [1, 17])
def test_step_without_lmhead_and_lmhead_only(M):
    p, host, ys, lm, lmhost = build(M, 1, LAYER[:4], None, 33000 + M)
    p.run_persistent()
    torch.cuda.synchronize()
    check_outputs(M, 1, host, ys, None, None, "no lm_head")
    p.close()
    T = M
    p, host, ys, lm, lmhost = build(M, T, [], (70000, 5120), 34000 + M)
    p.run_persistent()
    torch.cuda.synchronize()
    assert p.check() == 0
    check_outputs(M, T, host, ys, lm, lmhost, "lm_head only")
    p.close()


@pytest.mark.parametrize("M,T,sched", [(1, 1, "run_persistent"), (17, 17, "run_persistent"), (17, 17, "run"),
                                       (68, 17, "run"), (17, 17, "run_staged")])
def test_step_graph_replay(M, T, sched):
    """The step (one persistent launch, or the default schedule: one launch
    per stage at M >= 2, narrow matrices sliced) captured in a graph and
    replayed, with eager work and synchronisation between replays: every
    replay equals the eager run."""
    print(f"[case] graph replay M={M} {sched}", flush=True)
    p, host, ys, lm, lmhost = build(M, T, LAYER[:4], (9000, 5120), 35000 + M)
    getattr(p, sched)()
    torch.cuda.synchronize()
    eager = snapshot(ys, lm)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            getattr(p, sched)()
    torch.cuda.synchronize()
    for rep in range(4):
        for y in ys:
            y.fill_(0.0)
        lm[6].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same(eager, snapshot(ys, lm)), f"replay {rep}"
    assert p.check() == 0
    p.close()
