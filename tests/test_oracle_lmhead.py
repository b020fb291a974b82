"""Pins for the oracle's lm_head pass: argmax, top-2 / near-tie
classification and greedy accept (CPU only)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import exact_ref
import oracle
from verify_gemm_amd import synth


def _exact_logits(x, wq, ws, g):
    ys, abss = exact_ref.exact_gemm(x.tolist(), wq.tolist(), ws.tolist(), g)
    return ys, abss


def _lowest_index_max(row):
    best = max(row)
    return row.index(best)


@pytest.mark.parametrize("chunk", [1, 3, 7, 4096])
def test_argmax_and_top2_match_exact_brute_force(chunk):
    rng = np.random.default_rng(11)
    m, v, k = 4, 23, 32
    wq, ws = synth.gen_weights(rng, v, k)
    x = synth.gen_x(rng, m, k)
    r = oracle.lmhead_ref(x, wq, ws, 1.5, T=1, row_chunk=chunk)
    ys, abss = _exact_logits(x, wq, ws, 1.5)
    for i in range(m):
        row = ys[i]
        a = _lowest_index_max(row)
        assert r["argmax"][i] == a
        rest = [(val, j) for j, val in enumerate(row) if j != a]
        v2, j2 = sorted(rest, key=lambda t: (-t[0], t[1]))[0]
        assert r["idx2"][i] == j2
        assert r["top1"][i] == pytest.approx(float(row[a]), rel=1e-12, abs=1e-12)
        assert r["top2"][i] == pytest.approx(float(v2), rel=1e-12, abs=1e-12)
        b1 = 1e-3 * float(abss[i][a]) + 1e-6
        b2 = 1e-3 * float(abss[i][j2]) + 1e-6
        assert r["b1"][i] == pytest.approx(b1, rel=1e-12)
        assert r["b2"][i] == pytest.approx(b2, rel=1e-12)
        assert r["decisive"][i] == (float(row[a] - v2) > max(b1, b2))


@pytest.mark.parametrize("chunk", [1, 2, 5, 4096])
def test_ties_go_to_lowest_index_across_chunks(chunk):
    rng = np.random.default_rng(12)
    k = 32
    wq, ws = synth.gen_weights(rng, 9, k)
    # rows 2, 5 and 8 identical and dominant: force all-positive codes times positive x
    wq[[2, 5, 8]] = 0x77            # every element 6.0
    ws[[2, 5, 8]] = 0x48            # scale 4
    x = synth.f32_to_bf16_bits(np.ones((2, k), np.float32))
    r = oracle.lmhead_ref(x, wq, ws, 1.0, T=1, row_chunk=chunk)
    assert r["argmax"].tolist() == [2, 2]
    assert r["idx2"].tolist() == [5, 5]
    assert not r["decisive"].any()   # gap 0 is a near tie


def test_negative_zero_logits_tie_with_positive_zero():
    k = 16
    wq = np.array([[0x88] * 8, [0x00] * 8, [0x99] * 8], np.uint8)   # -0 codes, +0 codes, -0.5
    ws = np.full((3, 1), 0x38, np.uint8)
    x = synth.f32_to_bf16_bits(np.ones((1, k), np.float32))
    r = oracle.lmhead_ref(x, wq, ws, 1.0, T=1)
    assert r["argmax"].tolist() == [0]     # -0 == +0, the lower index wins
    assert r["idx2"].tolist() == [1]


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(-3, 3), min_size=2, max_size=12), st.integers(1, 5))
def test_top2_merge_matches_sort(vals, chunk):
    vals = [float(v) for v in vals]
    run = (np.array([-np.inf]), np.array([-1]), np.array([-np.inf]), np.array([-1]))
    for c0 in range(0, len(vals), chunk):
        seg = np.array([vals[c0:c0 + chunk]])
        cand = oracle.lmhead._chunk_top2(seg, c0)
        run = oracle.top2_merge(*run, *cand)
    order = sorted(range(len(vals)), key=lambda j: (-vals[j], j))
    assert int(run[1][0]) == order[0] and int(run[3][0]) == order[1]
    assert run[0][0] == vals[order[0]] and run[2][0] == vals[order[1]]


def test_accept_len_constructed():
    am = np.arange(100, 117)
    assert oracle.accept_len_ref(am[:16], am) == 16
    d = am[:16].copy(); d[0] = 7
    assert oracle.accept_len_ref(d, am) == 0
    for j in range(16):
        d = am[:16].copy(); d[j] = -1
        assert oracle.accept_len_ref(d, am) == j
    d = am[:16].copy(); d[3] = 0; d[9] = 0
    assert oracle.accept_len_ref(d, am) == 3
    assert oracle.accept_len_ref(np.zeros(0), np.array([5])) == 0


def test_accept_len_and_step_decisiveness_in_lmhead():
    rng = np.random.default_rng(13)
    t, s, v, k = 5, 3, 40, 32
    wq, ws = synth.gen_weights(rng, v, k)
    x = synth.gen_x(rng, t * s, k)
    base = oracle.lmhead_ref(x, wq, ws, 1.0, T=t)
    am = base["argmax"].reshape(s, t)
    drafts = am[:, :t - 1].copy()
    drafts[1, 2] = (drafts[1, 2] + 1) % v      # mismatch at j = 2
    drafts[2, 0] = (drafts[2, 0] + 1) % v      # mismatch at j = 0
    r = oracle.lmhead_ref(x, wq, ws, 1.0, T=t, drafts=drafts)
    assert r["accept_len"].tolist() == [t - 1, 2, 0]
    dec = r["decisive"].reshape(s, t)
    assert r["step_decisive"].tolist() == [bool(dec[0, :t - 1].all()), bool(dec[1, :3].all()),
                                           bool(dec[2, :1].all())]


def test_interval_decisive_matches_definition():
    rng = np.random.default_rng(14)
    m, v, k = 3, 17, 32
    wq, ws = synth.gen_weights(rng, v, k)
    x = synth.gen_x(rng, m, k)
    r = oracle.lmhead_ref(x, wq, ws, 1.0, T=1, interval=True, row_chunk=4)
    ys, abss = _exact_logits(x, wq, ws, 1.0)
    for i in range(m):
        a = _lowest_index_max(ys[i])
        lo = float(ys[i][a]) - (1e-3 * float(abss[i][a]) + 1e-6)
        hi = max(float(ys[i][j]) + 1e-3 * float(abss[i][j]) + 1e-6 for j in range(v) if j != a)
        assert r["interval_decisive"][i] == (lo > hi)
        # the interval test is at least as strict as the gap test
        assert (not r["interval_decisive"][i]) or r["decisive"][i]


def test_draft_generator_matches_target_with_p():
    rng = np.random.default_rng(15)
    am = rng.integers(0, 1000, (4000, 17))
    d = synth.gen_drafts(rng, am, 1000)
    frac = float(np.mean(d == am[:, :16]))
    assert 0.68 < frac < 0.72
