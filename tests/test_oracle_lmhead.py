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


# ---- tree verify and the sliced head --------------------------------------

def _agreed_forward(tokens, parents, argmax):
    """Agreed nodes by forward propagation from the root over child lists
    (the oracle walks each node up to the root instead)."""
    t = len(argmax)
    children = {p: [] for p in range(t)}
    for i in range(1, t):
        p = int(parents[i - 1])
        if 0 <= p < i:
            children[p].append(i)
    depth = {0: 0}
    frontier = [0]
    while frontier:
        nxt = []
        for p in frontier:
            for c in children[p]:
                if int(tokens[c - 1]) == int(argmax[p]):
                    depth[c] = depth[p] + 1
                    nxt.append(c)
        frontier = nxt
    best = max(depth.values())
    return best, min(n for n, d in depth.items() if d == best)


def test_tree_accept_hand_worked():
    # argmax of node p is the target's token after p
    am = [10, 20, 30, 40, 50, 60, 70, 80]
    # node:     1   2   3   4   5   6   7
    parents = [0, 0, 1, 1, 2, 3, 3]
    tokens = [10, 11, 20, 99, 30, 41, 40]
    # 1 agrees (10 == am[0]); 2 does not (11); 3 agrees below 1 (20 == am[1]);
    # 4 does not (99); 5 hangs below 2, which is not agreed; 6 does not (41 vs
    # am[3] = 40); 7 agrees below 3 (40) -> path 0-1-3-7 of depth 3, bonus am[7]
    assert oracle.lmhead.tree_accept_ref(tokens, parents, am) == (3, 7)
    # a second node at the same depth with a lower index wins the tie
    tokens_tie = [10, 11, 20, 99, 30, 40, 40]
    assert oracle.lmhead.tree_accept_ref(tokens_tie, parents, am) == (3, 6)
    # nothing agrees: only the root, depth 0, bonus am[0]
    assert oracle.lmhead.tree_accept_ref([1, 2, 3, 4, 5, 6, 7], parents, am) == (0, 0)


def test_tree_accept_invalid_parent_never_agrees():
    am = [5, 6, 7, 8]
    # node 2 names itself, node 3 a later node, as parent: neither can agree
    assert oracle.lmhead.tree_accept_ref([5, 6, 7], [0, 2, 3], am) == (1, 1)
    assert oracle.lmhead.tree_accept_ref([5, 5, 5], [-1, 0, 0], am) == (1, 2)
    # node 2 below the later node 3 (which agrees below the root) still fails
    assert oracle.lmhead.tree_accept_ref([5, 7, 5], [0, 3, 0], [5, 6, 7, 7]) == (1, 1)


@settings(max_examples=200, deadline=None)
@given(st.integers(0, 2**31 - 1))
def test_tree_accept_chain_is_greedy_accept(seed):
    rng = np.random.default_rng(seed)
    t = int(rng.integers(1, 18))
    am = rng.integers(0, 4, size=t)
    d = rng.integers(0, 4, size=t - 1)
    depth, node = oracle.lmhead.tree_accept_ref(d, np.arange(t - 1), am)
    assert depth == node == oracle.accept_len_ref(d, am)


@settings(max_examples=300, deadline=None)
@given(st.integers(0, 2**31 - 1))
def test_tree_accept_matches_forward_propagation(seed):
    rng = np.random.default_rng(seed)
    t = int(rng.integers(1, 24))
    am = rng.integers(0, 3, size=t)
    tokens = rng.integers(0, 3, size=t - 1)
    parents = np.array([rng.integers(-1, i + 1) for i in range(1, t)], dtype=np.int64)
    assert oracle.lmhead.tree_accept_ref(tokens, parents, am) == _agreed_forward(tokens, parents, am)


def test_star_tree_takes_lowest_agreeing_child():
    am = [3, 9, 9, 9, 9]
    assert oracle.lmhead.tree_accept_ref([1, 3, 2, 3], [0, 0, 0, 0], am) == (1, 2)


def test_lmhead_token_map_and_tree():
    rng = np.random.default_rng(21)
    m, v, k, t = 6, 40, 64, 6
    wq, ws = synth.gen_weights(rng, v, k)
    x = synth.gen_x(rng, m, k)
    base = oracle.lmhead_ref(x, wq, ws, 1.0, T=1)
    ident = oracle.lmhead_ref(x, wq, ws, 1.0, T=1, token_map=np.arange(v))
    assert np.array_equal(base["argmax"], ident["argmax"])
    perm = rng.permutation(v) + 1000
    mapped = oracle.lmhead_ref(x, wq, ws, 1.0, T=1, token_map=perm)
    assert np.array_equal(mapped["argmax_row"], base["argmax"])
    assert np.array_equal(mapped["argmax"], perm[base["argmax"]])
    # a chain given as parents gives the greedy result; a tree uses the rule
    am = mapped["argmax"]
    drafts = am[:t - 1].copy().reshape(1, t - 1)
    drafts[0, 3] += 1
    chain = oracle.lmhead_ref(x, wq, ws, 1.0, T=t, drafts=drafts, token_map=perm,
                              parents=np.arange(t - 1).reshape(1, t - 1))
    greedy = oracle.lmhead_ref(x, wq, ws, 1.0, T=t, drafts=drafts, token_map=perm)
    assert chain["accept_len"][0] == greedy["accept_len"][0] == 3
    star = np.zeros((1, t - 1), dtype=np.int64)
    tree = oracle.lmhead_ref(x, wq, ws, 1.0, T=t, drafts=np.full((1, t - 1), am[0]), token_map=perm,
                             parents=star)
    assert tree["accept_len"][0] == 1 and tree["accept_node"][0] == 1
