"""Planted mistakes: each plausible error in the oracle must make at least
one pin fail.  Mistakes are planted in the oracle on the CPU (monkeypatch),
never in the HIP path."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import lmhead as olm
from oracle import nvfp4 as onv
from verify_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(name):
    with open(os.path.join(GOLDEN, name)) as f:
        c = json.load(f)
    x = synth.f32_to_bf16_bits(np.array(c["x"], dtype=np.float32))
    wq = np.array([list(bytes.fromhex(h)) for h in c["wq_hex"]], dtype=np.uint8)
    ws = np.array([list(bytes.fromhex(h)) for h in c["ws_hex"]], dtype=np.uint8)
    return c, x, wq, ws


def pins_pass() -> bool:
    """The hand-worked cases, the spec's E2M1 value list and torch's E4M3
    decoder, evaluated against the (possibly mutated) oracle."""
    for name in ("case_a_1x16.json", "case_b_2x32.json"):
        c, x, wq, ws = _case(name)
        y, b = onv.nvfp4_gemm_ref(x, wq, ws, c["g"])
        if not np.array_equal(y, np.array(c["y"])):
            return False
        if not np.allclose(b, 1e-3 * np.array(c["abs_sum"]) + 1e-6, rtol=1e-15, atol=0):
            return False
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    t = onv.e2m1_table()
    if t[:8].tolist() != mags or t[8:].tolist() != [-v for v in mags]:
        return False
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = onv.e4m3_table()
    fin = ~np.isnan(ref)
    if not (np.array_equal(np.isnan(ours), ~fin) and np.array_equal(ours[fin], ref[fin])):
        return False
    return True


def test_unmutated_oracle_passes():
    assert pins_pass()


def _swap_nibbles(wq):
    wq = np.asarray(wq, dtype=np.uint8)
    codes = np.empty((wq.shape[0], 2 * wq.shape[1]), np.uint8)
    codes[:, 0::2] = wq >> 4
    codes[:, 1::2] = wq & 15
    return codes


MUTATIONS = {}


def mutation(fn):
    MUTATIONS[fn.__name__] = fn
    return fn


@mutation
def nibble_order_swapped(mp):
    mp.setattr(onv, "unpack_codes", _swap_nibbles)


@mutation
def e2m1_sign_dropped(mp):
    mp.setattr(onv, "_E2M1", np.abs(onv.e2m1_table()))
    mp.setattr(onv, "e2m1_table", lambda: np.abs(np.array([math.fabs(onv.e2m1_value(c)) for c in range(16)])))


@mutation
def e2m1_subnormal_wrong(mp):
    t = onv.e2m1_table().copy(); t[1] = 1.0; t[9] = -1.0
    mp.setattr(onv, "_E2M1", t)


@mutation
def e4m3_bias_off_by_one(mp):
    t = onv.e4m3_table() * 2.0
    mp.setattr(onv, "_E4M3", t)
    mp.setattr(onv, "e4m3_table", lambda: t)


@mutation
def e4m3_subnormal_scale_wrong(mp):
    t = onv.e4m3_table().copy()
    sub = [b for b in range(256) if (b >> 3) & 15 == 0]
    t[sub] = t[sub] / 2.0
    mp.setattr(onv, "_E4M3", t)
    mp.setattr(onv, "e4m3_table", lambda: t)


@mutation
def scale_block_index_transposed(mp):
    orig = onv.dequant

    def bad(wq, ws, g):
        ws = np.asarray(ws)
        return orig(wq, ws.T.reshape(ws.shape) if ws.shape[0] == ws.shape[1] else ws[:, ::-1], g)
    mp.setattr(onv, "dequant", bad)


@mutation
def gscale_dropped(mp):
    orig = onv.dequant
    mp.setattr(onv, "dequant", lambda wq, ws, g: orig(wq, ws, 1.0))


@mutation
def bound_uses_signed_sum(mp):
    def bad(x_bits, wq, ws, g, *, with_bound=True, row_chunk=4096):
        x = onv.bf16_bits_to_f64(x_bits)
        w = onv.dequant(wq, ws, g)
        y = x @ w.T
        return y, onv.tolerance_bound(np.abs(y))
    mp.setattr(onv, "nvfp4_gemm_ref", bad)


@mutation
def operand_transposed(mp):
    def bad(x_bits, wq, ws, g, *, with_bound=True, row_chunk=4096):
        x = onv.bf16_bits_to_f64(x_bits)
        w = onv.dequant(wq, ws, g)
        y = (x[:, ::-1] @ w.T)
        return y, onv.tolerance_bound(np.abs(x) @ np.abs(w).T)
    mp.setattr(onv, "nvfp4_gemm_ref", bad)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    MUTATIONS[name](monkeypatch)
    assert not pins_pass(), f"mutation {name} slipped past every pin"


def test_planted_argmax_tie_rule_is_caught(monkeypatch):
    """Highest-index-wins on ties must fail the tie pin."""
    def bad_chunk_top2(logits, base):
        flipped = logits[:, ::-1]
        a1 = logits.shape[1] - 1 - np.argmax(flipped, axis=1)
        rows = np.arange(logits.shape[0])
        v1 = logits[rows, a1]
        masked = logits.copy(); masked[rows, a1] = -np.inf
        a2 = np.argmax(masked, axis=1)
        return v1, a1 + base, masked[rows, a2], a2 + base
    monkeypatch.setattr(olm, "_chunk_top2", bad_chunk_top2)
    k = 32
    rng = np.random.default_rng(12)
    wq, ws = synth.gen_weights(rng, 9, k)
    wq[[2, 5, 8]] = 0x77; ws[[2, 5, 8]] = 0x48
    x = synth.f32_to_bf16_bits(np.ones((1, k), np.float32))
    r = olm.lmhead_ref(x, wq, ws, 1.0, T=1, row_chunk=4096)
    assert r["argmax"].tolist() != [2]


def test_planted_accept_off_by_one_is_caught(monkeypatch):
    def bad(drafts, argmax):
        n = 0
        while n < len(drafts) and int(drafts[n]) == int(argmax[n + 1]):
            n += 1
        return n
    am = np.arange(100, 117)
    assert bad(am[:16], am) != 16       # the constructed pin would fail
    assert oracle.accept_len_ref(am[:16], am) == 16


# ---- tree accept: plausible wrong rules must fail the tree pins ------------

def tree_pins_pass(fn) -> bool:
    """The hand-worked tree, the tie rule, the invalid-parent rule and the
    chain reduction, evaluated on a candidate tree-accept function."""
    am = [10, 20, 30, 40, 50, 60, 70, 80]
    parents = [0, 0, 1, 1, 2, 3, 3]
    if fn([10, 11, 20, 99, 30, 41, 40], parents, am) != (3, 7):
        return False
    if fn([10, 11, 20, 99, 30, 40, 40], parents, am) != (3, 6):
        return False
    if fn([5, 6, 7], [0, 2, 3], [5, 6, 7, 8]) != (1, 1):
        return False
    # node 2 hangs below the later node 3, whose own path agrees
    if fn([5, 7, 5], [0, 3, 0], [5, 6, 7, 7]) != (1, 1):
        return False
    rng = np.random.default_rng(5)
    for _ in range(50):
        t = int(rng.integers(2, 12))
        a = rng.integers(0, 3, size=t)
        d = rng.integers(0, 3, size=t - 1)
        if fn(d, np.arange(t - 1), a)[0] != olm.accept_len_ref(d, a):
            return False
    return True


def _walk_tree(rule):
    """A tree accept built like the oracle's but with `rule(c, p, tokens,
    argmax, parents)` deciding whether the step c -> p agrees, and ties
    going by `tie`."""
    def fn(tokens, parents, argmax, tie_high=False, count_nodes=False):
        tokens, parents, argmax = (np.asarray(v).reshape(-1) for v in (tokens, parents, argmax))
        best = (0, 0)
        for i in range(1, argmax.shape[0]):
            depth, c, ok = 0, i, True
            while c != 0 and depth <= argmax.shape[0]:   # bounded: a mutant may follow a cycle
                p = int(parents[c - 1])
                if not rule(c, p, tokens, argmax):
                    ok = False
                    break
                depth += 1
                c = p
            depth += 1 if (count_nodes and ok) else 0
            if ok and (depth > best[0] or (tie_high and depth == best[0] and depth > 0)):
                best = (depth, i)
        return best
    return fn


def test_tree_pins_pass_for_the_oracle():
    assert tree_pins_pass(olm.tree_accept_ref)


@pytest.mark.parametrize("mutant", ["child_argmax", "no_parent_check", "tie_high", "count_nodes"])
def test_planted_tree_mistake_is_caught(mutant):
    good = lambda c, p, t, a: 0 <= p < c and int(t[c - 1]) == int(a[p])
    if mutant == "child_argmax":      # compares with the child's own row
        fn = _walk_tree(lambda c, p, t, a: 0 <= p < c and int(t[c - 1]) == int(a[c]))
    elif mutant == "no_parent_check":  # follows parents that do not precede the child
        fn = _walk_tree(lambda c, p, t, a: -1 < p < len(a) and p != c and int(t[c - 1]) == int(a[p]))
    elif mutant == "tie_high":
        base = _walk_tree(good)
        fn = lambda t, p, a: base(t, p, a, tie_high=True)
    else:
        base = _walk_tree(good)
        fn = lambda t, p, a: base(t, p, a, count_nodes=True)
    assert not tree_pins_pass(fn)
