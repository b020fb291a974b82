"""The lm_head verify pass: argmax per row, near-tie classification and the
greedy accept-prefix length.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed
----------------
Logits l[m, v] are the NVFP4 GEMM of ``oracle.nvfp4`` with N = V rows.
Row m's token is argmax_v l[m, v]; among equal maxima the LOWEST index wins
(the numpy/torch argmax convention; the pages do not say).

Speculative verify (TandemLLM README, introduction and "Architecture: the
parts"): drafters propose tokens, the target checks them all in one pass,
the longest prefix the target agrees with is kept, and at the first wrong
guess the target's own token is emitted instead.  With T rows per sequence
and drafts d[0..T-2], row j's argmax is the target's choice for the
position that draft d[j] fills, so

    accept_len = the largest L <= T-1 with d[j] == argmax[j] for all j < L.

The emitted bonus token is argmax[accept_len]; it is not a separate output.

Tree verify (TandemLLM README, the flow diagram and "The parts": the
drafters' guesses form a tree, the target verifies the whole tree in one
pass and keeps the longest path it agrees with): node 0 of a T-node tree is
the last committed position, node i >= 1 holds drafted token tokens[i-1]
below parent parents[i-1].  See ``tree_accept_ref``; a chain (parent of
node i is i-1) is the greedy rule above.

Sliced head (dgx-spark-qwen38 README, opening section: the draft gets the
target's lm_head cut to 65,536 rows, with a map from rows to token ids):
head row r stands for token token_map[r]; the argmax is taken over rows
(lowest row among equal maxima) and reported as its token id, which is
what drafts are compared with.
A batch of M = S*T rows holds S independent sequences in contiguous blocks
of T rows (ling-engine README, "Six levers": several sequences share one
weight read).

Exactness limit: the pages concede that a batched verify may round the
other way where the top two logits are within an ulp (TandemLLM README,
introduction).  A row is *decisive* iff the oracle's top-2 gap exceeds the
acceptance bound of both contenders; only decisive rows (and steps whose
compared rows are all decisive) must match exactly.  The stricter
interval-overlap test is available with ``interval=True``.
"""
from __future__ import annotations

import numpy as np

from .fp8 import fp8_dequant
from .nvfp4 import bf16_bits_to_f64, dequant, tolerance_bound


def top2_merge(v1, i1, v2, i2, c1, j1, c2, j2):
    """Merge a running (best, second) per row with a new chunk's (best,
    second), where every index of the chunk is larger than every index seen
    so far (chunks are visited in increasing index order).  Order is value
    descending, then index ascending, so on equal values the running
    entries win.  All arguments are arrays over rows."""
    take_c1 = c1 > v1
    nv1 = np.where(take_c1, c1, v1)
    ni1 = np.where(take_c1, j1, i1)
    # Candidates for second place: if the chunk's best took first place,
    # the old best (lower index) against the chunk's second; otherwise the
    # old second (lower index) against the chunk's best.
    a_v = np.where(take_c1, v1, v2)
    a_i = np.where(take_c1, i1, i2)
    b_v = np.where(take_c1, c2, c1)
    b_i = np.where(take_c1, j2, j1)
    take_b = b_v > a_v
    return nv1, ni1, np.where(take_b, b_v, a_v), np.where(take_b, b_i, a_i)


def _chunk_top2(logits: np.ndarray, base: int):
    """Best and second-best (value, global index) per row of one chunk;
    first occurrence wins among equal values."""
    rows = np.arange(logits.shape[0])
    a1 = np.argmax(logits, axis=1)
    v1 = logits[rows, a1]
    if logits.shape[1] < 2:
        return v1, a1 + base, np.full_like(v1, -np.inf), np.full_like(a1, -1)
    masked = logits.copy()
    masked[rows, a1] = -np.inf
    a2 = np.argmax(masked, axis=1)
    return v1, a1 + base, masked[rows, a2], a2 + base


def accept_len_ref(drafts: np.ndarray, argmax: np.ndarray) -> int:
    """Greedy accept: the number of leading positions where the draft equals
    the target's argmax.  drafts has T-1 entries, argmax has T."""
    drafts = np.asarray(drafts).reshape(-1)
    argmax = np.asarray(argmax).reshape(-1)
    if drafts.shape[0] != argmax.shape[0] - 1:
        raise ValueError("need T-1 drafts for T argmax rows")
    length = 0
    while length < drafts.shape[0] and int(drafts[length]) == int(argmax[length]):
        length += 1
    return length


def tree_accept_ref(tokens: np.ndarray, parents: np.ndarray, argmax: np.ndarray) -> tuple[int, int]:
    """The longest agreed root path of a draft tree.

    tokens[i-1] and parents[i-1] belong to node i (1 <= i < T); argmax[p]
    (T entries) is the target's token after node p.  Node i is agreed iff
    the walk from it to the root only uses valid parents (each in [0, c)
    for its child c) and every step c -> parent p on the way has
    tokens[c-1] == argmax[p]; the root is agreed.  Returns (depth, node):
    the largest number of edges on an agreed node's path, and the lowest
    such node (0 if only the root is agreed).  The bonus token is
    argmax[node].  Each node's path is walked on its own (no reuse between
    nodes), so the definition can be read off directly."""
    tokens = np.asarray(tokens).reshape(-1)
    parents = np.asarray(parents).reshape(-1)
    argmax = np.asarray(argmax).reshape(-1)
    t = argmax.shape[0]
    if tokens.shape[0] != t - 1 or parents.shape[0] != t - 1:
        raise ValueError("need T-1 tokens and T-1 parents for T argmax rows")
    best_depth, best_node = 0, 0
    for i in range(1, t):
        depth, c, agreed = 0, i, True
        while c != 0:
            p = int(parents[c - 1])
            if not (0 <= p < c) or int(tokens[c - 1]) != int(argmax[p]):
                agreed = False
                break
            depth += 1
            c = p
        if agreed and depth > best_depth:
            best_depth, best_node = depth, i
    return best_depth, best_node


def _compared_rows(tokens, parents, argmax) -> list[int]:
    """Rows whose argmax the tree rule compares with a child's token: every
    agreed node that is the (valid) parent of some node."""
    t = argmax.shape[0]
    rows = set()
    for i in range(1, t):
        p = int(parents[i - 1])
        if 0 <= p < i:
            # p is agreed iff its own path to the root agrees
            c, ok = p, True
            while c != 0:
                q = int(parents[c - 1])
                if not (0 <= q < c) or int(tokens[c - 1]) != int(argmax[q]):
                    ok = False
                    break
                c = q
            if ok:
                rows.add(p)
    return sorted(rows)


def _row_bound(ax_row: np.ndarray, deq, v: int) -> float:
    """Acceptance bound of logit (row, v): one dot product of |x| and |w_v|."""
    w = deq(v, v + 1)[0]
    return float(tolerance_bound(np.dot(ax_row, np.abs(w))))


def lmhead_ref(x_bits: np.ndarray, wq: np.ndarray, ws: np.ndarray, g: float,
               T: int, drafts: np.ndarray | None = None, *,
               token_map: np.ndarray | None = None, parents: np.ndarray | None = None,
               fp8: bool = False, interval: bool = False, row_chunk: int = 4096) -> dict:
    """Run the lm_head verify pass on the CPU.

    x_bits uint16[M][K] (bf16 bits), wq uint8[V][K/2], ws uint8[V][K/16],
    g the tensor scale (part of every logit).  With ``fp8`` the head is FP8
    (``oracle.fp8``): wq is uint8[V][K] E4M3 bytes and ws the per-row
    scales float[V] or None.  M must be a multiple of T;
    drafts int[M/T][T-1] or None (then no accept lengths are computed).
    token_map int[V] or None: head row r stands for token token_map[r]
    (``argmax`` then holds token ids, ``argmax_row`` the rows).  parents
    int[M/T][T-1] or None: drafts are the tokens of a tree (see
    ``tree_accept_ref``) instead of a chain; then ``accept_node`` is also
    returned.

    Returns a dict with per-row ``argmax`` (int32), ``top1``/``top2`` logits,
    ``idx2``, the bounds ``b1``/``b2`` of the two contenders and
    ``decisive`` (gap > max(b1, b2)); with drafts, per-sequence
    ``accept_len`` (int32) and ``step_decisive`` (every row the accept
    decision reads, 0..min(L, T-2), is decisive); with ``interval=True``
    also ``interval_decisive`` (l_top1 - b1 > max over v != top1 of l_v + b_v).
    """
    x = bf16_bits_to_f64(x_bits)
    m, _k = x.shape
    if T < 1 or m % T:
        raise ValueError("M must be a positive multiple of T")
    wq = np.asarray(wq, dtype=np.uint8)
    if fp8:
        rs = None if ws is None else np.asarray(ws, dtype=np.float32)

        def deq(r0, r1):
            return fp8_dequant(wq[r0:r1], None if rs is None else rs[r0:r1], g)
    else:
        ws = np.asarray(ws, dtype=np.uint8)

        def deq(r0, r1):
            return dequant(wq[r0:r1], ws[r0:r1], g)
    nv = wq.shape[0]
    v1 = np.full(m, -np.inf); i1 = np.full(m, -1, dtype=np.int64)
    v2 = np.full(m, -np.inf); i2 = np.full(m, -1, dtype=np.int64)
    for r0 in range(0, nv, row_chunk):
        r1 = min(nv, r0 + row_chunk)
        logits = x @ deq(r0, r1).T
        v1, i1, v2, i2 = top2_merge(v1, i1, v2, i2, *_chunk_top2(logits, r0))
    ax = np.abs(x)
    b1 = np.array([_row_bound(ax[r], deq, int(i1[r])) for r in range(m)])
    b2 = np.array([_row_bound(ax[r], deq, int(i2[r])) if i2[r] >= 0 else 0.0
                   for r in range(m)])
    ids = i1 if token_map is None else np.asarray(token_map, dtype=np.int64)[i1]
    out = {
        "argmax": ids.astype(np.int32),
        "argmax_row": i1.astype(np.int32),
        "top1": v1, "top2": v2, "idx2": i2.astype(np.int32),
        "b1": b1, "b2": b2,
        "decisive": (v1 - v2) > np.maximum(b1, b2),
    }
    if interval:
        hi_other = np.full(m, -np.inf)
        rows = np.arange(m)
        for r0 in range(0, nv, row_chunk):
            r1 = min(nv, r0 + row_chunk)
            w = deq(r0, r1)
            hi = x @ w.T + tolerance_bound(ax @ np.abs(w).T)
            inside = (i1 >= r0) & (i1 < r1)
            hi[rows[inside], i1[inside] - r0] = -np.inf
            hi_other = np.maximum(hi_other, hi.max(axis=1))
        out["interval_decisive"] = (v1 - b1) > hi_other
    if drafts is not None:
        s = m // T
        d = np.asarray(drafts, dtype=np.int64).reshape(s, T - 1)
        acc = np.empty(s, dtype=np.int32)
        node = np.empty(s, dtype=np.int32)
        step_dec = np.empty(s, dtype=bool)
        par = None if parents is None else np.asarray(parents, dtype=np.int64).reshape(s, T - 1)
        for q in range(s):
            rows_q = slice(q * T, (q + 1) * T)
            am_q = out["argmax"][rows_q]
            if par is None:
                acc[q] = accept_len_ref(d[q], am_q)
                node[q] = acc[q]
                last = min(int(acc[q]), T - 2)
                step_dec[q] = bool(np.all(out["decisive"][q * T:q * T + last + 1]))
            else:
                acc[q], node[q] = tree_accept_ref(d[q], par[q], am_q)
                cmp_rows = [q * T + r for r in _compared_rows(d[q], par[q], am_q)]
                step_dec[q] = bool(np.all(out["decisive"][cmp_rows])) if cmp_rows else True
        out["accept_len"] = acc
        out["accept_node"] = node
        out["step_decisive"] = step_dec
    return out
