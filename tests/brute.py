"""Brute-force MISA on tiny inputs: pure Python loops over Python floats.

Written independently of the numpy oracle (no shared helpers) so that it can
pin the oracle: every sum is an explicit loop, and every selection is a rank
count (an element is selected iff fewer than `count` elements beat it, where
"beat" means a larger value, or an equal value and a lower id).
"""
from __future__ import annotations

NEG_INF = float("-inf")


def dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def relu(x):
    return x if x > 0.0 else 0.0


def mean_rows(rows):
    d = len(rows[0])
    out = [0.0] * d
    for r in rows:
        for i in range(d):
            out[i] += r[i]
    return [v / len(rows) for v in out]


def beats(va, ia, vb, ib):
    """True if entry a is ranked before entry b."""
    return va > vb or (va == vb and ia < ib)


def rank_select(values, ids, count):
    """Selected ids in selection order, by explicit rank counting."""
    n = len(values)
    ranked = [None] * n
    for a in range(n):
        rank = 0
        for b in range(n):
            if b != a and beats(values[b], ids[b], values[a], ids[a]):
                rank += 1
        ranked[a] = rank
    out = [None] * min(count, n)
    for a in range(n):
        if ranked[a] < count:
            out[ranked[a]] = ids[a]
    return out


def bf_route(qt, wt, keys, t, B, h, tail_mode="pool", weight="signed", agg="sum"):
    """qt: list of H vectors; keys: list of vectors.  Returns S, r, heads (ascending).

    Readings: tail_mode "pool" (the partial last block is a block too) or
    "drop"; weight "signed" (w S), "abs" (|w| S) or "none" (S); agg "sum" or
    "max" over the blocks (0 with no block)."""
    L = t + 1
    n_full = L // B
    blocks = [mean_rows(keys[m * B:(m + 1) * B]) for m in range(n_full)]
    if n_full * B < L and tail_mode == "pool":
        blocks.append(mean_rows(keys[n_full * B:L]))
    S = []
    for qj in qt:
        acc = 0.0
        for kb in blocks:
            term = relu(dot(qj, kb))
            if agg == "sum":
                acc += term
            elif term > acc:
                acc = term
        S.append(acc)
    r = []
    for j in range(len(qt)):
        if weight == "signed":
            f = wt[j]
        elif weight == "abs":
            f = wt[j] if wt[j] >= 0.0 else -wt[j]
        else:
            f = 1.0
        r.append(f * S[j])
    heads = sorted(rank_select(r, list(range(len(qt))), h))
    return S, r, heads, blocks


def bf_score(qt, wt, keys, t, heads, n_cols):
    out = []
    for s in range(n_cols):
        if s > t:
            out.append(NEG_INF)
            continue
        acc = 0.0
        for j in sorted(heads):
            acc += wt[j] * relu(dot(qt[j], keys[s]))
        out.append(acc)
    return out


def bf_topk(values, ids, k):
    vals = [v for v, i in zip(values, ids) if i >= 0]
    idl = [i for i in ids if i >= 0]
    vals = [v + 0.0 for v in vals]
    sel = rank_select(vals, idl, k)
    return sel + [-1] * (k - len(sel))


def bf_misa(qt, wt, keys, t, B, h, k):
    S, r, heads, _ = bf_route(qt, wt, keys, t, B, h)
    I = bf_score(qt, wt, keys, t, heads, len(keys))
    idx = bf_topk(I[:t + 1], list(range(t + 1)), k)
    return heads, I, idx


def bf_dagger(qt, wt, keys, t, B, h, kp, k):
    heads, I, cand = bf_misa(qt, wt, keys, t, B, h, kp)
    allh = list(range(len(qt)))
    D = []
    for c in cand:
        if c < 0:
            D.append(NEG_INF)
        else:
            acc = 0.0
            for j in allh:
                acc += wt[j] * relu(dot(qt[j], keys[c]))
            D.append(acc)
    return bf_topk(D, cand, k)


def bf_dense_topk(qt, wt, keys, t, k):
    I = bf_score(qt, wt, keys, t, list(range(len(qt))), len(keys))
    return bf_topk(I[:t + 1], list(range(t + 1)), k)
