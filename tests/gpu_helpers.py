"""Helpers of the GPU parity tests: upload generator inputs, tolerance and
selection-band checks (no indexer arithmetic here)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import long_context_sparse_block_amd as lcsb
import oracle

# Logits: bf16 inputs, fp32 accumulation -> within 1e-2 relative.  Near zero,
# where the signed head sum cancels, the scale is the row's magnitude:
#     |g - o| <= 1e-2 * max(|o|, 1e-3 * max_s |o[s]|)
REL_TOL = 1e-2
ROW_FLOOR = 1e-3
# Selections: element margins beyond 1e-2 |v| + 1e-6 rowmax around the
# boundary value v must be decided like the oracle decides them.
BAND_REL = 1e-2
BAND_ROW = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    return torch.device("cuda:0")


def upload(inp):
    dev = device()
    q = torch.from_numpy(inp.q.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(inp.w).to(dev)
    if inp.k_scale is None:
        k = torch.from_numpy(inp.k.view(np.int16)).to(dev).view(torch.bfloat16)
        ks = None
    else:
        k = torch.from_numpy(inp.k).to(dev)
        ks = torch.from_numpy(inp.k_scale).to(dev)
    return dict(q=q, w=w, k=k, k_scale=ks)


def shape_of(inp):
    c = inp.cfg
    return lcsb.make_shape(c.n_seq, c.q_per_seq, c.n_keys, inp.q_pos0, c.n_heads, c.block)


def logits_close(g: np.ndarray, o: np.ndarray):
    """g (fp32 from GPU) vs o (fp64 oracle), same shape; -inf must match exactly.
    Returns (ok, worst relative error in the tolerance's own scale)."""
    g = g.astype(np.float64)
    ninf_o = np.isneginf(o)
    if not np.array_equal(np.isneginf(g), ninf_o):
        return False, float("inf")
    fin = ~ninf_o
    if not fin.any():
        return True, 0.0
    of, gf = np.where(fin, o, 0.0), np.where(fin, g, 0.0)
    rowmax = np.abs(of).max(axis=-1, keepdims=True)
    scale = np.maximum(np.abs(of), ROW_FLOOR * rowmax)
    scale = np.where(scale > 0, scale, 1.0)
    err = np.abs(gf - of) / scale
    worst = float(err[fin].max())
    return worst <= REL_TOL, worst


# fp8 x fp8 matrix cores do not accumulate a dot product in fp32: the result
# of v_mfma_f32_16x16x128_f8f6f4 is off by up to about 2^-14 of the sum of the
# |products| (measured), as on other fp8 tensor hardware.  The stated 1e-2
# relative bound is for bf16 inputs with fp32 accumulation; for the fp8-query
# kernels the bound is derived from that accumulation instead: each head's
# dot product may be off by EPS_F8 * sum_i |q_ji k_si| (4x the measured
# error; ReLU does not enlarge it), and the fp32 head sum adds a few
# roundings of its terms' magnitude.
EPS_F8 = 2.0 ** -12


def rounding_close(g: np.ndarray, ctx, i: int, heads, eps_dot: float, eps_epi: float):
    """g: one GPU row of logits (fp32) for query i of ctx (an oracle
    SeqContext) over `heads`.  -inf must match the oracle exactly; every
    finite entry must lie within the rounding bound
        sum_j |w_j| * eps_dot * sum_i |q_ji k_si|  +  eps_epi * sum_j |w_j| ReLU(q_j . k_s)
    (the dot products' accumulation error, which ReLU does not enlarge, and
    the fp32 epilogue's roundings of the head sum).  Returns (ok, worst error
    in units of the bound)."""
    t = ctx.t(i)
    heads = np.sort(np.asarray(heads))
    qt, wt = ctx.q[i][heads], ctx.w[i][heads]
    keys = ctx.keys[:t + 1]
    o = ctx.score(i, heads)
    g = g.astype(np.float64)
    if not np.array_equal(np.isneginf(g[:len(o)]), np.isneginf(o)):
        return False, float("inf")
    aw = np.abs(wt)[:, None]
    mag = (aw * (np.abs(qt) @ np.abs(keys).T)).sum(axis=0)
    terms = (aw * np.maximum(qt @ keys.T, 0.0)).sum(axis=0)
    bound = eps_dot * mag + eps_epi * terms + 1e-30
    err = np.abs(g[:t + 1] - o[:t + 1]) / bound
    worst = float(err.max()) if err.size else 0.0
    return worst <= 1.0, worst


def fp8_mfma_close(g: np.ndarray, ctx, i: int, heads):
    """fp8-query logits (ctx built with q8=True) within the derived fp8 bound."""
    return rounding_close(g, ctx, i, heads, EPS_F8, 2.0 ** -20)


# Regression guard beside the 1e-2 bar for the bf16-query kernels.  Their
# only error is rounding, and its worst case follows from the arithmetic:
#  * a (query head, key) dot product is 128 bf16 x bf16 products (each exact
#    in fp32) summed by the matrix core: at most 127 fp32 roundings of partial
#    sums bounded by sum_i |q_i k_i|, i.e. 2^-17 of it with round-to-nearest
#    (2^-16 if the core truncates); EPS_BF16_DOT = 2^-15 allows twice that;
#  * the epilogue (ReLU, the fma chain over a quad of heads, the quad and
#    16-head group adds, the fp8 scale) rounds at most 11 times a partial sum
#    bounded by sum_j |w_j| ReLU(q_j . k_s): 11 * 2^-24 < 2^-20; EPS_EPI =
#    2^-19.
# On the workloads this is 20 to 100 times tighter than 1e-2 relative, so a
# slip of 1 % in one head's term fails it (tests/test_tight_bounds.py).
EPS_BF16_DOT = 2.0 ** -15
EPS_BF16_EPI = 2.0 ** -19


def bf16_tight_close(g: np.ndarray, ctx, i: int, heads):
    """bf16-query logits within the derived rounding bound."""
    return rounding_close(g, ctx, i, heads, EPS_BF16_DOT, EPS_BF16_EPI)


# Pooling's rounding bound: a mean of n keys summed in fp32 (in slices whose
# sums are added in order) and scaled once is off by at most (n + 1) 2^-24 of
# the mean of |k| over those keys; doubled for margin.
def pool_bound(keys_abs_mean: np.ndarray, n: int) -> np.ndarray:
    return 2 * (n + 1) * 2.0 ** -24 * keys_abs_mean + 1e-30


# The router's rounding bound, per head j of query t, given the pooled keys
# it was fed (n = the query's complete blocks):
#  * a pooled-key dot product: the key split into bf16 hi + lo parts (off by
#    at most 2^-16 of |pooled|) and 256 products summed by the matrix core
#    (2^-16 of the sum of |products|): 2^-15 of sum_i |q_i pooled_i|; the
#    partial block's mean goes through the matrix core the same way;
#  * the block sum: each lane adds n/16 terms, then 4 butterfly adds, the
#    parts of a split sum and the partial block's term: (n/16 + 16) 2^-24 of S;
#  * r = w S: one more rounding.
# The block-sum and partial-block terms are doubled for margin; the dot
# products' term is their worst case itself (with random data the error is two
# orders of magnitude below it).
EPS_ROUTE_DOT = 2.0 ** -15


def route_reference(ctx, i: int, pooled=None, tail=None):
    """The oracle's (S, r) for query i, from the given pooled keys and partial
    block mean (the GPU's, widened), or from its own when they are None."""
    t = ctx.t(i)
    pooled = ctx.pooled if pooled is None else np.asarray(pooled, np.float64)
    tl = ctx.tail(i)
    if tl is not None and tail is not None:
        tl = np.asarray(tail, np.float64)
    return oracle.head_importance(ctx.q[i], ctx.w[i], pooled, tl, t, ctx.B)


def route_bound(ctx, i: int, pooled=None, tail=None):
    """Per-head bound on |r_gpu - r_ref| for query i of ctx (route_reference)."""
    t, B = ctx.t(i), ctx.B
    n_full = (t + 1) // B
    pooled = ctx.pooled if pooled is None else np.asarray(pooled, np.float64)
    aq = np.abs(ctx.q[i])                                   # [H, d]
    S, r = route_reference(ctx, i, pooled, tail)
    bound = EPS_ROUTE_DOT * (aq @ np.abs(pooled[:n_full]).sum(axis=0))
    tl = ctx.tail(i)
    if tl is not None:
        tl = tl if tail is None else np.asarray(tail, np.float64)
        bound = bound + EPS_ROUTE_DOT * (aq @ np.abs(tl))
    bound = bound + 2 * (n_full / 16 + 16) * 2.0 ** -24 * S
    return np.abs(ctx.w[i]) * bound + 2.0 ** -23 * np.abs(r) + 1e-30


def route_tight_close(gr: np.ndarray, ctx, i: int, pooled=None, tail=None):
    """One query's GPU router scores r against route_reference within
    route_bound.  Returns (ok, worst error in units of the bound)."""
    _, r = route_reference(ctx, i, pooled, tail)
    err = np.abs(gr.astype(np.float64) - r) / route_bound(ctx, i, pooled, tail)
    worst = float(err.max()) if err.size else 0.0
    return worst <= 1.0, worst


def band_check(values: np.ndarray, ids: np.ndarray, picked: np.ndarray, count: int):
    """Is `picked` (ids) a valid top-`count` of (values, ids) up to the band?
    Returns (ok, n_inside_band_disagreements)."""
    keep = ids >= 0
    values, ids = values[keep], ids[keep]
    count = min(count, len(ids))
    picked = picked[picked >= 0]
    if len(picked) != count or len(set(picked.tolist())) != count:
        return False, -1
    if count == 0:
        return True, 0
    order = np.argsort(-values, kind="stable")
    v = values[order[count - 1]]
    rowmax = np.abs(values[np.isfinite(values)]).max() if np.isfinite(values).any() else 0.0
    delta = BAND_REL * abs(v) + BAND_ROW * rowmax
    pos = {int(i): p for p, i in enumerate(ids)}
    psel = np.zeros(len(ids), bool)
    for i in picked:
        if int(i) not in pos:
            return False, -1
        psel[pos[int(i)]] = True
    must = values > v + delta
    must_not = values < v - delta
    if (must & ~psel).any() or (must_not & psel).any():
        return False, -1
    oracle_sel = np.zeros(len(ids), bool)
    oracle_sel[order[:count]] = True
    return True, int((oracle_sel != psel).sum() // 2)


def recall(picked: np.ndarray, ref: np.ndarray) -> float:
    r = ref[ref >= 0]
    if len(r) == 0:
        return 1.0
    return len(set(picked[picked >= 0].tolist()) & set(r.tolist())) / len(r)


def sample_rows(M: int, n: int):
    if M <= n:
        return list(range(M))
    rows = np.unique(np.linspace(0, M - 1, n).round().astype(int))
    return rows.tolist()


def f64(t):
    return t.detach().cpu().numpy().astype(np.float64)


_CTX = {}


def ctx_of(inp, b):
    """Oracle context of sequence b (widened keys + pooled keys), cached per input set."""
    key = (id(inp), b)
    if key not in _CTX:
        if len(_CTX) > 8:
            _CTX.clear()
        _CTX[key] = (inp, oracle.SeqContext(inp, b))
    return _CTX[key][1]


def run_stages(inp, t=None, h=None, rows_for_logits=None):
    t = upload(inp) if t is None else t
    sh = shape_of(inp)
    h = inp.cfg.h if h is None else h
    pooled, tail = lcsb.misa_pool_keys(sh, t["k"], t["k_scale"])
    heads, r = lcsb.misa_route_heads(sh, t["q"], t["w"], pooled, tail, h, want_scores=True)
    logits = lcsb.misa_sparse_head_logits(sh, t["q"], t["w"], t["k"], heads, k_scale=t["k_scale"])
    torch.cuda.synchronize()
    return dict(t=t, sh=sh, pooled=pooled, tail=tail, heads=heads, r=r, logits=logits)


def check_pool(inp, st, rows=None, seqs=None):
    M = inp.cfg.q_per_seq
    rows = range(M) if rows is None else rows
    seqs = range(inp.cfg.n_seq) if seqs is None else seqs
    for b in seqs:
        ctx = ctx_of(inp, b)
        gp = f64(st["pooled"][b])
        B = ctx.B
        if ctx.pooled.size:
            n_full = ctx.pooled.shape[0]
            absmean = np.abs(ctx.keys[:n_full * B]).reshape(n_full, B, -1).mean(axis=1)
            err = np.abs(gp[:n_full] - ctx.pooled) / pool_bound(absmean, B)
            assert err.max() <= 1.0, f"pooled keys seq {b}: {err.max():.3g} of the rounding bound"
        gt = st["tail"][b]
        for i in rows:
            tl = ctx.tail(i)
            g = f64(gt[i])
            if tl is None:
                assert not g.any()
            else:
                t = ctx.t(i)
                start = ((t + 1) // B) * B
                absmean = np.abs(ctx.keys[start:t + 1]).mean(axis=0)
                err = np.abs(g - tl) / pool_bound(absmean, t + 1 - start)
                assert err.max() <= 1.0, f"tail seq {b} query {i}: {err.max():.3g} of the rounding bound"


def check_route(inp, st, rows=None, seqs=None):
    M, H, h = inp.cfg.q_per_seq, inp.cfg.n_heads, st["heads"].shape[-1]
    rows = list(range(M)) if rows is None else rows
    seqs = range(inp.cfg.n_seq) if seqs is None else seqs
    gh = st["heads"].cpu().numpy()
    gr = st["r"].cpu().numpy().astype(np.float64)
    worst, inside, tight = 0.0, 0, 0.0
    for b in seqs:
        ctx = ctx_of(inp, b)
        gp = f64(st["pooled"][b])
        gt = f64(st["tail"][b])
        for i in rows:
            S, r, heads = ctx.route(i, h)
            ok, wst = logits_close(gr[b, i][None], r[None])
            assert ok, f"router scores seq {b} query {i}: worst {wst}"
            worst = max(worst, wst)
            ok, wt = route_tight_close(gr[b, i], ctx, i, gp, gt[i])
            assert ok, f"router scores seq {b} query {i}: {wt:.3g} of the rounding bound"
            tight = max(tight, wt)
            assert np.all(np.diff(gh[b, i]) > 0), "heads not ascending/distinct"
            ok, n_in = band_check(r, np.arange(H), gh[b, i], h)
            assert ok, f"heads seq {b} query {i}: gpu {gh[b, i]} oracle {heads}"
            inside += n_in
    check_route.tight = tight   # worst share of the rounding bound of the last call
    return worst, inside


def check_logits(inp, st, rows=None, seqs=None):
    M = inp.cfg.q_per_seq
    rows = list(range(M)) if rows is None else rows
    seqs = range(inp.cfg.n_seq) if seqs is None else seqs
    gh = st["heads"].cpu().numpy()
    worst, tight = 0.0, 0.0
    N = inp.cfg.n_keys
    for b in seqs:
        ctx = ctx_of(inp, b)
        idx = torch.tensor(rows, device=st["logits"].device)
        g = st["logits"][b].index_select(0, idx)[:, :N].cpu().numpy()
        for n, i in enumerate(rows):
            o = ctx.score(i, gh[b, i])
            ok, wst = logits_close(g[n][None], o[None])
            assert ok, f"logits seq {b} query {i}: worst {wst}"
            worst = max(worst, wst)
            ok, wt = bf16_tight_close(g[n], ctx, i, gh[b, i])
            assert ok, f"logits seq {b} query {i}: {wt:.3g} of the rounding bound"
            tight = max(tight, wt)
    check_logits.tight = tight   # worst share of the rounding bound of the last call
    return worst


def check_topk_exact(inp, logits, k, idx, vals, rows=None, seqs=None):
    """top-k of the GPU's own logits: the oracle decides on the same fp32 values."""
    M = inp.cfg.q_per_seq
    rows = list(range(M)) if rows is None else rows
    seqs = range(inp.cfg.n_seq) if seqs is None else seqs
    for b in seqs:
        ridx = torch.tensor(rows, device=logits.device)
        g = logits[b].index_select(0, ridx).cpu().numpy().astype(np.float64)
        gi = idx[b].index_select(0, ridx).cpu().numpy()
        gv = vals[b].index_select(0, ridx).cpu().numpy() if vals is not None else None
        for n, i in enumerate(rows):
            t = inp.q_pos0 + i
            oi, ov = oracle.topk_prefix(g[n], t, k)
            assert np.array_equal(gi[n], oi), f"top-k seq {b} query {i}"
            if gv is not None:
                assert np.array_equal(gv[n].astype(np.float64), ov)
