"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the same stage calls, the same kernels and grids).

The oracle computes sampled outputs one query at a time: 256 evenly spaced
queries including the first and the last (for the decode batch, every one of
its 64 sequences).  Every check of the small-shape suite is applied to those
rows, including the rounding-bound guards of the logits, the router scores
and the pooled keys; whole-tensor properties (the indexer equals its stages,
-inf exactly beyond the causal prefix, heads ascending, distinct and in
range, ids in range and distinct, values non-increasing along each row with
equal values in ascending id order) are checked on every row.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_block_amd as lcsb
import oracle
from gpu_helpers import (band_check, bf16_tight_close, check_logits, check_pool, check_route, check_topk_exact,
                         ctx_of, logits_close, recall, run_stages, sample_rows, say, upload)
from long_context_sparse_block_amd import inputs as gen

pytestmark = pytest.mark.gpu

BIG = ["dsv32_prefill_m8k_n32k", "final_chunk_m8k_n128k_fp8", "glm5_decode_64x1_n128k",
       "dagger_prefill_m4k_n128k"]


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    lcsb.load()


N_ROWS = 256   # sampled queries per long chunk


def rows_of(cfg):
    """(sequences, queries) the oracle checks: every sequence of a decode
    batch, else N_ROWS evenly spaced queries including the first and last."""
    if cfg.n_seq > 1:
        return list(range(cfg.n_seq)), list(range(cfg.q_per_seq))
    return [0], sample_rows(cfg.q_per_seq, N_ROWS)


def check_heads_tensor(heads, H):
    """Every row's routed heads: in [0, H), strictly ascending (so distinct)."""
    assert bool((heads >= 0).all()) and bool((heads < H).all()), "head id out of range"
    if heads.shape[-1] > 1:
        assert bool((heads[..., 1:] > heads[..., :-1]).all()), "heads not ascending / distinct"


def check_sorted_tensor(idx, vals):
    """Every row of a sorted selection: values non-increasing, equal values in
    ascending id order, padding (-1, -inf) only at the end."""
    v, i = vals[..., :-1], vals[..., 1:]
    a, b = idx[..., :-1], idx[..., 1:]
    assert not bool(torch.isnan(vals).any())
    assert bool((v >= i).all()), "values not non-increasing"
    tie = (v == i) & (b >= 0)
    assert bool((a[tie] < b[tie]).all()), "equal values not in ascending id order"
    pad = idx < 0
    assert bool(torch.isneginf(vals[pad]).all()), "padding without -inf"
    # once padded, padded to the end
    assert not bool((pad[..., :-1] & ~pad[..., 1:]).any()), "padding before a selected id"


def whole_tensor_checks(inp, st, idx, vals=None):
    """Properties that hold at any size, checked on every row on the GPU."""
    cfg = inp.cfg
    N, M, K = cfg.n_keys, cfg.q_per_seq, idx.shape[-1]
    dev = idx.device
    check_heads_tensor(st["heads"], cfg.n_heads)
    if vals is not None:
        check_sorted_tensor(idx, vals)
    t = inp.q_pos0 + torch.arange(M, device=dev)
    # ids: -1 only as trailing padding, otherwise in [0, t], distinct per row
    valid = idx >= 0
    assert bool((idx[valid] >= 0).all())
    assert bool((idx <= t.view(1, M, 1)).all())
    s, _ = torch.sort(idx, dim=-1)
    dup = (s[..., 1:] == s[..., :-1]) & (s[..., 1:] >= 0)
    assert not bool(dup.any()), "duplicate ids in a row"
    n_expect = torch.clamp(t + 1, max=K)
    assert torch.equal(valid.sum(-1), n_expect.view(1, M).expand(cfg.n_seq, M))
    # logits: -inf exactly after the causal prefix, finite inside it
    lg = st["logits"][..., :N]
    col = torch.arange(N, device=dev).view(1, 1, N)
    after = col > t.view(1, M, 1)
    for b in range(cfg.n_seq):
        assert bool((torch.isneginf(lg[b]) == after[0]).all()), "-inf must mark exactly s > t"
        assert not bool(torch.isnan(lg[b]).any() or torch.isposinf(lg[b]).any())


@pytest.fixture(scope="module")
def big():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            cfg = gen.CONFIGS[name]
            say("generating", name)
            inp = gen.generate(cfg)
            st = run_stages(inp)
            cache[name] = (inp, st)
        return cache[name]
    return get


@pytest.mark.parametrize("name", BIG)
def test_fullsize_staged_parity(big, name):
    inp, st = big(name)
    cfg = inp.cfg
    seqs, rows = rows_of(cfg)
    say(f"full-size staged parity {name}: {len(seqs)} sequence(s) x {len(rows)} queries")
    worst_r = worst_l = tight_r = tight_l = 0.0
    inside = 0
    for b in seqs:   # one sequence at a time: its oracle context is built once
        check_pool(inp, st, rows=rows, seqs=[b])
        wr, ins = check_route(inp, st, rows=rows, seqs=[b])
        tight_r, worst_r, inside = max(tight_r, check_route.tight), max(worst_r, wr), inside + ins
        wl = check_logits(inp, st, rows=rows, seqs=[b])
        tight_l, worst_l = max(tight_l, check_logits.tight), max(worst_l, wl)
    sh = st["sh"]
    first_k = cfg.k_prime if cfg.k_prime else cfg.topk
    idx, vals = lcsb.misa_topk(sh, st["logits"], first_k)
    check_topk_exact(inp, st["logits"], first_k, idx, vals, rows=rows, seqs=seqs)
    whole_tensor_checks(inp, st, idx, vals)
    say(f"  router worst {worst_r:.2e} ({tight_r:.3f} of its rounding bound; in-band disagreements {inside}), "
        f"logits worst {worst_l:.2e} ({tight_l:.3f} of the rounding bound)")


@pytest.mark.parametrize("name", BIG)
def test_fullsize_indexer(big, name):
    inp, st = big(name)
    cfg = inp.cfg
    t, sh = st["t"], st["sh"]
    say("full-size indexer", name)
    idx, vals = lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk, k_prime=cfg.k_prime,
                                  k_scale=t["k_scale"])
    if cfg.k_prime:
        cand, _ = lcsb.misa_topk(sh, st["logits"], cfg.k_prime, want_vals=False)
        D = lcsb.dsa_dense_logits(sh, t["q"], t["w"], t["k"], k_scale=t["k_scale"], cand=cand)
        sidx, svals = lcsb.misa_topk(sh, D, cfg.topk, cand=cand)
    else:
        sidx, svals = lcsb.misa_topk(sh, st["logits"], cfg.topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, sidx) and torch.equal(vals, svals), "indexer != its stages"
    whole_tensor_checks(inp, st, idx, vals)
    seqs, rows = rows_of(cfg)
    say(f"  {len(seqs)} sequence(s) x {len(rows)} queries against the oracle")
    gi = idx.cpu().numpy()
    gh = st["heads"].cpu().numpy()
    gc = cand.cpu().numpy() if cfg.k_prime else None
    recs, dense_recs = [], []
    for b in seqs:
        ctx = ctx_of(inp, b)
        for n, i in enumerate(rows):
            T = inp.q_pos0 + i
            # the selection given the GPU's routed heads (valid by the router
            # checks, in-band choices included) is decided like the oracle
            # decides it from its own scores of those heads
            I = ctx.score(i, gh[b, i])
            if cfg.k_prime:
                ok, _ = band_check(I[:T + 1], np.arange(T + 1), gc[b, i], cfg.k_prime)
                assert ok, f"candidate set seq {b} query {i}"
                c = gc[b, i].astype(np.int64)
                Do = oracle.score_candidates(ctx.q[i], ctx.w[i], ctx.keys, c)
                ok, _ = band_check(Do, c, gi[b, i], cfg.topk)
                assert ok, f"final set seq {b} query {i}"
                out = ctx.misa_dagger(i, cfg.h, cfg.k_prime, cfg.topk)
                if n % 4 == 0:   # reported, not a pass/fail (a quarter of the rows: the dense oracle is slow)
                    dense_recs.append(recall(gi[b, i], ctx.dense_topk(i, cfg.topk)["idx"]))
            else:
                ok, _ = band_check(I[:T + 1], np.arange(T + 1), gi[b, i], cfg.topk)
                assert ok, f"token set seq {b} query {i}"
                out = ctx.misa(i, cfg.h, cfg.topk)
            recs.append(recall(gi[b, i], out["idx"]))
    say(f"  recall vs oracle: mean {np.mean(recs):.6f} min {np.min(recs):.4f}")
    if dense_recs:
        say(f"  MISA-dagger recall vs the dense top-k: mean {np.mean(dense_recs):.4f} "
            f"min {np.min(dense_recs):.4f}")
    assert np.mean(recs) >= 0.999
    if cfg.k_prime:
        # the re-rank stage on sampled rows: bitwise equal to the dense logits of the
        # candidate tokens, within tolerance of the oracle, exact final selection
        D_np = D.cpu().numpy()
        c_np = cand.cpu().numpy()
        ctx = ctx_of(inp, 0)
        for i in rows[::8]:
            o = oracle.score_candidates(ctx.q[i], ctx.w[i], ctx.keys, c_np[0, i].astype(np.int64))
            ok, wst = logits_close(D_np[0, i, :cfg.k_prime][None], o[None])
            assert ok, f"rerank query {i} worst {wst}"
            oi, _ = oracle.topk_row(D_np[0, i, :cfg.k_prime].astype(np.float64), c_np[0, i].astype(np.int64),
                                    cfg.topk)
            assert np.array_equal(gi[0, i], oi)


def test_fullsize_dense_comparator_rows(big):
    inp, st = big("final_chunk_m8k_n128k_fp8")
    cfg = inp.cfg
    t, sh = st["t"], st["sh"]
    rows = sample_rows(cfg.q_per_seq, 32)
    say(f"full-size dense comparator, {len(rows)} rows")
    dense = lcsb.dsa_dense_logits(sh, t["q"], t["w"], t["k"], k_scale=t["k_scale"])
    g = dense[0, rows, :cfg.n_keys].cpu().numpy()
    del dense
    ctx = ctx_of(inp, 0)
    tight = 0.0
    for n, i in enumerate(rows):
        ok, wst = logits_close(g[n][None], ctx.dense(i)[None])
        assert ok, f"dense query {i} worst {wst}"
        ok, wt = bf16_tight_close(g[n], ctx, i, np.arange(cfg.n_heads))
        assert ok, f"dense query {i}: {wt:.3g} of the rounding bound"
        tight = max(tight, wt)
    say(f"  worst {tight:.3f} of the rounding bound")
