"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the same stage calls, the same kernels and grids).

The oracle computes sampled outputs one query at a time: evenly spaced
queries including the first and the last (or, for the decode batch, evenly
spaced sequences).  Every check of the small-shape suite is applied to those
rows; whole-tensor properties (the indexer equals its stages, -inf beyond the
causal prefix, ids in range and distinct) are checked on every row.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_block_amd as lcsb
import oracle
from gpu_helpers import (band_check, check_logits, check_pool, check_route, check_topk_exact, ctx_of,
                         logits_close, recall, run_stages, sample_rows, say, upload)
from long_context_sparse_block_amd import inputs as gen

pytestmark = pytest.mark.gpu

BIG = ["dsv32_prefill_m8k_n32k", "final_chunk_m8k_n128k_fp8", "glm5_decode_64x1_n128k",
       "dagger_prefill_m4k_n128k"]


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    lcsb.load()


def whole_tensor_checks(inp, st, idx):
    """Properties that hold at any size, checked on every row on the GPU."""
    cfg = inp.cfg
    N, M, K = cfg.n_keys, cfg.q_per_seq, idx.shape[-1]
    dev = idx.device
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
    say("full-size staged parity", name)
    if cfg.n_seq > 1:
        seqs, rows = sample_rows(cfg.n_seq, 12), list(range(cfg.q_per_seq))
    else:
        seqs, rows = [0], sample_rows(cfg.q_per_seq, 40)
    check_pool(inp, st, rows=rows, seqs=seqs)
    worst_r, inside = check_route(inp, st, rows=rows, seqs=seqs)
    worst_l = check_logits(inp, st, rows=rows, seqs=seqs)
    sh = st["sh"]
    first_k = cfg.k_prime if cfg.k_prime else cfg.topk
    idx, vals = lcsb.misa_topk(sh, st["logits"], first_k)
    check_topk_exact(inp, st["logits"], first_k, idx, vals, rows=rows, seqs=seqs)
    whole_tensor_checks(inp, st, idx)
    say(f"  router worst {worst_r:.2e} (in-band disagreements {inside}), logits worst {worst_l:.2e}")


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
    if cfg.n_seq > 1:
        seqs, rows = sample_rows(cfg.n_seq, 12), list(range(cfg.q_per_seq))
    else:
        seqs, rows = [0], sample_rows(cfg.q_per_seq, 24)
    gi = idx.cpu().numpy()
    gh = st["heads"].cpu().numpy()
    recs, dense_recs = [], []
    for b in seqs:
        ctx = ctx_of(inp, b)
        for i in rows:
            T = inp.q_pos0 + i
            if cfg.k_prime:
                out = ctx.misa_dagger(i, cfg.h, cfg.k_prime, cfg.topk)
                dense = ctx.dense_topk(i, cfg.topk)["idx"]
                dense_recs.append(recall(gi[b, i], dense))
            else:
                out = ctx.misa(i, cfg.h, cfg.topk)
                if np.array_equal(np.sort(out["heads"]), gh[b, i]):
                    ok, _ = band_check(out["I"][:T + 1], np.arange(T + 1), gi[b, i], cfg.topk)
                    assert ok, f"token set seq {b} query {i}"
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
        for i in rows[:8]:
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
    say("full-size dense comparator, sampled rows")
    dense = lcsb.dsa_dense_logits(sh, t["q"], t["w"], t["k"], k_scale=t["k_scale"])
    rows = sample_rows(cfg.q_per_seq, 6)
    g = dense[0, rows, :cfg.n_keys].cpu().numpy()
    del dense
    ctx = ctx_of(inp, 0)
    for n, i in enumerate(rows):
        ok, wst = logits_close(g[n][None], ctx.dense(i)[None])
        assert ok, f"dense query {i} worst {wst}"
