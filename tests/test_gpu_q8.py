"""GPU parity of the fp8 query path (misa_quantize_q, misa_sparse_head_logits_q8).

  * quantisation: codes and scales bit-exact against the oracle (integer
    outputs), including zero rows, values that land in e4m3fn's subnormal
    range, and exact midpoints between codes (ties to even);
  * fp8 scoring: every logit against the oracle's routed score of the
    dequantised queries and keys, within the stated 1e-2 relative tolerance
    and within the bound derived from the fp8 matrix cores' accumulation
    (fp8_mfma_close);
  * the top-k of those logits against the oracle's, up to the tolerance band;
  * the fused selection (misa_sparse_head_topk_q8) bit for bit against its
    staged form (fp8 logits, then misa_topk): ids, values and order, the set
    when unsorted; the staged top-k exactly against the oracle's top-k of
    the same logits; inputs that defeat the sampled threshold (every row
    re-scored), all-negative weights with a ragged query tile, k up to 6000,
    decode, prefixes too short for the fused path, and the full-size chunk;
  * the fp8-query indexer (misa_indexer_q8, MISA and MISA-dagger) bit for bit
    against the same steps as separate calls, and its ids against the
    oracle's fp8-query indexer (recall);
  * the fp8-query dense comparator (dsa_dense_logits_q8): every logit against
    the oracle's all-head score of the dequantised inputs within the derived
    fp8 bound (64 signed head terms cancel far more than 8, so the 1e-2
    relative bound stated for bf16 inputs and fp32 accumulation does not
    carry over), for 1 to 4 blocks of 16 heads and a ragged query tile, and
    sampled rows at full size.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_block_amd as lcsb
import oracle
from gpu_helpers import (band_check, check_topk_exact, fp8_mfma_close, logits_close, recall, sample_rows, say,
                         shape_of, upload)
from long_context_sparse_block_amd import inputs as gen

pytestmark = pytest.mark.gpu


def to_bf16_bits(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def special_rows(q):
    """Overwrite a few (query, head) rows of q (bf16 bits [n_seq, M, H, 128])."""
    q[0, 0, 0] = 0                                              # all zero: scale 1, codes 0
    # amax 1, the rest k * 2^-18: 448 k 2^-18 spans e4m3fn's subnormals (below 2^-6) and low normals
    tiny = np.concatenate([[1.0], np.ldexp(np.arange(1, 128, dtype=np.float64), -18)])
    q[0, 1, 0] = to_bf16_bits(tiny * np.where(np.arange(128) % 2, 1.0, -1.0))
    # amax 448 -> scale 1: the values themselves are rounded, midpoints included
    mids = np.array([448.0, 1.0625, 1.1875, 17.0, -19.0, 2.5 * 2 ** -9, 1.5 * 2 ** -9, -5.25, 0.0, 3.0])
    row = np.resize(mids, 128)
    q[0, 2, 1] = to_bf16_bits(row)
    assert np.all(oracle.bf16_bits_to_f64(q[0, 2, 1]) == row)   # all exact in bf16


def test_quantize_q_bitwise():
    say("fp8 quantisation")
    cfg = gen.small_config(name="q8_quant", n_seq=2, m=37, n=3000, hh=48, b=64, h=8, k=64,
                           kdtype=gen.KDTYPE_FP8, seed=46)
    inp = gen.generate(cfg)
    special_rows(inp.q)
    t = upload(inp)
    sh = shape_of(inp)
    q8, qs = lcsb.misa_quantize_q(sh, t["q"])
    torch.cuda.synchronize()
    oc, osc = oracle.quantize_q_e4m3(inp.q)
    np.testing.assert_array_equal(q8.cpu().numpy(), oc)
    np.testing.assert_array_equal(qs.cpu().numpy(), osc)


Q8_CASES = [
    dict(name="q8_ragged", n_seq=1, m=40, n=3000, hh=48, b=64, h=5, k=256),
    dict(name="q8_h8", n_seq=1, m=64, n=4100, hh=32, b=128, h=8, k=512),
    dict(name="q8_decode", n_seq=3, m=1, n=2500, hh=32, b=64, h=8, k=256),
]


@pytest.mark.parametrize("case", Q8_CASES, ids=lambda c: c["name"])
def test_q8_logits_and_topk_against_oracle(case):
    c = dict(case)
    name = c.pop("name")
    say("fp8 scoring", name)
    cfg = gen.small_config(name=name, kdtype=gen.KDTYPE_FP8, seed=47, **c)
    inp = gen.generate(cfg)
    t = upload(inp)
    sh = shape_of(inp)
    pooled, tail = lcsb.misa_pool_keys(sh, t["k"], t["k_scale"])
    heads = lcsb.misa_route_heads(sh, t["q"], t["w"], pooled, tail, cfg.h)
    q8, qs = lcsb.misa_quantize_q(sh, t["q"])
    logits = lcsb.misa_sparse_head_logits_q8(sh, q8, qs, t["w"], t["k"], heads, t["k_scale"])
    idx, vals = lcsb.misa_topk(sh, logits, cfg.topk)
    torch.cuda.synchronize()
    N = cfg.n_keys
    gh = heads.cpu().numpy()
    gl = logits.cpu().numpy()[..., :N]
    gi = idx.cpu().numpy()
    worst = 0.0
    for b in range(cfg.n_seq):
        ctx = oracle.SeqContext(inp, b, q8=True)
        for i in range(cfg.q_per_seq):
            o = ctx.score(i, gh[b, i])
            ok, wst = logits_close(gl[b, i][None], o[None])
            assert ok, f"fp8 logits seq {b} query {i}: worst {wst}"
            ok, wb = fp8_mfma_close(gl[b, i], ctx, i, gh[b, i])
            assert ok, f"fp8 logits seq {b} query {i}: {wb} of the fp8 bound"
            worst = max(worst, wst)
            T = ctx.t(i)
            ok, _ = band_check(o[:T + 1], np.arange(T + 1), gi[b, i], cfg.topk)
            assert ok, f"fp8 top-k seq {b} query {i}"
    say(f"  worst relative logit error {worst:.2e}")


def q8_stages(inp):
    """pool -> route (bf16 q) -> fp8 quantisation -> fp8 logits, all on the GPU."""
    cfg = inp.cfg
    t = upload(inp)
    sh = shape_of(inp)
    pooled, tail = lcsb.misa_pool_keys(sh, t["k"], t["k_scale"])
    heads = lcsb.misa_route_heads(sh, t["q"], t["w"], pooled, tail, cfg.h)
    q8, qs = lcsb.misa_quantize_q(sh, t["q"])
    logits = lcsb.misa_sparse_head_logits_q8(sh, q8, qs, t["w"], t["k"], heads, t["k_scale"])
    return dict(t=t, sh=sh, heads=heads, q8=q8, qs=qs, logits=logits)


def check_q8_selection(inp, st, k):
    """fused == staged, bit for bit (sorted), and the same set (unsorted)."""
    t, sh = st["t"], st["sh"]
    si, sv = lcsb.misa_topk(sh, st["logits"], k)
    fi, fv = lcsb.misa_sparse_head_topk_q8(sh, st["q8"], st["qs"], t["w"], t["k"], st["heads"], k, t["k_scale"])
    ui, _ = lcsb.misa_sparse_head_topk_q8(sh, st["q8"], st["qs"], t["w"], t["k"], st["heads"], k, t["k_scale"],
                                          sorted=False, want_vals=False)
    torch.cuda.synchronize()
    assert torch.equal(fi, si) and torch.equal(fv, sv), "fused fp8 selection != fp8 logits + top-k"
    assert torch.equal(torch.sort(ui, dim=-1)[0], torch.sort(si, dim=-1)[0]), "unsorted: not the same set"
    return fi, fv


def fp8_keys_from(inp, kf):
    """Re-encode float keys [n_seq, N, 128] as the inputs' fp8 keys (per-key
    scale amax / 448, e4m3fn codes of k / scale)."""
    amax = np.abs(kf).max(axis=-1)
    sc = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    inp.k[...] = gen.to_e4m3_codes(kf / sc[..., None])
    inp.k_scale[...] = sc


FUSED_Q8_CASES = [
    dict(name="q8_fused_h8_ragged", n_seq=1, m=72, n=40000, hh=32, b=64, h=8, k=2048),
    dict(name="q8_fused_h5", n_seq=1, m=40, n=36001, hh=48, b=128, h=5, k=1000),
    dict(name="q8_fused_decode", n_seq=6, m=1, n=50000, hh=32, b=64, h=8, k=2048),
    dict(name="q8_fused_k6000", n_seq=1, m=40, n=40000, hh=16, b=64, h=8, k=6000),
    dict(name="q8_short_prefix", n_seq=1, m=64, n=4100, hh=32, b=128, h=8, k=512),
]


@pytest.mark.parametrize("case", FUSED_Q8_CASES, ids=lambda c: c["name"])
def test_q8_fused_selection_equals_staged_and_oracle(case):
    c = dict(case)
    name = c.pop("name")
    say("fused fp8 selection", name)
    cfg = gen.small_config(name=name, kdtype=gen.KDTYPE_FP8, seed=48, **c)
    inp = gen.generate(cfg)
    st = q8_stages(inp)
    fi, fv = check_q8_selection(inp, st, cfg.topk)
    rows = sample_rows(cfg.q_per_seq, 6)
    check_topk_exact(inp, st["logits"], cfg.topk, fi, fv, rows=rows)
    gh = st["heads"].cpu().numpy()
    gi = fi.cpu().numpy()
    for b in range(cfg.n_seq):
        ctx = oracle.SeqContext(inp, b, q8=True)
        for i in rows:
            o = ctx.score(i, gh[b, i])
            T = ctx.t(i)
            ok, _ = band_check(o[:T + 1], np.arange(T + 1), gi[b, i], cfg.topk)
            assert ok, f"fp8 fused top-k seq {b} query {i}"


def test_q8_fused_rows_the_sample_misjudges():
    """Every key at a multiple of the sampling stride (32) gets a huge score,
    so the sampled threshold admits far fewer than k candidates: every row is
    flagged, re-scored into fp8 logits and selected from them."""
    say("fused fp8 selection: threshold defeated")
    cfg = gen.small_config(name="q8_adv", m=48, n=40000, hh=16, b=64, h=8, k=2048, kdtype=gen.KDTYPE_FP8,
                           seed=49, plant=False)
    inp = gen.generate(cfg)
    q = oracle.bf16_bits_to_f64(inp.q).astype(np.float32)
    kf = oracle.e4m3fn_to_f64(inp.k).astype(np.float32) * inp.k_scale[..., None]
    u = np.ones(128, np.float32) / np.sqrt(128.0)
    q += 4.0 * u
    kf[:, ::32, :] += 40.0 * u
    inp.q[...] = gen.to_bf16_bits(q)
    fp8_keys_from(inp, kf)
    inp.w[...] = np.abs(inp.w)
    st = q8_stages(inp)
    fi, fv = check_q8_selection(inp, st, cfg.topk)
    check_topk_exact(inp, st["logits"], cfg.topk, fi, fv)


def test_q8_fused_selection_in_a_smaller_workspace():
    """misa_sparse_head_topk_q8 and misa_indexer_q8 with room for one query tile
    of logits (every row flagged, two sequences of 48 queries: 4 re-scoring
    batches) give the fast plan's result bit for bit."""
    say("fused fp8 selection in a smaller workspace")
    cfg = gen.small_config(name="q8_slab", n_seq=2, m=48, n=40000, hh=16, b=64, h=8, k=2048, kdtype=gen.KDTYPE_FP8,
                           seed=50, plant=False)
    inp = gen.generate(cfg)
    q = oracle.bf16_bits_to_f64(inp.q).astype(np.float32)
    kf = oracle.e4m3fn_to_f64(inp.k).astype(np.float32) * inp.k_scale[..., None]
    u = np.ones(128, np.float32) / np.sqrt(128.0)
    q += 4.0 * u
    kf[:, ::32, :] += 40.0 * u
    inp.q[...] = gen.to_bf16_bits(q)
    fp8_keys_from(inp, kf)
    inp.w[...] = np.abs(inp.w)
    st = q8_stages(inp)
    t, sh = st["t"], st["sh"]
    tile = 32 * 40000 * 4
    si, sv = lcsb.misa_topk(sh, st["logits"], cfg.topk)
    full = lcsb.misa_sparse_head_topk_workspace_bytes(sh, gen.KDTYPE_FP8, cfg.h, cfg.topk)
    ws = torch.empty(full - 3 * tile, dtype=torch.uint8, device="cuda")
    fi, fv = lcsb.misa_sparse_head_topk_q8(sh, st["q8"], st["qs"], t["w"], t["k"], st["heads"], cfg.topk,
                                           t["k_scale"], ws=ws)
    ii, iv = lcsb.misa_indexer_q8(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk, t["k_scale"])
    full_ix = lcsb.misa_indexer_q8_workspace_bytes(sh, cfg.h, cfg.topk)
    ji, jv = lcsb.misa_indexer_q8(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk, t["k_scale"],
                                  ws=torch.empty(full_ix - 3 * tile, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(fi, si) and torch.equal(fv, sv)
    assert torch.equal(ji, ii) and torch.equal(jv, iv)
    assert torch.equal(ii, si) and torch.equal(iv, sv)


def test_q8_fused_nonpositive_scores_ragged_query_tile():
    """All head weights negative: scores <= 0, many exactly 0, thresholds <= 0;
    M = 37 leaves padding lanes whose zero scores must reach no row."""
    say("fused fp8 selection: scores <= 0, ragged query tile")
    cfg = gen.small_config(name="q8_neg", m=37, n=40000, hh=16, b=64, h=4, k=256, kdtype=gen.KDTYPE_FP8,
                           seed=50, plant=False)
    inp = gen.generate(cfg)
    inp.w[...] = -np.abs(inp.w)
    st = q8_stages(inp)
    fi, fv = check_q8_selection(inp, st, cfg.topk)
    assert float(fv.max()) <= 0.0 and int((fv == 0).sum()) > 0
    check_topk_exact(inp, st["logits"], cfg.topk, fi, fv)


def test_q8_fused_selection_full_size():
    """The benchmark's chunk (M = 8192, N = 131072, fp8 keys, H = 64, B = 128,
    top-2048): fused == staged on every row, the staged top-k exact on
    sampled rows, and sampled rows within the band of the oracle's scores."""
    cfg = gen.CONFIGS["final_chunk_m8k_n128k_fp8"]
    say("fused fp8 selection, full size", cfg.name)
    inp = gen.generate(cfg)
    st = q8_stages(inp)
    fi, fv = check_q8_selection(inp, st, cfg.topk)
    rows = sample_rows(cfg.q_per_seq, 24)
    check_topk_exact(inp, st["logits"], cfg.topk, fi, fv, rows=rows)
    gh = st["heads"].cpu().numpy()
    gi = fi.cpu().numpy()
    ctx = oracle.SeqContext(inp, 0, q8=True)
    for i in rows[::3]:
        o = ctx.score(i, gh[0, i])
        T = ctx.t(i)
        ok, _ = band_check(o[:T + 1], np.arange(T + 1), gi[0, i], cfg.topk)
        assert ok, f"fp8 fused top-k query {i}"


DENSE_Q8_CASES = [
    dict(name="dq8_h64_ragged", n_seq=1, m=37, n=3000, hh=64, b=64, h=8, k=64),
    dict(name="dq8_h48", n_seq=1, m=16, n=2100, hh=48, b=64, h=8, k=64),
    dict(name="dq8_h16_decode", n_seq=3, m=1, n=2500, hh=16, b=64, h=8, k=64),
    dict(name="dq8_h20", n_seq=1, m=9, n=700, hh=20, b=32, h=4, k=64),
]


@pytest.mark.parametrize("case", DENSE_Q8_CASES, ids=lambda c: c["name"])
def test_dense_q8_logits_against_oracle(case):
    c = dict(case)
    name = c.pop("name")
    say("fp8 dense scoring", name)
    cfg = gen.small_config(name=name, kdtype=gen.KDTYPE_FP8, seed=51, **c)
    inp = gen.generate(cfg)
    t = upload(inp)
    sh = shape_of(inp)
    q8, qs = lcsb.misa_quantize_q(sh, t["q"])
    logits = lcsb.dsa_dense_logits_q8(sh, q8, qs, t["w"], t["k"], t["k_scale"])
    torch.cuda.synchronize()
    N = cfg.n_keys
    gl = logits.cpu().numpy()[..., :N]
    worst = 0.0
    for b in range(cfg.n_seq):
        ctx = oracle.SeqContext(inp, b, q8=True)
        for i in range(cfg.q_per_seq):
            ok, wb = fp8_mfma_close(gl[b, i], ctx, i, np.arange(cfg.n_heads))
            assert ok, f"fp8 dense logits seq {b} query {i}: {wb} of the fp8 bound"
            worst = max(worst, wb)
    say(f"  worst error {worst:.3f} of the derived fp8 bound")


def test_dense_q8_full_size_rows():
    """Dense fp8 logits of the benchmark's chunk on sampled rows, and -inf
    exactly after each query's prefix on every row."""
    cfg = gen.CONFIGS["final_chunk_m8k_n128k_fp8"]
    say("fp8 dense scoring, full size", cfg.name)
    inp = gen.generate(cfg)
    t = upload(inp)
    sh = shape_of(inp)
    q8, qs = lcsb.misa_quantize_q(sh, t["q"])
    logits = lcsb.dsa_dense_logits_q8(sh, q8, qs, t["w"], t["k"], t["k_scale"])
    N, M = cfg.n_keys, cfg.q_per_seq
    tpos = inp.q_pos0 + torch.arange(M, device=logits.device)
    col = torch.arange(N, device=logits.device).view(1, N)
    after = col > tpos.view(M, 1)
    lg = logits[0, :, :N]
    assert bool((torch.isneginf(lg) == after).all())
    assert not bool(torch.isnan(lg).any() or torch.isposinf(lg).any())
    rows = sample_rows(M, 6)
    g = lg.index_select(0, torch.tensor(rows, device=lg.device)).cpu().numpy()
    ctx = oracle.SeqContext(inp, 0, q8=True)
    for n, i in enumerate(rows):
        ok, wb = fp8_mfma_close(g[n], ctx, i, np.arange(cfg.n_heads))
        assert ok, f"fp8 dense logits query {i}: {wb} of the fp8 bound"


INDEXER_Q8_CASES = [
    dict(name="iq8_fused", n_seq=1, m=40, n=40000, hh=32, b=64, h=8, k=2048),
    dict(name="iq8_dagger", n_seq=1, m=48, n=36000, hh=32, b=64, h=8, k=1024, kp=4096),
    dict(name="iq8_short_decode", n_seq=3, m=1, n=3000, hh=16, b=64, h=5, k=256),
]


@pytest.mark.parametrize("case", INDEXER_Q8_CASES, ids=lambda c: c["name"])
def test_fp8_indexer_equals_its_steps_and_oracle(case):
    c = dict(case)
    name, kp = c.pop("name"), c.pop("kp", 0)
    say("fp8-query indexer", name)
    cfg = gen.small_config(name=name, kdtype=gen.KDTYPE_FP8, seed=53, kp=kp, **c)
    inp = gen.generate(cfg)
    st = q8_stages(inp)
    t, sh = st["t"], st["sh"]
    ii, iv = lcsb.misa_indexer_q8(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk, t["k_scale"], k_prime=kp)
    if kp == 0:
        si, sv = lcsb.misa_sparse_head_topk_q8(sh, st["q8"], st["qs"], t["w"], t["k"], st["heads"], cfg.topk,
                                               t["k_scale"])
    else:
        cand, _ = lcsb.misa_sparse_head_topk_q8(sh, st["q8"], st["qs"], t["w"], t["k"], st["heads"], kp,
                                                t["k_scale"], sorted=False, want_vals=False)
        dl = lcsb.dsa_dense_logits(sh, t["q"], t["w"], t["k"], k_scale=t["k_scale"], cand=cand)
        si, sv = lcsb.misa_topk(sh, dl, cfg.topk, cand=cand)
    torch.cuda.synchronize()
    assert torch.equal(ii, si) and torch.equal(iv, sv), "misa_indexer_q8 != its steps"
    gi = ii.cpu().numpy()
    recs = []
    for b in range(cfg.n_seq):
        ctx = oracle.SeqContext(inp, b, q8=True)
        ctx_bf16 = oracle.SeqContext(inp, b)
        for i in sample_rows(cfg.q_per_seq, 6):
            # routing on bf16 q, routed scoring on the fp8 queries
            heads = ctx_bf16.route(i, cfg.h)[2]
            I = ctx.score(i, heads)
            if kp:
                # the k' candidates re-ranked with bf16 q and every head
                cand_o = oracle.topk_prefix(I, ctx.t(i), kp)[0]
                D = oracle.score_candidates(ctx_bf16.q[i], ctx_bf16.w[i], ctx_bf16.keys, cand_o)
                ref = oracle.topk_row(D, cand_o, cfg.topk)[0]
            else:
                ref = oracle.topk_prefix(I, ctx.t(i), cfg.topk)[0]
            recs.append(recall(gi[b, i], ref))
    assert np.mean(recs) >= 0.999, np.mean(recs)
