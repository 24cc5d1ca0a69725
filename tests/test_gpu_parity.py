"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Staged checks feed each kernel the inputs its oracle stage gets (the router
the GPU's pooled keys, the scoring kernel the GPU's routed heads, the top-k
the GPU's own logits), so every stage is compared on equal footing:
  * pooled keys / tails and the fp8 decode: fp32 vs fp64, relative 1e-5;
  * router scores r and logits: within 1e-2 relative (row-scaled near 0);
  * routed heads and MISA token sets: bit-exact outside the tolerance band;
  * top-k of given logits: bit-exact (the decision is taken on the same fp32
    values on both sides);
  * GPU identities, bitwise: routed scoring with every head == dense DSA;
    MISA-dagger with k' >= L == dense top-k; repeated runs identical.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_block_amd as lcsb
import oracle
from gpu_helpers import (band_check, check_logits, check_pool, check_route, check_topk_exact, f64,
                         logits_close, recall, run_stages, sample_rows, say, shape_of, upload)
from long_context_sparse_block_amd import inputs as gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    lcsb.load()


# ---------------------------------------------------------------------------
# fp8 decode and pooling
# ---------------------------------------------------------------------------

def test_fp8_decode_all_codes_through_pooling():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # 254 finite codes
    N = len(codes)
    k = np.stack([np.roll(codes, -s)[:128] for s in range(N)]).astype(np.uint8)
    scale = np.where(np.arange(N) % 2 == 0, 1.0, 0.25).astype(np.float32)   # powers of two: exact
    sh = lcsb.make_shape(1, 1, N, N - 1, 1, 1)
    dev = torch.device("cuda:0")
    kt = torch.from_numpy(k[None]).to(dev)
    st = torch.from_numpy(scale[None]).to(dev)
    pooled, tail = lcsb.misa_pool_keys(sh, kt, st)
    got = f64(pooled[0])
    expect = oracle.e4m3fn_to_f64(k) * scale[:, None].astype(np.float64)
    assert np.array_equal(got, expect)
    nz = expect != 0          # a block sum starts at +0, so a lone -0.0 pools to +0.0
    assert np.array_equal(np.signbit(got[nz]), np.signbit(expect[nz]))
    assert not f64(tail).any()


def test_fp8_decode_all_codes_through_scoring():
    """Every finite e4m3 code through the scoring kernels' fp8 -> bf16 widening.
    Query i reads dimension i // 2 with sign +-1 through a one-hot head, so each
    logit is exactly ReLU(+-decode(code)) * sigma: the routed kernel (h = 1),
    the dense kernel (H = 2, the second head weighted 0) and the candidate
    re-rank kernel must all reproduce the oracle's decoder value for value."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # 254 finite codes
    n_code = len(codes)
    M = 256                                  # 128 dims x 2 signs
    N = n_code + M                           # queries at t >= n_code see every code row
    k = np.zeros((N, 128), np.uint8)
    k[:n_code] = np.stack([np.roll(codes, -s)[:128] for s in range(n_code)])
    scale = np.where(np.arange(N) % 2 == 0, 1.0, 0.25).astype(np.float32)
    q = np.zeros((M, 2, 128), np.float32)
    for i in range(M):
        q[i, 0, i // 2] = 1.0 if i % 2 == 0 else -1.0
    w = np.zeros((M, 2), np.float32)
    w[:, 0] = 1.0
    dev = torch.device("cuda:0")
    sh = lcsb.make_shape(1, M, N, n_code, 2, 64)
    qt = torch.from_numpy(q[None]).to(dev).to(torch.bfloat16)
    wt = torch.from_numpy(w[None]).to(dev)
    kt = torch.from_numpy(k[None]).to(dev)
    st = torch.from_numpy(scale[None]).to(dev)
    heads = torch.zeros((1, M, 1), dtype=torch.int32, device=dev)
    dec = oracle.e4m3fn_to_f64(k[:n_code]) * scale[:n_code, None].astype(np.float64)   # [code row, dim]
    sign = np.where(np.arange(M) % 2 == 0, 1.0, -1.0)
    expect = np.maximum(sign[:, None] * dec[:, np.arange(M) // 2].T, 0.0)            # [query, code row]
    routed = f64(lcsb.misa_sparse_head_logits(sh, qt, wt, kt, heads, k_scale=st)[0])
    dense = f64(lcsb.dsa_dense_logits(sh, qt, wt, kt, k_scale=st)[0])
    cand = torch.arange(n_code, dtype=torch.int32, device=dev).repeat(M, 1)[None].contiguous()
    gather = f64(lcsb.dsa_dense_logits(sh, qt, wt, kt, k_scale=st, cand=cand)[0])
    for name, got in (("routed", routed[:, :n_code]), ("dense", dense[:, :n_code]), ("gather", gather[:, :n_code])):
        bad = np.argwhere(got != expect)
        assert len(bad) == 0, f"{name}: {len(bad)} mismatches, first {bad[:3].tolist()}"


@pytest.mark.parametrize("kdtype", [gen.KDTYPE_BF16, gen.KDTYPE_FP8])
@pytest.mark.parametrize("n", [517, 640])
def test_logit_columns_past_n(kdtype, n):
    """Routed and dense logits leave columns roundup4(N)..ld-1 untouched; the
    columns N..roundup4(N)-1 hold either their old value or -inf."""
    say("columns past N", kdtype, n)
    cfg = gen.small_config(m=40, n=n, b=16, k=32, kdtype=kdtype, seed=31)
    inp = gen.generate(cfg)
    d = upload(inp)
    sh = shape_of(inp)
    dev = torch.device("cuda:0")
    ld = (n + 3) // 4 * 4 + 12
    heads = torch.tensor(np.tile(np.arange(cfg.h, dtype=np.int32), (1, cfg.q_per_seq, 1)), device=dev)
    r4 = (n + 3) // 4 * 4
    for name in ("routed", "dense"):
        lg = torch.full((1, cfg.q_per_seq, ld), float("nan"), device=dev)
        if name == "routed":
            lcsb.misa_sparse_head_logits(sh, d["q"], d["w"], d["k"], heads, k_scale=d["k_scale"], logits=lg)
        else:
            lcsb.dsa_dense_logits(sh, d["q"], d["w"], d["k"], k_scale=d["k_scale"], logits=lg)
        x = lg.cpu().numpy()
        assert not np.isnan(x[..., :n]).any(), name
        assert np.isnan(x[..., r4:]).all(), f"{name}: columns past roundup4(N) were written"
        pad = x[..., n:r4]
        assert (np.isnan(pad) | np.isneginf(pad)).all(), name


POOL_CASES = [
    dict(m=37, n=1000, b=64), dict(m=64, n=512, b=1), dict(m=20, n=300, b=3),
    dict(m=16, n=40, b=64), dict(m=33, n=777, b=128, kdtype=gen.KDTYPE_FP8),
    dict(m=1, n=4096, b=64, n_seq=3), dict(m=10, n=600, b=7, q_pos0=100),
]


@pytest.mark.parametrize("case", POOL_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_pool_parity(case):
    c = dict(case)
    inp = gen.generate(gen.small_config(m=c.pop("m"), n=c.pop("n"), b=c.pop("b"), hh=16, h=4, k=16,
                                        kdtype=c.pop("kdtype", gen.KDTYPE_BF16), n_seq=c.pop("n_seq", 1),
                                        q_pos0=c.pop("q_pos0", None), seed=21))
    say("pool case", case)
    st = run_stages(inp)
    check_pool(inp, st)


# ---------------------------------------------------------------------------
# staged parity on small workloads, including ragged and degenerate shapes
# ---------------------------------------------------------------------------

STAGE_CASES = [
    dict(name="tiny", cfg=gen.CONFIGS["tiny_prefill_m256_n4k"]),
    dict(name="ragged", cfg=gen.small_config(m=37, n=1003, hh=64, b=64, h=8, k=100, seed=5)),
    dict(name="fp8", cfg=gen.small_config(m=70, n=2049, hh=64, b=128, h=8, k=300,
                                          kdtype=gen.KDTYPE_FP8, seed=6)),
    dict(name="h1_B1", cfg=gen.small_config(m=9, n=300, hh=16, b=1, h=1, k=40, seed=7)),
    dict(name="h5_B3_H48", cfg=gen.small_config(m=45, n=650, hh=48, b=3, h=5, k=64, seed=8)),
    dict(name="h12_H32", cfg=gen.small_config(m=40, n=900, hh=32, b=64, h=12, k=128, seed=9)),
    dict(name="h24_fp8", cfg=gen.small_config(m=21, n=700, hh=64, b=32, h=24, k=77,
                                              kdtype=gen.KDTYPE_FP8, seed=10)),
    dict(name="Bbig", cfg=gen.small_config(m=30, n=200, hh=64, b=512, h=8, k=50, seed=11)),
    dict(name="decode", cfg=gen.small_config(n_seq=5, m=1, n=3000, hh=32, b=64, h=8, k=256, seed=12)),
    dict(name="mid_chunk", cfg=gen.small_config(m=50, n=1500, hh=64, b=64, h=8, k=120, q_pos0=600,
                                                seed=13)),
    dict(name="short_prefix", cfg=gen.small_config(m=40, n=40, hh=16, b=8, h=4, k=64, seed=14)),
]


@pytest.fixture(scope="module")
def staged():
    cache = {}

    def get(name):
        if name not in cache:
            case = next(c for c in STAGE_CASES if c["name"] == name)
            inp = gen.generate(case["cfg"])
            cache[name] = (inp, run_stages(inp))
        return cache[name]
    return get


@pytest.mark.parametrize("name", [c["name"] for c in STAGE_CASES])
def test_staged_parity(staged, name):
    say("staged case", name)
    inp, st = staged(name)
    cfg = inp.cfg
    check_pool(inp, st)
    worst_r, inside = check_route(inp, st)
    worst_l = check_logits(inp, st)
    idx, vals = lcsb.misa_topk(st["sh"], st["logits"], cfg.topk)
    check_topk_exact(inp, st["logits"], cfg.topk, idx, vals)
    # masked region beyond each query is -inf, padding beyond N untouched by contract
    say(f"  router worst {worst_r:.2e} (band disagreements {inside}); logits worst {worst_l:.2e}")


@pytest.mark.parametrize("name", ["tiny", "fp8", "h5_B3_H48", "decode", "mid_chunk"])
def test_dense_logits_parity_and_routed_all_heads_identity(staged, name):
    say("dense case", name)
    inp, st = staged(name)
    cfg = inp.cfg
    t = st["t"]
    sh = st["sh"]
    dense = lcsb.dsa_dense_logits(sh, t["q"], t["w"], t["k"], k_scale=t["k_scale"])
    allh = torch.arange(cfg.n_heads, dtype=torch.int32, device=dense.device)
    allh = allh.expand(cfg.n_seq, cfg.q_per_seq, cfg.n_heads).contiguous()
    routed_all = lcsb.misa_sparse_head_logits(sh, t["q"], t["w"], t["k"], allh, k_scale=t["k_scale"])
    torch.cuda.synchronize()
    N = cfg.n_keys
    assert torch.equal(dense[..., :N], routed_all[..., :N]), "h = H routed scoring != dense DSA"
    rows = sample_rows(cfg.q_per_seq, 24)
    for b in range(cfg.n_seq):
        ctx = oracle.SeqContext(inp, b)
        g = dense[b, rows, :N].cpu().numpy()
        for n, i in enumerate(rows):
            ok, wst = logits_close(g[n][None], ctx.dense(i)[None])
            assert ok, f"dense seq {b} query {i} worst {wst}"


def test_topk_candidate_mode_ties_and_padding():
    rng = np.random.default_rng(3)
    M, n_cols, k = 7, 1003, 300
    vals = (rng.integers(-6, 7, (1, M, n_cols)) / 2.0).astype(np.float32)
    vals[rng.random(vals.shape) < 0.1] = -0.0
    ids = np.stack([rng.permutation(5000)[:n_cols] for _ in range(M)])[None].astype(np.int32)
    ids[rng.random(ids.shape) < 0.2] = -1
    ids[0, 3, :] = -1                       # a row with no candidate at all
    ids[0, 4, 50:] = -1                      # fewer candidates than k
    sh = lcsb.make_shape(1, M, 5000, 0, 1, 1)
    dev = torch.device("cuda:0")
    ld = (n_cols + 3) // 4 * 4
    lg = torch.full((1, M, ld), float("nan"), device=dev)
    lg[..., :n_cols] = torch.from_numpy(vals).to(dev)
    idx, v = lcsb.misa_topk(sh, lg, k, cand=torch.from_numpy(ids).to(dev))
    gi, gv = idx.cpu().numpy(), v.cpu().numpy()
    for i in range(M):
        oi, ov = oracle.topk_row(vals[0, i].astype(np.float64), ids[0, i].astype(np.int64), k)
        assert np.array_equal(gi[0, i], oi), f"row {i}"
        assert np.array_equal(gv[0, i].astype(np.float64), ov)


@pytest.mark.parametrize("kind", ["all_equal", "two_values", "neg_zero_mix", "short_rows", "wide"])
def test_topk_degenerate_rows(kind):
    rng = np.random.default_rng(4)
    M, N, k = 6, 20000, 2048
    if kind == "all_equal":
        vals = np.full((1, M, N), 0.5, np.float32)
    elif kind == "two_values":
        vals = np.where(rng.random((1, M, N)) < 0.5, 1.0, 2.0).astype(np.float32)
    elif kind == "neg_zero_mix":
        vals = np.where(rng.random((1, M, N)) < 0.5, -0.0, 0.0).astype(np.float32)
        vals[0, :, ::97] = 1e-30
    elif kind == "short_rows":
        N = 3000
        vals = rng.standard_normal((1, M, N)).astype(np.float32)
    else:
        k = 8192
        vals = rng.standard_normal((1, M, N)).astype(np.float32)
    q_pos0 = N - M if kind != "short_rows" else 1000
    M_ = M
    sh = lcsb.make_shape(1, M_, N, q_pos0, 1, 1)
    dev = torch.device("cuda:0")
    ld = (N + 3) // 4 * 4
    lg = torch.zeros((1, M_, ld), device=dev)
    lg[..., :N] = torch.from_numpy(vals).to(dev)
    idx, v = lcsb.misa_topk(sh, lg, k)
    check_topk_exact_arrays(vals, q_pos0, k, idx.cpu().numpy(), v.cpu().numpy())


def check_topk_exact_arrays(vals, q_pos0, k, gi, gv):
    for i in range(vals.shape[1]):
        oi, ov = oracle.topk_prefix(vals[0, i].astype(np.float64), q_pos0 + i, k)
        assert np.array_equal(gi[0, i], oi), f"row {i}"
        assert np.array_equal(gv[0, i].astype(np.float64), ov)


# ---------------------------------------------------------------------------
# whole indexer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "ragged", "fp8", "decode", "h12_H32"])
def test_indexer_matches_stages_and_oracle(staged, name):
    say("indexer case", name)
    inp, st = staged(name)
    cfg = inp.cfg
    t = st["t"]
    sh = st["sh"]
    idx, vals = lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk, k_scale=t["k_scale"])
    sidx, svals = lcsb.misa_topk(sh, st["logits"], cfg.topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, sidx) and torch.equal(vals, svals), "indexer != its stages"
    gi = idx.cpu().numpy()
    gh = st["heads"].cpu().numpy()
    recs = []
    for b in range(cfg.n_seq):
        ctx = oracle.SeqContext(inp, b)
        for i in range(cfg.q_per_seq):
            out = ctx.misa(i, cfg.h, cfg.topk)
            recs.append(recall(gi[b, i], out["idx"]))
            if np.array_equal(np.sort(out["heads"]), gh[b, i]):
                T = inp.q_pos0 + i
                ok, _ = band_check(out["I"][:T + 1], np.arange(T + 1), gi[b, i], cfg.topk)
                assert ok, f"token set seq {b} query {i}"
    say(f"  recall mean {np.mean(recs):.6f} min {np.min(recs):.4f}")
    assert np.mean(recs) >= 0.999


def test_indexer_is_deterministic(staged):
    inp, st = staged("fp8")
    cfg = inp.cfg
    t = st["t"]
    outs = [lcsb.misa_indexer(st["sh"], t["q"], t["w"], t["k"], cfg.h, cfg.topk, k_prime=2 * cfg.topk,
                              k_scale=t["k_scale"]) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0]) and torch.equal(o[1], outs[0][1])


# ---------------------------------------------------------------------------
# fused scoring -> top-k (the indexer's path when every prefix is >= 32768 keys)
# ---------------------------------------------------------------------------

def _staged_selection(inp, st, k_prime):
    """The indexer's result rebuilt from the separate stage calls."""
    cfg, t, sh = inp.cfg, st["t"], st["sh"]
    if not k_prime:
        return lcsb.misa_topk(sh, st["logits"], cfg.topk)
    cand, _ = lcsb.misa_topk(sh, st["logits"], k_prime, want_vals=False, sorted=False)
    D = lcsb.dsa_dense_logits(sh, t["q"], t["w"], t["k"], k_scale=t["k_scale"], cand=cand)
    return lcsb.misa_topk(sh, D, cfg.topk, cand=cand)


def _check_sparse_head_topk(inp, st):
    """misa_sparse_head_topk == misa_topk(misa_sparse_head_logits): the sorted
    result exactly, the unsorted one as a set per row."""
    cfg, t, sh = inp.cfg, st["t"], st["sh"]
    fi, fv = lcsb.misa_sparse_head_topk(sh, t["q"], t["w"], t["k"], st["heads"], cfg.topk, k_scale=t["k_scale"])
    ti, tv = lcsb.misa_topk(sh, st["logits"], cfg.topk)
    ui, _ = lcsb.misa_sparse_head_topk(sh, t["q"], t["w"], t["k"], st["heads"], cfg.topk, k_scale=t["k_scale"],
                                       sorted=False, want_vals=False)
    torch.cuda.synchronize()
    assert torch.equal(fi, ti) and torch.equal(fv, tv), "fused selection != logits + top-k"
    a, b = torch.sort(ui, dim=-1)[0], torch.sort(ti, dim=-1)[0]
    assert torch.equal(a, b), "unsorted fused selection is not the same set"


@pytest.mark.parametrize("name", ["tiny", "fp8", "decode"])
def test_sparse_head_topk_short_prefixes_equals_logits_topk(staged, name):
    """Prefixes too short for the fused path: logits in the workspace, then top-k."""
    inp, st = staged(name)
    _check_sparse_head_topk(inp, st)


FUSED_CASES = [
    dict(name="fused_bf16", n_seq=1, m=96, n=40000, hh=32, b=64, h=8, k=2048, kdtype=gen.KDTYPE_BF16),
    dict(name="fused_fp8_h5", n_seq=1, m=40, n=36001, hh=48, b=128, h=5, k=1000, kdtype=gen.KDTYPE_FP8),
    dict(name="fused_dagger", n_seq=1, m=64, n=40000, hh=32, b=64, h=8, k=1024, kp=4096,
         kdtype=gen.KDTYPE_BF16),
    dict(name="fused_decode", n_seq=6, m=1, n=50000, hh=32, b=64, h=8, k=2048, kdtype=gen.KDTYPE_BF16),
    dict(name="fused_2seq_fp8", n_seq=2, m=70, n=38000, hh=32, b=64, h=8, k=2048, kdtype=gen.KDTYPE_FP8),
    dict(name="fused_mid_prefix", n_seq=1, m=64, n=20000, hh=32, b=64, h=8, k=2048, kdtype=gen.KDTYPE_BF16),
    # few router workgroups (2 per sequence, the second with one query) over 625 blocks: the
    # indexer's router splits each block sum into 4 parts (the last ragged) and a finishing pass
    dict(name="fused_split_router_h64", n_seq=2, m=5, n=40000, hh=64, b=64, h=8, k=2048,
         kdtype=gen.KDTYPE_FP8),
    # the edge of the few-query passes: 8 queries per sequence still run one-wave workgroups (every
    # lane row of the wave holds a query), 9 the four-wave ones
    dict(name="fused_8q", n_seq=2, m=8, n=40000, hh=32, b=64, h=8, k=2048, kdtype=gen.KDTYPE_BF16),
    dict(name="fused_9q_fp8", n_seq=2, m=9, n=40000, hh=32, b=64, h=8, k=2048, kdtype=gen.KDTYPE_FP8),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: c["name"])
def test_fused_indexer_equals_stages_and_oracle(case):
    c = dict(case)
    name, kp = c.pop("name"), c.pop("kp", 0)
    say("fused indexer", name)
    cfg = gen.small_config(name=name, n_seq=c["n_seq"], m=c["m"], n=c["n"], hh=c["hh"], b=c["b"], h=c["h"],
                           k=c["k"], kdtype=c["kdtype"], seed=41)
    inp = gen.generate(cfg)
    st = run_stages(inp)
    idx, vals = lcsb.misa_indexer(st["sh"], st["t"]["q"], st["t"]["w"], st["t"]["k"], cfg.h, cfg.topk,
                                  k_prime=kp, k_scale=st["t"]["k_scale"])
    sidx, svals = _staged_selection(inp, st, kp)
    torch.cuda.synchronize()
    # (with few queries the indexer's router adds its block sum in parts over
    # several workgroups; the staged misa_route_heads adds the same parts in the
    # same order in one workgroup, so the heads agree bit for bit)
    assert torch.equal(idx, sidx) and torch.equal(vals, svals), "fused indexer != its stages"
    _check_sparse_head_topk(inp, st)
    gi = idx.cpu().numpy()
    recs = []
    for b in range(cfg.n_seq):
        ctx = oracle.SeqContext(inp, b)
        for i in sample_rows(cfg.q_per_seq, 6):
            out = ctx.misa_dagger(i, cfg.h, kp, cfg.topk) if kp else ctx.misa(i, cfg.h, cfg.topk)
            recs.append(recall(gi[b, i], out["idx"]))
    assert np.mean(recs) >= 0.999, np.mean(recs)


@pytest.mark.parametrize("topk", [3000, 6000])
def test_fused_selection_larger_k_equals_logits_topk(topk):
    """k above 2048 takes the region selects with 8192- and 16384-candidate
    lists (the MISA-dagger candidate pass uses the latter): sorted result
    bitwise equal to logits + top-k, unsorted the same set, and each row's
    set checked against the oracle's top-k of the same logits."""
    say("fused selection, k =", topk)
    cfg = gen.small_config(name=f"fused_k{topk}", m=40, n=40000, hh=16, b=64, h=8, k=topk,
                           kdtype=gen.KDTYPE_FP8, seed=45)
    inp = gen.generate(cfg)
    st = run_stages(inp)
    _check_sparse_head_topk(inp, st)
    fi, fv = lcsb.misa_sparse_head_topk(st["sh"], st["t"]["q"], st["t"]["w"], st["t"]["k"], st["heads"], topk,
                                        k_scale=st["t"]["k_scale"])
    torch.cuda.synchronize()
    check_topk_exact(inp, st["logits"], topk, fi, fv)


def test_fused_indexer_rows_the_sample_misjudges():
    """Every sampled key position (multiples of the sampling stride, 32 here)
    gets a huge score, so the sampled threshold admits far fewer than k
    candidates in every row: each row must be re-scored and selected from full
    logits, and the result must still equal the staged pipeline."""
    say("fused indexer: threshold defeated")
    cfg = gen.small_config(name="fused_adv", m=48, n=40000, hh=16, b=64, h=8, k=2048, seed=43, plant=False)
    inp = gen.generate(cfg)
    q = oracle.bf16_bits_to_f64(inp.q).astype(np.float32)
    kf = oracle.bf16_bits_to_f64(inp.k).astype(np.float32)
    u = np.ones(128, np.float32) / np.sqrt(128.0)
    q += 4.0 * u
    kf[:, ::32, :] += 40.0 * u
    inp.q[...] = gen.to_bf16_bits(q)
    inp.k[...] = gen.to_bf16_bits(kf)
    inp.w[...] = np.abs(inp.w)
    st = run_stages(inp)
    idx, vals = lcsb.misa_indexer(st["sh"], st["t"]["q"], st["t"]["w"], st["t"]["k"], cfg.h, cfg.topk)
    sidx, svals = _staged_selection(inp, st, 0)
    torch.cuda.synchronize()
    assert torch.equal(idx, sidx) and torch.equal(vals, svals)
    check_topk_exact(inp, st["logits"], cfg.topk, idx, vals)
    _check_sparse_head_topk(inp, st)


def test_fused_select_tied_list_past_4096():
    """4,400 keys of every query's prefix share one key vector far above the
    others, so in every row they tie on one score: the sampled threshold (about
    one sample in nine is a tied key) admits exactly them, a list of more than
    4096 and at most 4608 entries in one rank bucket.  The compact list ranks a
    crowded bucket only up to 4096 entries, so each row must be flagged and
    selected from full logits; ties go to the lower token id."""
    say("fused select: tied list past 4096")
    cfg = gen.small_config(name="fused_tied", m=1024, n=40000, hh=16, b=64, h=8, k=2048, seed=47, plant=False)
    inp = gen.generate(cfg)
    q = oracle.bf16_bits_to_f64(inp.q).astype(np.float32)
    kf = oracle.bf16_bits_to_f64(inp.k).astype(np.float32)
    u = np.ones(128, np.float32) / np.sqrt(128.0)
    q += 4.0 * u
    tied = np.random.default_rng(48).choice(inp.q_pos0 - 500, size=4400, replace=False)
    kf[:, tied, :] = 40.0 * u
    inp.q[...] = gen.to_bf16_bits(q)
    inp.k[...] = gen.to_bf16_bits(kf)
    inp.w[...] = np.abs(inp.w)
    st = run_stages(inp)
    sh, t = st["sh"], st["t"]
    idx, vals = lcsb.misa_sparse_head_topk(sh, t["q"], t["w"], t["k"], st["heads"], cfg.topk)
    sidx, svals = lcsb.misa_topk(sh, st["logits"], cfg.topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, sidx) and torch.equal(vals, svals)
    # every row's top-k: the 2048 lowest tied ids, all at one value
    gi = idx.cpu().numpy()[0]
    lowest = np.sort(tied)[:cfg.topk]
    for i in sample_rows(cfg.q_per_seq, 16):
        assert np.array_equal(gi[i], lowest), f"query {i}"
    check_topk_exact(inp, st["logits"], cfg.topk, idx, vals)


def _threshold_defeated(inp):
    """Every key at a multiple of the sampling stride (32) gets a huge score,
    so the sampled threshold admits far fewer than k candidates: every row is
    flagged for the re-scoring."""
    q = oracle.bf16_bits_to_f64(inp.q).astype(np.float32)
    kf = oracle.bf16_bits_to_f64(inp.k).astype(np.float32)
    u = np.ones(128, np.float32) / np.sqrt(128.0)
    q += 4.0 * u
    kf[:, ::32, :] += 40.0 * u
    inp.q[...] = gen.to_bf16_bits(q)
    inp.k[...] = gen.to_bf16_bits(kf)
    inp.w[...] = np.abs(inp.w)
    return inp


@pytest.mark.parametrize("room", ["least", "two_tiles", "three_tiles"])
def test_fused_indexer_in_a_smaller_workspace(room):
    """Below the fast plan's workspace the flagged rows are re-scored through a
    logits slab a few query tiles at a time (the least workspace: one tile,
    and candidate regions sized closer to the expected candidates).  Two
    sequences of 48 queries (2 tiles each, the second ragged) with every row
    flagged: the result equals the fast plan's bit for bit, in 4, 2 and 2
    batches."""
    say(f"fused indexer in a smaller workspace ({room})")
    cfg = gen.small_config(name="fused_slab", n_seq=2, m=48, n=40000, hh=16, b=64, h=8, k=2048, seed=46,
                           plant=False)
    inp = _threshold_defeated(gen.generate(cfg))
    st = run_stages(inp)
    sh, t = st["sh"], st["t"]
    full = lcsb.misa_indexer_workspace_bytes(sh, cfg.kdtype, cfg.h, cfg.topk)
    least = lcsb.misa_indexer_workspace_min_bytes(sh, cfg.kdtype, cfg.h, cfg.topk)
    tile = 32 * 40000 * 4
    # (regions of 128-key ranges hold at most 32 groups in either plan, so the
    # least workspace is the fast one with a slab of one tile)
    assert least == full - 3 * tile
    size = dict(least=least, two_tiles=full - 2 * tile, three_tiles=full - tile)[room]
    ref_i, ref_v = lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk)
    ws = torch.empty(size, dtype=torch.uint8, device="cuda")
    idx, vals = lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk, ws=ws)
    sidx, svals = _staged_selection(inp, st, 0)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_i) and torch.equal(vals, ref_v)
    assert torch.equal(idx, sidx) and torch.equal(vals, svals)
    with pytest.raises(lcsb.MisaError):
        lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk,
                          ws=torch.empty(least - 256, dtype=torch.uint8, device="cuda"))


def test_fused_indexer_nonpositive_scores_ragged_query_tile():
    """All head weights negative: every score is <= 0 and a good share of each
    row is exactly 0 (no routed head with a positive dot product), so the row
    thresholds are <= 0 and the top-k is decided by index among equal zeros.
    M = 37 leaves a query tile with padding lanes, whose zero scores would
    pass such a threshold; they belong to no row and must not reach any
    row's candidates."""
    say("fused indexer: scores <= 0, ragged query tile")
    cfg = gen.small_config(name="fused_neg", m=37, n=40000, hh=16, b=64, h=4, k=256, seed=44, plant=False)
    inp = gen.generate(cfg)
    inp.w[...] = -np.abs(inp.w)
    st = run_stages(inp)
    idx, vals = lcsb.misa_indexer(st["sh"], st["t"]["q"], st["t"]["w"], st["t"]["k"], cfg.h, cfg.topk)
    sidx, svals = _staged_selection(inp, st, 0)
    torch.cuda.synchronize()
    assert float(svals.max()) <= 0.0 and int((svals == 0).sum()) > 0
    assert torch.equal(idx, sidx) and torch.equal(vals, svals)
    check_topk_exact(inp, st["logits"], cfg.topk, idx, vals)
    _check_sparse_head_topk(inp, st)


@pytest.mark.parametrize("kdtype", [gen.KDTYPE_BF16, gen.KDTYPE_FP8])
def test_dagger_with_all_candidates_is_dense_topk(kdtype):
    # k' >= L: every prefix token is a candidate, the re-rank is the dense indexer
    cfg = gen.small_config(m=48, n=2000, hh=64, b=64, h=8, k=256, kp=2048, kdtype=kdtype, seed=31)
    inp = gen.generate(cfg)
    t = upload(inp)
    sh = shape_of(inp)
    idx, vals = lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk, k_prime=cfg.k_prime,
                                  k_scale=t["k_scale"])
    dense = lcsb.dsa_dense_logits(sh, t["q"], t["w"], t["k"], k_scale=t["k_scale"])
    didx, dvals = lcsb.misa_topk(sh, dense, cfg.topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, didx) and torch.equal(vals, dvals)
    ctx = oracle.SeqContext(inp, 0)
    gi = idx.cpu().numpy()
    for i in sample_rows(cfg.q_per_seq, 12):
        T = inp.q_pos0 + i
        ok, _ = band_check(ctx.dense(i)[:T + 1], np.arange(T + 1), gi[0, i], cfg.topk)
        assert ok, f"query {i}"


def test_dagger_rerank_parity():
    cfg = gen.small_config(m=40, n=3000, hh=64, b=64, h=8, k=128, kp=512, seed=32)
    inp = gen.generate(cfg)
    st = run_stages(inp)
    t, sh = st["t"], st["sh"]
    cand, _ = lcsb.misa_topk(sh, st["logits"], cfg.k_prime)
    D = lcsb.dsa_dense_logits(sh, t["q"], t["w"], t["k"], cand=cand)
    fidx, fvals = lcsb.misa_topk(sh, D, cfg.topk, cand=cand)
    idx, vals = lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk, k_prime=cfg.k_prime)
    torch.cuda.synchronize()
    assert torch.equal(idx, fidx) and torch.equal(vals, fvals)
    dense = lcsb.dsa_dense_logits(sh, t["q"], t["w"], t["k"])
    torch.cuda.synchronize()
    ctx = oracle.SeqContext(inp, 0)
    gc, gD = cand.cpu().numpy()[0], D.cpu().numpy()[0]
    gdense = dense.cpu().numpy()[0]
    gfi = fidx.cpu().numpy()[0]
    for i in range(cfg.q_per_seq):
        # re-ranked score of a candidate is bitwise the dense logit of that token
        ok_c = gc[i] >= 0
        assert np.array_equal(gD[i, :cfg.k_prime][ok_c], gdense[i, gc[i][ok_c]])
        o = oracle.score_candidates(ctx.q[i], ctx.w[i], ctx.keys, gc[i].astype(np.int64))
        ok, wst = logits_close(gD[i, :cfg.k_prime][None], o[None])
        assert ok, f"rerank query {i} worst {wst}"
        oi, _ = oracle.topk_row(gD[i, :cfg.k_prime].astype(np.float64), gc[i].astype(np.int64), cfg.topk)
        assert np.array_equal(gfi[i], oi)


@pytest.mark.parametrize("kind", ["sample_too_high", "sample_too_low", "ascending"])
def test_topk_rows_that_defeat_the_sampled_threshold(kind):
    # the top-k samples every 32nd 128-byte line to pick its first threshold;
    # these rows make that guess wrong in both directions, forcing the exact
    # fallback stream (rescan without threshold, or lock-step with compaction)
    M, N, k = 3, 131072, 2048
    line = np.arange(N) // 32
    sampled = (line % 32) == 0
    rng = np.random.default_rng(5)
    base = rng.standard_normal((1, M, N)).astype(np.float32)
    if kind == "sample_too_high":
        vals = base.copy()
        vals[0, :, sampled & (np.arange(N) % 32 == 7)] = 100.0     # 128 huge values, all sampled
    elif kind == "sample_too_low":
        vals = np.where(sampled, base - 10.0, base + 10.0).astype(np.float32)
    else:
        vals = np.broadcast_to(np.arange(N, dtype=np.float32), (1, M, N)).copy()
    sh = lcsb.make_shape(1, M, N, N - M, 1, 1)
    lg = torch.from_numpy(vals).to(torch.device("cuda:0"))
    idx, v = lcsb.misa_topk(sh, lg, k)
    check_topk_exact_arrays(vals, N - M, k, idx.cpu().numpy(), v.cpu().numpy())


@pytest.mark.parametrize("n,k,q0", [(40001, 2048, None), (50003, 8192, None), (16384, 2048, None),
                                    (20000, 2048, 8170), (20000, 2048, 7000), (20000, 4096, 0)])
def test_topk_long_rows_split_path(n, k, q0):
    """Rows of buffers long enough for the long-row paths (the one-kernel
    top-k for k <= 4096, the threshold / filter / list kernels above):
    ragged lengths, causal prefixes (rows from 1 to 40 keys, rows of about
    7000 keys that keep every element, rows crossing 8192 keys where the
    sampled threshold starts), repeated values."""
    say("long-row top-k", n, k, q0)
    M = 40
    rng = np.random.default_rng(n + k)
    vals = rng.standard_normal((1, M, n)).astype(np.float32)
    vals[0, :, ::7] = np.round(vals[0, :, ::7], 1)          # many exact ties
    q_pos0 = n - M if q0 is None else q0
    sh = lcsb.make_shape(1, M, n, q_pos0, 1, 1)
    dev = torch.device("cuda:0")
    ld = (n + 3) // 4 * 4
    lg = torch.full((1, M, ld), float("nan"), device=dev)
    lg[..., :n] = torch.from_numpy(vals).to(dev)
    idx, v = lcsb.misa_topk(sh, lg, k)
    check_topk_exact_arrays(vals, q_pos0, k, idx.cpu().numpy(), v.cpu().numpy())
    idx2, _ = lcsb.misa_topk(sh, lg, k, sorted=False)
    for i in range(M):
        assert set(idx2[0, i].cpu().numpy().tolist()) == set(idx[0, i].cpu().numpy().tolist())


@pytest.mark.parametrize("kind", ["ties", "sample_too_high", "sample_too_low", "all_equal", "short_prefixes"])
def test_topk_one_kernel_and_chunked_paths_agree(kind):
    """Rows of at least 16384 keys: 512 rows or more take the one-kernel top-k,
    fewer take the chunked threshold / filter / list kernels.  Both are exact,
    so the same rows through each agree bit for bit (ids, values, order), and
    sampled rows equal the oracle.  The kinds defeat the sampled threshold in
    both directions, tie everything, or keep every element (prefixes shorter
    than the sample)."""
    say("one-kernel vs chunked top-k", kind)
    M, N, k = 512, 20000, 2048
    rng = np.random.default_rng(31)
    vals = rng.standard_normal((1, M, N)).astype(np.float32)
    line = np.arange(N) // 32
    sampled = (line % 4) == 0          # around the lines a 20000-key row's sample reads
    if kind == "ties":
        vals = np.round(vals, 1)
    elif kind == "sample_too_high":
        vals[0, :, sampled & (np.arange(N) % 32 == 7)] = 100.0
    elif kind == "sample_too_low":
        vals = np.where(sampled, vals - 10.0, vals + 10.0).astype(np.float32)
    elif kind == "all_equal":
        vals[...] = 0.25
    q_pos0 = 300 if kind == "short_prefixes" else N - M
    dev = torch.device("cuda:0")
    lg = torch.from_numpy(vals).to(dev)
    one, one_v = lcsb.misa_topk(lcsb.make_shape(1, M, N, q_pos0, 1, 1), lg, k)
    a, a_v = lcsb.misa_topk(lcsb.make_shape(1, 256, N, q_pos0, 1, 1), lg[:, :256].contiguous(), k)
    b, b_v = lcsb.misa_topk(lcsb.make_shape(1, 256, N, q_pos0 + 256, 1, 1), lg[:, 256:].contiguous(), k)
    torch.cuda.synchronize()
    assert torch.equal(one[:, :256], a) and torch.equal(one[:, 256:], b)
    assert torch.equal(one_v[:, :256], a_v) and torch.equal(one_v[:, 256:], b_v)
    rows = [0, 1, 255, 256, 511] + list(rng.choice(M, 5, replace=False))
    gi, gv = one.cpu().numpy(), one_v.cpu().numpy()
    for i in rows:
        oi, ov = oracle.topk_prefix(vals[0, i].astype(np.float64), q_pos0 + i, k)
        assert np.array_equal(gi[0, i], oi), f"row {i}"
        assert np.array_equal(gv[0, i].astype(np.float64), ov)


@pytest.mark.parametrize("k", [300, 2048, 8192])
def test_topk_unsorted_returns_the_same_set(k):
    rng = np.random.default_rng(6)
    M, N = 4, 20000
    vals = rng.standard_normal((1, M, N)).astype(np.float32)
    vals[0, 1, :] = np.round(vals[0, 1, :])            # ties
    sh = lcsb.make_shape(1, M, N, N - M, 1, 1)
    lg = torch.from_numpy(vals).to(torch.device("cuda:0"))
    si, sv = lcsb.misa_topk(sh, lg, k)
    ui, uv = lcsb.misa_topk(sh, lg, k, sorted=False)
    si, ui, uv = si.cpu().numpy(), ui.cpu().numpy(), uv.cpu().numpy()
    for i in range(M):
        n_ok = (si[0, i] >= 0).sum()
        assert np.all(ui[0, i, n_ok:] == -1)
        assert sorted(ui[0, i, :n_ok].tolist()) == sorted(si[0, i, :n_ok].tolist())
        assert np.array_equal(uv[0, i, :n_ok], vals[0, i, ui[0, i, :n_ok]])
