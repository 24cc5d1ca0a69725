"""Pins of the fp64 oracle against things other than itself (CPU only).

* a hand-derived worked example (tests/golden/handworked_tiny.json), bf16 and fp8 keys;
* the OCP e4m3fn definition and torch's float8/bfloat16 casts (library routines);
* a pure-Python brute force (tests/brute.py) on tiny random inputs, with exact ties;
* closed forms: B = 1 (every key its own block) and B >= L (one partial block);
* invariances of the method: head relabelling, positive rescaling of w and k,
  key order inside a block;
* numpy lexsort as an independent top-k order, including -0.0 / +0.0;
* the MISA-dagger identities: k' >= L gives the dense top-k, k' = k keeps the MISA set.
"""
import numpy as np
import pytest
import torch

import brute
import oracle
from long_context_sparse_block_amd import inputs as gen
from oracle_helpers import fval, inputs_from_arrays, load_golden, random_tiny

D = 128


def golden_inputs(fp8):
    g = load_golden("handworked_tiny.json")
    M, H, N = g["q_per_seq"], g["n_heads"], g["n_keys"]
    q = np.zeros((M, H, D), np.float32)
    q[:, :, :2] = np.array(g["q_dim01"], np.float32)
    w = np.array(g["w"], np.float32)
    if fp8:
        codes = np.zeros((N, D), np.uint8)
        codes[:, :2] = np.array(g["keys_fp8"]["codes_dim01"], np.uint8)
        inp = inputs_from_arrays(q, w, k_codes=codes, k_scale=g["keys_fp8"]["scale"],
                                 q_pos0=g["q_pos0"], block=g["block"], h=g["h"], topk=3)
    else:
        k = np.zeros((N, D), np.float32)
        k[:, :2] = np.array(g["keys_dim01"], np.float32)
        inp = inputs_from_arrays(q, w, k_f32=k, q_pos0=g["q_pos0"], block=g["block"], h=g["h"], topk=3)
    return g, inp


@pytest.mark.parametrize("fp8", [False, True])
def test_golden_handworked(fp8):
    g, inp = golden_inputs(fp8)
    e = g["expect"]
    ctx = oracle.SeqContext(inp, 0)
    assert np.array_equal(ctx.keys[:, :2], np.array(g["keys_dim01"], float))
    assert np.array_equal(ctx.pooled[:, :2], np.array(e["pooled_dim01"], float))
    assert not ctx.pooled[:, 2:].any()
    for i in range(2):
        tl = ctx.tail(i)
        if e["tail_dim01"][i] is None:
            assert tl is None
        else:
            assert np.array_equal(tl[:2], np.array(e["tail_dim01"][i], float))
        S, r, heads = ctx.route(i, g["h"])
        assert np.array_equal(S, np.array(e["S"][i], float))
        assert np.array_equal(r, np.array(e["r"][i], float))
        assert heads.tolist() == e["heads"][i]
        I = ctx.score(i, heads)
        assert np.array_equal(I, np.array(fval(e["I"][i])))
        out = ctx.misa(i, g["h"], 3)
        assert out["idx"].tolist() == e["misa_top3_idx"][i]
        assert np.array_equal(out["vals"], np.array(fval(e["misa_top3_vals"][i])))
        assert np.array_equal(ctx.dense(i), np.array(fval(e["dense_I"][i])))
        assert ctx.dense_topk(i, 3)["idx"].tolist() == e["dense_top3_idx"][i]
        assert ctx.misa_dagger(i, g["h"], 4, 3)["idx"].tolist() == e["dagger_kp4_top3_idx"][i]
        assert ctx.misa_dagger(i, g["h"], 6, 3)["idx"].tolist() == e["dagger_kp6_top3_idx"][i]
    out = ctx.misa(0, g["h"], 7)
    assert out["idx"].tolist() == e["misa_top7_idx_q0"]
    assert np.array_equal(out["vals"], np.array(fval(e["misa_top7_vals_q0"])))


def test_e4m3fn_decoder_definition_points():
    # OCP FP8 E4M3: bias 7, max normal 448 = 0x7E, min subnormal 2^-9 = 0x01, NaN = s.1111.111
    c = np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x7E, 0xFE, 0x48, 0xB8, 0x7F, 0xFF], np.uint8)
    v = oracle.e4m3fn_to_f64(c)
    exp = [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 448.0, -448.0, 4.0, -1.0]
    assert np.array_equal(v[:10], exp)
    assert np.signbit(v[1])
    assert np.isnan(v[10]) and np.isnan(v[11])


def test_e4m3fn_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    got = oracle.e4m3fn_to_f64(codes)
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~ok)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 16, 4096).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]   # drop inf/nan patterns
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), ref)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("B", [1, 2, 3, 4, 7, 64])
def test_oracle_vs_brute_force(seed, B):
    # odd seeds: coarse values (exact ties in the scores fed to top-k); even seeds:
    # continuous values, where every selection of the whole pipeline must agree
    quant = 2 if seed % 2 else None
    M, N, H, d = 3, 13, 5, 6
    q, w, k, q_pos0 = random_tiny(seed * 31 + B, M=M, N=N, H=H, d=d, quant=quant)
    h = 1 + seed % 3
    kk = 4 + seed
    inp = inputs_from_arrays(q, w, k_f32=k, q_pos0=q_pos0, block=B, h=h, topk=kk)
    ctx = oracle.SeqContext(inp, 0)
    keys = ctx.keys.tolist()
    for i in range(M):
        qt, wt = ctx.q[i].tolist(), ctx.w[i].tolist()
        t = q_pos0 + i
        S, r, heads = ctx.route(i, h)
        bS, br, bheads, bblocks = brute.bf_route(qt, wt, keys, t, B, h)
        np.testing.assert_allclose(S, bS, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r, br, rtol=1e-12, atol=1e-12)
        n_full = (t + 1) // B
        np.testing.assert_allclose(ctx.pooled[:n_full], np.array(bblocks[:n_full]).reshape(n_full, d),
                                   rtol=1e-12, atol=1e-12)
        tl = ctx.tail(i)
        if n_full * B == t + 1:
            assert tl is None and len(bblocks) == n_full
        else:
            np.testing.assert_allclose(tl, bblocks[-1], rtol=1e-12, atol=1e-12)
        I = ctx.score(i, heads)
        bI = brute.bf_score(qt, wt, keys, t, heads.tolist(), N)
        np.testing.assert_allclose(I, bI, rtol=1e-12, atol=1e-12)
        # top-k of identical values: exact, ties included
        idx, _ = oracle.topk_prefix(I, t, kk)
        assert idx.tolist() == brute.bf_topk(I[:t + 1].tolist(), list(range(t + 1)), kk)
        D = ctx.dense(i)
        didx, _ = oracle.topk_prefix(D, t, kk)
        assert didx.tolist() == brute.bf_topk(D[:t + 1].tolist(), list(range(t + 1)), kk)
        if not quant:
            assert heads.tolist() == bheads
            assert ctx.misa(i, h, kk)["idx"].tolist() == brute.bf_misa(qt, wt, keys, t, B, h, kk)[2]
            assert didx.tolist() == brute.bf_dense_topk(qt, wt, keys, t, kk)
            for kp in (kk, kk + 3, t + 1, t + 5):
                assert ctx.misa_dagger(i, h, kp, kk)["idx"].tolist() == \
                    brute.bf_dagger(qt, wt, keys, t, B, h, kp, kk)


def test_route_B1_closed_form():
    # B = 1: every key is a block of its own, no partial block; S_j = sum_s<=t ReLU(q_j.k_s)
    q, w, k, q_pos0 = random_tiny(5, M=4, N=20, H=6, d=8)
    inp = inputs_from_arrays(q, w, k_f32=k, q_pos0=q_pos0, block=1, h=3, topk=4)
    ctx = oracle.SeqContext(inp, 0)
    per_head_token = np.einsum("mhd,nd->mhn", q.astype(np.float64), k.astype(np.float64))
    for i in range(4):
        t = q_pos0 + i
        assert ctx.tail(i) is None
        S, r, _ = ctx.route(i, 3)
        expect = np.maximum(per_head_token[i, :, :t + 1], 0).sum(axis=1)
        np.testing.assert_allclose(S, expect, rtol=1e-13)


def test_route_single_partial_block():
    # B > L: no complete block; the router sees one pooled key, the prefix mean
    q, w, k, q_pos0 = random_tiny(6, M=3, N=9, H=4, d=5)
    B = 64
    inp = inputs_from_arrays(q, w, k_f32=k, q_pos0=q_pos0, block=B, h=2, topk=3)
    ctx = oracle.SeqContext(inp, 0)
    assert ctx.pooled.shape[0] == 0
    for i in range(3):
        t = q_pos0 + i
        mean = k[:t + 1].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(ctx.tail(i), mean, rtol=1e-13)
        S, _, _ = ctx.route(i, 2)
        np.testing.assert_allclose(S, np.maximum(q[i].astype(np.float64) @ mean, 0), rtol=1e-13)


def test_pool_invariant_to_key_order_within_block():
    q, w, k, q_pos0 = random_tiny(7, M=2, N=16, H=3, d=4, quant=4)
    B = 4
    perm = np.arange(16)
    for m in range(4):
        perm[m * B:(m + 1) * B] = perm[m * B:(m + 1) * B][::-1]
    a = oracle.SeqContext(inputs_from_arrays(q, w, k_f32=k, q_pos0=q_pos0, block=B), 0)
    b = oracle.SeqContext(inputs_from_arrays(q, w, k_f32=k[perm], q_pos0=q_pos0, block=B), 0)
    assert np.array_equal(a.pooled, b.pooled)


def test_router_head_relabelling_equivariant_and_scale_invariant():
    q, w, k, q_pos0 = random_tiny(8, M=4, N=40, H=8, d=8)
    B, h = 4, 3
    base = oracle.SeqContext(inputs_from_arrays(q, w, k_f32=k, q_pos0=q_pos0, block=B), 0)
    perm = np.array([3, 7, 0, 5, 1, 6, 2, 4])
    relab = oracle.SeqContext(inputs_from_arrays(q[:, perm], w[:, perm], k_f32=k, q_pos0=q_pos0, block=B), 0)
    scaled = oracle.SeqContext(inputs_from_arrays(q, w * np.float32(4.0), k_f32=k * np.float32(0.5),
                                                  q_pos0=q_pos0, block=B), 0)
    for i in range(4):
        _, _, hb = base.route(i, h)
        _, _, hp = relab.route(i, h)
        assert sorted(perm[hp].tolist()) == hb.tolist()
        _, _, hs = scaled.route(i, h)
        assert hs.tolist() == hb.tolist()
        # I scales by 4 * 0.5 = 2 exactly (powers of two)
        assert np.array_equal(scaled.score(i, hb), 2.0 * base.score(i, hb))


def test_relu_gives_exact_zero_for_antialigned_keys():
    d = 8
    q = np.zeros((1, 2, d), np.float32)
    q[0, 0, 0] = 1.0
    q[0, 1, 1] = 1.0
    k = np.zeros((5, d), np.float32)
    k[:, 0] = -1.0
    k[:, 1] = -2.0
    w = np.array([[0.5, -0.75]], np.float32)
    inp = inputs_from_arrays(q, w, k_f32=k, q_pos0=4, block=2, h=2, topk=5)
    ctx = oracle.SeqContext(inp, 0)
    I = ctx.score(0, np.array([0, 1]))
    assert np.all(I == 0.0)
    S, r, heads = ctx.route(0, 1)
    assert np.all(S == 0.0) and heads.tolist() == [0]


def test_topk_against_lexsort_with_ties_and_signed_zeros():
    rng = np.random.default_rng(11)
    for trial in range(20):
        n = int(rng.integers(1, 3000))
        v = rng.integers(-5, 6, n).astype(np.float64) / 4.0   # many exact ties
        v[rng.random(n) < 0.2] = -0.0
        v[rng.random(n) < 0.05] = float("-inf")
        k = int(rng.integers(1, n + 20))
        idx, vals = oracle.topk_row(v, np.arange(n), k)
        order = np.lexsort((np.arange(n), -(v + 0.0)))[:k]    # primary key last
        assert idx[:len(order)].tolist() == order.tolist()
        assert np.all(idx[len(order):] == -1)
        assert np.all(np.isneginf(vals[len(order):]))


def test_topk_ties_break_on_candidate_token_id_not_position():
    vals = np.array([1.0, 2.0, 1.0, 2.0, 1.0])
    ids = np.array([40, 30, 10, -1, 20])       # -1 is not a candidate
    idx, v = oracle.topk_row(vals, ids, 4)
    assert idx.tolist() == [30, 10, 20, 40]
    assert v.tolist() == [2.0, 1.0, 1.0, 1.0]


def test_misa_h_equals_H_is_the_dense_indexer():
    q, w, k, q_pos0 = random_tiny(12, M=4, N=30, H=6, d=7)
    inp = inputs_from_arrays(q, w, k_f32=k, q_pos0=q_pos0, block=4, h=6, topk=9)
    ctx = oracle.SeqContext(inp, 0)
    for i in range(4):
        out = ctx.misa(i, 6, 9)
        assert out["heads"].tolist() == list(range(6))
        t = q_pos0 + i
        bI = brute.bf_score(ctx.q[i].tolist(), ctx.w[i].tolist(), ctx.keys.tolist(), t, list(range(6)), 30)
        np.testing.assert_allclose(out["I"], bI, rtol=1e-12)
        assert out["idx"].tolist() == ctx.dense_topk(i, 9)["idx"].tolist()


def test_dagger_identities():
    q, w, k, q_pos0 = random_tiny(13, M=5, N=50, H=6, d=8)
    inp = inputs_from_arrays(q, w, k_f32=k, q_pos0=q_pos0, block=5, h=2, topk=7)
    ctx = oracle.SeqContext(inp, 0)
    for i in range(5):
        t = q_pos0 + i
        dense = ctx.dense_topk(i, 7)["idx"].tolist()
        for kp in (t + 1, t + 9):                      # k' >= L: exactly the dense top-k
            assert ctx.misa_dagger(i, 2, kp, 7)["idx"].tolist() == dense
        m = ctx.misa(i, 2, 7)["idx"]
        dg = ctx.misa_dagger(i, 2, 7, 7)["idx"]        # k' = k: same set, dense order
        assert sorted(m.tolist()) == sorted(dg.tolist())


def test_planted_heads_are_routed_on_generated_workload():
    cfg = gen.small_config(m=32, n=2048, hh=16, b=64, h=4, k=64, seed=3)
    inp = gen.generate(cfg)
    ctx = oracle.SeqContext(inp, 0)
    planted = set(inp.plant_heads[0].tolist())
    hits = 0
    for i in range(cfg.q_per_seq):
        _, _, heads = ctx.route(i, cfg.h)
        hits += len(planted & set(heads.tolist()))
    frac = hits / (cfg.q_per_seq * len(planted))
    assert 0.5 < frac <= 1.0
    # tokens of the planted blocks dominate the top-k
    blocks = inp.plant_blocks[0]
    out = ctx.misa(cfg.q_per_seq - 1, cfg.h, cfg.topk)
    in_plant = np.isin(out["idx"] // cfg.block, blocks).mean()
    assert in_plant > 0.5
