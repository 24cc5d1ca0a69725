"""The router's other readings (CPU only).

The pages say that each indexer head is scored against the mean-pooled block
keys and that these affinities are aggregated along the blocks into one
importance per head (gist.science summary of MISA, "Metodologia: MISA" item
1; agents-report summary, the HISA comparison), but they print no formula.
The oracle implements the reading this repository takes (partial last block
pooled, signed weight, sum over blocks) and, for comparison only, the others:
the partial block dropped, |w| or no weight, max instead of sum.

* every reading is pinned by the pure-Python brute force and by closed forms;
* on the generated workloads, the share of queries whose routed heads change
  between readings is measured and printed (the figures quoted in the design
  notes), with the planted heads routed under every reading.
"""
import dataclasses
import itertools

import numpy as np
import pytest

import brute
import oracle
from long_context_sparse_block_amd import inputs as gen
from oracle_helpers import inputs_from_arrays, random_tiny

READINGS = [dict(tail_mode=t, weight=w, agg=a)
            for t, w, a in itertools.product(*oracle.ROUTER_READINGS.values())]
DEFAULT = dict(tail_mode="pool", weight="signed", agg="sum")


def _name(rd):
    return f"tail={rd['tail_mode']},weight={rd['weight']},agg={rd['agg']}"


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("B", [1, 3, 4, 7, 64])
def test_every_reading_against_brute_force(seed, B):
    M, N, H, d = 3, 13, 5, 6
    q, w, k, q_pos0 = random_tiny(seed * 17 + B, M=M, N=N, H=H, d=d)
    h = 1 + seed % 3
    ctx = oracle.SeqContext(inputs_from_arrays(q, w, k_f32=k, q_pos0=q_pos0, block=B, h=h), 0)
    keys = ctx.keys.tolist()
    for i in range(M):
        t = q_pos0 + i
        for rd in READINGS:
            S, r, heads = ctx.route(i, h, reading=rd)
            bS, br, bheads, _ = brute.bf_route(ctx.q[i].tolist(), ctx.w[i].tolist(), keys, t, B, h, **rd)
            np.testing.assert_allclose(S, bS, rtol=1e-12, atol=1e-12, err_msg=_name(rd))
            np.testing.assert_allclose(r, br, rtol=1e-12, atol=1e-12, err_msg=_name(rd))
            assert heads.tolist() == bheads, _name(rd)


def test_default_reading_is_the_oracle_router():
    q, w, k, q_pos0 = random_tiny(21, M=4, N=30, H=6, d=8)
    ctx = oracle.SeqContext(inputs_from_arrays(q, w, k_f32=k, q_pos0=q_pos0, block=4, h=2), 0)
    for i in range(4):
        S0, r0, h0 = ctx.route(i, 2)
        S1, r1, h1 = ctx.route(i, 2, reading=DEFAULT)
        np.testing.assert_allclose(S1, S0, rtol=1e-14)
        np.testing.assert_allclose(r1, r0, rtol=1e-14)
        assert h1.tolist() == h0.tolist()


def test_closed_forms_of_the_readings():
    q, w, k, q_pos0 = random_tiny(22, M=4, N=20, H=6, d=8)
    per_token = np.einsum("mhd,nd->mhn", q.astype(np.float64), k.astype(np.float64))
    # B = 1: every key is a complete block, so dropping the partial block changes
    # nothing, and max over blocks is the largest ReLU(q_j . k_s) over s <= t
    ctx = oracle.SeqContext(inputs_from_arrays(q, w, k_f32=k, q_pos0=q_pos0, block=1, h=3), 0)
    for i in range(4):
        t = q_pos0 + i
        relu_terms = np.maximum(per_token[i, :, :t + 1], 0.0)
        for wt in oracle.ROUTER_READINGS["weight"]:
            a = ctx.route(i, 3, reading=dict(tail_mode="pool", weight=wt, agg="sum"))
            b = ctx.route(i, 3, reading=dict(tail_mode="drop", weight=wt, agg="sum"))
            np.testing.assert_allclose(a[1], b[1], rtol=1e-14)
        S, r, _ = ctx.route(i, 3, reading=dict(tail_mode="pool", weight="none", agg="max"))
        np.testing.assert_allclose(S, relu_terms.max(axis=1), rtol=1e-13)
        np.testing.assert_allclose(r, S, rtol=0)
        _, r, _ = ctx.route(i, 3, reading=dict(tail_mode="pool", weight="abs", agg="max"))
        np.testing.assert_allclose(r, np.abs(w[i].astype(np.float64)) * S, rtol=1e-14)
    # one partial block and nothing else (B > L): with the block dropped every
    # head scores 0, and the tie rule routes the lowest head ids
    ctx = oracle.SeqContext(inputs_from_arrays(q[:, :, :], w, k_f32=k[:9], q_pos0=5, block=64, h=3), 0)
    for i in range(4):
        S, r, heads = ctx.route(i, 3, reading=dict(tail_mode="drop", weight="signed", agg="sum"))
        assert not S.any() and heads.tolist() == [0, 1, 2]
        # ... and with it kept, sum and max over the single block coincide
        a = ctx.route(i, 3, reading=dict(tail_mode="pool", weight="signed", agg="sum"))
        b = ctx.route(i, 3, reading=dict(tail_mode="pool", weight="signed", agg="max"))
        np.testing.assert_allclose(a[0], b[0], rtol=0)
    # positive weights: signed, |w| and (for the selection) w itself agree
    wpos = np.abs(w) + np.float32(0.25)
    ctx = oracle.SeqContext(inputs_from_arrays(q, wpos, k_f32=k, q_pos0=q_pos0, block=3, h=2), 0)
    for i in range(4):
        a = ctx.route(i, 2, reading=dict(tail_mode="pool", weight="signed", agg="sum"))
        b = ctx.route(i, 2, reading=dict(tail_mode="pool", weight="abs", agg="sum"))
        np.testing.assert_allclose(a[1], b[1], rtol=0)
        assert a[2].tolist() == b[2].tolist()


def _workloads():
    """(name, config, sequences, rows) sampled from every generated workload:
    the tiny chunk whole, 64 evenly spaced queries of the long chunks, the
    first 4 sequences of the decode batch (sequence b's draws do not depend on
    how many sequences follow it)."""
    C = gen.CONFIGS
    out = [("tiny_prefill_m256_n4k", C["tiny_prefill_m256_n4k"], 1, None)]
    for name in ("dsv32_prefill_m8k_n32k", "final_chunk_m8k_n128k_fp8", "dagger_prefill_m4k_n128k"):
        out.append((name, C[name], 1, 64))
    out.append(("glm5_decode_64x1_n128k", dataclasses.replace(C["glm5_decode_64x1_n128k"], n_seq=4), 4, None))
    return out


def test_how_much_the_routed_heads_depend_on_the_reading(capsys):
    lines = []
    for name, cfg, n_seq, n_rows in _workloads():
        inp = gen.generate(cfg)
        M = cfg.q_per_seq
        rows = list(range(M)) if n_rows is None else \
            np.unique(np.linspace(0, M - 1, n_rows).round().astype(int)).tolist()
        changed = {_name(rd): 0 for rd in READINGS}
        moved = {_name(rd): 0 for rd in READINGS}
        planted_hits = {_name(rd): 0 for rd in READINGS}
        n_q = 0
        for b in range(n_seq):
            ctx = oracle.SeqContext(inp, b)
            planted = set(inp.plant_heads[b].tolist())
            for i in rows:
                base = set(ctx.route(i, cfg.h)[2].tolist())
                n_q += 1
                for rd in READINGS:
                    heads = set(ctx.route(i, cfg.h, reading=rd)[2].tolist())
                    changed[_name(rd)] += heads != base
                    moved[_name(rd)] += len(heads - base)
                    planted_hits[_name(rd)] += len(planted & heads) / max(1, len(planted))
        for rd in READINGS:
            key = _name(rd)
            lines.append(f"{name:28s} {key:40s} queries with other heads {changed[key] / n_q:6.3f}  "
                         f"heads replaced per query {moved[key] / n_q:5.2f}  "
                         f"planted heads routed {planted_hits[key] / n_q:5.3f}")
            # the plant is built to be visible under every reading (a planted
            # head whose weight is near 0 can still lose under a weighted one)
            assert planted_hits[key] / n_q >= 0.75, (name, key)
        assert changed[_name(DEFAULT)] == 0
    with capsys.disabled():
        print("\nrouted heads under the other router readings (vs tail=pool, weight=signed, agg=sum):")
        print("\n".join(lines))
