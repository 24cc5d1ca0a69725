"""GPU parity of the fp8 query path (misa_quantize_q, misa_sparse_head_logits_q8).

  * quantisation: codes and scales bit-exact against the oracle (integer
    outputs), including zero rows, values that land in e4m3fn's subnormal
    range, and exact midpoints between codes (ties to even);
  * fp8 scoring: every logit against the oracle's routed score of the
    dequantised queries and keys, within the scoring tolerance (the fp8 matrix
    cores accumulate at slightly less than fp32 precision);
  * the top-k of those logits against the oracle's, up to the tolerance band.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_block_amd as lcsb
import oracle
from gpu_helpers import band_check, logits_close, say, shape_of, upload
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
            worst = max(worst, wst)
            T = ctx.t(i)
            ok, _ = band_check(o[:T + 1], np.arange(T + 1), gi[b, i], cfg.topk)
            assert ok, f"fp8 top-k seq {b} query {i}"
    say(f"  worst relative logit error {worst:.2e}")
