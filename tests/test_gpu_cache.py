"""GPU parity of the pooled-key cache and the chunked-prefill driver.

Block means do not depend on which call pools them, so every cached path
must equal the one-call indexer bit for bit (ids and values):
  * misa_prefill_chunked over a whole prompt == one misa_indexer call over
    the same queries (bf16 and fp8 keys, two sequences, MISA-dagger, a ragged
    last chunk), and == a loop of misa_indexer_cached calls sharing one cache;
  * decode steps with the cache (one query per sequence, the cache grown by
    misa_indexer_cached and misa_pool_keys_cached) == misa_indexer from
    scratch at every step, across block boundaries;
  * the GLM-5-shaped 64K prompt (H = 32) in chunks of 8192, with sampled
    rows against the oracle.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_block_amd as lcsb
import oracle
from gpu_helpers import recall, sample_rows, say, shape_of, upload
from long_context_sparse_block_amd import inputs as gen

pytestmark = pytest.mark.gpu


def whole(st, cfg, kp=0):
    return lcsb.misa_indexer(st["sh"], st["t"]["q"], st["t"]["w"], st["t"]["k"], cfg.h, cfg.topk, k_prime=kp,
                             k_scale=st["t"]["k_scale"])


def staged(inp):
    return dict(t=upload(inp), sh=shape_of(inp))


PROMPT_CASES = [
    dict(name="prompt_bf16", n_seq=1, m=40000, n=40000, hh=32, b=64, h=8, k=2048, chunk=8192),
    dict(name="prompt_fp8_2seq", n_seq=2, m=20000, n=21000, hh=16, b=128, h=5, k=512, chunk=6000,
         kdtype=gen.KDTYPE_FP8),
    dict(name="prompt_dagger", n_seq=1, m=36000, n=36000, hh=32, b=64, h=8, k=1024, kp=4096, chunk=8192),
]


@pytest.mark.parametrize("case", PROMPT_CASES, ids=lambda c: c["name"])
def test_chunked_prefill_equals_one_call(case):
    c = dict(case)
    name, chunk, kp = c.pop("name"), c.pop("chunk"), c.pop("kp", 0)
    say("chunked prefill", name)
    cfg = gen.small_config(name=name, seed=60, q_pos0=c["n"] - c["m"], plant=False, **c)
    inp = gen.generate(cfg)
    st = staged(inp)
    t = st["t"]
    ci, cv = lcsb.misa_prefill_chunked(st["sh"], t["q"], t["w"], t["k"], cfg.h, cfg.topk, chunk=chunk, k_prime=kp,
                                       k_scale=t["k_scale"])
    wi, wv = whole(st, cfg, kp)
    torch.cuda.synchronize()
    assert torch.equal(ci, wi) and torch.equal(cv, wv), "chunked prefill != one call"
    # the same chunks through misa_indexer_cached, one cache per sequence
    M, N = cfg.q_per_seq, cfg.n_keys
    for b in range(cfg.n_seq):
        cache = lcsb.PooledCache(1, N // cfg.block)
        for c0 in range(0, M, chunk):
            m = min(chunk, M - c0)
            q0 = inp.q_pos0 + c0
            sh = lcsb.make_shape(1, m, q0 + m, q0, cfg.n_heads, cfg.block)
            ks = None if t["k_scale"] is None else t["k_scale"][b:b + 1, :q0 + m].contiguous()
            ii, vv = lcsb.misa_indexer_cached(sh, t["q"][b:b + 1, c0:c0 + m].contiguous(),
                                              t["w"][b:b + 1, c0:c0 + m].contiguous(),
                                              t["k"][b:b + 1, :q0 + m].contiguous(), cfg.h, cfg.topk, cache,
                                              k_prime=kp, k_scale=ks)
            torch.cuda.synchronize()
            assert torch.equal(ii[0], wi[b, c0:c0 + m]) and torch.equal(vv[0], wv[b, c0:c0 + m]), \
                f"cached indexer, sequence {b}, chunk at {c0}"


def test_decode_steps_with_the_cache():
    say("decode with the pooled-key cache")
    S, N0, steps, B, H = 3, 5000, 70, 64, 32
    cfg = gen.small_config(name="decode_cache", n_seq=S, m=1, n=N0 + steps, hh=H, b=B, h=8, k=512, seed=61,
                           plant=False)
    inp = gen.generate(cfg)
    kfull = torch.from_numpy(inp.k.view(np.int16)).cuda().view(torch.bfloat16)
    rng = np.random.default_rng(62)
    cache = lcsb.PooledCache(S, (N0 + steps) // B)
    # prime the cache with the first N0 - 1 keys (no query)
    sh0 = lcsb.make_shape(S, 0, N0 - 1, N0 - 1, H, B)
    lcsb.misa_pool_keys_cached(sh0, kfull[:, :N0 - 1].contiguous(), cache)
    for step in range(steps):
        N = N0 + step
        sh = lcsb.make_shape(S, 1, N, N - 1, H, B)
        q = torch.from_numpy(gen.to_bf16_bits(rng.standard_normal((S, 1, H, 128)).astype(np.float32))
                             .view(np.int16)).cuda().view(torch.bfloat16)
        w = torch.from_numpy((rng.standard_normal((S, 1, H)) / 8).astype(np.float32)).cuda()
        k = kfull[:, :N].contiguous()
        ci, cv = lcsb.misa_indexer_cached(sh, q, w, k, cfg.h, cfg.topk, cache)
        ri, rv = lcsb.misa_indexer(sh, q, w, k, cfg.h, cfg.topk)
        torch.cuda.synchronize()
        assert torch.equal(ci, ri) and torch.equal(cv, rv), f"decode step {step} (N = {N})"
        assert cache.n_cached == N // B


def test_glm5_prompt_chunked_prefill():
    """GLM-5 shape (H = 32, B = 64, fp8 keys), a 64K prompt in 8 chunks of
    8192: equal to one call, and sampled rows against the oracle."""
    cfg = gen.CONFIGS["glm5_prompt_m64k_h32_fp8"]
    say("chunked prefill", cfg.name)
    inp = gen.generate(cfg)
    st = staged(inp)
    t = st["t"]
    ci, cv = lcsb.misa_prefill_chunked(st["sh"], t["q"], t["w"], t["k"], cfg.h, cfg.topk, chunk=8192,
                                       k_scale=t["k_scale"])
    wi, wv = whole(st, cfg)
    torch.cuda.synchronize()
    assert torch.equal(ci, wi) and torch.equal(cv, wv), "chunked prefill != one call"
    gi = ci.cpu().numpy()
    ctx = oracle.SeqContext(inp, 0)
    recs = []
    for i in sample_rows(cfg.q_per_seq, 10):
        recs.append(recall(gi[0, i], ctx.misa(i, cfg.h, cfg.topk)["idx"]))
    assert np.mean(recs) >= 0.999, np.mean(recs)
