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
    rows against the oracle;
  * a paged key cache (shuffled pages, spare pages, a partial last page)
    gathered back bit for bit, an out-of-range page id giving zero keys, and
    the indexer on the gathered keys equal to the indexer on the originals;
  * misa_indexer_paged, reading the pages in place, == misa_indexer_cached on
    the contiguous keys (decode and a short chunk, bf16 and fp8, pages of 64
    to 256 keys, from an empty cache and from a previous step's cache).
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


@pytest.mark.parametrize("kdtype,page_keys", [(gen.KDTYPE_FP8, 64), (gen.KDTYPE_BF16, 48)])
def test_paged_keys_gather(kdtype, page_keys):
    say("paged key cache", kdtype, page_keys)
    cfg = gen.small_config(name="paged", n_seq=3, m=16, n=5000, hh=16, b=64, h=4, k=128, kdtype=kdtype, seed=63)
    inp = gen.generate(cfg)
    S, N = cfg.n_seq, cfg.n_keys
    per_seq = -(-N // page_keys)
    max_pages = per_seq + 2
    n_pages = S * per_seq + 7
    rng = np.random.default_rng(64)
    ids = rng.permutation(n_pages)[:S * per_seq].reshape(S, per_seq).astype(np.int32)
    table = np.full((S, max_pages), -1, np.int32)
    table[:, :per_seq] = ids
    kdt = inp.k.dtype
    pages = np.zeros((n_pages, page_keys, 128), kdt)
    pscale = np.zeros((n_pages, page_keys), np.float32)
    for b in range(S):
        for p in range(per_seq):
            rows = inp.k[b, p * page_keys:(p + 1) * page_keys]
            pages[ids[b, p], :len(rows)] = rows
            if inp.k_scale is not None:
                pscale[ids[b, p], :len(rows)] = inp.k_scale[b, p * page_keys:(p + 1) * page_keys]
    dev = "cuda"
    if kdtype == gen.KDTYPE_FP8:
        kp = torch.from_numpy(pages).to(dev)
        sp = torch.from_numpy(pscale).to(dev)
    else:
        kp = torch.from_numpy(pages.view(np.int16)).to(dev).view(torch.bfloat16)
        sp = None
    tt = torch.from_numpy(table).to(dev)
    sh = shape_of(inp)
    kg, sg = lcsb.misa_gather_keys_paged(sh, kp, tt, scale_pages=sp)
    st = staged(inp)
    torch.cuda.synchronize()
    assert torch.equal(kg.view(torch.uint8), st["t"]["k"].view(torch.uint8))
    if sg is not None:
        assert torch.equal(sg, st["t"]["k_scale"])
    t = st["t"]
    ia, va = lcsb.misa_indexer(sh, t["q"], t["w"], kg, cfg.h, cfg.topk, k_scale=sg)
    ib, vb = whole(st, cfg)
    torch.cuda.synchronize()
    assert torch.equal(ia, ib) and torch.equal(va, vb)
    # an out-of-range page id: its keys come back as zeros (scale 1), nothing read
    bad = tt.clone()
    bad[1, 2] = n_pages
    kb, sb = lcsb.misa_gather_keys_paged(sh, kp, bad, scale_pages=sp)
    torch.cuda.synchronize()
    lo, hi = 2 * page_keys, min(3 * page_keys, N)
    assert not bool(kb[1, lo:hi].view(torch.uint8).any())
    if sb is not None:
        assert bool((sb[1, lo:hi] == 1.0).all())
    assert torch.equal(kb[0], kg[0]) and torch.equal(kb[1, :lo], kg[1, :lo])


def paged_copy(inp, page_keys, seed):
    """The inputs' keys laid into shuffled pages of page_keys keys, with spare
    pages and a partial last page: (k_pages, scale_pages, table) on the GPU."""
    S, N = inp.cfg.n_seq, inp.cfg.n_keys
    per_seq = -(-N // page_keys)
    max_pages = per_seq + 2
    n_pages = S * per_seq + 7
    rng = np.random.default_rng(seed)
    ids = rng.permutation(n_pages)[:S * per_seq].reshape(S, per_seq).astype(np.int32)
    table = np.full((S, max_pages), -1, np.int32)
    table[:, :per_seq] = ids
    pages = np.zeros((n_pages, page_keys, 128), inp.k.dtype)
    pscale = np.zeros((n_pages, page_keys), np.float32)
    for b in range(S):
        for p in range(per_seq):
            rows = inp.k[b, p * page_keys:(p + 1) * page_keys]
            pages[ids[b, p], :len(rows)] = rows
            if inp.k_scale is not None:
                pscale[ids[b, p], :len(rows)] = inp.k_scale[b, p * page_keys:(p + 1) * page_keys]
    if inp.k_scale is not None:
        kp, sp = torch.from_numpy(pages).cuda(), torch.from_numpy(pscale).cuda()
    else:
        kp, sp = torch.from_numpy(pages.view(np.int16)).cuda().view(torch.bfloat16), None
    return kp, sp, torch.from_numpy(table).cuda()


@pytest.mark.parametrize("kdtype,page_keys,m", [(gen.KDTYPE_BF16, 64, 1), (gen.KDTYPE_FP8, 128, 1),
                                                (gen.KDTYPE_BF16, 256, 24), (gen.KDTYPE_FP8, 64, 24)])
def test_paged_indexer_reads_the_pages_in_place(kdtype, page_keys, m):
    say("paged indexer", kdtype, page_keys, m)
    cfg = gen.small_config(name="paged_ix", n_seq=3, m=m, n=20011, hh=16, b=64, h=8, k=512, kdtype=kdtype,
                           seed=71 + m)
    inp = gen.generate(cfg)
    kp, sp, tt = paged_copy(inp, page_keys, 72)
    st = staged(inp)
    sh, t = st["sh"], st["t"]
    S, N, B = cfg.n_seq, cfg.n_keys, cfg.block
    wi, wv = whole(st, cfg)
    # from an empty cache
    ca, cb = lcsb.PooledCache(S, N // B), lcsb.PooledCache(S, N // B)
    pi, pv = lcsb.misa_indexer_paged(sh, t["q"], t["w"], kp, tt, cfg.h, cfg.topk, ca, scale_pages=sp)
    ci, cv = lcsb.misa_indexer_cached(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk, cb, k_scale=t["k_scale"])
    torch.cuda.synchronize()
    assert torch.equal(pi, ci) and torch.equal(pv, cv), "paged != cached (empty cache)"
    assert torch.equal(pi, wi) and torch.equal(pv, wv), "paged != one call"
    assert torch.equal(ca.pooled, cb.pooled) and torch.equal(ca.split, cb.split)
    # from a previous step's cache: blocks of the first N - 700 keys pooled before
    prev = lcsb.make_shape(S, 0, N - 700, N - 700, cfg.n_heads, B)
    pk = t["k"][:, :N - 700].contiguous()
    pks = None if t["k_scale"] is None else t["k_scale"][:, :N - 700].contiguous()
    cc = lcsb.PooledCache(S, N // B)
    lcsb.misa_pool_keys_cached(prev, pk, cc, k_scale=pks)
    pi2, pv2 = lcsb.misa_indexer_paged(sh, t["q"], t["w"], kp, tt, cfg.h, cfg.topk, cc, scale_pages=sp)
    torch.cuda.synchronize()
    assert torch.equal(pi2, wi) and torch.equal(pv2, wv), "paged != one call (previous cache)"
    assert torch.equal(cc.pooled, ca.pooled)
    # an empty step only brings the cache up to date
    cd = lcsb.PooledCache(S, N // B)
    none = lcsb.make_shape(S, 0, N, N, cfg.n_heads, B)
    lcsb.misa_indexer_paged(none, t["q"][:, :0], t["w"][:, :0], kp, tt, cfg.h, cfg.topk, cd, scale_pages=sp)
    torch.cuda.synchronize()
    assert torch.equal(cd.pooled, ca.pooled)
