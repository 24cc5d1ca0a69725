"""misa_indexer_noalloc (the indexer for callers that cannot allocate: its
scratch is the library's fixed device buffer) through the C ABI, against
misa_indexer on the same inputs: bit for bit (same kernels, same layout),
over calls in a row on the shared buffer, each smaller than the one before
(the buffer keeps the previous call's contents)."""
import numpy as np
import pytest
import torch

import long_context_sparse_block_amd as lcsb
from gpu_helpers import say, shape_of, upload
from long_context_sparse_block_amd import inputs as gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")
    lcsb.load()


# largest first: a decode batch over 50000 keys (the fused path), a prefill
# chunk with fp8 keys, then MISA-dagger on a small chunk
CASES = [
    dict(name="decode_fused", n_seq=6, m=1, n=50000, hh=32, b=64, h=8, k=2048, kdtype=gen.KDTYPE_BF16, kp=0),
    dict(name="prefill_fp8", n_seq=1, m=256, n=4096, hh=64, b=64, h=8, k=256, kdtype=gen.KDTYPE_FP8, kp=0),
    dict(name="dagger_small", n_seq=2, m=40, n=1500, hh=16, b=32, h=4, k=64, kdtype=gen.KDTYPE_BF16, kp=128),
]


def _run(case, seed):
    c = dict(case)
    name, kp = c.pop("name"), c.pop("kp")
    cfg = gen.small_config(name=name, n_seq=c["n_seq"], m=c["m"], n=c["n"], hh=c["hh"], b=c["b"], h=c["h"],
                           k=c["k"], kdtype=c["kdtype"], seed=seed)
    inp = gen.generate(cfg)
    t = upload(inp)
    sh = shape_of(inp)
    need = lcsb.misa_indexer_workspace_bytes(sh, cfg.kdtype, cfg.h, cfg.topk, kp)
    assert need <= lcsb.NOALLOC_SCRATCH_BYTES, (name, need)
    say(f"no-alloc indexer {name}: {need / 2**20:.1f} MiB of scratch")
    ref_i, ref_v = lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk, k_prime=kp, k_scale=t["k_scale"])
    # the outputs are allocated here, before the call: the entry point itself allocates nothing
    idx = torch.full_like(ref_i, -7)
    vals = torch.full_like(ref_v, 7.0)
    lcsb.misa_indexer_noalloc(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk, k_prime=kp, k_scale=t["k_scale"],
                              idx=idx, vals=vals)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_i), name
    assert torch.equal(vals, ref_v), name
    return idx


def test_noalloc_equals_indexer_on_calls_in_a_row():
    for n, case in enumerate(CASES):
        _run(case, seed=71 + n)


def test_noalloc_repeat_after_a_larger_call():
    # the small case again right after the largest: stale contents of the
    # buffer must not leak into the result
    _run(CASES[0], seed=80)
    a = _run(CASES[2], seed=81)
    b = _run(CASES[2], seed=81)
    assert torch.equal(a, b)


def test_noalloc_refuses_an_oversized_request():
    cfg = gen.small_config(name="big", n_seq=1, m=8, n=4096, hh=8, b=64, h=4, k=64, seed=5)
    inp = gen.generate(cfg)
    t = upload(inp)
    big = lcsb.make_shape(1, 8192, 131072, 131072 - 8192, 64, 128)
    assert lcsb.misa_indexer_workspace_bytes(big, gen.KDTYPE_BF16, 8, 2048) > lcsb.NOALLOC_SCRATCH_BYTES
    st = lcsb.load().misa_indexer_noalloc(
        lcsb._lib.ctypes.byref(big), lcsb._lib._ptr(t["q"]), lcsb._lib._ptr(t["w"]), lcsb._lib._ptr(t["k"]), 0,
        None, 8, 2048, 0, lcsb._lib._ptr(torch.empty(1, dtype=torch.int32, device="cuda")), None, None)
    assert st == lcsb.MISA_ERR_SCRATCH
