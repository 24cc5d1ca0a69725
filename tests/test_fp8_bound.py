"""The derived tolerance of the fp8-query kernels (gpu_helpers.fp8_mfma_close),
checked on the CPU: rows that differ from the oracle only by the fp8 matrix
cores' accumulation error pass, and plausible kernel mistakes fail."""
import numpy as np

import oracle
from gpu_helpers import EPS_F8, fp8_mfma_close
from long_context_sparse_block_amd import inputs as gen


def context():
    cfg = gen.small_config(name="fp8_bound", n_seq=1, m=8, n=1500, hh=64, b=64, h=8, k=64,
                           kdtype=gen.KDTYPE_FP8, seed=52)
    return oracle.SeqContext(gen.generate(cfg), 0, q8=True)


def test_accumulation_error_of_the_modelled_size_passes():
    ctx = context()
    rng = np.random.default_rng(3)
    heads = np.arange(64)
    for i in range(4):
        t = ctx.t(i)
        q, w, keys = ctx.q[i], ctx.w[i], ctx.keys[:t + 1]
        dots = q @ keys.T
        absd = np.abs(q) @ np.abs(keys).T
        # every dot product off by a quarter of the allowance (the measured
        # accumulation error), with random signs; then fp32 rounding
        noisy = dots + rng.choice([-1.0, 1.0], dots.shape) * (EPS_F8 / 4) * absd
        g = np.full(ctx.keys.shape[0], -np.inf)
        g[:t + 1] = (w[:, None] * np.maximum(noisy, 0.0)).sum(axis=0)
        ok, worst = fp8_mfma_close(g.astype(np.float32), ctx, i, heads)
        assert ok, worst


def test_a_dropped_or_misplaced_head_fails():
    ctx = context()
    heads = np.arange(64)
    i = 5
    t = ctx.t(i)
    q, w, keys = ctx.q[i], ctx.w[i], ctx.keys[:t + 1]
    o = ctx.dense(i)
    term = w[:, None] * np.maximum(q @ keys.T, 0.0)
    # heads of typical weight (a head whose weight is a hundredth of the
    # others' contributes less than any tolerance can see)
    by_w = np.argsort(np.abs(w))
    j, j2 = int(by_w[32]), int(by_w[-1])
    dropped = o.copy()
    dropped[:t + 1] -= term[j]
    assert not fp8_mfma_close(dropped.astype(np.float32), ctx, i, heads)[0]
    w2 = w.copy()
    w2[[j, j2]] = w2[[j2, j]]   # two heads' weights swapped
    swapped = o.copy()
    swapped[:t + 1] = (w2[:, None] * np.maximum(q @ keys.T, 0.0)).sum(axis=0)
    assert not fp8_mfma_close(swapped.astype(np.float32), ctx, i, heads)[0]
    # one key's logit off by a whole head term
    one = o.copy()
    s = int(np.argmax(np.abs(term[j])))
    one[s] += term[j, s]
    assert not fp8_mfma_close(one.astype(np.float32), ctx, i, heads)[0]
    # a causal-mask mistake
    late = o.copy()
    late[t] = -np.inf
    assert not fp8_mfma_close(late.astype(np.float32), ctx, i, heads)[0]
