"""The indexer under HIP graph capture.

The library allocates, frees, clears and synchronises nothing (every buffer,
scratch included, comes from the caller), so a serving loop can capture a
whole indexer call in a graph and replay it.  Checked here: misa_indexer
(fused path, fp8 keys) and misa_indexer_q8 captured once, replayed several
times with eager work and synchronisation between replays and new inputs
copied into the captured buffers; every replay equals the eager call on the
same inputs, bit for bit.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_block_amd as lcsb
from gpu_helpers import say, shape_of, upload
from long_context_sparse_block_amd import inputs as gen

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fp8_query", [False, True])
def test_indexer_graph_replays_equal_eager(fp8_query):
    say("graph capture, fp8 queries" if fp8_query else "graph capture")
    cfg = gen.small_config(name="graph", m=64, n=40000, hh=32, b=64, h=8, k=1024, kdtype=gen.KDTYPE_FP8, seed=70)
    inputs = [upload(gen.generate(cfg, seed=s)) for s in (70, 71, 72)]
    sh = shape_of(gen.generate(cfg, seed=70))
    t0 = inputs[0]
    q, w, k, ks = (t0[n].clone() for n in ("q", "w", "k", "k_scale"))
    nbytes = (lcsb.misa_indexer_q8_workspace_bytes(sh, cfg.h, cfg.topk) if fp8_query
              else lcsb.misa_indexer_workspace_bytes(sh, cfg.kdtype, cfg.h, cfg.topk))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    idx = torch.empty((1, cfg.q_per_seq, cfg.topk), dtype=torch.int32, device=q.device)
    vals = torch.empty((1, cfg.q_per_seq, cfg.topk), dtype=torch.float32, device=q.device)

    def call(q_, w_, k_, ks_, idx_=None, vals_=None, ws_=None):
        if fp8_query:
            return lcsb.misa_indexer_q8(sh, q_, w_, k_, cfg.h, cfg.topk, ks_, idx=idx_, vals=vals_, ws=ws_)
        return lcsb.misa_indexer(sh, q_, w_, k_, cfg.h, cfg.topk, k_scale=ks_, idx=idx_, vals=vals_, ws=ws_)

    call(q, w, k, ks, idx, vals, ws)   # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            call(q, w, k, ks, idx, vals, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(6):
        t = inputs[rep % 3]
        q.copy_(t["q"]), w.copy_(t["w"]), k.copy_(t["k"]), ks.copy_(t["k_scale"])
        idx.fill_(-7)
        vals.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ei, ev = call(t["q"], t["w"], t["k"], t["k_scale"])   # eager, its own buffers
        torch.cuda.synchronize()
        assert torch.equal(idx, ei) and torch.equal(vals, ev), f"replay {rep}"
