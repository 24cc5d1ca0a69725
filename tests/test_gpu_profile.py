"""The profiling hook (misa_profile_stage) through the C ABI: the events it
records bracket the named stage inside a call on the call's stream, the
stage's time is positive and below the whole call's, results do not change,
and a stage the call does not run leaves the events alone."""
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


def _events():
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s = torch.cuda.current_stream()
    a.record(s)
    b.record(s)
    torch.cuda.synchronize()
    return a, b, a.elapsed_time(b)


def test_profile_stage_brackets_the_stages_of_the_fused_indexer():
    say("profiling hook on the fused indexer")
    cfg = gen.small_config(name="prof", n_seq=1, m=64, n=40000, hh=32, b=64, h=8, k=1024, seed=91)
    inp = gen.generate(cfg)
    t = upload(inp)
    sh = shape_of(inp)
    ref_i, ref_v = lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s = torch.cuda.current_stream()
    e0.record(s)
    lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk)
    e1.record(s)
    torch.cuda.synchronize()
    whole = e0.elapsed_time(e1)
    total = 0.0
    for stage in ("pool", "route", "score_sample", "sample_threshold", "score_candidates", "region_select",
                  "rescore"):
        a, b, before = _events()
        lcsb.misa_profile_stage(stage, a, b)
        try:
            idx, vals = lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk)
        finally:
            lcsb.misa_profile_stage(None)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        assert ms != before, f"stage {stage} was not recorded"
        assert 0 < ms < whole * 1.5, (stage, ms, whole)
        total += ms
        assert torch.equal(idx, ref_i) and torch.equal(vals, ref_v)
    say(f"  whole call {whole:.3f} ms, stages {total:.3f} ms")
    # the dagger stages are not run by a MISA call: the events stay as they were
    a, b, before = _events()
    lcsb.misa_profile_stage("rerank", a, b)
    try:
        lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk)
    finally:
        lcsb.misa_profile_stage(None)
    torch.cuda.synchronize()
    assert a.elapsed_time(b) == before
    # turned off: calls record nothing
    a, b, before = _events()
    lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk)
    torch.cuda.synchronize()
    assert a.elapsed_time(b) == before


def test_profile_stage_on_the_dagger_rerank():
    cfg = gen.small_config(name="prof_dag", n_seq=1, m=32, n=3000, hh=64, b=64, h=8, k=128, kp=512, seed=92)
    inp = gen.generate(cfg)
    t = upload(inp)
    sh = shape_of(inp)
    for stage in ("rerank", "final_topk"):
        a, b, before = _events()
        lcsb.misa_profile_stage(stage, a, b)
        try:
            lcsb.misa_indexer(sh, t["q"], t["w"], t["k"], cfg.h, cfg.topk, k_prime=cfg.k_prime)
        finally:
            lcsb.misa_profile_stage(None)
        torch.cuda.synchronize()
        assert a.elapsed_time(b) != before and a.elapsed_time(b) > 0
