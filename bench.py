"""Benchmark of the MISA indexer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]

A step is one pass of the MISA indexer over one prefill chunk resident in
HBM: one misa_indexer call through the C ABI (block pooling -> head routing
-> routed-head token scoring fused with the top-k selection), timed with HIP
events on the launch stream.  The headline workload is the long-context final
prefill chunk: M = 8192 queries against N = 131072 fp8 keys, H_I = 64 heads,
h = 8, B = 128, top-2048.

Printed: one JSON line.  value = scored (query, key, head) triples per second
(G/s) of the whole step; ms_per_step = indexer milliseconds per chunk;
roofline = the dominant kernel (the routed scoring that keeps the top-k
candidates), timed on its own inside the step through the library's
profiling hook, against the bf16 MFMA peak; stages = every stage's time and
roofline fraction.  Extras, each on its own seeded workload: MISA-dagger at
its own shape (M = 4096, bf16 keys, k' = 8192 -> 2048) with the split of time
between stages and its recall of the dense top-k; the same-GPU dense DSA
indexer; the fp8-query path; the 32K DeepSeek-V3.2 chunk and the tiny chunk;
the GLM-5 decode batch; a whole GLM-5 prompt through the chunked-prefill
driver.  cpu_baseline = the fp64 oracle on the host cores over a bounded
sample of the headline chunk.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, TFLOP/s
METRIC = "indexer ms per chunk & G(query·key·head)/s at M=8192,N=131K; MFMA util %"
UNIT = "G(query·key·head)/s"
FUSED_STAGES = ("pool", "route", "score_sample", "sample_threshold", "score_candidates", "region_select",
                "rescore")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="final_chunk_m8k_n128k_fp8")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="only the headline chunk")
    p.add_argument("--no-prefill", action="store_true", help="skip the decode and chunked-prefill legs")
    p.add_argument("--cpu-queries", type=int, default=1536, help="queries in the oracle timing sample")
    p.add_argument("--cpu-dense-queries", type=int, default=32, help="queries in the dense-oracle timing sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a 1 GiB device copy (reference kernel for HBM byte counters)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work per unit: 256 flops per scored triple,
# 4 bytes per causal-valid logit written and read once, 132/256 bytes per key
# ---------------------------------------------------------------------------

def work(cfg, q_pos0):
    M, N, H, h, B = cfg.q_per_seq, cfg.n_keys, cfg.n_heads, cfg.h, cfg.block
    t = q_pos0 + np.arange(M, dtype=np.int64)
    pairs = int((t + 1).sum()) * cfg.n_seq                       # causal (query, key) pairs
    n_full = (t + 1) // B
    blocks = int((n_full + ((t + 1) % B != 0)).sum()) * cfg.n_seq  # (query, block) pairs incl. tail
    key_bytes = N * (128 + 4 if cfg.kdtype == 1 else 256) * cfg.n_seq
    return dict(
        pairs=pairs,
        triples=pairs * h,
        score_flops=pairs * h * 256,
        score_bytes=pairs * 4,
        dense_flops=pairs * H * 256,
        route_flops=blocks * H * 256,
        pool_bytes=key_bytes + cfg.n_seq * (N // B) * 512 + cfg.n_seq * M * 512,
        topk_bytes=pairs * 4 + cfg.n_seq * M * cfg.topk * 8,
    )


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_sparse_block_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "score_candidates": ("score.hip", "score_shared.h", "misa_common.h"),
    "select": ("score.hip", "score_shared.h", "topk.hip", "misa_common.h"),
    "staged_score": ("score.hip", "score_shared.h", "misa_common.h"),
    "staged_topk": ("topk.hip", "misa_common.h"),
    "route": ("route.hip", "misa_common.h"),
    "pool": ("pool.hip", "misa_common.h"),
}


def measured_traffic(stage, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path) or stage not in KERNEL_SOURCES:
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(workload, {}).get(stage)
    if not ent or ent.get("source_hash") != src_hash(*KERNEL_SOURCES[stage]):
        return None
    return ent.get("bytes_per_launch")


def say(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class Bench:
    def __init__(self, torch, lcsb, gen, dev):
        self.torch, self.lcsb, self.gen, self.dev = torch, lcsb, gen, dev
        self.stream = torch.cuda.current_stream()

    def load(self, name):
        """Seeded inputs of a workload, resident on the GPU."""
        torch, gen = self.torch, self.gen
        cfg = gen.CONFIGS[name]
        t0 = time.perf_counter()
        inp = gen.generate(cfg)
        say(f"generated {name} in {time.perf_counter() - t0:.1f}s")
        dev = self.dev
        q = torch.from_numpy(inp.q.view(np.int16)).to(dev).view(torch.bfloat16)
        w = torch.from_numpy(inp.w).to(dev)
        if inp.k_scale is None:
            k = torch.from_numpy(inp.k.view(np.int16)).to(dev).view(torch.bfloat16)
            ks = None
        else:
            k = torch.from_numpy(inp.k).to(dev)
            ks = torch.from_numpy(inp.k_scale).to(dev)
        sh = self.lcsb.make_shape(cfg.n_seq, cfg.q_per_seq, cfg.n_keys, inp.q_pos0, cfg.n_heads, cfg.block)
        return dict(cfg=cfg, inp=inp, q=q, w=w, k=k, ks=ks, sh=sh, W=work(cfg, inp.q_pos0))

    def timed(self, stages, steps, warmup):
        """stages: list of (name, fn).  Returns per-stage mean ms and step ms
        (HIP events on the launch stream around each call)."""
        torch, stream = self.torch, self.stream
        for _ in range(warmup):
            for _, fn in stages:
                fn()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        for s in range(steps):
            evs[s][0].record(stream)
            for j, (_, fn) in enumerate(stages):
                fn()
                evs[s][j + 1].record(stream)
        torch.cuda.synchronize()
        self.wall = (time.perf_counter() - wall0) * 1e3 / steps
        per = {}
        for j, (name, _) in enumerate(stages):
            per[name] = float(np.mean([evs[s][j].elapsed_time(evs[s][j + 1]) for s in range(steps)]))
        self.samples = [evs[s][0].elapsed_time(evs[s][-1]) for s in range(steps)]
        return per, float(np.mean(self.samples))

    def stage_ms(self, fn, stages, steps):
        """Mean ms of each named stage inside calls of fn, timed with the
        library's profiling hook (HIP events recorded by the library on the
        call's stream just before and after the stage's kernels).  A stage
        the call does not run reads 0."""
        torch, lcsb, stream = self.torch, self.lcsb, self.stream
        out = {}
        for stg in stages:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            b.record(stream)
            torch.cuda.synchronize()
            before = a.elapsed_time(b)   # unchanged unless the library records them again
            lcsb.misa_profile_stage(stg, a, b)
            try:
                fn()
                ts = []
                for _ in range(steps):
                    fn()
                    torch.cuda.synchronize()
                    ts.append(a.elapsed_time(b))
            finally:
                lcsb.misa_profile_stage(None)
            if any(t != before for t in ts):
                out[stg] = float(np.mean(ts))
        return out

    def recovered(self, a, ref):
        """Per row: the share of ref's ids (>= 0) that a also holds."""
        torch = self.torch
        s_, _ = torch.sort(torch.cat([a, ref], dim=-1), dim=-1)
        both = ((s_[..., 1:] == s_[..., :-1]) & (s_[..., 1:] >= 0)).sum(-1).float()
        return both / (ref >= 0).sum(-1).clamp(min=1).float()


def roof_mfma(flops, ms, peak=PEAK_BF16_TFLOPS):
    a = flops / (ms * 1e-3) / 1e12
    return dict(bound="mfma", achieved=a, peak=peak, unit="TFLOP/s", frac=a / peak)


def roof_hbm(nbytes, ms):
    a = nbytes / (ms * 1e-3) / 1e9
    return dict(bound="hbm", achieved=a, peak=PEAK_HBM_GBS, unit="GB/s", frac=a / PEAK_HBM_GBS)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU: the indexer shards by query across GPUs "
                                   "with no exchange (see DESIGN.md), but only the 1-GPU path is "
                                   "built and measured; run with --gpus 1"}))
        sys.exit(2)
    import torch

    import long_context_sparse_block_amd as lcsb
    from long_context_sparse_block_amd import inputs as gen

    dev = torch.device("cuda:0")
    lcsb.load()
    B_ = Bench(torch, lcsb, gen, dev)
    X = B_.load(args.workload)
    cfg, sh, q, w, k, ks, W = X["cfg"], X["sh"], X["q"], X["w"], X["k"], X["ks"], X["W"]
    S, M, N, H, h, B, K = cfg.n_seq, cfg.q_per_seq, cfg.n_keys, cfg.n_heads, cfg.h, cfg.block, cfg.topk
    ld = (N + 3) // 4 * 4
    n_full = N // B
    pooled = torch.empty((S, max(n_full, 1), 128), dtype=torch.float32, device=dev)
    tail = torch.empty((S, M, 128), dtype=torch.float32, device=dev)
    heads = torch.empty((S, M, h), dtype=torch.int32, device=dev)
    idx = torch.empty((S, M, K), dtype=torch.int32, device=dev)
    vals = torch.empty((S, M, K), dtype=torch.float32, device=dev)
    stream = B_.stream

    # ---- the step: one misa_indexer call -------------------------------------------------------
    ix_ws = torch.empty(lcsb.misa_indexer_workspace_bytes(sh, cfg.kdtype, h, K), dtype=torch.uint8, device=dev)

    def step():
        lcsb.misa_indexer(sh, q, w, k, h, K, k_scale=ks, idx=idx, vals=vals, ws=ix_ws)

    _, step_ms = B_.timed([("indexer", step)], args.steps, args.warmup)
    wall_ms = B_.wall
    warm_pct = [float(np.percentile(B_.samples, p)) for p in (10, 50, 90)]
    # cold: a 1 GiB write before each sample evicts L2 and the 256 MB last-level cache
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(10):
        flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    cold_pct = [float(np.percentile(cold, p)) for p in (10, 50, 90)]
    # the same call captured in a HIP graph and replayed
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    _, graph_ms = B_.timed([("graph", graph.replay)], args.steps, args.warmup)
    del graph
    say(f"MISA step (misa_indexer) {step_ms:.3f} ms (wall {wall_ms:.3f}); warm p10/p50/p90 {warm_pct}; "
        f"cold p10/p50/p90 {cold_pct}; graph replay {graph_ms:.3f} ms")
    # each stage inside the step, timed on its own through the profiling hook
    inner = B_.stage_ms(step, FUSED_STAGES, args.steps)
    say(f"stages inside the step {inner}")

    # the same path as separate calls, and the staged scoring + top-k (rows a3 and a4 on their own)
    sel_ws = torch.empty(lcsb.misa_sparse_head_topk_workspace_bytes(sh, cfg.kdtype, h, K), dtype=torch.uint8,
                         device=dev)
    per, calls_ms = B_.timed([
        ("pool", lambda: lcsb.misa_pool_keys(sh, k, ks, pooled=pooled, tail=tail)),
        ("route", lambda: lcsb.misa_route_heads(sh, q, w, pooled[:, :n_full], tail, h, heads=heads)),
        ("select", lambda: lcsb.misa_sparse_head_topk(sh, q, w, k, heads, K, k_scale=ks, idx=idx, vals=vals,
                                                      ws=sel_ws)),
    ], args.steps, args.warmup)
    say(f"as separate calls {calls_ms:.3f} ms {per}")
    del sel_ws
    logits = torch.empty((S, M, ld), dtype=torch.float32, device=dev)
    tk_ws = torch.empty(max(lcsb.misa_topk_workspace_bytes(sh, N, K), 1), dtype=torch.uint8, device=dev)
    sper, _ = B_.timed([
        ("staged_score", lambda: lcsb.misa_sparse_head_logits(sh, q, w, k, heads, k_scale=ks, logits=logits)),
        ("staged_topk", lambda: lcsb.misa_topk(sh, logits, K, idx=idx, vals=vals, ws=tk_ws)),
    ], max(3, args.steps // 2), 2)
    say(f"staged score + top-k {sper}")

    def stage_roof(name, ms):
        if name in ("select", "staged_score", "score_candidates"):
            r = roof_mfma(W["score_flops"], ms)
        elif name == "route":
            r = roof_mfma(W["route_flops"], ms)
        elif name == "pool":
            r = roof_hbm(W["pool_bytes"], ms)
        elif name == "staged_topk":
            r = roof_hbm(W["topk_bytes"], ms)
        else:
            return dict(ms=ms)
        r["traffic"] = measured_traffic(name, cfg.name)
        r["ms"] = ms
        return r

    stages_out = {name: stage_roof(name, ms) for name, ms in list(per.items()) + list(sper.items())}
    stages_out["staged_score"]["logit_write_GBs"] = W["score_bytes"] / (sper["staged_score"] * 1e-3) / 1e9
    step_stages = {name: stage_roof(name, ms) for name, ms in inner.items()}
    cand_ms = inner["score_candidates"]
    roofline = {kk: v for kk, v in stage_roof("score_candidates", cand_ms).items() if kk != "ms"}
    roofline["kernel"] = "k_score_h8 candidate scoring (stage score_candidates of the step's misa_indexer call)"
    roofline["kernel_ms"] = cand_ms

    extras = {}
    if not args.no_extras:
        # ---- the dense DSA indexer on the same chunk, and the recall of its top-k ------------------
        dper, dstep = B_.timed([
            ("dense_score", lambda: lcsb.dsa_dense_logits(sh, q, w, k, k_scale=ks, logits=logits)),
            ("topk", lambda: lcsb.misa_topk(sh, logits, K, idx=idx, vals=vals, ws=tk_ws)),
        ], max(3, args.steps // 4), 2)
        extras["dense"] = dict(ms_per_step=dstep, stage_ms=dper,
                               dense_score_TFLOPs=W["dense_flops"] / (dper["dense_score"] * 1e-3) / 1e12,
                               dense_score_frac=W["dense_flops"] / (dper["dense_score"] * 1e-3) / 1e12
                               / PEAK_BF16_TFLOPS,
                               misa_speedup=dstep / step_ms)
        say(f"dense {dstep:.3f} ms {dper}")
        dense_idx, _ = lcsb.misa_topk(sh, logits, K, want_vals=False, ws=tk_ws)   # logits: the dense ones
        misa_idx, _ = lcsb.misa_indexer(sh, q, w, k, h, K, k_scale=ks, want_vals=False)
        quality = {"misa": B_.recovered(misa_idx, dense_idx)}
        if cfg.kdtype == 1:
            q8_idx, _ = lcsb.misa_indexer_q8(sh, q, w, k, h, K, ks, want_vals=False)
            quality["misa_fp8_query"] = B_.recovered(q8_idx, dense_idx)
            quality["misa_fp8_query_vs_misa"] = B_.recovered(q8_idx, misa_idx)
            del q8_idx
        extras["recall_vs_dense_topk"] = {n: dict(mean=float(r.mean()), min=float(r.min()))
                                          for n, r in quality.items()}
        say(f"recall vs the dense top-k {extras['recall_vs_dense_topk']}")
        del dense_idx, misa_idx, quality
        if cfg.kdtype == 1:
            # ---- the fp8-query path: per-row quantisation, routed scoring on fp8 matrix cores -----
            q8, qs = lcsb.misa_quantize_q(sh, q)
            iq_ws = torch.empty(lcsb.misa_indexer_q8_workspace_bytes(sh, h, K), dtype=torch.uint8, device=dev)
            qper, qstep = B_.timed([("indexer_q8", lambda: lcsb.misa_indexer_q8(sh, q, w, k, h, K, ks, idx=idx,
                                                                                vals=vals, ws=iq_ws))],
                                   max(3, args.steps // 2), 2)
            del iq_ws
            lper, _ = B_.timed([("score_q8", lambda: lcsb.misa_sparse_head_logits_q8(
                sh, q8, qs, w, k, heads, ks, logits=logits))], max(3, args.steps // 4), 2)
            dqper, dqstep = B_.timed([
                ("quantize_q", lambda: lcsb.misa_quantize_q(sh, q, q8=q8, q_scale=qs)),
                ("dense_score_q8", lambda: lcsb.dsa_dense_logits_q8(sh, q8, qs, w, k, ks, logits=logits)),
                ("topk", lambda: lcsb.misa_topk(sh, logits, K, idx=idx, vals=vals, ws=tk_ws)),
            ], max(3, args.steps // 4), 2)
            extras["fp8_query_path"] = dict(
                ms_per_step=qstep, vs_bf16_step=step_ms / qstep, triples_G_per_s=W["triples"] / (qstep * 1e-3) / 1e9,
                score_q8_ms=lper["score_q8"],
                score_q8_frac_of_fp8_peak=W["score_flops"] / (lper["score_q8"] * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                dense_q8_ms_per_step=dqstep, dense_q8_stage_ms=dqper,
                dense_score_q8_frac_of_fp8_peak=W["dense_flops"] / (dqper["dense_score_q8"] * 1e-3) / 1e12
                / PEAK_FP8_TFLOPS,
                misa_q8_speedup_vs_dense_q8=dqstep / qstep)
            say(f"fp8 query path: misa_indexer_q8 {qstep:.3f} ms; fp8 logits {lper['score_q8']:.3f} ms; "
                f"fp8 dense {dqstep:.3f} ms {dqper}")
            del q8, qs
    del logits, tk_ws, ix_ws
    torch.cuda.empty_cache()

    if not args.no_extras:
        extras["misa_dagger"] = dagger_leg(B_, args)
        torch.cuda.empty_cache()
        extras["dsv32_chunk"] = chunk_leg(B_, "dsv32_prefill_m8k_n32k", args, dense=True)
        extras["tiny_chunk"] = chunk_leg(B_, "tiny_prefill_m256_n4k", args, dense=False)
        torch.cuda.empty_cache()
    if not args.no_extras and not args.no_prefill:
        extras["decode"] = decode_leg(B_, args)
        torch.cuda.empty_cache()
        extras["chunked_prefill"] = prefill_leg(B_, args)
        torch.cuda.empty_cache()

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(X["inp"], args.cpu_queries, args.cpu_dense_queries, W)

    value = W["triples"] / (step_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": value,
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian q/k/w with planted head-block affinity)",
        "config": {"workload": cfg.name, "n_seq": S, "M": M, "N": N, "H_I": H, "h": h, "B": B, "topk": K,
                   "k_dtype": "fp8_e4m3" if cfg.kdtype == 1 else "bf16", "head_dim": 128},
        "roofline": roofline,
        # the metric's MFMA utilisation: the dominant kernel's algorithmic flops over
        # its measured time and the bf16 dense peak (hardware MFMA-busy counters
        # per kernel are in the committed profiles)
        "mfma_util_pct": round(100.0 * roofline["frac"], 1),
        "step": "one misa_indexer call: pool, route, fused routed scoring + top-k",
        "step_stages": step_stages,
        "stages": stages_out,
        "separate_calls_ms": calls_ms,
        "step_ms_p10_p50_p90": warm_pct,
        "cold_step_ms_p10_p50_p90": cold_pct,
        "graph_replay_ms": graph_ms,
        "cpu_baseline": cpu,
    }
    line.update(extras)
    print(json.dumps(line))


def dagger_leg(B_, args):
    """MISA-dagger at its own shape: M = 4096 queries over 131072 bf16 keys, B = 64,
    k' = 8192 candidates re-ranked by all 64 heads down to top-2048; the split of
    time between stages, and the recall of the dense indexer's top-k."""
    torch, lcsb = B_.torch, B_.lcsb
    X = B_.load("dagger_prefill_m4k_n128k")
    cfg, sh, q, w, k, ks, W = X["cfg"], X["sh"], X["q"], X["w"], X["k"], X["ks"], X["W"]
    S, M, N, H, h, K, kp = cfg.n_seq, cfg.q_per_seq, cfg.n_keys, cfg.n_heads, cfg.h, cfg.topk, cfg.k_prime
    dev = B_.dev
    idx = torch.empty((S, M, K), dtype=torch.int32, device=dev)
    vals = torch.empty((S, M, K), dtype=torch.float32, device=dev)
    ws = torch.empty(lcsb.misa_indexer_workspace_bytes(sh, cfg.kdtype, h, K, kp), dtype=torch.uint8, device=dev)

    def step():
        lcsb.misa_indexer(sh, q, w, k, h, K, k_prime=kp, k_scale=ks, idx=idx, vals=vals, ws=ws)

    steps = max(5, args.steps // 2)
    _, ms = B_.timed([("dagger", step)], steps, 2)
    inner = B_.stage_ms(step, FUSED_STAGES + ("rerank", "final_topk"), steps)
    step()
    dag_idx = idx.clone()
    del ws
    # the plain MISA step on the same chunk, for the cost of the re-rank
    ws2 = torch.empty(lcsb.misa_indexer_workspace_bytes(sh, cfg.kdtype, h, K), dtype=torch.uint8, device=dev)
    _, misa_ms = B_.timed([("misa", lambda: lcsb.misa_indexer(sh, q, w, k, h, K, k_scale=ks, idx=idx, vals=vals,
                                                             ws=ws2))], steps, 2)
    misa_idx = idx.clone()
    del ws2
    # the dense top-k of the same chunk
    logits = lcsb.dsa_dense_logits(sh, q, w, k, k_scale=ks)
    dense_idx, _ = lcsb.misa_topk(sh, logits, K, want_vals=False)
    del logits
    rec_d = B_.recovered(dag_idx, dense_idx)
    rec_m = B_.recovered(misa_idx, dense_idx)
    # IoU of the MISA-dagger and dense top-k sets: |A & D| / |A | D|
    inter = rec_d * (dense_idx >= 0).sum(-1).float()
    union = (dag_idx >= 0).sum(-1).float() + (dense_idx >= 0).sum(-1).float() - inter
    iou = inter / union.clamp(min=1)
    rerank_flops = S * M * kp * H * 256
    out = dict(workload=cfg.name, k_prime=kp, topk=K, ms_per_step=ms, misa_ms_per_step=misa_ms, stage_ms=inner,
               candidate_pass_ms=sum(inner[s] for s in FUSED_STAGES[2:]),
               rerank=roof_mfma(rerank_flops, inner["rerank"]),
               score_candidates=roof_mfma(W["score_flops"], inner["score_candidates"]),
               recall_vs_dense_topk=dict(mean=float(rec_d.mean()), min=float(rec_d.min())),
               iou_vs_dense_topk=dict(mean=float(iou.mean()), min=float(iou.min())),
               misa_recall_vs_dense_topk=dict(mean=float(rec_m.mean()), min=float(rec_m.min())))
    say(f"MISA-dagger {cfg.name}: {ms:.3f} ms (MISA {misa_ms:.3f} ms) {inner}; recall of the dense top-k "
        f"{out['recall_vs_dense_topk']}, IoU {out['iou_vs_dense_topk']}")
    return out


def chunk_leg(B_, name, args, dense):
    """misa_indexer on another seeded chunk: step time, throughput, stages."""
    torch, lcsb = B_.torch, B_.lcsb
    X = B_.load(name)
    cfg, sh, q, w, k, ks, W = X["cfg"], X["sh"], X["q"], X["w"], X["k"], X["ks"], X["W"]
    S, M, N, h, K = cfg.n_seq, cfg.q_per_seq, cfg.n_keys, cfg.h, cfg.topk
    dev = B_.dev
    idx = torch.empty((S, M, K), dtype=torch.int32, device=dev)
    vals = torch.empty((S, M, K), dtype=torch.float32, device=dev)
    ws = torch.empty(lcsb.misa_indexer_workspace_bytes(sh, cfg.kdtype, h, K), dtype=torch.uint8, device=dev)

    def step():
        lcsb.misa_indexer(sh, q, w, k, h, K, k_scale=ks, idx=idx, vals=vals, ws=ws)

    _, ms = B_.timed([("step", step)], args.steps, args.warmup)
    inner = B_.stage_ms(step, FUSED_STAGES, max(5, args.steps // 2))
    out = dict(workload=name, ms_per_step=ms, triples_G_per_s=W["triples"] / (ms * 1e-3) / 1e9, stage_ms=inner)
    if "score_candidates" in inner:
        out["score_candidates"] = roof_mfma(W["score_flops"], inner["score_candidates"])
    if dense:
        logits = torch.empty((S, M, (N + 3) // 4 * 4), dtype=torch.float32, device=dev)
        tk = torch.empty(max(lcsb.misa_topk_workspace_bytes(sh, N, K), 1), dtype=torch.uint8, device=dev)
        dper, dms = B_.timed([
            ("dense_score", lambda: lcsb.dsa_dense_logits(sh, q, w, k, k_scale=ks, logits=logits)),
            ("topk", lambda: lcsb.misa_topk(sh, logits, K, idx=idx, vals=vals, ws=tk)),
        ], max(3, args.steps // 4), 2)
        out.update(dense_ms_per_step=dms, dense_stage_ms=dper, misa_speedup=dms / ms)
        del logits, tk
    say(f"{name}: {ms:.3f} ms {inner}" + (f"; dense {out['dense_ms_per_step']:.3f} ms" if dense else ""))
    return out


def decode_leg(B_, args):
    """The GLM-5 decode batch (64 sequences x 1 query over 131072 bf16 keys each,
    H = 32, B = 64), seeded: misa_indexer from scratch, and misa_indexer_cached
    with the previous step's pooled-key cache (K read once)."""
    torch, lcsb = B_.torch, B_.lcsb
    X = B_.load("glm5_decode_64x1_n128k")
    dc, sh, q, w, k = X["cfg"], X["sh"], X["q"], X["w"], X["k"]
    Sd, Nd, Hd, Bd = dc.n_seq, dc.n_keys, dc.n_heads, dc.block
    dev = B_.dev
    idd = torch.empty((Sd, 1, dc.topk), dtype=torch.int32, device=dev)
    vad = torch.empty((Sd, 1, dc.topk), dtype=torch.float32, device=dev)
    wsd = torch.empty(lcsb.misa_indexer_workspace_bytes(sh, dc.kdtype, dc.h, dc.topk), dtype=torch.uint8, device=dev)
    wsc = torch.empty(lcsb.misa_indexer_cached_workspace_bytes(sh, dc.kdtype, dc.h, dc.topk), dtype=torch.uint8,
                      device=dev)
    cache = lcsb.PooledCache(Sd, Nd // Bd)
    prev = lcsb.make_shape(Sd, 0, Nd - 1, Nd - 1, Hd, Bd)
    lcsb.misa_pool_keys_cached(prev, k[:, :Nd - 1].contiguous(), cache)   # the previous step's cache

    def cached_step():
        cache.n_cached = (Nd - 1) // Bd
        lcsb.misa_indexer_cached(sh, q, w, k, dc.h, dc.topk, cache, idx=idd, vals=vad, ws=wsc)

    # the same keys in a paged cache (pages of 64 keys, shuffled over a pool
    # with spare pages), read in place by misa_indexer_paged
    page_keys = 64
    per_seq = Nd // page_keys
    n_pages = Sd * per_seq + 64
    g = torch.Generator(device="cpu").manual_seed(11)
    ids = torch.randperm(n_pages, generator=g)[:Sd * per_seq].view(Sd, per_seq).to(torch.int32)
    pages = torch.empty((n_pages, page_keys, 128), dtype=k.dtype, device=dev)
    pages[ids.view(-1).to(dev).long()] = k.view(Sd * per_seq, page_keys, 128)
    table = ids.to(dev)
    wsp = torch.empty(lcsb.misa_indexer_paged_workspace_bytes(sh, dc.kdtype, dc.h, dc.topk), dtype=torch.uint8,
                      device=dev)
    cache_p = lcsb.PooledCache(Sd, Nd // Bd)
    lcsb.misa_pool_keys_cached(prev, k[:, :Nd - 1].contiguous(), cache_p)
    idp = torch.empty_like(idd)
    vap = torch.empty_like(vad)

    def paged_step():
        cache_p.n_cached = (Nd - 1) // Bd
        lcsb.misa_indexer_paged(sh, q, w, pages, table, dc.h, dc.topk, cache_p, idx=idp, vals=vap, ws=wsp)

    dper, _ = B_.timed([("scratch", lambda: lcsb.misa_indexer(sh, q, w, k, dc.h, dc.topk, idx=idd, vals=vad,
                                                               ws=wsd)),
                        ("cached", cached_step), ("paged", paged_step)], max(5, args.steps // 2), 2)
    same = bool(torch.equal(idp, idd) and torch.equal(vap, vad))
    kbytes = Sd * Nd * 256
    out = dict(workload=dc.name, ms_from_scratch=dper["scratch"], ms_with_pooled_cache=dper["cached"],
               ms_paged_in_place=dper["paged"], paged_equals_contiguous=same, page_keys=page_keys,
               key_bytes=kbytes, cached_key_read=roof_hbm(kbytes, dper["cached"]),
               paged_key_read=roof_hbm(kbytes, dper["paged"]),
               stages_paged=B_.stage_ms(paged_step, ("pool", "route", "score_sample", "sample_threshold",
                                                     "score_candidates", "region_select", "rescore"), 10))
    say(f"decode {dc.name}: {dper['scratch']:.3f} ms from scratch, {dper['cached']:.3f} ms with the pooled-key "
        f"cache, {dper['paged']:.3f} ms on pages read in place (same result: {same})")
    return out


def prefill_leg(B_, args):
    """A whole GLM-5-shaped prompt (65536 tokens from the first, H = 32, fp8 keys),
    seeded, through the chunked-prefill driver in chunks of 8192 with the
    pooled-key cache carried across chunks; the last chunk is checked against
    one misa_indexer call on it."""
    torch, lcsb = B_.torch, B_.lcsb
    X = B_.load("glm5_prompt_m64k_h32_fp8")
    cfg, sh, q, w, k, ks = X["cfg"], X["sh"], X["q"], X["w"], X["k"], X["ks"]
    N, H, B, h, K, chunk = cfg.n_keys, cfg.n_heads, cfg.block, cfg.h, cfg.topk, 8192
    dev = B_.dev
    idxp = torch.empty((1, N, K), dtype=torch.int32, device=dev)
    valp = torch.empty((1, N, K), dtype=torch.float32, device=dev)
    pf_ws = torch.empty(lcsb.misa_prefill_workspace_bytes(sh, cfg.kdtype, h, K, 0, chunk), dtype=torch.uint8,
                        device=dev)
    _, ms = B_.timed([("prefill", lambda: lcsb.misa_prefill_chunked(sh, q, w, k, h, K, chunk=chunk, k_scale=ks,
                                                                     idx=idxp, vals=valp, ws=pf_ws))], 3, 1)
    last = lcsb.make_shape(1, chunk, N, N - chunk, H, B)
    ref_idx, _ = lcsb.misa_indexer(last, q[:, N - chunk:].contiguous(), w[:, N - chunk:].contiguous(), k, h, K,
                                   k_scale=ks)
    out = dict(workload=cfg.name, prompt_tokens=N, chunk=chunk, n_chunks=N // chunk, ms=ms,
               triples_G_per_s=h * (N * (N + 1) / 2) / (ms * 1e-3) / 1e9,
               last_chunk_equals_indexer=bool(torch.equal(idxp[:, N - chunk:], ref_idx)))
    say(f"chunked prefill of {N} tokens in chunks of {chunk}: {ms:.2f} ms")
    return out


def cpu_baseline(inp, n_queries, n_dense, W):
    """The fp64 oracle, as it stands, on samples of the chunk's queries: the MISA
    pipeline (route, score, top-k) and the dense indexer, each extrapolated
    linearly to the chunk."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:   # threadpoolctl missing: report the affinity size
        threads = len(os.sched_getaffinity(0))
    cfg = inp.cfg
    M = cfg.q_per_seq
    rows = np.unique(np.linspace(0, M - 1, min(n_queries, M)).round().astype(int))
    t0 = time.perf_counter()
    ctx = oracle.SeqContext(inp, 0)
    t_setup = time.perf_counter() - t0
    t1 = time.perf_counter()
    for i in rows:
        ctx.misa(int(i), cfg.h, cfg.topk)
    t_rows = time.perf_counter() - t1
    per_chunk = (t_setup + t_rows * M / len(rows)) * cfg.n_seq
    drows = np.unique(np.linspace(0, M - 1, min(n_dense, M)).round().astype(int))
    t2 = time.perf_counter()
    for i in drows:
        ctx.dense_topk(int(i), cfg.topk)
    t_dense = time.perf_counter() - t2
    dense_chunk = (t_setup + t_dense * M / len(drows)) * cfg.n_seq
    return dict(value=W["triples"] / per_chunk / 1e9, unit=UNIT, cores=int(threads), kind="oracle",
                seconds_per_chunk_extrapolated=per_chunk, sample_seconds=t_setup + t_rows,
                sample=f"{len(rows)} evenly spaced of {M} queries of sequence 0 (key widening + pooling of "
                       f"the whole sequence, then route/score/top-k per sampled query), extrapolated "
                       f"linearly to the chunk",
                dense_seconds_per_chunk_extrapolated=dense_chunk, dense_sample_seconds=t_dense,
                dense_sample=f"{len(drows)} evenly spaced queries through the oracle's dense indexer and top-k, "
                             f"extrapolated linearly to the chunk",
                cpu_model=cpu_model(), host_cpus=os.cpu_count(), affinity=len(os.sched_getaffinity(0)))


if __name__ == "__main__":
    main()
