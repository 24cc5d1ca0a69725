"""Benchmark of the MISA indexer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the MISA indexer over one prefill chunk resident in
HBM: block pooling -> head routing -> routed-head token scoring fused with
the top-k selection (misa_sparse_head_topk: the logits are not written), each
issued through the C ABI on the launch stream with HIP events between them.
The default workload is the long-context final prefill chunk: M = 8192
queries against N = 131072 fp8 keys, H_I = 64 heads, h = 8, B = 128,
top-2048.

Printed: one JSON line.  value = scored (query, key, head) triples per second
(G/s) of the whole step; ms_per_step = indexer milliseconds per chunk;
roofline = the dominant stage (the fused scoring + selection) against the
bf16 MFMA peak, with its scoring work; stages = every stage's time and
roofline fraction, plus the same chunk through the separate logits kernel
and top-k kernel (staged_score, staged_topk); misa_dagger and dense = the
chunk through the MISA-dagger pipeline (k' = 8192) and through the dense
all-head DSA indexer, timed in the same run; cpu_baseline = the fp64 oracle
on the host cores over a bounded sample of the same chunk.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="final_chunk_m8k_n128k_fp8")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip the MISA-dagger and dense timings")
    p.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill timing")
    p.add_argument("--cpu-queries", type=int, default=1536, help="queries in the oracle timing sample")
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
        route_bytes=cfg.n_seq * M * H * (256 + 4) + cfg.n_seq * (N // B) * 512 + cfg.n_seq * M * 512,
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
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(workload, {}).get(stage)
    if not ent or ent.get("source_hash") != src_hash(*KERNEL_SOURCES[stage]):
        return None
    return ent.get("bytes_per_launch")


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

    cfg = gen.CONFIGS[args.workload]
    t0 = time.perf_counter()
    inp = gen.generate(cfg)
    print(f"[bench] generated {cfg.name} in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    lcsb.load()
    q = torch.from_numpy(inp.q.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(inp.w).to(dev)
    if inp.k_scale is None:
        k = torch.from_numpy(inp.k.view(np.int16)).to(dev).view(torch.bfloat16)
        ks = None
    else:
        k = torch.from_numpy(inp.k).to(dev)
        ks = torch.from_numpy(inp.k_scale).to(dev)
    sh = lcsb.make_shape(cfg.n_seq, cfg.q_per_seq, cfg.n_keys, inp.q_pos0, cfg.n_heads, cfg.block)
    S, M, N, H, h, B, K = cfg.n_seq, cfg.q_per_seq, cfg.n_keys, cfg.n_heads, cfg.h, cfg.block, cfg.topk
    ld = (N + 3) // 4 * 4
    n_full = N // B
    pooled = torch.empty((S, max(n_full, 1), 128), dtype=torch.float32, device=dev)
    tail = torch.empty((S, M, 128), dtype=torch.float32, device=dev)
    heads = torch.empty((S, M, h), dtype=torch.int32, device=dev)
    logits = torch.empty((S, M, ld), dtype=torch.float32, device=dev)
    idx = torch.empty((S, M, K), dtype=torch.int32, device=dev)
    vals = torch.empty((S, M, K), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    W = work(cfg, inp.q_pos0)
    kp = 8192
    tk_ws_bytes = max(lcsb.misa_topk_workspace_bytes(sh, N, K), lcsb.misa_topk_workspace_bytes(sh, N, kp),
                      lcsb.misa_topk_workspace_bytes(sh, kp, K), 1)
    tk_ws = torch.empty(tk_ws_bytes, dtype=torch.uint8, device=dev)   # top-k scratch, allocated once
    sel_ws = torch.empty(max(lcsb.misa_sparse_head_topk_workspace_bytes(sh, cfg.kdtype, h, K),
                             lcsb.misa_sparse_head_topk_workspace_bytes(sh, cfg.kdtype, h, kp)), dtype=torch.uint8,
                         device=dev)

    def run_timed(stages, steps, warmup):
        """stages: list of (name, fn).  Returns per-stage mean ms and step ms."""
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
        wall = (time.perf_counter() - wall0) * 1e3 / steps
        per = {}
        for j, (name, _) in enumerate(stages):
            per[name] = float(np.mean([evs[s][j].elapsed_time(evs[s][j + 1]) for s in range(steps)]))
        samples = [evs[s][0].elapsed_time(evs[s][-1]) for s in range(steps)]
        run_timed.samples = samples   # per-step ms of the last call
        return per, float(np.mean(samples)), wall

    misa_stages = [
        ("pool", lambda: lcsb.misa_pool_keys(sh, k, ks, pooled=pooled, tail=tail)),
        ("route", lambda: lcsb.misa_route_heads(sh, q, w, pooled[:, :n_full], tail, h, heads=heads)),
        ("select", lambda: lcsb.misa_sparse_head_topk(sh, q, w, k, heads, K, k_scale=ks, idx=idx, vals=vals,
                                                      ws=sel_ws)),
    ]
    # the step: the whole indexer as one C call (pool, route, fused selection;
    # the router stages pooled keys the pooling kernel has already split)
    ix_ws = torch.empty(lcsb.misa_indexer_workspace_bytes(sh, cfg.kdtype, h, K), dtype=torch.uint8, device=dev)
    _, step_ms, wall_ms = run_timed([("indexer", lambda: lcsb.misa_indexer(sh, q, w, k, h, K, k_scale=ks, idx=idx,
                                                                           vals=vals, ws=ix_ws))],
                                    args.steps, args.warmup)
    warm_pct = [float(np.percentile(run_timed.samples, p)) for p in (10, 50, 90)]
    # cold: a 1 GiB write before each sample evicts L2 and the 256 MB last-level cache
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(10):
        flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lcsb.misa_indexer(sh, q, w, k, h, K, k_scale=ks, idx=idx, vals=vals, ws=ix_ws)
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    cold_pct = [float(np.percentile(cold, p)) for p in (10, 50, 90)]
    # the same call captured in a HIP graph and replayed (no launch gaps
    # between its kernels; the library allocates and synchronises nothing)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            lcsb.misa_indexer(sh, q, w, k, h, K, k_scale=ks, idx=idx, vals=vals, ws=ix_ws)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    _, graph_ms, _ = run_timed([("graph", graph.replay)], args.steps, args.warmup)
    del graph, ix_ws
    print(f"[bench] MISA step (misa_indexer) {step_ms:.3f} ms (wall {wall_ms:.3f}); warm p10/p50/p90 "
          f"{warm_pct}; cold (1 GiB flush before each) p10/p50/p90 {cold_pct}; graph replay {graph_ms:.3f} ms",
          file=sys.stderr, flush=True)
    # the same path as separate calls, for the time split by stage
    per, calls_ms, _ = run_timed(misa_stages, args.steps, args.warmup)
    print(f"[bench] as separate calls {calls_ms:.3f} ms {per}", file=sys.stderr, flush=True)
    # the same scoring and selection as two kernels with materialised logits
    staged = [
        ("staged_score", lambda: lcsb.misa_sparse_head_logits(sh, q, w, k, heads, k_scale=ks, logits=logits)),
        ("staged_topk", lambda: lcsb.misa_topk(sh, logits, K, idx=idx, vals=vals, ws=tk_ws)),
    ]
    sper, sstep, _ = run_timed(staged, max(3, args.steps // 2), 2)
    print(f"[bench] staged score + top-k {sstep:.3f} ms {sper}", file=sys.stderr, flush=True)

    def roof(stage, ms):
        if stage in ("select", "staged_score"):
            a = W["score_flops"] / (ms * 1e-3) / 1e12
            r = dict(bound="mfma", achieved=a, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s")
        elif stage == "route":
            a = W["route_flops"] / (ms * 1e-3) / 1e12
            r = dict(bound="mfma", achieved=a, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s")
        else:
            nbytes = W["pool_bytes"] if stage == "pool" else W["topk_bytes"]
            a = nbytes / (ms * 1e-3) / 1e9
            r = dict(bound="hbm", achieved=a, peak=PEAK_HBM_GBS, unit="GB/s")
        r["frac"] = r["achieved"] / r["peak"]
        r["traffic"] = measured_traffic(stage, cfg.name) if stage in KERNEL_SOURCES else None
        r["ms"] = ms
        return r

    stages_out = {name: roof(name, ms) for name, ms in list(per.items()) + list(sper.items())}
    dominant = max(per, key=per.get)
    roofline = {kk: v for kk, v in stages_out[dominant].items() if kk != "ms"}
    roofline["kernel"] = dominant
    # the logits kernel also streams the logits out: report that rate beside its MFMA rate
    stages_out["staged_score"]["logit_write_GBs"] = W["score_bytes"] / (sper["staged_score"] * 1e-3) / 1e9

    extras = {}
    if not args.no_extras:
        cand = torch.empty((S, M, kp), dtype=torch.int32, device=dev)
        dlog = torch.empty((S, M, kp), dtype=torch.float32, device=dev)
        dagger_stages = misa_stages[:2] + [
            ("select_kprime", lambda: lcsb.misa_sparse_head_topk(sh, q, w, k, heads, kp, k_scale=ks, sorted=False,
                                                                 idx=cand, want_vals=False, ws=sel_ws)),
            ("rerank", lambda: lcsb.dsa_dense_logits(sh, q, w, k, k_scale=ks, cand=cand, logits=dlog)),
            ("topk_final", lambda: lcsb.misa_topk(sh, dlog, K, cand=cand, idx=idx, vals=vals, ws=tk_ws)),
        ]
        dper, dstep, _ = run_timed(dagger_stages, max(3, args.steps // 4), 2)
        extras["misa_dagger"] = dict(k_prime=kp, ms_per_step=dstep, stage_ms=dper,
                                     rerank_TFLOPs=S * M * kp * H * 256 / (dper["rerank"] * 1e-3) / 1e12)
        dense_stages = [
            ("dense_score", lambda: lcsb.dsa_dense_logits(sh, q, w, k, k_scale=ks, logits=logits)),
            ("topk", lambda: lcsb.misa_topk(sh, logits, K, idx=idx, vals=vals, ws=tk_ws)),
        ]
        nper, nstep, _ = run_timed(dense_stages, max(3, args.steps // 4), 2)
        extras["dense"] = dict(ms_per_step=nstep, stage_ms=nper,
                               dense_score_TFLOPs=W["dense_flops"] / (nper["dense_score"] * 1e-3) / 1e12,
                               dense_score_frac=W["dense_flops"] / (nper["dense_score"] * 1e-3) / 1e12
                               / PEAK_BF16_TFLOPS,
                               misa_speedup=nstep / step_ms)
        print(f"[bench] dagger {dstep:.3f} ms {dper}; dense {nstep:.3f} ms {nper}", file=sys.stderr, flush=True)
        # selection quality on every row (reported, not a pass/fail): the share
        # of the dense indexer's top-k that MISA and MISA-dagger recover
        dense_idx, _ = lcsb.misa_topk(sh, logits, K, want_vals=False, ws=tk_ws)   # logits: the dense ones
        misa_idx, _ = lcsb.misa_indexer(sh, q, w, k, h, K, k_scale=ks, want_vals=False)
        dag_idx, _ = lcsb.misa_indexer(sh, q, w, k, h, K, k_prime=kp, k_scale=ks, want_vals=False)

        def recovered(a, ref):
            s_, _ = torch.sort(torch.cat([a, ref], dim=-1), dim=-1)
            both = ((s_[..., 1:] == s_[..., :-1]) & (s_[..., 1:] >= 0)).sum(-1).float()
            return both / (ref >= 0).sum(-1).clamp(min=1).float()

        sels = [("misa", misa_idx), ("misa_dagger", dag_idx)]
        if cfg.kdtype == 1:
            sels.append(("misa_fp8_query", lcsb.misa_indexer_q8(sh, q, w, k, h, K, ks, want_vals=False)[0]))
        quality = {}
        for name, sel in sels:
            r = recovered(sel, dense_idx)
            quality[name] = dict(mean=float(r.mean()), min=float(r.min()))
        if cfg.kdtype == 1:   # fp8 queries against bf16 queries, same routing
            r = recovered(sels[2][1], misa_idx)
            quality["misa_fp8_query_vs_misa"] = dict(mean=float(r.mean()), min=float(r.min()))
        extras["recall_vs_dense_topk"] = quality
        print(f"[bench] recall vs the dense top-k {quality}", file=sys.stderr, flush=True)
        del dense_idx, misa_idx, dag_idx, sels
        if cfg.kdtype == 1:
            # the fp8 query path: per-row quantisation, then routed scoring on
            # the fp8 matrix cores, fused with the selection (the step) and as
            # full logits (beside the bf16 staged scoring)
            q8, qs = lcsb.misa_quantize_q(sh, q)
            q8_stages = misa_stages[:2] + [
                ("quantize_q", lambda: lcsb.misa_quantize_q(sh, q, q8=q8, q_scale=qs)),
                ("select_q8", lambda: lcsb.misa_sparse_head_topk_q8(sh, q8, qs, w, k, heads, K, ks, idx=idx,
                                                                    vals=vals, ws=sel_ws)),
            ]
            qper, qcalls, _ = run_timed(q8_stages, max(3, args.steps // 2), 2)
            iq_ws = torch.empty(lcsb.misa_indexer_q8_workspace_bytes(sh, h, K), dtype=torch.uint8, device=dev)
            _, qstep, _ = run_timed([("indexer_q8", lambda: lcsb.misa_indexer_q8(sh, q, w, k, h, K, ks, idx=idx,
                                                                                 vals=vals, ws=iq_ws))],
                                    max(3, args.steps // 2), 2)
            del iq_ws
            lper, _, _ = run_timed([("score_q8", lambda: lcsb.misa_sparse_head_logits_q8(
                sh, q8, qs, w, k, heads, ks, logits=logits))], max(3, args.steps // 4), 2)
            # the fp8-query dense comparator: quantisation, all-head fp8 logits, top-k
            dq_stages = [
                ("quantize_q", lambda: lcsb.misa_quantize_q(sh, q, q8=q8, q_scale=qs)),
                ("dense_score_q8", lambda: lcsb.dsa_dense_logits_q8(sh, q8, qs, w, k, ks, logits=logits)),
                ("topk", lambda: lcsb.misa_topk(sh, logits, K, idx=idx, vals=vals, ws=tk_ws)),
            ]
            dqper, dqstep, _ = run_timed(dq_stages, max(3, args.steps // 4), 2)
            extras["fp8_query_path"] = dict(
                ms_per_step=qstep, separate_calls_ms=qcalls, stage_ms=qper, vs_bf16_step=step_ms / qstep,
                triples_G_per_s=W["triples"] / (qstep * 1e-3) / 1e9,
                select_q8_TFLOPs=W["score_flops"] / (qper["select_q8"] * 1e-3) / 1e12,
                score_q8_ms=lper["score_q8"],
                score_q8_TFLOPs=W["score_flops"] / (lper["score_q8"] * 1e-3) / 1e12,
                score_q8_frac_of_fp8_peak=W["score_flops"] / (lper["score_q8"] * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                vs_bf16_score=sper["staged_score"] / lper["score_q8"],
                dense_q8_ms_per_step=dqstep, dense_q8_stage_ms=dqper,
                dense_score_q8_TFLOPs=W["dense_flops"] / (dqper["dense_score_q8"] * 1e-3) / 1e12,
                dense_score_q8_frac_of_fp8_peak=W["dense_flops"] / (dqper["dense_score_q8"] * 1e-3) / 1e12
                / PEAK_FP8_TFLOPS,
                misa_q8_speedup_vs_dense_q8=dqstep / qstep)
            print(f"[bench] fp8 query path: misa_indexer_q8 {qstep:.3f} ms, as calls {qcalls:.3f} ms {qper}; "
                  f"fp8 logits {lper['score_q8']:.3f} ms; "
                  f"fp8 dense {dqstep:.3f} ms {dqper}", file=sys.stderr, flush=True)

    if not args.no_extras and not args.no_prefill and cfg.n_seq == 1 and inp.q_pos0 + M == N:
        # the whole prompt this chunk ends: N queries from the first token in
        # chunks of M, with the pooled-key cache carried across chunks (the
        # earlier chunks' queries drawn on the GPU, same distribution; the
        # keys are the chunk's)
        gq = torch.Generator(device=dev).manual_seed(cfg.seed + 1000)
        qp = torch.randn((1, N, H, 128), generator=gq, device=dev, dtype=torch.float32).to(torch.bfloat16)
        wp = torch.randn((1, N, H), generator=gq, device=dev, dtype=torch.float32) / 8
        qp[:, N - M:] = q
        wp[:, N - M:] = w
        shp = lcsb.make_shape(1, N, N, 0, H, B)
        idxp = torch.empty((1, N, K), dtype=torch.int32, device=dev)
        valp = torch.empty((1, N, K), dtype=torch.float32, device=dev)
        pf_ws = torch.empty(lcsb.misa_prefill_workspace_bytes(shp, cfg.kdtype, h, K, 0, M), dtype=torch.uint8, device=dev)
        pper, pstep, _ = run_timed([("prefill", lambda: lcsb.misa_prefill_chunked(
            shp, qp, wp, k, h, K, chunk=M, k_scale=ks, idx=idxp, vals=valp, ws=pf_ws))], 3, 1)
        ref_idx, _ = lcsb.misa_indexer(sh, q, w, k, h, K, k_scale=ks)   # the step's own result
        extras["chunked_prefill"] = dict(
            prompt_tokens=N, chunk=M, n_chunks=N // M, ms=pstep,
            triples_G_per_s=cfg.h * (N * (N + 1) / 2) / (pstep * 1e-3) / 1e9,
            last_chunk_equals_step=bool(torch.equal(idxp[:, N - M:], ref_idx)))
        del ref_idx
        print(f"[bench] chunked prefill of {N} tokens in chunks of {M}: {pstep:.2f} ms", file=sys.stderr,
              flush=True)
        del qp, wp, idxp, valp, pf_ws

    if not args.no_extras and not args.no_prefill:
        # decode: the GLM-5-shaped batch of 64 sequences x 1 query over 131072
        # keys each (bf16 keys, H = 32, B = 64), drawn on the GPU with the
        # same distributions; from scratch, and with the pooled-key cache of
        # the previous step (only the new key's block is pooled, K is read once)
        dc = gen.CONFIGS["glm5_decode_64x1_n128k"]
        gd = torch.Generator(device=dev).manual_seed(dc.seed)
        Sd, Nd, Hd, Bd = dc.n_seq, dc.n_keys, dc.n_heads, dc.block
        kd_ = torch.randn((Sd, Nd, 128), generator=gd, device=dev, dtype=torch.float32).to(torch.bfloat16)
        qd_ = torch.randn((Sd, 1, Hd, 128), generator=gd, device=dev, dtype=torch.float32).to(torch.bfloat16)
        wd_ = torch.randn((Sd, 1, Hd), generator=gd, device=dev, dtype=torch.float32) / 8
        shd = lcsb.make_shape(Sd, 1, Nd, Nd - 1, Hd, Bd)
        idd = torch.empty((Sd, 1, dc.topk), dtype=torch.int32, device=dev)
        vad = torch.empty((Sd, 1, dc.topk), dtype=torch.float32, device=dev)
        wsd = torch.empty(lcsb.misa_indexer_workspace_bytes(shd, dc.kdtype, dc.h, dc.topk), dtype=torch.uint8, device=dev)
        wsc = torch.empty(lcsb.misa_indexer_cached_workspace_bytes(shd, dc.kdtype, dc.h, dc.topk), dtype=torch.uint8,
                          device=dev)
        cache = lcsb.PooledCache(Sd, Nd // Bd)
        prev = lcsb.make_shape(Sd, 0, Nd - 1, Nd - 1, Hd, Bd)
        lcsb.misa_pool_keys_cached(prev, kd_[:, :Nd - 1].contiguous(), cache)   # the previous step's cache

        def cached_step():
            cache.n_cached = (Nd - 1) // Bd
            lcsb.misa_indexer_cached(shd, qd_, wd_, kd_, dc.h, dc.topk, cache, idx=idd, vals=vad, ws=wsc)

        dper, _, _ = run_timed([("scratch", lambda: lcsb.misa_indexer(shd, qd_, wd_, kd_, dc.h, dc.topk, idx=idd,
                                                                       vals=vad, ws=wsd)),
                                ("cached", cached_step)], 5, 2)
        kbytes = Sd * Nd * 256
        extras["decode"] = dict(workload=dc.name, ms_from_scratch=dper["scratch"], ms_with_pooled_cache=dper["cached"],
                                key_bytes=kbytes,
                                cached_key_read_GBs=kbytes / (dper["cached"] * 1e-3) / 1e9)
        print(f"[bench] decode {dc.name}: {dper['scratch']:.3f} ms from scratch, {dper['cached']:.3f} ms with the "
              f"pooled-key cache", file=sys.stderr, flush=True)
        del kd_, qd_, wd_, wsd, wsc, cache

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_queries, W)

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
        # the metric's MFMA utilisation: the dominant call's algorithmic flops
        # over its measured time and the bf16 dense peak (the hardware
        # MFMA-busy counters per kernel are in the committed profiles)
        "mfma_util_pct": round(100.0 * roofline["frac"], 1) if roofline.get("frac") is not None else None,
        "stages": stages_out,
        "step": "one misa_indexer call: pool, route, fused routed scoring + top-k",
        "separate_calls_ms": calls_ms,
        "step_ms_p10_p50_p90": warm_pct,
        "cold_step_ms_p10_p50_p90": cold_pct,
        "graph_replay_ms": graph_ms,
        "cpu_baseline": cpu,
    }
    line.update(extras)
    print(json.dumps(line))


def cpu_baseline(inp, n_queries, W):
    """The fp64 oracle, as it stands, on a sample of the chunk's queries."""
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
    return dict(value=W["triples"] / per_chunk / 1e9, unit=UNIT, cores=int(threads), kind="oracle",
                seconds_per_chunk_extrapolated=per_chunk, sample_seconds=t_setup + t_rows,
                sample=f"{len(rows)} evenly spaced of {M} queries of sequence 0 (key widening + pooling of "
                       f"the whole sequence, then route/score/top-k per sampled query), extrapolated "
                       f"linearly to the chunk",
                host_cpus=os.cpu_count(), affinity=len(os.sched_getaffinity(0)))


if __name__ == "__main__":
    main()
