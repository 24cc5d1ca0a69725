"""Seeded synthetic inputs for the MISA indexer.

This module only draws random numbers and casts them to the storage formats
the indexer consumes.  It holds none of the indexer's arithmetic, so both the
HIP path and the fp64 oracle can take their inputs from it.

Workloads follow the shapes of the MISA pages: DeepSeek-V3.2-shaped prefill
chunks with H_I = 64 indexer heads and GLM-5-shaped decode with H_I = 32 (MISA
technical summary on gist.science, "Resultados Experimentais"; agents-report
summary, "實驗與主要結果"), chunked prefill of 8192 queries against a 128K key
cache with an fp8 key cache (GitHub issue "Clarification on the Figure 3
baseline ...", the measured configuration list).  The pages evaluate on
LongBench and Needle-in-a-Haystack with trained weights; those are not
available, so seeded Gaussian tensors with a planted head/block affinity stand
in for them.

Recipe (per sequence, numpy PCG64 seeded generator, draws in this order):
  1. plant heads P (4 distinct heads), plant blocks (8 distinct blocks among
     those lying entirely before the first query), a unit direction u;
  2. q ~ N(0,1) fp32 [M, H, d]; k ~ N(0,1) fp32 [N, d]; w ~ N(0,1)/8 fp32 [M, H];
  3. q[:, P, :] += a*u; every key of the 8 plant blocks += a*u; w[:, P] = |w[:, P]|;
  4. q and bf16 keys: round-to-nearest-even cast to bf16.  fp8 keys: per-token
     scale sigma_s = max_i |k_s,i| / 448 (fp32), codes = e4m3fn RNE cast of
     k_s / sigma_s (clamped to +-448).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

KDTYPE_BF16 = 0
KDTYPE_FP8 = 1


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    n_seq: int
    q_per_seq: int
    n_keys: int
    n_heads: int
    block: int
    h: int
    topk: int
    kdtype: int = KDTYPE_BF16
    k_prime: int = 0
    head_dim: int = 128
    seed: int = 0
    plant_heads: int = 4
    plant_blocks: int = 8
    plant_a: float = 8.0
    first_query: int = -1   # absolute position of query 0; -1 = causal tail of the cache

    @property
    def q_pos0(self) -> int:
        # by default every chunk is the causal tail of its key cache
        return self.n_keys - self.q_per_seq if self.first_query < 0 else self.first_query


def _plant_scale(n_keys: int, block: int) -> float:
    # a = 8 at 64 blocks, growing with sqrt(#blocks) so the plant stays visible
    return 8.0 * math.sqrt((n_keys // block) / 64.0)


def _cfg(name, n_seq, m, n, hh, b, h, k, kdtype=KDTYPE_BF16, kp=0, seed=0):
    return Config(name=name, n_seq=n_seq, q_per_seq=m, n_keys=n, n_heads=hh, block=b,
                  h=h, topk=k, kdtype=kdtype, k_prime=kp, seed=seed,
                  plant_a=_plant_scale(n, b))


# The workloads (tiny chunk, DeepSeek-V3.2 chunk, 128K final chunk with fp8
# keys, GLM-5 decode batch, MISA-dagger prefill, GLM-5 64K prompt).
CONFIGS = {
    "tiny_prefill_m256_n4k": _cfg("tiny_prefill_m256_n4k", 1, 256, 4096, 64, 64, 8, 256, seed=101),
    "dsv32_prefill_m8k_n32k": _cfg("dsv32_prefill_m8k_n32k", 1, 8192, 32768, 64, 64, 8, 2048, seed=102),
    "final_chunk_m8k_n128k_fp8": _cfg("final_chunk_m8k_n128k_fp8", 1, 8192, 131072, 64, 128, 8, 2048,
                                      kdtype=KDTYPE_FP8, seed=103),
    "glm5_decode_64x1_n128k": _cfg("glm5_decode_64x1_n128k", 64, 1, 131072, 32, 64, 8, 2048, seed=104),
    "dagger_prefill_m4k_n128k": _cfg("dagger_prefill_m4k_n128k", 1, 4096, 131072, 64, 64, 8, 2048,
                                     kp=8192, seed=105),
    # a whole GLM-5-shaped prompt (H = 32) from its first token, for the
    # chunked-prefill driver (chunks of 8192; no block lies before the first
    # query, so nothing is planted)
    "glm5_prompt_m64k_h32_fp8": _cfg("glm5_prompt_m64k_h32_fp8", 1, 65536, 65536, 32, 64, 8, 2048,
                                     kdtype=KDTYPE_FP8, seed=106),
}


def small_config(name="small", n_seq=1, m=64, n=512, hh=64, b=64, h=8, k=64,
                 kdtype=KDTYPE_BF16, kp=0, seed=7, q_pos0=None, plant=True):
    """A reduced workload with the same recipe (for parity tests and smoke)."""
    return Config(name=name, n_seq=n_seq, q_per_seq=m, n_keys=n, n_heads=hh, block=b, h=h,
                  topk=k, kdtype=kdtype, k_prime=kp, seed=seed,
                  plant_heads=min(4, hh) if plant else 0,
                  plant_blocks=8 if plant else 0,
                  plant_a=_plant_scale(n, max(b, 1)) if plant else 0.0,
                  first_query=-1 if q_pos0 is None else q_pos0)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """RNE cast fp32 -> bf16, returned as the raw uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """RNE cast fp32 -> OCP fp8 e4m3fn, returned as uint8 codes."""
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


@dataclasses.dataclass
class Inputs:
    cfg: Config
    q_pos0: int
    q: np.ndarray            # uint16 bf16 bits [n_seq, M, H, d]
    w: np.ndarray            # float32 [n_seq, M, H]
    k: np.ndarray            # uint16 bf16 bits [n_seq, N, d]  or uint8 e4m3 codes
    k_scale: np.ndarray | None  # float32 [n_seq, N] (fp8 only)
    plant_heads: np.ndarray  # int [n_seq, plant_heads]
    plant_blocks: np.ndarray  # int [n_seq, plant_blocks]


def generate(cfg: Config, seed: int | None = None) -> Inputs:
    seed = cfg.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    S, M, N, H, d, B = cfg.n_seq, cfg.q_per_seq, cfg.n_keys, cfg.n_heads, cfg.head_dim, cfg.block
    q_pos0 = cfg.q_pos0
    assert 0 <= q_pos0 and q_pos0 + M <= N
    q = np.empty((S, M, H, d), np.uint16)
    w = np.empty((S, M, H), np.float32)
    fp8 = cfg.kdtype == KDTYPE_FP8
    k = np.empty((S, N, d), np.uint8 if fp8 else np.uint16)
    ks = np.empty((S, N), np.float32) if fp8 else None
    n_ph, n_pb = cfg.plant_heads, cfg.plant_blocks
    ph = np.zeros((S, n_ph), np.int64)
    pb = np.zeros((S, n_pb), np.int64)
    n_vis = q_pos0 // B
    for b in range(S):
        if n_ph > 0 and n_vis >= n_pb:
            ph[b] = np.sort(rng.choice(H, n_ph, replace=False))
            pb[b] = np.sort(rng.choice(n_vis, n_pb, replace=False))
            u = rng.standard_normal(d).astype(np.float32)
            u /= np.float32(np.linalg.norm(u))
            planted = True
        else:
            planted = False
        qf = rng.standard_normal((M, H, d), dtype=np.float32)
        kf = rng.standard_normal((N, d), dtype=np.float32)
        wf = rng.standard_normal((M, H), dtype=np.float32) / np.float32(8.0)
        if planted:
            a = np.float32(cfg.plant_a)
            qf[:, ph[b], :] += a * u
            for blk in pb[b]:
                kf[blk * B:(blk + 1) * B, :] += a * u
            wf[:, ph[b]] = np.abs(wf[:, ph[b]])
        q[b] = to_bf16_bits(qf)
        w[b] = wf
        if fp8:
            sig = (np.abs(kf).max(axis=1) / np.float32(448.0)).astype(np.float32)
            sig = np.where(sig > 0, sig, np.float32(1.0)).astype(np.float32)
            ks[b] = sig
            k[b] = to_e4m3_codes(kf / sig[:, None])
        else:
            k[b] = to_bf16_bits(kf)
    return Inputs(cfg=cfg, q_pos0=q_pos0, q=q, w=w, k=k, k_scale=ks, plant_heads=ph, plant_blocks=pb)
