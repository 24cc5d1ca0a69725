"""Small helpers shared by the oracle pin tests (no indexer arithmetic here)."""
from __future__ import annotations

import json
import os

import numpy as np

from long_context_sparse_block_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def fval(x):
    if x is None:
        return None
    if isinstance(x, str):
        return float(x)
    if isinstance(x, list):
        return [fval(v) for v in x]
    return float(x)


def inputs_from_arrays(q_f32, w_f32, k_f32=None, k_codes=None, k_scale=None, q_pos0=0, block=1,
                       h=1, topk=1, k_prime=0):
    """Wrap explicit arrays (one sequence) into a generator Inputs record.

    q_f32 [M,H,d] and k_f32 [N,d] must be exactly representable in bf16."""
    q_f32 = np.asarray(q_f32, np.float32)
    M, H, d = q_f32.shape
    if k_codes is not None:
        N = k_codes.shape[0]
        kdt = gen.KDTYPE_FP8
    else:
        N = np.asarray(k_f32).shape[0]
        kdt = gen.KDTYPE_BF16
    cfg = gen.Config(name="explicit", n_seq=1, q_per_seq=M, n_keys=N, n_heads=H, block=block, h=h,
                     topk=topk, kdtype=kdt, k_prime=k_prime, head_dim=d, first_query=q_pos0,
                     plant_heads=0, plant_blocks=0, plant_a=0.0)
    qb = gen.to_bf16_bits(q_f32)[None]
    assert np.array_equal(_widen(qb[0]), q_f32), "q not bf16-exact"
    if k_codes is not None:
        kk = np.asarray(k_codes, np.uint8)[None]
        ks = np.asarray(k_scale, np.float32)[None]
    else:
        kk = gen.to_bf16_bits(np.asarray(k_f32, np.float32))[None]
        assert np.array_equal(_widen(kk[0]), np.asarray(k_f32, np.float32)), "k not bf16-exact"
        ks = None
    return gen.Inputs(cfg=cfg, q_pos0=q_pos0, q=qb, w=np.asarray(w_f32, np.float32)[None], k=kk,
                      k_scale=ks, plant_heads=np.zeros((1, 0), np.int64),
                      plant_blocks=np.zeros((1, 0), np.int64))


def _widen(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def random_tiny(seed, M=3, N=11, H=5, d=6, q_pos0=None, quant=None):
    """Tiny random inputs (bf16-exact).  quant: round values to multiples of 1/quant
    (creates exact ties)."""
    rng = np.random.default_rng(seed)
    q_pos0 = N - M if q_pos0 is None else q_pos0
    q = rng.standard_normal((M, H, d)).astype(np.float32)
    k = rng.standard_normal((N, d)).astype(np.float32)
    w = (rng.standard_normal((M, H)) / 4).astype(np.float32)
    if quant:
        q = np.round(q * quant) / quant
        k = np.round(k * quant) / quant
        w = np.round(w * quant * 4) / (quant * 4)
    q = _widen(gen.to_bf16_bits(q))
    k = _widen(gen.to_bf16_bits(k))
    return q, w.astype(np.float32), k, q_pos0
