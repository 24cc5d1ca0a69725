"""ctypes binding of libmisa (the C ABI in include/misa.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks dtype / shape / device on the host, and passes raw
device pointers plus the current HIP stream to the library.  There is no
fallback: if libmisa.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmisa.so")

MISA_OK = 0
MISA_ERR_INVALID_ARG = -1
MISA_ERR_UNSUPPORTED = -2
MISA_ERR_WORKSPACE = -3
MISA_ERR_HIP = -4
MISA_K_BF16 = 0
MISA_K_FP8_E4M3 = 1
HEAD_DIM = 128
MAX_HEADS = 64
MAX_TOPK = 8192

EXPORTED = ("misa_status_str", "misa_pool_keys", "misa_route_heads", "misa_sparse_head_logits",
            "dsa_dense_logits", "misa_topk", "misa_topk_workspace_bytes", "misa_sparse_head_topk",
            "misa_sparse_head_topk_workspace_bytes", "misa_indexer", "misa_indexer_workspace_bytes",
            "misa_indexer_workspace_min_bytes",
            "misa_quantize_q", "misa_sparse_head_logits_q8", "misa_sparse_head_topk_q8", "dsa_dense_logits_q8",
            "misa_pool_keys_cached", "misa_indexer_cached", "misa_indexer_cached_workspace_bytes",
            "misa_prefill_chunked", "misa_prefill_workspace_bytes", "misa_indexer_q8",
            "misa_indexer_q8_workspace_bytes", "misa_gather_keys_paged", "misa_indexer_noalloc",
            "misa_profile_stage", "misa_indexer_paged", "misa_indexer_paged_workspace_bytes")
STAGES = dict(pool=1, route=2, score_sample=3, sample_threshold=4, score_candidates=5, region_select=6,
              rescore=7, rerank=8, final_topk=9, score_logits=10, logits_topk=11)
MISA_ERR_SCRATCH = -5
NOALLOC_SCRATCH_BYTES = 256 << 20   # MISA_NOALLOC_SCRATCH_BYTES of misa.h


class MisaShape(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("q_per_seq", ctypes.c_int32), ("n_keys", ctypes.c_int64),
                ("q_pos0", ctypes.c_int64), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block", ctypes.c_int32)]


class MisaError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        super().__init__(f"{where}: {text} (status {status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmisa.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libmisa.so not found at {path}: build it with "
                           "`python -m long_context_sparse_block_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    S = ctypes.POINTER(MisaShape)
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.misa_status_str.restype = ctypes.c_char_p
    lib.misa_status_str.argtypes = [ctypes.c_int]
    sigs = {
        "misa_pool_keys": [S, P, ctypes.c_int, P, P, P, P],
        "misa_route_heads": [S, P, P, P, P, i32, P, P, P],
        "misa_sparse_head_logits": [S, P, P, P, ctypes.c_int, P, P, i32, P, i64, P],
        "dsa_dense_logits": [S, P, P, P, ctypes.c_int, P, P, i32, P, i64, P],
        "misa_topk": [S, P, i64, P, i32, i32, i32, P, P, P, sz, P],
        "misa_sparse_head_topk": [S, P, P, P, ctypes.c_int, P, P, i32, i32, i32, P, P, P, sz, P],
        "misa_indexer": [S, P, P, P, ctypes.c_int, P, i32, i32, i32, P, P, P, sz, P],
        "misa_indexer_noalloc": [S, P, P, P, ctypes.c_int, P, i32, i32, i32, P, P, P],
        "misa_profile_stage": [i32, P, P],
        "misa_quantize_q": [S, P, P, P, P],
        "misa_sparse_head_logits_q8": [S, P, P, P, P, ctypes.c_int, P, P, i32, P, i64, P],
        "misa_sparse_head_topk_q8": [S, P, P, P, P, ctypes.c_int, P, P, i32, i32, i32, P, P, P, sz, P],
        "dsa_dense_logits_q8": [S, P, P, P, P, ctypes.c_int, P, P, i64, P],
        "misa_pool_keys_cached": [S, P, ctypes.c_int, P, i64, P, P, i64, P, P],
        "misa_indexer_cached": [S, P, P, P, ctypes.c_int, P, i32, i32, i32, i64, P, P, i64, P, P, P, sz, P],
        "misa_prefill_chunked": [S, P, P, P, ctypes.c_int, P, i32, i32, i32, i32, P, P, P, sz, P],
        "misa_indexer_q8": [S, P, P, P, ctypes.c_int, P, i32, i32, i32, P, P, P, sz, P],
        "misa_gather_keys_paged": [S, P, ctypes.c_int, P, P, i64, i64, i32, P, P, P],
        "misa_indexer_paged": [S, P, P, P, ctypes.c_int, P, P, i64, i64, i32, i32, i32, i64, P, P, i64, P, P, P,
                               sz, P],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.misa_topk_workspace_bytes.argtypes = [S, i32, i32]
    lib.misa_topk_workspace_bytes.restype = sz
    lib.misa_sparse_head_topk_workspace_bytes.argtypes = [S, ctypes.c_int, i32, i32]
    lib.misa_sparse_head_topk_workspace_bytes.restype = sz
    lib.misa_indexer_workspace_bytes.argtypes = [S, ctypes.c_int, i32, i32, i32]
    lib.misa_indexer_workspace_bytes.restype = sz
    lib.misa_indexer_workspace_min_bytes.argtypes = [S, ctypes.c_int, i32, i32, i32]
    lib.misa_indexer_workspace_min_bytes.restype = sz
    lib.misa_indexer_cached_workspace_bytes.argtypes = [S, ctypes.c_int, i32, i32, i32]
    lib.misa_indexer_cached_workspace_bytes.restype = sz
    lib.misa_indexer_q8_workspace_bytes.argtypes = [S, i32, i32, i32]
    lib.misa_indexer_q8_workspace_bytes.restype = sz
    lib.misa_prefill_workspace_bytes.argtypes = [S, ctypes.c_int, i32, i32, i32, i32]
    lib.misa_prefill_workspace_bytes.restype = sz
    lib.misa_indexer_paged_workspace_bytes.argtypes = [S, ctypes.c_int, i32, i32]
    lib.misa_indexer_paged_workspace_bytes.restype = sz
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().misa_status_str(status).decode()


def _check(status: int, where: str):
    if status != MISA_OK:
        raise MisaError(status, where, status_str(status))


def make_shape(n_seq, q_per_seq, n_keys, q_pos0, n_heads, block, head_dim=HEAD_DIM) -> MisaShape:
    return MisaShape(int(n_seq), int(q_per_seq), int(n_keys), int(q_pos0), int(n_heads), int(head_dim),
                     int(block))


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, shape, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _kdtype(k):
    if k.dtype == torch.bfloat16:
        return MISA_K_BF16
    if k.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MISA_K_FP8_E4M3
    raise ValueError(f"k: dtype {k.dtype} (expected bfloat16 or float8_e4m3fn/uint8 codes)")


def _check_keys(shape, k, k_scale):
    kd = _kdtype(k)
    _need(k, k.dtype, (shape.n_seq, shape.n_keys, HEAD_DIM), "k")
    if kd == MISA_K_FP8_E4M3:
        _need(k_scale, torch.float32, (shape.n_seq, shape.n_keys), "k_scale")
    return kd


def misa_pool_keys(shape: MisaShape, k, k_scale=None, pooled=None, tail=None, stream=None):
    """Block mean-pooled keys [n_seq, N//B, 128] and per-query tails [n_seq, M, 128] (fp32)."""
    kd = _check_keys(shape, k, k_scale)
    n_full = shape.n_keys // shape.block
    dev = k.device
    if pooled is None:
        pooled = torch.empty((shape.n_seq, max(n_full, 1), HEAD_DIM), dtype=torch.float32, device=dev)
    if tail is None:
        tail = torch.empty((shape.n_seq, shape.q_per_seq, HEAD_DIM), dtype=torch.float32, device=dev)
    st = load().misa_pool_keys(ctypes.byref(shape), _ptr(k), kd, _ptr(k_scale), _ptr(pooled), _ptr(tail),
                               _stream(stream))
    _check(st, "misa_pool_keys")
    return pooled[:, :n_full], tail


def misa_route_heads(shape: MisaShape, q, w, pooled, tail, h: int, heads=None, scores=None,
                     want_scores=False, stream=None):
    """Routed heads [n_seq, M, h] (int32, ascending) and optionally r = w*S [n_seq, M, H]."""
    M, H = shape.q_per_seq, shape.n_heads
    _need(q, torch.bfloat16, (shape.n_seq, M, H, HEAD_DIM), "q")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    if heads is None:
        heads = torch.empty((shape.n_seq, M, h), dtype=torch.int32, device=q.device)
    if scores is None and want_scores:
        scores = torch.empty((shape.n_seq, M, H), dtype=torch.float32, device=q.device)
    st = load().misa_route_heads(ctypes.byref(shape), _ptr(q), _ptr(w), _ptr(pooled.contiguous()),
                                 _ptr(tail), int(h), _ptr(heads), _ptr(scores), _stream(stream))
    _check(st, "misa_route_heads")
    return (heads, scores) if want_scores else heads


def _ld(n):
    return (int(n) + 3) // 4 * 4


def misa_sparse_head_logits(shape: MisaShape, q, w, k, heads, k_scale=None, logits=None, stream=None):
    """Routed-head logits [n_seq, M, ld] (fp32, -inf beyond each query's prefix)."""
    kd = _check_keys(shape, k, k_scale)
    M, H = shape.q_per_seq, shape.n_heads
    _need(q, torch.bfloat16, (shape.n_seq, M, H, HEAD_DIM), "q")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    h = heads.shape[-1]
    _need(heads, torch.int32, (shape.n_seq, M, h), "heads")
    if logits is None:
        logits = torch.empty((shape.n_seq, M, _ld(shape.n_keys)), dtype=torch.float32, device=q.device)
    st = load().misa_sparse_head_logits(ctypes.byref(shape), _ptr(q), _ptr(w), _ptr(k), kd, _ptr(k_scale),
                                        _ptr(heads), int(h), _ptr(logits), int(logits.shape[-1]),
                                        _stream(stream))
    _check(st, "misa_sparse_head_logits")
    return logits


def dsa_dense_logits(shape: MisaShape, q, w, k, k_scale=None, cand=None, logits=None, stream=None):
    """All-head DSA logits: over every key ([n_seq, M, ld]) or over candidates ([n_seq, M, n_cand])."""
    kd = _check_keys(shape, k, k_scale)
    M, H = shape.q_per_seq, shape.n_heads
    _need(q, torch.bfloat16, (shape.n_seq, M, H, HEAD_DIM), "q")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    n_cand = 0
    if cand is not None:
        n_cand = cand.shape[-1]
        _need(cand, torch.int32, (shape.n_seq, M, n_cand), "cand")
    if logits is None:
        cols = _ld(n_cand) if cand is not None else _ld(shape.n_keys)
        logits = torch.empty((shape.n_seq, M, cols), dtype=torch.float32, device=q.device)
    st = load().dsa_dense_logits(ctypes.byref(shape), _ptr(q), _ptr(w), _ptr(k), kd, _ptr(k_scale),
                                 _ptr(cand), int(n_cand), _ptr(logits), int(logits.shape[-1]),
                                 _stream(stream))
    _check(st, "dsa_dense_logits")
    return logits


def misa_topk(shape: MisaShape, logits, k: int, n_cols=None, cand=None, idx=None, vals=None,
              want_vals=True, sorted=True, ws=None, stream=None):
    """Top-k ids [n_seq, M, k] (int32, -1 padded) and values (fp32, -inf padded);
    sorted=False returns the same set in an unspecified order."""
    M = shape.q_per_seq
    _need(logits, torch.float32, (shape.n_seq, M, logits.shape[-1]), "logits")
    if cand is not None:
        n_cols = cand.shape[-1]
        _need(cand, torch.int32, (shape.n_seq, M, n_cols), "cand")
    elif n_cols is None:
        n_cols = shape.n_keys
    lib = load()
    if idx is None:
        idx = torch.empty((shape.n_seq, M, k), dtype=torch.int32, device=logits.device)
    if vals is None and want_vals:
        vals = torch.empty((shape.n_seq, M, k), dtype=torch.float32, device=logits.device)
    need = lib.misa_topk_workspace_bytes(ctypes.byref(shape), int(n_cols), int(k))
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=logits.device)
    st = lib.misa_topk(ctypes.byref(shape), _ptr(logits), int(logits.shape[-1]), _ptr(cand), int(n_cols),
                       int(k), int(bool(sorted)), _ptr(idx), _ptr(vals), _ptr(ws), int(ws.numel() if ws is not None else 0),
                       _stream(stream))
    _check(st, "misa_topk")
    return idx, vals


def misa_topk_workspace_bytes(shape: MisaShape, n_cols: int, k: int) -> int:
    return int(load().misa_topk_workspace_bytes(ctypes.byref(shape), int(n_cols), int(k)))


def misa_sparse_head_topk_workspace_bytes(shape: MisaShape, kdtype: int, h: int, topk: int) -> int:
    """kdtype: MISA_K_BF16 or MISA_K_FP8_E4M3 (the key type of the call)."""
    return int(load().misa_sparse_head_topk_workspace_bytes(ctypes.byref(shape), int(kdtype), int(h), int(topk)))


def misa_sparse_head_topk(shape: MisaShape, q, w, k, heads, topk: int, k_scale=None, sorted=True, idx=None,
                          vals=None, want_vals=True, ws=None, stream=None):
    """Routed scoring + top-k in one call (no logits where they can be avoided);
    the same result as misa_topk(misa_sparse_head_logits(...), topk)."""
    kd = _check_keys(shape, k, k_scale)
    M, H = shape.q_per_seq, shape.n_heads
    _need(q, torch.bfloat16, (shape.n_seq, M, H, HEAD_DIM), "q")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    h = heads.shape[-1]
    _need(heads, torch.int32, (shape.n_seq, M, h), "heads")
    if idx is None:
        idx = torch.empty((shape.n_seq, M, topk), dtype=torch.int32, device=q.device)
    if vals is None and want_vals:
        vals = torch.empty((shape.n_seq, M, topk), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(max(misa_sparse_head_topk_workspace_bytes(shape, kd, h, topk), 1), dtype=torch.uint8,
                         device=q.device)
    st = load().misa_sparse_head_topk(ctypes.byref(shape), _ptr(q), _ptr(w), _ptr(k), kd, _ptr(k_scale),
                                      _ptr(heads), int(h), int(topk), int(bool(sorted)), _ptr(idx), _ptr(vals),
                                      _ptr(ws), int(ws.numel()), _stream(stream))
    _check(st, "misa_sparse_head_topk")
    return idx, vals


def misa_quantize_q(shape: MisaShape, q, q8=None, q_scale=None, stream=None):
    """Per-(query, head) fp8 queries: e4m3fn codes [n_seq, M, H, 128] (uint8) and
    fp32 scales [n_seq, M, H]."""
    M, H = shape.q_per_seq, shape.n_heads
    _need(q, torch.bfloat16, (shape.n_seq, M, H, HEAD_DIM), "q")
    if q8 is None:
        q8 = torch.empty((shape.n_seq, M, H, HEAD_DIM), dtype=torch.uint8, device=q.device)
    if q_scale is None:
        q_scale = torch.empty((shape.n_seq, M, H), dtype=torch.float32, device=q.device)
    st = load().misa_quantize_q(ctypes.byref(shape), _ptr(q), _ptr(q8), _ptr(q_scale), _stream(stream))
    _check(st, "misa_quantize_q")
    return q8, q_scale


def misa_sparse_head_logits_q8(shape: MisaShape, q8, q_scale, w, k, heads, k_scale, logits=None, stream=None):
    """Routed-head logits [n_seq, M, ld] from fp8 queries and fp8 keys (h <= 8)."""
    kd = _check_keys(shape, k, k_scale)
    M, H = shape.q_per_seq, shape.n_heads
    _need(q8, torch.uint8, (shape.n_seq, M, H, HEAD_DIM), "q8")
    _need(q_scale, torch.float32, (shape.n_seq, M, H), "q_scale")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    h = heads.shape[-1]
    _need(heads, torch.int32, (shape.n_seq, M, h), "heads")
    if logits is None:
        logits = torch.empty((shape.n_seq, M, _ld(shape.n_keys)), dtype=torch.float32, device=q8.device)
    st = load().misa_sparse_head_logits_q8(ctypes.byref(shape), _ptr(q8), _ptr(q_scale), _ptr(w), _ptr(k), kd,
                                           _ptr(k_scale), _ptr(heads), int(h), _ptr(logits),
                                           int(logits.shape[-1]), _stream(stream))
    _check(st, "misa_sparse_head_logits_q8")
    return logits


def misa_sparse_head_topk_q8(shape: MisaShape, q8, q_scale, w, k, heads, topk: int, k_scale, sorted=True, idx=None,
                             vals=None, want_vals=True, ws=None, stream=None):
    """misa_sparse_head_topk on fp8 queries and fp8 keys (h <= 8): the same
    result as misa_topk(misa_sparse_head_logits_q8(...), topk)."""
    kd = _check_keys(shape, k, k_scale)
    M, H = shape.q_per_seq, shape.n_heads
    _need(q8, torch.uint8, (shape.n_seq, M, H, HEAD_DIM), "q8")
    _need(q_scale, torch.float32, (shape.n_seq, M, H), "q_scale")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    h = heads.shape[-1]
    _need(heads, torch.int32, (shape.n_seq, M, h), "heads")
    if idx is None:
        idx = torch.empty((shape.n_seq, M, topk), dtype=torch.int32, device=q8.device)
    if vals is None and want_vals:
        vals = torch.empty((shape.n_seq, M, topk), dtype=torch.float32, device=q8.device)
    if ws is None:
        ws = torch.empty(max(misa_sparse_head_topk_workspace_bytes(shape, kd, h, topk), 1), dtype=torch.uint8,
                         device=q8.device)
    st = load().misa_sparse_head_topk_q8(ctypes.byref(shape), _ptr(q8), _ptr(q_scale), _ptr(w), _ptr(k), kd,
                                         _ptr(k_scale), _ptr(heads), int(h), int(topk), int(bool(sorted)),
                                         _ptr(idx), _ptr(vals), _ptr(ws), int(ws.numel()), _stream(stream))
    _check(st, "misa_sparse_head_topk_q8")
    return idx, vals


def dsa_dense_logits_q8(shape: MisaShape, q8, q_scale, w, k, k_scale, logits=None, stream=None):
    """All-head (dense DSA) logits [n_seq, M, ld] from fp8 queries and fp8 keys."""
    kd = _check_keys(shape, k, k_scale)
    M, H = shape.q_per_seq, shape.n_heads
    _need(q8, torch.uint8, (shape.n_seq, M, H, HEAD_DIM), "q8")
    _need(q_scale, torch.float32, (shape.n_seq, M, H), "q_scale")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    if logits is None:
        logits = torch.empty((shape.n_seq, M, _ld(shape.n_keys)), dtype=torch.float32, device=q8.device)
    st = load().dsa_dense_logits_q8(ctypes.byref(shape), _ptr(q8), _ptr(q_scale), _ptr(w), _ptr(k), kd,
                                    _ptr(k_scale), _ptr(logits), int(logits.shape[-1]), _stream(stream))
    _check(st, "dsa_dense_logits_q8")
    return logits


def misa_indexer_workspace_bytes(shape: MisaShape, kdtype: int, h: int, topk: int, k_prime: int = 0) -> int:
    return int(load().misa_indexer_workspace_bytes(ctypes.byref(shape), int(kdtype), int(h), int(topk),
                                                   int(k_prime)))


def misa_indexer_workspace_min_bytes(shape: MisaShape, kdtype: int, h: int, topk: int, k_prime: int = 0) -> int:
    """The least workspace misa_indexer takes (same results, the flagged-row
    re-scoring in batches)."""
    return int(load().misa_indexer_workspace_min_bytes(ctypes.byref(shape), int(kdtype), int(h), int(topk),
                                                       int(k_prime)))


def misa_indexer(shape: MisaShape, q, w, k, h: int, topk: int, k_prime: int = 0, k_scale=None,
                 idx=None, vals=None, want_vals=True, ws=None, stream=None):
    """The whole MISA (k_prime = 0) or MISA-dagger (k_prime >= topk) indexer."""
    kd = _check_keys(shape, k, k_scale)
    M, H = shape.q_per_seq, shape.n_heads
    _need(q, torch.bfloat16, (shape.n_seq, M, H, HEAD_DIM), "q")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    if idx is None:
        idx = torch.empty((shape.n_seq, M, topk), dtype=torch.int32, device=q.device)
    if vals is None and want_vals:
        vals = torch.empty((shape.n_seq, M, topk), dtype=torch.float32, device=q.device)
    need = misa_indexer_workspace_bytes(shape, kd, h, topk, k_prime)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = load().misa_indexer(ctypes.byref(shape), _ptr(q), _ptr(w), _ptr(k), kd, _ptr(k_scale), int(h),
                             int(topk), int(k_prime), _ptr(idx), _ptr(vals), _ptr(ws), int(ws.numel()),
                             _stream(stream))
    _check(st, "misa_indexer")
    return idx, vals


def misa_indexer_noalloc(shape: MisaShape, q, w, k, h: int, topk: int, k_prime: int = 0, k_scale=None,
                         idx=None, vals=None, want_vals=True, stream=None):
    """misa_indexer with the library's fixed device scratch instead of a
    workspace (for callers that cannot allocate; the outputs must still be
    given to avoid an allocation here).  Raises MisaError (MISA_ERR_SCRATCH)
    when the request needs more than NOALLOC_SCRATCH_BYTES."""
    kd = _check_keys(shape, k, k_scale)
    M, H = shape.q_per_seq, shape.n_heads
    _need(q, torch.bfloat16, (shape.n_seq, M, H, HEAD_DIM), "q")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    if idx is None:
        idx = torch.empty((shape.n_seq, M, topk), dtype=torch.int32, device=q.device)
    if vals is None and want_vals:
        vals = torch.empty((shape.n_seq, M, topk), dtype=torch.float32, device=q.device)
    st = load().misa_indexer_noalloc(ctypes.byref(shape), _ptr(q), _ptr(w), _ptr(k), kd, _ptr(k_scale), int(h),
                                     int(topk), int(k_prime), _ptr(idx), _ptr(vals), _stream(stream))
    _check(st, "misa_indexer_noalloc")
    return idx, vals


def misa_profile_stage(stage, start_event=None, stop_event=None):
    """Bracket the kernels of `stage` (a name of STAGES, or None to stop) in the
    calls this host thread makes next with two torch.cuda.Event(enable_timing=True)."""
    if stage is None:
        _check(load().misa_profile_stage(0, None, None), "misa_profile_stage")
        return
    _check(load().misa_profile_stage(int(STAGES[stage]), ctypes.c_void_p(start_event.cuda_event),
                                     ctypes.c_void_p(stop_event.cuda_event)), "misa_profile_stage")


class PooledCache:
    """Caller-owned pooled-key cache of n_seq sequences (misa.h): block means
    [n_seq, cap_blocks, 128] fp32 and their bf16 hi/lo rows
    [n_seq, 2, cap_blocks, 128]; n_cached counts the valid leading blocks."""

    def __init__(self, n_seq: int, cap_blocks: int, device="cuda"):
        self.pooled = torch.empty((n_seq, cap_blocks, HEAD_DIM), dtype=torch.float32, device=device)
        self.split = torch.empty((n_seq, 2, cap_blocks, HEAD_DIM), dtype=torch.int16, device=device)
        self.cap_blocks = int(cap_blocks)
        self.n_cached = 0


def misa_pool_keys_cached(shape: MisaShape, k, cache: PooledCache, k_scale=None, tail=None, stream=None):
    """Pool the blocks completed since the cache was last brought up to date
    (and the shape's query tails); returns tail [n_seq, M, 128]."""
    kd = _check_keys(shape, k, k_scale)
    if tail is None:
        tail = torch.empty((shape.n_seq, max(shape.q_per_seq, 1), HEAD_DIM), dtype=torch.float32, device=k.device)
    st = load().misa_pool_keys_cached(ctypes.byref(shape), _ptr(k), kd, _ptr(k_scale), int(cache.n_cached),
                                      _ptr(cache.pooled), _ptr(cache.split), cache.cap_blocks, _ptr(tail),
                                      _stream(stream))
    _check(st, "misa_pool_keys_cached")
    cache.n_cached = shape.n_keys // shape.block
    return tail


def misa_indexer_cached_workspace_bytes(shape: MisaShape, kdtype: int, h: int, topk: int, k_prime: int = 0) -> int:
    return int(load().misa_indexer_cached_workspace_bytes(ctypes.byref(shape), int(kdtype), int(h), int(topk),
                                                          int(k_prime)))


def misa_indexer_cached(shape: MisaShape, q, w, k, h: int, topk: int, cache: PooledCache, k_prime: int = 0,
                        k_scale=None, idx=None, vals=None, want_vals=True, ws=None, stream=None):
    """misa_indexer with the pooled keys kept in `cache` across calls (the
    cache is brought up to date first; same result as misa_indexer)."""
    kd = _check_keys(shape, k, k_scale)
    M, H = shape.q_per_seq, shape.n_heads
    _need(q, torch.bfloat16, (shape.n_seq, M, H, HEAD_DIM), "q")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    if idx is None:
        idx = torch.empty((shape.n_seq, M, topk), dtype=torch.int32, device=q.device)
    if vals is None and want_vals:
        vals = torch.empty((shape.n_seq, M, topk), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(max(misa_indexer_cached_workspace_bytes(shape, kd, h, topk, k_prime), 1),
                         dtype=torch.uint8, device=q.device)
    st = load().misa_indexer_cached(ctypes.byref(shape), _ptr(q), _ptr(w), _ptr(k), kd, _ptr(k_scale), int(h),
                                    int(topk), int(k_prime), int(cache.n_cached), _ptr(cache.pooled),
                                    _ptr(cache.split), cache.cap_blocks, _ptr(idx), _ptr(vals), _ptr(ws),
                                    int(ws.numel()), _stream(stream))
    _check(st, "misa_indexer_cached")
    cache.n_cached = shape.n_keys // shape.block
    return idx, vals


def misa_prefill_workspace_bytes(shape: MisaShape, kdtype: int, h: int, topk: int, k_prime: int = 0,
                                 chunk: int = 8192) -> int:
    return int(load().misa_prefill_workspace_bytes(ctypes.byref(shape), int(kdtype), int(h), int(topk),
                                                   int(k_prime), int(chunk)))


def misa_prefill_chunked(shape: MisaShape, q, w, k, h: int, topk: int, chunk: int = 8192, k_prime: int = 0,
                         k_scale=None, idx=None, vals=None, want_vals=True, ws=None, stream=None):
    """The indexer over a whole prompt in chunks of `chunk` queries with an
    incremental pooled-key cache (same result as one misa_indexer call)."""
    kd = _check_keys(shape, k, k_scale)
    M, H = shape.q_per_seq, shape.n_heads
    _need(q, torch.bfloat16, (shape.n_seq, M, H, HEAD_DIM), "q")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    if idx is None:
        idx = torch.empty((shape.n_seq, M, topk), dtype=torch.int32, device=q.device)
    if vals is None and want_vals:
        vals = torch.empty((shape.n_seq, M, topk), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(max(misa_prefill_workspace_bytes(shape, kd, h, topk, k_prime, chunk), 1),
                         dtype=torch.uint8, device=q.device)
    st = load().misa_prefill_chunked(ctypes.byref(shape), _ptr(q), _ptr(w), _ptr(k), kd, _ptr(k_scale), int(h),
                                     int(topk), int(k_prime), int(chunk), _ptr(idx), _ptr(vals), _ptr(ws),
                                     int(ws.numel()), _stream(stream))
    _check(st, "misa_prefill_chunked")
    return idx, vals


def misa_indexer_q8_workspace_bytes(shape: MisaShape, h: int, topk: int, k_prime: int = 0) -> int:
    return int(load().misa_indexer_q8_workspace_bytes(ctypes.byref(shape), int(h), int(topk), int(k_prime)))


def misa_indexer_q8(shape: MisaShape, q, w, k, h: int, topk: int, k_scale, k_prime: int = 0, idx=None, vals=None,
                    want_vals=True, ws=None, stream=None):
    """misa_indexer with the routed scoring on fp8 queries (fp8 keys, h <= 8)."""
    kd = _check_keys(shape, k, k_scale)
    M, H = shape.q_per_seq, shape.n_heads
    _need(q, torch.bfloat16, (shape.n_seq, M, H, HEAD_DIM), "q")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    if idx is None:
        idx = torch.empty((shape.n_seq, M, topk), dtype=torch.int32, device=q.device)
    if vals is None and want_vals:
        vals = torch.empty((shape.n_seq, M, topk), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(max(misa_indexer_q8_workspace_bytes(shape, h, topk, k_prime), 1), dtype=torch.uint8,
                         device=q.device)
    st = load().misa_indexer_q8(ctypes.byref(shape), _ptr(q), _ptr(w), _ptr(k), kd, _ptr(k_scale), int(h),
                                int(topk), int(k_prime), _ptr(idx), _ptr(vals), _ptr(ws), int(ws.numel()),
                                _stream(stream))
    _check(st, "misa_indexer_q8")
    return idx, vals


def misa_gather_keys_paged(shape: MisaShape, k_pages, block_table, scale_pages=None, k_out=None, scale_out=None,
                           stream=None):
    """Contiguous keys [n_seq, n_keys, 128] (and fp8 scales [n_seq, n_keys]) from
    a paged cache: k_pages [n_pages, page_keys, 128], block_table int32
    [n_seq, max_pages]."""
    kd = _kdtype(k_pages)
    n_pages, page_keys = int(k_pages.shape[0]), int(k_pages.shape[1])
    _need(k_pages, k_pages.dtype, (n_pages, page_keys, HEAD_DIM), "k_pages")
    if kd == MISA_K_FP8_E4M3:
        _need(scale_pages, torch.float32, (n_pages, page_keys), "scale_pages")
    _need(block_table, torch.int32, (shape.n_seq, block_table.shape[-1]), "block_table")
    if k_out is None:
        k_out = torch.empty((shape.n_seq, shape.n_keys, HEAD_DIM), dtype=k_pages.dtype, device=k_pages.device)
    if scale_out is None and kd == MISA_K_FP8_E4M3:
        scale_out = torch.empty((shape.n_seq, shape.n_keys), dtype=torch.float32, device=k_pages.device)
    st = load().misa_gather_keys_paged(ctypes.byref(shape), _ptr(k_pages), kd, _ptr(scale_pages), _ptr(block_table),
                                       int(block_table.shape[-1]), n_pages, page_keys, _ptr(k_out), _ptr(scale_out),
                                       _stream(stream))
    _check(st, "misa_gather_keys_paged")
    return k_out, scale_out


def misa_indexer_paged_workspace_bytes(shape: MisaShape, kdtype: int, h: int, topk: int) -> int:
    return int(load().misa_indexer_paged_workspace_bytes(ctypes.byref(shape), int(kdtype), int(h), int(topk)))


def misa_indexer_paged(shape: MisaShape, q, w, k_pages, block_table, h: int, topk: int, cache: PooledCache,
                       scale_pages=None, idx=None, vals=None, want_vals=True, ws=None, stream=None):
    """misa_indexer_cached on keys read in place from a paged cache: k_pages
    [n_pages, page_keys, 128] (bf16, or e4m3 codes with scale_pages [n_pages,
    page_keys]), block_table int32 [n_seq, max_pages]."""
    kd = _kdtype(k_pages)
    n_pages, page_keys = int(k_pages.shape[0]), int(k_pages.shape[1])
    _need(k_pages, k_pages.dtype, (n_pages, page_keys, HEAD_DIM), "k_pages")
    if kd == MISA_K_FP8_E4M3:
        _need(scale_pages, torch.float32, (n_pages, page_keys), "scale_pages")
    _need(block_table, torch.int32, (shape.n_seq, block_table.shape[-1]), "block_table")
    M, H = shape.q_per_seq, shape.n_heads
    _need(q, torch.bfloat16, (shape.n_seq, M, H, HEAD_DIM), "q")
    _need(w, torch.float32, (shape.n_seq, M, H), "w")
    if idx is None:
        idx = torch.empty((shape.n_seq, M, topk), dtype=torch.int32, device=q.device)
    if vals is None and want_vals:
        vals = torch.empty((shape.n_seq, M, topk), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(max(misa_indexer_paged_workspace_bytes(shape, kd, h, topk), 1), dtype=torch.uint8,
                         device=q.device)
    st = load().misa_indexer_paged(ctypes.byref(shape), _ptr(q), _ptr(w), _ptr(k_pages), kd, _ptr(scale_pages),
                                   _ptr(block_table), int(block_table.shape[-1]), n_pages, page_keys, int(h),
                                   int(topk), int(cache.n_cached), _ptr(cache.pooled), _ptr(cache.split),
                                   cache.cap_blocks, _ptr(idx), _ptr(vals), _ptr(ws), int(ws.numel()),
                                   _stream(stream))
    _check(st, "misa_indexer_paged")
    cache.n_cached = shape.n_keys // shape.block
    return idx, vals
