"""The C ABI library on the CPU: it loads, exports every function misa.h declares,
and rejects bad arguments on the host before anything touches a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import long_context_sparse_block_amd as lcsb
from long_context_sparse_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "misa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmisa.so is not built (python -m long_context_sparse_block_amd.build)")
    return _lib.load()


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    assert names == sorted(_lib.EXPORTED), names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def shape(**kw):
    base = dict(n_seq=1, q_per_seq=4, n_keys=64, q_pos0=60, n_heads=8, block=16)
    base.update(kw)
    return lcsb.make_shape(**base)


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation first


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert lib.misa_status_str(code)
    assert b"unknown" in lib.misa_status_str(7)


@pytest.mark.parametrize("kw,code", [
    (dict(n_seq=0), -1), (dict(q_per_seq=-1), -1), (dict(n_keys=0), -1), (dict(q_pos0=-1), -1),
    (dict(q_pos0=61), -1), (dict(n_heads=0), -1), (dict(n_heads=65), -1), (dict(block=0), -1),
    (dict(head_dim=64), -2),
])
def test_pool_rejects_bad_shapes(lib, kw, code):
    s = shape(**kw)
    st = lib.misa_pool_keys(ctypes.byref(s), FAKE, 0, None, FAKE, FAKE, None)
    assert st == code


def test_null_shape_and_pointers(lib):
    assert lib.misa_pool_keys(None, FAKE, 0, None, FAKE, FAKE, None) == -1
    s = shape()
    assert lib.misa_pool_keys(ctypes.byref(s), None, 0, None, FAKE, FAKE, None) == -1
    assert lib.misa_pool_keys(ctypes.byref(s), FAKE, 1, None, FAKE, FAKE, None) == -1   # fp8 needs scale
    assert lib.misa_pool_keys(ctypes.byref(s), FAKE, 5, None, FAKE, FAKE, None) == -1   # bad dtype
    misaligned = ctypes.c_void_p(0x10004)
    assert lib.misa_pool_keys(ctypes.byref(s), misaligned, 0, None, FAKE, FAKE, None) == -1


def test_route_checks_h(lib):
    s = shape()
    for h in (0, 9):
        assert lib.misa_route_heads(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, h, FAKE, None, None) == -1


def test_logits_check_ld_and_h(lib):
    s = shape()
    f = lib.misa_sparse_head_logits
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, FAKE, 0, FAKE, 64, None) == -1
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, FAKE, 2, FAKE, 60, None) == -1   # ld < N
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, FAKE, 2, FAKE, 66, None) == -1   # ld % 4
    g = lib.dsa_dense_logits
    assert g(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, None, 0, FAKE, 62, None) == -1
    assert g(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, FAKE, 0, FAKE, 64, None) == -1   # n_cand 0
    assert g(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, FAKE, 80, FAKE, 64, None) == -1  # ld < n_cand


def test_topk_checks(lib):
    s = shape()
    f = lib.misa_topk
    assert f(ctypes.byref(s), FAKE, 64, None, 64, 0, 1, FAKE, None, None, 0, None) == -1
    assert f(ctypes.byref(s), FAKE, 64, None, 64, 8193, 1, FAKE, None, None, 0, None) == -1
    assert f(ctypes.byref(s), FAKE, 64, None, 65, 4, 1, FAKE, None, None, 0, None) == -1     # ld < n_cols
    assert f(ctypes.byref(s), FAKE, 64, None, 64, 4, 1, None, None, None, 0, None) == -1     # idx null


def test_indexer_checks_and_workspace(lib):
    s = shape()
    f = lib.misa_indexer
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, 9, 4, 0, FAKE, None, FAKE, 1 << 30, None) == -1
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, 2, 4, 3, FAKE, None, FAKE, 1 << 30, None) == -1
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, 2, 4, 0, FAKE, None, None, 0, None) == -3
    need = lib.misa_indexer_workspace_bytes(ctypes.byref(s), 0, 2, 4, 0)
    assert need > 0
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, 2, 4, 0, FAKE, None, FAKE, need - 1, None) == -3
    # MISA-dagger needs room for candidates and their re-ranked scores
    need_d = lib.misa_indexer_workspace_bytes(ctypes.byref(s), 0, 2, 4, 16)
    assert need_d > need


def test_sparse_head_topk_checks_and_workspace(lib):
    s = shape()
    f = lib.misa_sparse_head_topk
    # h out of range, topk out of range, missing heads, missing workspace
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, FAKE, 9, 4, 1, FAKE, None, FAKE, 1 << 30, None) == -1
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, FAKE, 2, 0, 1, FAKE, None, FAKE, 1 << 30, None) == -1
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, None, 2, 4, 1, FAKE, None, FAKE, 1 << 30, None) == -1
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, FAKE, 2, 4, 1, FAKE, None, None, 0, None) == -3
    need = lib.misa_sparse_head_topk_workspace_bytes(ctypes.byref(s), 0, 2, 4)
    assert need > 0
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, FAKE, 2, 4, 1, FAKE, None, FAKE, need - 1, None) == -3
    # the long-context chunk takes the fused path: sampled scores and candidate
    # regions instead of the whole-row top-k's lists, beside the full logits
    # kept for rows the candidates cannot settle
    big = lcsb.make_shape(1, 8192, 131072, 131072 - 8192, 64, 128)
    fused = lib.misa_sparse_head_topk_workspace_bytes(ctypes.byref(big), 1, 8, 2048)
    # target 3072 candidates per row, 8 key ranges of 16384 keys over a shortest
    # prefix of 122881: 410 expected groups per range, doubled, + 512, rounded
    # up to 256 = 1536 groups of 4 scores (16 bytes) and their first key (4)
    # plus the bf16 copy of the keys the scoring stages by direct loads (131072 x 256)
    # (the sampled scores share their memory with the logits slab)
    assert fused == (8192 * 131072 * 4 + 131072 * 256 + 2 * 8192 * 4 + 8192 * 8 * 4 + 8192 * 8 * 1536 * 20)
    # bf16 keys are staged as they are: no widened copy
    assert lib.misa_sparse_head_topk_workspace_bytes(ctypes.byref(big), 0, 8, 2048) == fused - 131072 * 256


def test_only_fp8_keys_reserve_a_widened_copy(lib):
    # a prefill chunk of 256 queries over 131072 keys takes the fused path,
    # whose direct-load staging reads a bf16 copy of fp8 keys (131072 x 256 B)
    s = lcsb.make_shape(1, 256, 131072, 131072 - 256, 32, 64)
    bf = lib.misa_indexer_workspace_bytes(ctypes.byref(s), 0, 8, 2048, 0)
    f8 = lib.misa_indexer_workspace_bytes(ctypes.byref(s), 1, 8, 2048, 0)
    assert f8 - bf == 131072 * 256
    # the fp8-query indexer feeds fp8 keys to the fp8 matrix cores directly
    q8 = lib.misa_indexer_q8_workspace_bytes(ctypes.byref(s), 8, 2048, 0)
    assert q8 < f8
    # the decode batch (64 sequences x 131072 keys, one query each) scores into
    # whole logits rows (64 x 131072 x 4 B = 32 MiB) and stages fp8 keys
    # through registers: no copy of the keys (it would be 2 GiB)
    d = lcsb.make_shape(64, 1, 131072, 131071, 32, 64)
    bf = lib.misa_indexer_workspace_bytes(ctypes.byref(d), 0, 8, 2048, 0)
    assert lib.misa_indexer_workspace_bytes(ctypes.byref(d), 1, 8, 2048, 0) == bf
    assert 64 * 131072 * 4 <= bf < (256 << 20)


def test_fp8_query_calls_check_their_arguments(lib):
    s = shape()
    # quantisation: null or misaligned pointers
    assert lib.misa_quantize_q(ctypes.byref(s), None, FAKE, FAKE, None) == -1
    assert lib.misa_quantize_q(ctypes.byref(s), FAKE, ctypes.c_void_p(0x10004), FAKE, None) == -1
    assert lib.misa_quantize_q(ctypes.byref(s), FAKE, FAKE, None, None) == -1
    lq = lib.misa_sparse_head_logits_q8
    # bf16 keys are refused (the fp8 MFMA takes fp8 on both sides), h above 8 too
    assert lq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 0, None, FAKE, 2, FAKE, 64, None) == -2
    assert lq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 9, FAKE, 64, None) == -1   # h > H
    s16 = shape(n_heads=16)
    assert lq(ctypes.byref(s16), FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 9, FAKE, 64, None) == -2
    assert lq(ctypes.byref(s), FAKE, None, FAKE, FAKE, 1, FAKE, FAKE, 2, FAKE, 64, None) == -1   # no q scale
    assert lq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 2, FAKE, 62, None) == -1   # ld < N
    dq = lib.dsa_dense_logits_q8
    assert dq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 0, None, FAKE, 64, None) == -2    # bf16 keys
    assert dq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1, None, FAKE, 64, None) == -1    # fp8 needs scales
    assert dq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 66, None) == -1    # ld % 4
    assert dq(ctypes.byref(s), FAKE, FAKE, None, FAKE, 1, FAKE, FAKE, 64, None) == -1    # no weights
    tq = lib.misa_sparse_head_topk_q8
    need = lib.misa_sparse_head_topk_workspace_bytes(ctypes.byref(s), 0, 2, 4)
    assert tq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 0, None, FAKE, 2, 4, 1, FAKE, None, FAKE, need, None) == -2
    assert tq(ctypes.byref(s16), FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 9, 4, 1, FAKE, None, FAKE, 1 << 30,
              None) == -2
    assert tq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 2, 0, 1, FAKE, None, FAKE, need, None) == -1
    assert tq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1, FAKE, None, 2, 4, 1, FAKE, None, FAKE, need, None) == -1
    assert tq(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, 2, 4, 1, FAKE, None, FAKE, need - 1,
              None) == -3


def test_fp8_indexer_checks(lib):
    s = shape()
    f = lib.misa_indexer_q8
    need = lib.misa_indexer_q8_workspace_bytes(ctypes.byref(s), 2, 4, 0)
    assert need > lib.misa_indexer_workspace_bytes(ctypes.byref(s), 0, 2, 4, 0)   # + fp8 q and its scales
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, 2, 4, 0, FAKE, None, FAKE, need, None) == -2   # bf16 keys
    s16 = shape(n_heads=16)
    assert f(ctypes.byref(s16), FAKE, FAKE, FAKE, 1, FAKE, 9, 16, 0, FAKE, None, FAKE, 1 << 30, None) == -2
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 1, FAKE, 2, 4, 2, FAKE, None, FAKE, 1 << 30, None) == -1   # k' < k
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 1, FAKE, 2, 4, 0, FAKE, None, FAKE, need - 1, None) == -3


def test_paged_gather_checks(lib):
    s = shape()   # 64 keys
    g = lib.misa_gather_keys_paged
    assert g(ctypes.byref(s), FAKE, 0, None, None, 4, 8, 16, FAKE, None, None) == -1       # no block table
    assert g(ctypes.byref(s), FAKE, 0, None, FAKE, 3, 8, 16, FAKE, None, None) == -1       # 3 pages < 64 / 16
    assert g(ctypes.byref(s), FAKE, 0, None, FAKE, 4, 8, 0, FAKE, None, None) == -1        # empty pages
    assert g(ctypes.byref(s), FAKE, 1, FAKE, FAKE, 4, 8, 16, FAKE, None, None) == -1       # fp8 needs scale_out
    assert g(ctypes.byref(s), FAKE, 1, None, FAKE, 4, 8, 16, FAKE, FAKE, None) == -1       # fp8 needs page scales


def test_paged_indexer_checks_its_arguments(lib):
    s = lcsb.make_shape(2, 1, 300, 299, 16, 64)   # decode: 2 sequences x 300 keys, 4 complete blocks
    f = lib.misa_indexer_paged
    need = lib.misa_indexer_paged_workspace_bytes(ctypes.byref(s), 0, 8, 64)
    assert need > 0

    def call(kd=0, sc=None, table=FAKE, max_pages=5, n_pages=10, page_keys=64, h=8, cap=4, ws_bytes=need):
        return f(ctypes.byref(s), FAKE, FAKE, FAKE, kd, sc, table, max_pages, n_pages, page_keys, h, 64, 0, FAKE,
                 FAKE, cap, FAKE, None, FAKE, ws_bytes, None)
    assert call(table=None) == -1          # no block table
    assert call(page_keys=48) == -1        # pages must hold whole 64-key tiles
    assert call(page_keys=32) == -1
    assert call(max_pages=4) == -1         # 4 pages of 64 < 300 keys
    assert call(n_pages=0) == -1
    assert call(kd=1) == -1                # fp8 pages need their scales
    assert call(cap=3) == -1               # cache smaller than the 4 complete blocks
    assert call(h=17) == -1                # more heads than the shape has
    assert call(h=9) == -2                 # the routed kernel that reads pages takes h <= 8
    assert call(ws_bytes=need - 1) == -3   # workspace too small
    # the fast plan: the re-scoring slab holds every query tile, and fp8 pages
    # are never widened into the workspace (unlike contiguous fp8 keys)
    big = lcsb.make_shape(1, 8192, 131072, 131072 - 8192, 64, 128)
    paged = lib.misa_indexer_paged_workspace_bytes(ctypes.byref(big), 1, 8, 2048)
    assert paged >= 8192 * 131072 * 4
    cached = lib.misa_indexer_cached_workspace_bytes(ctypes.byref(big), 1, 8, 2048, 0)
    assert cached - paged == 131072 * 256


def test_workspace_queries_of_a_cache_update_without_queries(lib):
    # no queries over more than 256 complete blocks: the router's part split
    # must not divide by its (zero) workgroup count
    # (such a call only brings the cache up to date and needs no workspace
    # beyond the pooled keys misa_indexer keeps in its own)
    s = lcsb.make_shape(3, 0, 20011, 20011, 16, 64)
    for kd in (0, 1):
        assert lib.misa_indexer_cached_workspace_bytes(ctypes.byref(s), kd, 8, 512, 0) == 0
        assert lib.misa_indexer_paged_workspace_bytes(ctypes.byref(s), kd, 8, 512) == 0
        assert lib.misa_indexer_workspace_bytes(ctypes.byref(s), kd, 8, 512, 0) > 0


def test_pooled_cache_calls_check_their_arguments(lib):
    s = shape()   # 64 keys, block 16: 4 complete blocks
    pc = lib.misa_pool_keys_cached
    assert pc(ctypes.byref(s), FAKE, 0, None, 0, FAKE, FAKE, 3, FAKE, None) == -1     # cap < N / B
    assert pc(ctypes.byref(s), FAKE, 0, None, 5, FAKE, FAKE, 4, FAKE, None) == -1     # n_cached > N / B
    assert pc(ctypes.byref(s), FAKE, 0, None, -1, FAKE, FAKE, 4, FAKE, None) == -1    # n_cached < 0
    assert pc(ctypes.byref(s), FAKE, 0, None, 0, None, FAKE, 4, FAKE, None) == -1     # no pooled rows
    assert pc(ctypes.byref(s), FAKE, 0, None, 0, FAKE, None, 4, FAKE, None) == -1     # no hi/lo rows
    assert pc(ctypes.byref(s), FAKE, 0, None, 0, FAKE, FAKE, 4, None, None) == -1     # queries need tails
    ic = lib.misa_indexer_cached
    need = lib.misa_indexer_cached_workspace_bytes(ctypes.byref(s), 0, 2, 4, 0)
    full = lib.misa_indexer_workspace_bytes(ctypes.byref(s), 0, 2, 4, 0)
    assert 0 < need < full   # the pooled keys live in the cache, not the workspace
    assert ic(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, 2, 4, 0, 0, FAKE, FAKE, 3, FAKE, None, FAKE, need,
              None) == -1
    assert ic(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, 9, 4, 0, 0, FAKE, FAKE, 4, FAKE, None, FAKE, need,
              None) == -1
    assert ic(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, 2, 4, 0, 0, FAKE, FAKE, 4, FAKE, None, FAKE, need - 1,
              None) == -3
    pf = lib.misa_prefill_chunked
    pneed = lib.misa_prefill_workspace_bytes(ctypes.byref(s), 0, 2, 4, 0, 2)
    assert pneed > 0 and lib.misa_prefill_workspace_bytes(ctypes.byref(s), 0, 2, 4, 0, 0) == 0
    assert pf(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, 2, 4, 0, 0, FAKE, None, FAKE, pneed, None) == -1
    assert pf(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, 2, 4, 0, 2, FAKE, None, FAKE, pneed - 1, None) == -3
    assert pf(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, 2, 4, 3, 2, FAKE, None, FAKE, pneed, None) == -1


def test_prefill_workspace_of_a_128k_prompt(lib):
    # 16 chunks of 8192: the one-sequence cache (1024 blocks of 128: 0.5 MB of
    # means + 0.5 MB of bf16 hi/lo rows) plus the last chunk's indexer
    # workspace, the largest (the full-prefix chunk of the benchmark)
    s = lcsb.make_shape(1, 131072, 131072, 0, 64, 128)
    need = lib.misa_prefill_workspace_bytes(ctypes.byref(s), 1, 8, 2048, 0, 8192)
    last = lcsb.make_shape(1, 8192, 131072, 131072 - 8192, 64, 128)
    ix = lib.misa_indexer_cached_workspace_bytes(ctypes.byref(last), 1, 8, 2048, 0)
    assert need == 1024 * 128 * 4 + 2 * 1024 * 128 * 2 + ix


def test_empty_query_set_is_a_no_op(lib):
    s = shape(q_per_seq=0, q_pos0=64)
    assert lib.misa_sparse_head_logits(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, FAKE, 2, FAKE, 64,
                                       None) == 0
    assert lib.misa_topk(ctypes.byref(s), FAKE, 64, None, 64, 4, 1, FAKE, None, None, 0, None) == 0


def test_workspace_size_of_the_long_context_chunk(lib):
    s = lcsb.make_shape(1, 8192, 131072, 131072 - 8192, 64, 128)
    need = lib.misa_indexer_workspace_bytes(ctypes.byref(s), 1, 8, 2048, 0)
    # the fp32 logits of the chunk (8192 x 131072 x 4 bytes; the fused path
    # writes them only for rows its candidates cannot settle, and the sampled
    # scores share their memory), the candidate regions (8192 rows x 8 key
    # ranges x 1536 groups of 4 scores and a key, 20 bytes) and the bf16 keys
    main = 8192 * 131072 * 4 + 8192 * 8 * 1536 * 20 + 131072 * 256
    assert main <= need < main * 1.01


def test_least_workspace_of_the_long_context_chunk(lib):
    s = lcsb.make_shape(1, 8192, 131072, 131072 - 8192, 64, 128)
    full = lib.misa_indexer_workspace_bytes(ctypes.byref(s), 1, 8, 2048, 0)
    least = lib.misa_indexer_workspace_min_bytes(ctypes.byref(s), 1, 8, 2048, 0)
    # the sampled scores (8192 x 4096 x 4 bytes = 128 MiB) double as the
    # logits slab (8 query tiles of 32 rows x 131072 scores, 16 MiB each), the
    # regions take 640 groups (410 expected + a quarter + 128, rounded up to
    # 64), and the bf16 keys
    main = 8192 * 4096 * 4 + 8192 * 8 * 640 * 20 + 131072 * 256
    assert main <= least < main * 1.01
    assert least < (1 << 30) < full
    # a workspace below the least is refused before anything is enqueued
    f = lib.misa_indexer
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 1, FAKE, 8, 2048, 0, FAKE, None, FAKE, least - 1, None) == -3
    assert lib.misa_indexer_workspace_min_bytes(ctypes.byref(s), 1, 0, 2048, 0) == 0


def test_short_prefixes_have_no_lean_plan(lib):
    # rows that the fused path does not take (prefixes of 1 .. 4096 keys) are
    # selected from full logits, whatever the workspace
    s = lcsb.make_shape(1, 4096, 4096, 0, 64, 64)
    assert lib.misa_indexer_workspace_min_bytes(ctypes.byref(s), 0, 8, 256, 0) == \
        lib.misa_indexer_workspace_bytes(ctypes.byref(s), 0, 8, 256, 0)


def test_noalloc_indexer_refuses_requests_beyond_its_scratch(lib):
    # argument errors first, as misa_indexer
    s = shape()
    f = lib.misa_indexer_noalloc
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 0, None, 9, 4, 0, FAKE, None, None) == -1
    assert f(ctypes.byref(s), FAKE, FAKE, FAKE, 1, None, 2, 4, 0, FAKE, None, None) == -1   # fp8 without scales
    # the long-context chunk needs gigabytes of scratch: refused before anything is enqueued
    big = lcsb.make_shape(1, 8192, 131072, 131072 - 8192, 64, 128)
    assert lib.misa_indexer_workspace_bytes(ctypes.byref(big), 1, 8, 2048, 0) > lcsb.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), FAKE, FAKE, FAKE, 1, FAKE, 8, 2048, 0, FAKE, None, None) == lcsb.MISA_ERR_SCRATCH
    assert "fixed device buffer" in lcsb.status_str(lcsb.MISA_ERR_SCRATCH)
    # a decode batch of 64 sequences x 131072 bf16 keys fits
    dec = lcsb.make_shape(64, 1, 131072, 131071, 32, 64)
    assert lib.misa_indexer_workspace_bytes(ctypes.byref(dec), 0, 8, 2048, 0) <= lcsb.NOALLOC_SCRATCH_BYTES


def test_region_capacity_never_exceeds_a_key_range(lib):
    # 64 queries over 32768 keys: 512 key ranges of 64 keys, each of which holds
    # at most 16 groups of 4 keys, so no region reserves more than that
    s = lcsb.make_shape(1, 64, 32768, 32768 - 64, 64, 64)
    need = lib.misa_indexer_workspace_bytes(ctypes.byref(s), 0, 8, 2048, 0)
    assert need < (32 << 20)


def test_profile_stage_checks_its_arguments(lib):
    assert lib.misa_profile_stage(99, FAKE, FAKE) == -1        # unknown stage
    assert lib.misa_profile_stage(5, None, FAKE) == -1         # null event
    assert lib.misa_profile_stage(0, None, None) == 0          # off

