// Host-side launchers of the MISA kernels (internal; the public ABI is misa.h).
// Each returns hipSuccess or the error of the launch.  Arguments have been
// validated by the caller (misa_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "misa.h"

namespace misa {

// pooled: [n_seq][ld_blk][128] block means (ld_blk < 0: N/B).  split
// (nullable): also write the pooled keys' bf16 hi and lo (pooled - hi) rows,
// per sequence ld_blk hi rows then ld_blk lo rows, for launch_route.
// n_cached: block rows [0, n_cached) already hold these keys' means (an
// incremental cache); only later complete blocks are pooled.
// Paged keys: key t of sequence b is row table[b * max_pages + t / page_keys]
// * page_keys + t % page_keys of the page pool.  page_keys is a multiple of
// 64, so a 64-key scoring tile never straddles two pages.
struct KeyPages {
  const int32_t* table;
  int64_t max_pages, n_pages;
  int page_keys;
};

// Routed-head logits (h <= 8, the k_score_h8 arithmetic) with the keys read in
// place from a page pool through the block table (page_keys % 64 == 0)
hipError_t launch_score_paged(const misa_shape& s, const uint16_t* q, const float* w, const void* k_pages,
                              int kdtype, const float* scale_pages, const int32_t* heads, int h, float* logits,
                              int64_t ld, const KeyPages& pages, hipStream_t st);
// pages (nullable): k and k_scale are page pools read through the block table
hipError_t launch_pool(const misa_shape& s, const void* k, int kdtype, const float* k_scale,
                       float* pooled, float* tail, uint16_t* split, hipStream_t st, int64_t n_cached = 0,
                       int64_t ld_blk = -1, const KeyPages* pages = nullptr);

// split (nullable): launch_pool's hi/lo rows, staged directly instead of
// splitting `pooled` in every workgroup (same values); ld_blk as launch_pool.
// part_ws (nullable, with split): [rows][route_parts(s) + 1][H] floats that let
// a launch with few workgroups (decode) split each block sum over more of them
// (the last slot holds the partial block's term).
constexpr int kMaxRouteParts = 8;
int route_parts(const misa_shape& s);   // 1: no split
hipError_t launch_route(const misa_shape& s, const uint16_t* q, const float* w, const float* pooled,
                        const uint16_t* split, const float* tail, int h, int32_t* heads, float* scores,
                        hipStream_t st, int64_t ld_blk = -1, float* part_ws = nullptr);

// Key-range split of a scoring grid: n_ksplits ranges of KR keys (a multiple
// of the tile KT), about `target` workgroups (several per CU) in the grid.
void plan_split(int64_t N, int n_seq, int n_qtiles, int KT, int* n_ksplits, int64_t* KR, int64_t target = 2048);

// Paged key cache -> contiguous [n_seq][N][128] keys (and fp8 scales [n_seq][N]).
hipError_t launch_gather_pages(const misa_shape& s, const void* pages, int kdtype, const float* page_scales,
                               const int32_t* table, int64_t max_pages, int64_t n_pages, int page_keys, void* out,
                               float* out_scale, hipStream_t st);

// Per-(query, head) fp8 quantisation of q: q8 codes [n_seq][M][H][128] and
// scales q_scale [n_seq][M][H].
hipError_t launch_quant_q(const misa_shape& s, const uint16_t* q, uint8_t* q8, float* q_scale, hipStream_t st);
// Routed-head logits from fp8 queries and fp8 keys (h <= 8); row_flag: only
// the workgroups holding a flagged row run (re-scoring after a fused pass).
// A re-scoring batch through a logits slab: query tiles [first, first +
// tiles) of the flattened (sequence, query tile) order, 32 queries a tile;
// the queries of the tile in slot s go to slab rows s * tr .. s * tr + tr - 1
// (tr = min(32, queries per sequence)).
struct SlabBatch {
  int64_t first;
  int tiles, tr;
};
hipError_t launch_score_q8(const misa_shape& s, const uint8_t* q8, const float* q_scale, const float* w,
                          const uint8_t* k, const float* k_scale, const int32_t* heads, int h, float* logits,
                          int64_t ld, hipStream_t st, const uint32_t* row_flag = nullptr,
                          const SlabBatch* slab = nullptr);

// heads == nullptr: all H heads (dense DSA indexer); otherwise h routed heads per query.
hipError_t launch_score(const misa_shape& s, const uint16_t* q, const float* w, const void* k,
                        int kdtype, const float* k_scale, const int32_t* heads, int h,
                        float* logits, int64_t ld, hipStream_t st);

hipError_t launch_score_gather(const misa_shape& s, const uint16_t* q, const float* w, const void* k,
                               int kdtype, const float* k_scale, const int32_t* cand, int n_cand,
                               float* logits, int64_t ld, hipStream_t st);

// sorted = false writes the selected set in no particular order (candidate lists).
hipError_t launch_topk(const misa_shape& s, const float* logits, int64_t ld, const int32_t* cand,
                       int n_cols, int k, int32_t* idx, float* vals, void* ws, size_t ws_bytes,
                       hipStream_t st, bool sorted = true);

size_t topk_workspace_bytes(const misa_shape& s, int n_cols, int k);

// ---------------------------------------------------------------------------
// Fused scoring -> top-k (the indexer's path for h <= 8 and long prefixes):
//  1. scores of a key sample (every kstride-th key) -> sample logits;
//  2. per-row threshold from the sample row (k_s-th largest sampled score);
//  3. routed-head scoring that keeps only scores >= the row threshold, as
//     candidates in per-(row, key range) regions, writing no logits;
//  4. exact top-k of each row's candidates; a row whose regions overflowed or
//     hold fewer than k candidates is flagged, re-scored into full logits and
//     selected from them, so the result is exact for every input.
// ---------------------------------------------------------------------------
// key ranges of one row the region select can take (its LDS prefix table)
constexpr int kMaxRegionSplits = 1024;

struct FusedPlan {
  bool ok;             // the fused path applies
  int kstride;         // key sampling stride of step 1
  int64_t n_sample;    // sampled keys per row (<= 4096)
  int64_t ld_sample;   // row stride of the sample logits
  int cap_list;        // candidates the select kernel can hold per row
  int target;          // candidates aimed for per row
  int n_splits;        // key ranges of the scoring grid
  int64_t key_range;   // keys per range
  int cap_region;      // candidate groups of 4 keys one (row, key range) region holds
};
FusedPlan plan_fused(const misa_shape& s, int h, int k);
// the fast plan with candidate regions sized closer to the expected
// candidates (the least-workspace plan)
FusedPlan lean_plan(const FusedPlan& fast, const misa_shape& s);

// The fused path's scoring launches: direct == true takes bf16 keys in `k`
// whatever kdtype is (fp8 keys widened by launch_widen_fp8; kdtype then says
// that k_scale applies) and stages them by direct global -> LDS loads;
// direct == false takes the keys as they are and stages them through
// registers (fp8 widened on the way into LDS: the same bf16 tiles).
hipError_t launch_widen_fp8(const misa_shape& s, const void* k, uint16_t* out, hipStream_t st);
hipError_t launch_score_sampled(const misa_shape& s, const uint16_t* q, const float* w, const void* k, int kdtype,
                                const float* k_scale, const int32_t* heads, int h, const FusedPlan& p,
                                float* sample_logits, hipStream_t st, bool direct = true,
                                const KeyPages* pages = nullptr);
// candidate regions: groups of 4 consecutive scores (gvals, float4 each) and
// their first key (gkeys), cap_region groups per (row, key range)
hipError_t launch_score_cands(const misa_shape& s, const uint16_t* q, const float* w, const void* k, int kdtype,
                              const float* k_scale, const int32_t* heads, int h, const FusedPlan& p,
                              const float* thr, float* gvals, int32_t* gkeys, uint32_t* rcount, hipStream_t st,
                              bool direct = true, const KeyPages* pages = nullptr);
// logits rows, into a slab batch, of the workgroups that hold a row with
// row_flag != 0
hipError_t launch_score_rescore(const misa_shape& s, const uint16_t* q, const float* w, const void* k,
                                int kdtype, const float* k_scale, const int32_t* heads, int h,
                                const uint32_t* row_flag, float* slab, int64_t ld, const SlabBatch& sb,
                                hipStream_t st, bool direct = true, const KeyPages* pages = nullptr);
// thr[row] from the sample logits; row_flag[row] = 0
hipError_t launch_topk_sample_thresh(const misa_shape& s, const FusedPlan& p, const float* sample_logits,
                                     float* thr, uint32_t* row_flag, hipStream_t st);
// top-k of the candidate regions; rows it cannot settle get row_flag = 1
hipError_t launch_topk_regions(const misa_shape& s, const FusedPlan& p, int k, const float* thr,
                               const float* gvals, const int32_t* gkeys, const uint32_t* rcount, uint32_t* row_flag,
                               int32_t* idx, float* vals, bool sorted, hipStream_t st);
// Dense (all H heads) logits from fp8 queries and fp8 keys: the fp8-query
// DSA comparator.
hipError_t launch_dense_q8(const misa_shape& s, const uint8_t* q8, const float* q_scale, const float* w,
                           const uint8_t* k, const float* k_scale, float* logits, int64_t ld, hipStream_t st);
// the fp8-query versions of the two scoring passes above (fp8 keys, h <= 8)
hipError_t launch_score_q8_sampled(const misa_shape& s, const uint8_t* q8, const float* q_scale, const float* w,
                                   const uint8_t* k, const float* k_scale, const int32_t* heads, int h,
                                   const FusedPlan& p, float* sample_logits, hipStream_t st);
hipError_t launch_score_q8_cands(const misa_shape& s, const uint8_t* q8, const float* q_scale, const float* w,
                                 const uint8_t* k, const float* k_scale, const int32_t* heads, int h,
                                 const FusedPlan& p, const float* thr, float* gvals, int32_t* gkeys, uint32_t* rcount,
                                 hipStream_t st);
// whole-row top-k of the flagged rows of a slab batch
hipError_t launch_topk_flagged(const misa_shape& s, int k, const float* slab, int64_t ld, const SlabBatch& sb,
                               const uint32_t* row_flag, int32_t* idx, float* vals, bool sorted, hipStream_t st);

}  // namespace misa
