// Pieces shared by the token-scoring kernels (bf16 k_score_h8 / k_score_q64
// and fp8 k_score_q8): tile coordinates, the output descriptor of a scoring
// pass, and its two epilogues (logits rows, or candidate groups appended to
// per-(row, key range) regions).
#pragma once

#include "misa_common.h"

namespace misa {

// Head ids are a documented precondition (in [0, H)); clamping keeps a bad id
// from turning into an out-of-bounds load.
__device__ __forceinline__ int clamp_head(int j, int H) { return j < 0 ? 0 : (j >= H ? H - 1 : j); }

struct TileCoords {
  int qt;            // query tile
  int64_t k0, k1;    // key range [k0, k1)
};

__device__ __forceinline__ TileCoords tile_coords(int n_qtiles, int n_ksplits, int64_t KR, int64_t N) {
  const int64_t total = (int64_t)n_qtiles * n_ksplits;
  const int64_t T = xcd_remap(blockIdx.x, total);
  TileCoords c;
  c.qt = (int)(T % n_qtiles);
  const int64_t ks = T / n_qtiles;
  c.k0 = ks * KR;
  c.k1 = c.k0 + KR < N ? c.k0 + KR : N;
  return c;
}

// -inf for keys [from, to) of queries [qa, qb) (all of them lie after every
// query); query qi's logits row is row orow0 + qi
__device__ __forceinline__ void fill_neg_inf(float* logits, int64_t ld, int64_t orow0, int qa, int qb,
                                             int64_t from, int64_t to, int tid, int nt) {
  if (from >= to) return;
  const float ninf = -__builtin_inff();
  const int64_t span = to - from;
  for (int qi = qa; qi < qb; ++qi) {
    float* row = logits + (orow0 + qi) * ld;
    // from is a multiple of 4 (tile aligned) and ld % 4 == 0
    const int64_t n4 = span / 4;
    for (int64_t e = tid; e < n4; e += nt)
      __builtin_nontemporal_store(f32x4{ninf, ninf, ninf, ninf}, reinterpret_cast<f32x4*>(row + from) + e);
    for (int64_t e = n4 * 4 + tid; e < span; e += nt) row[from + e] = ninf;
  }
}

// Four consecutive scores through a uniform_rsrc descriptor (offsets past its
// size are dropped).  The store takes raw 32-bit patterns.  policy kStream
// marks it non-temporal: full logits rows are far larger than L2 and the
// last-level cache, and streaming them out keeps the key tiles, which every
// query tile re-reads, resident in L2.
__device__ __forceinline__ void store_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4 v, int policy = 0) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  if (policy == kStream)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)byte_off, 0, kStream);
  else
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)byte_off, 0, 0);
}
__device__ __forceinline__ void store_i32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, int v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)byte_off, 0, 0);
}

// Where a scoring pass (k_score_h8, k_score_q8) puts its results.
//  MODE kLogits: logits[row][u] for key u of the scored key sequence (u ks).
//  MODE kCands: no logits; every group of 4 consecutive keys (4c .. 4c+3)
//    holding a score >= thr[row] (a finite threshold, so masked -inf scores
//    never qualify) is appended to the region of that row and of the
//    workgroup's key range, region (row * n_splits + split) of `cap` groups:
//    its 4 scores to gvals, its first key to gkeys.  rcount[row * n_splits +
//    split] receives the number of groups found (more than cap: the region
//    overflowed and holds only the first cap).
//  row_flag != nullptr: only workgroups holding a row with row_flag[row] != 0
//    run (re-scoring of the rows a candidate pass could not settle).
//  slab_tiles > 0 (kLogits): one batch of a re-scoring that runs through a
//    logits slab.  The grid covers slab_tiles consecutive query tiles of the
//    flattened (sequence, query tile) order, from tile slab_first on (tiles
//    past n_flat have no work); query qi of the tile in slot s writes slab row
//    s * slab_tr + (qi - first query of the tile).
struct ScoreOut {
  float* logits;
  int64_t ld;
  const float* thr;
  f32x4* gvals;
  int32_t* gkeys;
  uint32_t* rcount;
  int cap;
  const uint32_t* row_flag;
  int slab_tiles = 0, slab_first = 0, slab_tr = 0, n_flat = 0;
};
constexpr int kLogits = 0;
constexpr int kCands = 1;

constexpr uint32_t kDrop = 0x80000000u;   // a byte offset past every store resource

// The workgroup's sequence b, query tile (qt, QT queries a tile), key range
// [k0, k1), and the logits row base orow0 (query qi of the tile writes row
// orow0 + qi).  valid == false: a slab batch's slot past the last tile (no
// work; uniform over the workgroup).  SLAB: slab batches are possible (only
// logits passes take them).
struct WgTile {
  int b, qt;
  int64_t k0, k1, orow0;
  bool valid;
};
template <int QT, bool SLAB>
__device__ __forceinline__ WgTile wg_tile(const ScoreOut& o, int M, int n_qtiles, int n_ksplits, int64_t KR,
                                          int64_t N) {
  WgTile t;
  if (SLAB && o.slab_tiles > 0) {
    const int64_t T = xcd_remap(blockIdx.x, (int64_t)o.slab_tiles * n_ksplits);
    const int slot = (int)(T % o.slab_tiles);
    const int64_t flat = (int64_t)o.slab_first + slot;
    t.valid = flat < (int64_t)o.n_flat;
    t.b = (int)(flat / n_qtiles);
    t.qt = (int)(flat % n_qtiles);
    t.k0 = (T / o.slab_tiles) * KR;
    t.orow0 = (int64_t)slot * o.slab_tr - (int64_t)t.qt * QT;
  } else {
    const TileCoords c = tile_coords(n_qtiles, n_ksplits, KR, N);
    t.valid = true;
    t.b = blockIdx.y;
    t.qt = c.qt;
    t.k0 = c.k0;
    t.orow0 = (int64_t)t.b * M;
  }
  t.k1 = t.k0 + KR < N ? t.k0 + KR : N;
  return t;
}

// kCands set-up for the lane's output query qo (qoc = min(qo, M - 1)) of a
// workgroup holding rows qa .. qb-1 of sequence row base qrow0: its threshold
// (finite, so masked -inf scores never qualify; +inf past the last query,
// whose scores belong to no row) and the group offset of its region from the
// workgroup's first
__device__ __forceinline__ void cand_lane(const ScoreOut& o, int64_t qrow0, int qa, int qb, int qo, int qoc,
                                          int n_ksplits, float& thr, uint32_t& reg) {
  thr = (qo < qb) ? __builtin_fmaxf(o.thr[qrow0 + qoc], -__FLT_MAX__) : __builtin_inff();
  reg = (uint32_t)(qoc - qa) * (uint32_t)n_ksplits * (uint32_t)o.cap;
}

// kCands store descriptors: regions of rows qa..qb-1 in key range `split`;
// row r's starts (r - qa) * n_ksplits * cap groups after row qa's (fits 31
// bits: checked on the host)
__device__ __forceinline__ void cand_rsrc(const ScoreOut& o, int64_t qrow0, int qa, int qb, int n_ksplits,
                                          int split, __amdgpu_buffer_rsrc_t* r) {
  const int64_t g0 = ((qrow0 + qa) * n_ksplits + split) * (int64_t)o.cap;
  const uint32_t span = (uint32_t)(((int64_t)(qb - 1 - qa) * n_ksplits + 1) * o.cap);
  r[0] = uniform_rsrc(o.gvals + g0, span * 16u);
  r[1] = uniform_rsrc(o.gkeys + g0, span * 4u);
}

// Largest of four scores that are finite or -inf: v_max3 and v_max without the
// NaN-quieting operand canonicalisation that fmaxf costs (two more VALU
// instructions per group).
__device__ __forceinline__ float max4(f32x4 v) {
  float m;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(v[0]), "v"(v[1]), "v"(v[2]));
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(m), "v"(v[3]));
  return m;
}

// kCands epilogue of one tile: the lane holds 4 consecutive scores `v` (keys
// kg .. kg+3) of its output query; the 16 lanes of lane group `gmask` hold one
// query.  A group with a score at or above thr is appended whole; positions
// come from one ballot and the running count `run` (no atomics).  Every lane
// issues both stores (dropped unless the group qualifies and the region has
// room), so a wave's count of stores per tile is fixed.
__device__ __forceinline__ void append_group(const __amdgpu_buffer_rsrc_t* r, f32x4 v, float thr, uint64_t gmask,
                                             uint32_t& run, uint32_t reg, int cap, int kg) {
  const float vmax = max4(v);
  const bool pass = vmax >= thr;
  const uint64_t m = __ballot(pass) & gmask;
  const uint32_t pos = run + lanes_below(m);
  run += (uint32_t)__popcll(m);
  const bool put = pass && pos < (uint32_t)cap;
  // the group's slot, or one whose byte offsets lie past both descriptors:
  // kDrop for the scores; kDrop / 4 for the keys, past their range because a
  // workgroup's regions take fewer than 2^31 bytes of scores (4x their keys)
  const uint32_t slot = put ? reg + pos : (kDrop >> 4);
  store_f32x4(r[0], slot << 4, v);
  store_i32(r[1], slot << 2, kg);
}

}  // namespace misa
