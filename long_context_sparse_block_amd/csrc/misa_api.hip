// extern "C" entry points of libmisa: argument validation on the host, then
// asynchronous launches on the caller's stream.  Nothing here allocates,
// frees or synchronises; the indexer carves its scratch from the caller's
// workspace.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "misa.h"
#include "misa_launch.h"

// Fixed device scratch of misa_indexer_noalloc (callers that cannot allocate:
// HIP graph capture, serving loops, harnesses that forbid allocation).  Every
// GPU the library runs on holds one copy until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: kernels get
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MISA_NOALLOC_SCRATCH_BYTES];

namespace {

using misa::launch_pool;
using misa::launch_route;
using misa::launch_score;
using misa::launch_score_gather;
using misa::launch_topk;

constexpr size_t kAlign = 256;

constexpr int64_t kMaxKeys = (int64_t)1 << 26;
constexpr int64_t kMaxLogitLd = (int64_t)1 << 27;   // 4 rows of ld floats < 2^31 bytes

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

misa_status check_shape(const misa_shape* s) {
  if (s == nullptr) return MISA_ERR_INVALID_ARG;
  if (s->n_seq < 1 || s->q_per_seq < 0 || s->n_keys < 1 || s->q_pos0 < 0) return MISA_ERR_INVALID_ARG;
  if (s->q_pos0 + s->q_per_seq > s->n_keys) return MISA_ERR_INVALID_ARG;
  if (s->n_heads < 1 || s->n_heads > MISA_MAX_HEADS) return MISA_ERR_INVALID_ARG;
  if (s->head_dim != MISA_HEAD_DIM) return MISA_ERR_UNSUPPORTED;
  if (s->block < 1) return MISA_ERR_INVALID_ARG;
  // grid dimensions, 32-bit row counters and 32-bit buffer offsets
  if (s->n_keys > kMaxKeys) return MISA_ERR_UNSUPPORTED;
  if (s->n_seq > 65535) return MISA_ERR_UNSUPPORTED;
  return MISA_OK;
}

misa_status check_keys(const void* k, misa_kdtype kdtype, const float* k_scale) {
  if (kdtype != MISA_K_BF16 && kdtype != MISA_K_FP8_E4M3) return MISA_ERR_INVALID_ARG;
  if (k == nullptr || !aligned16(k)) return MISA_ERR_INVALID_ARG;
  if (kdtype == MISA_K_FP8_E4M3 && k_scale == nullptr) return MISA_ERR_INVALID_ARG;
  return MISA_OK;
}

inline misa_status from_hip(hipError_t e) { return e == hipSuccess ? MISA_OK : MISA_ERR_HIP; }

#define MISA_TRY(expr)                 \
  do {                                 \
    misa_status _st = (expr);          \
    if (_st != MISA_OK) return _st;    \
  } while (0)

// Workspace of the routed scoring + top-k selection (misa_sparse_head_topk,
// and the first selection of misa_indexer), placed from offset `off`.
//
// Fused path: the sample logits and the slab of the flagged-row re-scoring
// share one buffer (the sample is dead once the thresholds are taken).  The
// slab holds slab_tiles query tiles of tr rows; the re-scoring walks the
// tiles in batches of that many.  With room for every tile (the fast plan)
// it is one batch; a smaller workspace (down to the lean plan, whose slab
// is no larger than the sample, and whose candidate regions are sized to the
// expected candidates with a smaller margin) takes more batches, each a
// scoring and a top-k launch that only flagged rows give work.
struct SelectLayout {
  size_t logits, kwide, sample, thr, flag, rcount, gvals, gkeys, topk_ws, end;
  int64_t ld;
  int slab_tiles, tr, n_flat;
  bool widen;   // fp8 keys widened into kwide for the direct-load staging
  misa::FusedPlan fused;
};

// wide_keys: reserve the bf16 copy of fp8 keys that the direct-load staging
// of the bf16-query scoring reads (fp8 keys, bf16 queries).  end_limit: the
// workspace's end (the caller's bytes); the fast plan when it fits, else the
// largest slab that fits, else the lean plan (whose end then lies past
// end_limit: the caller's check refuses the workspace).
SelectLayout select_layout(const misa_shape& s, int h, int k, size_t off, bool wide_keys,
                           size_t end_limit = SIZE_MAX, bool paged = false) {
  SelectLayout L{};
  const int64_t rows = (int64_t)s.n_seq * s.q_per_seq;
  L.ld = (s.n_keys + 3) / 4 * 4;
  L.fused = misa::plan_fused(s, h, k);
  if (!L.fused.ok) {
    L.logits = off;   // full logits
    off += align_up((size_t)rows * (size_t)L.ld * sizeof(float));
    L.topk_ws = off;
    off += align_up(misa::topk_workspace_bytes(s, (int)s.n_keys, k));
    L.end = off;
    return L;
  }
  const int n_qtiles = (s.q_per_seq + 31) / 32;
  L.n_flat = s.n_seq * n_qtiles;
  // a widened copy pays when the keys are read by several query tiles; with
  // one query tile per sequence (decode) each key is read once, so fp8 keys
  // are staged as they are, through registers
  L.widen = wide_keys && n_qtiles > 1 && !paged;   // paged keys are read in place, never copied
  L.tr = std::min(32, (int)s.q_per_seq);
  const size_t tile_bytes = (size_t)L.tr * (size_t)L.ld * sizeof(float);
  auto place = [&](const misa::FusedPlan& p, int64_t slab_tiles) {
    size_t o = off;
    L.fused = p;
    L.kwide = o;   // bf16 copy of fp8 keys
    if (L.widen) o += align_up((size_t)s.n_seq * (size_t)s.n_keys * 128 * sizeof(uint16_t));   // d = 128
    L.thr = o;
    o += align_up((size_t)rows * sizeof(float));
    L.flag = o;
    o += align_up((size_t)rows * sizeof(uint32_t));
    L.rcount = o;
    o += align_up((size_t)rows * p.n_splits * sizeof(uint32_t));
    const size_t groups = (size_t)rows * p.n_splits * (size_t)p.cap_region;
    L.gvals = o;
    o += align_up(groups * 4 * sizeof(float));
    L.gkeys = o;
    o += align_up(groups * sizeof(int32_t));
    L.sample = L.logits = o;   // last: the part a workspace's size decides
    const size_t sample_bytes = (size_t)rows * (size_t)p.ld_sample * sizeof(float);
    L.slab_tiles = (int)std::max<int64_t>(1, slab_tiles);
    o += align_up(std::max(sample_bytes, (size_t)L.slab_tiles * tile_bytes));
    L.end = o;
    return sample_bytes;
  };
  place(L.fused, L.n_flat);
  if (L.end <= end_limit) return L;   // the fast plan: every tile in one batch
  const misa::FusedPlan fast = L.fused;
  for (const misa::FusedPlan& p : {fast, misa::lean_plan(fast, s)}) {
    const size_t sample_bytes = place(p, 1);
    const size_t fixed = L.sample;
    // as many tiles as the workspace holds, at least those the sample's bytes hold
    // (tiles whose bytes fit the room rounded down to the alignment still fit
    // once rounded up)
    const int64_t room = end_limit > fixed ? (int64_t)((end_limit - fixed) / kAlign * kAlign / tile_bytes) : 0;
    const int64_t free_tiles = (int64_t)(sample_bytes / tile_bytes);
    place(p, std::min<int64_t>(L.n_flat, std::max<int64_t>(room, free_tiles)));
    if (L.end <= end_limit) return L;
  }
  return L;   // the lean plan at its least: end_limit is below it
}

// fp8 queries (misa_quantize_q's codes and scales): the selection scores with
// fp8 x fp8 matrix cores instead of bf16 q
struct QuantQ {
  const uint8_t* q8;
  const float* q_scale;
};

// misa_profile_stage: per host thread, the stage whose kernels calls bracket
// with the caller's events (MISA_STAGE_NONE: none)
struct ProfileHook {
  int stage;
  hipEvent_t start, stop;
};
thread_local ProfileHook t_profile = {MISA_STAGE_NONE, nullptr, nullptr};

inline misa_status stage_begin(int stage, hipStream_t st) {
  if (t_profile.stage != stage) return MISA_OK;
  return from_hip(hipEventRecord(t_profile.start, st));
}
inline misa_status stage_end(int stage, hipStream_t st) {
  if (t_profile.stage != stage) return MISA_OK;
  return from_hip(hipEventRecord(t_profile.stop, st));
}

// Routed scoring + exact top-k (see misa_sparse_head_topk); qq != nullptr:
// fp8 queries and fp8 keys (misa_sparse_head_topk_q8).
// pages != nullptr: k / k_scale are page pools read through the block table
// (the layout from select_layout with paged = true).
misa_status run_select(const misa_shape& s, const SelectLayout& L, char* base, const uint16_t* q, const float* w,
                       const void* k, int kdtype, const float* k_scale, const int32_t* heads, int h, int topk,
                       bool sorted, int32_t* idx, float* vals, hipStream_t st, const QuantQ* qq = nullptr,
                       const misa::KeyPages* pages = nullptr) {
  float* logits = reinterpret_cast<float*>(base + L.logits);
  const uint8_t* k8 = static_cast<const uint8_t*>(k);
  if (!L.fused.ok) {
    MISA_TRY(stage_begin(MISA_STAGE_SCORE_LOGITS, st));
    if (pages != nullptr)
      MISA_TRY(from_hip(misa::launch_score_paged(s, q, w, k, kdtype, k_scale, heads, h, logits, L.ld, *pages, st)));
    else if (qq != nullptr)
      MISA_TRY(from_hip(misa::launch_score_q8(s, qq->q8, qq->q_scale, w, k8, k_scale, heads, h, logits, L.ld, st)));
    else
      MISA_TRY(from_hip(launch_score(s, q, w, k, kdtype, k_scale, heads, h, logits, L.ld, st)));
    MISA_TRY(stage_end(MISA_STAGE_SCORE_LOGITS, st));
    MISA_TRY(stage_begin(MISA_STAGE_LOGITS_TOPK, st));
    MISA_TRY(from_hip(launch_topk(s, logits, L.ld, nullptr, (int)s.n_keys, topk, idx, vals, base + L.topk_ws,
                                  L.end - L.topk_ws, st, sorted)));
    return stage_end(MISA_STAGE_LOGITS_TOPK, st);
  }
  const misa::FusedPlan& p = L.fused;
  float* sample = reinterpret_cast<float*>(base + L.sample);
  float* thr = reinterpret_cast<float*>(base + L.thr);
  uint32_t* flag = reinterpret_cast<uint32_t*>(base + L.flag);
  uint32_t* rcount = reinterpret_cast<uint32_t*>(base + L.rcount);
  float* gvals = reinterpret_cast<float*>(base + L.gvals);
  int32_t* gkeys = reinterpret_cast<int32_t*>(base + L.gkeys);
  if (qq != nullptr) {   // (the fp8-query calls take contiguous keys)
    MISA_TRY(stage_begin(MISA_STAGE_SCORE_SAMPLE, st));
    MISA_TRY(from_hip(misa::launch_score_q8_sampled(s, qq->q8, qq->q_scale, w, k8, k_scale, heads, h, p, sample, st)));
    MISA_TRY(stage_end(MISA_STAGE_SCORE_SAMPLE, st));
    MISA_TRY(stage_begin(MISA_STAGE_SAMPLE_THRESHOLD, st));
    MISA_TRY(from_hip(misa::launch_topk_sample_thresh(s, p, sample, thr, flag, st)));
    MISA_TRY(stage_end(MISA_STAGE_SAMPLE_THRESHOLD, st));
    MISA_TRY(stage_begin(MISA_STAGE_SCORE_CANDIDATES, st));
    MISA_TRY(from_hip(misa::launch_score_q8_cands(s, qq->q8, qq->q_scale, w, k8, k_scale, heads, h, p, thr, gvals,
                                                  gkeys, rcount, st)));
    MISA_TRY(stage_end(MISA_STAGE_SCORE_CANDIDATES, st));
    MISA_TRY(stage_begin(MISA_STAGE_REGION_SELECT, st));
    MISA_TRY(
        from_hip(misa::launch_topk_regions(s, p, topk, thr, gvals, gkeys, rcount, flag, idx, vals, sorted, st)));
    MISA_TRY(stage_end(MISA_STAGE_REGION_SELECT, st));
    MISA_TRY(stage_begin(MISA_STAGE_RESCORE, st));
    for (int64_t first = 0; first < L.n_flat; first += L.slab_tiles) {
      const misa::SlabBatch sb{first, (int)std::min<int64_t>(L.slab_tiles, L.n_flat - first), L.tr};
      MISA_TRY(from_hip(
          misa::launch_score_q8(s, qq->q8, qq->q_scale, w, k8, k_scale, heads, h, logits, L.ld, st, flag, &sb)));
      MISA_TRY(from_hip(misa::launch_topk_flagged(s, topk, logits, L.ld, sb, flag, idx, vals, sorted, st)));
    }
    return stage_end(MISA_STAGE_RESCORE, st);
  }
  // the scoring launches stage bf16 keys by direct loads into LDS (fp8 keys
  // widened once), or fp8 keys read once through registers
  const void* kb = k;
  const bool direct = kdtype != MISA_K_FP8_E4M3 || L.widen;
  if (kdtype == MISA_K_FP8_E4M3 && L.widen) {
    uint16_t* kwide = reinterpret_cast<uint16_t*>(base + L.kwide);
    MISA_TRY(from_hip(misa::launch_widen_fp8(s, k, kwide, st)));
    kb = kwide;
  }
  MISA_TRY(stage_begin(MISA_STAGE_SCORE_SAMPLE, st));
  MISA_TRY(from_hip(
      misa::launch_score_sampled(s, q, w, kb, kdtype, k_scale, heads, h, p, sample, st, direct, pages)));
  MISA_TRY(stage_end(MISA_STAGE_SCORE_SAMPLE, st));
  MISA_TRY(stage_begin(MISA_STAGE_SAMPLE_THRESHOLD, st));
  MISA_TRY(from_hip(misa::launch_topk_sample_thresh(s, p, sample, thr, flag, st)));
  MISA_TRY(stage_end(MISA_STAGE_SAMPLE_THRESHOLD, st));
  MISA_TRY(stage_begin(MISA_STAGE_SCORE_CANDIDATES, st));
  MISA_TRY(from_hip(
      misa::launch_score_cands(s, q, w, kb, kdtype, k_scale, heads, h, p, thr, gvals, gkeys, rcount, st, direct,
                               pages)));
  MISA_TRY(stage_end(MISA_STAGE_SCORE_CANDIDATES, st));
  MISA_TRY(stage_begin(MISA_STAGE_REGION_SELECT, st));
  MISA_TRY(from_hip(misa::launch_topk_regions(s, p, topk, thr, gvals, gkeys, rcount, flag, idx, vals, sorted, st)));
  MISA_TRY(stage_end(MISA_STAGE_REGION_SELECT, st));
  // the rows the regions could not settle: whole logits rows through the
  // slab, a batch of query tiles at a time
  MISA_TRY(stage_begin(MISA_STAGE_RESCORE, st));
  for (int64_t first = 0; first < L.n_flat; first += L.slab_tiles) {
    const misa::SlabBatch sb{first, (int)std::min<int64_t>(L.slab_tiles, L.n_flat - first), L.tr};
    MISA_TRY(from_hip(misa::launch_score_rescore(s, q, w, kb, kdtype, k_scale, heads, h, flag, logits, L.ld, sb, st,
                                                 direct, pages)));
    MISA_TRY(from_hip(misa::launch_topk_flagged(s, topk, logits, L.ld, sb, flag, idx, vals, sorted, st)));
  }
  return stage_end(MISA_STAGE_RESCORE, st);
}

struct IndexerLayout {
  size_t pooled, split, tail, heads, rpart, q8, qscale, cand, dlog, ftopk, ftopk_bytes, total;
  int64_t ld_d;
  SelectLayout sel;
};

// own_pool: the pooled keys (and their bf16 hi/lo rows) live in the
// workspace; otherwise in a caller-owned cache (misa_indexer_cached).
// end_limit: the workspace's size (the selection is planned to fit it; see
// select_layout).
IndexerLayout indexer_layout(const misa_shape& s, int kdtype, int h, int topk, int k_prime, bool own_pool = true,
                             bool quant_q = false, size_t end_limit = SIZE_MAX, bool paged = false) {
  IndexerLayout L{};
  const int64_t rows = (int64_t)s.n_seq * s.q_per_seq;
  const int64_t n_full = s.n_keys / s.block;
  L.ld_d = (k_prime + 3) / 4 * 4;
  size_t off = 0;
  if (own_pool) {
    L.pooled = off;
    off += align_up((size_t)s.n_seq * (size_t)(n_full > 0 ? n_full : 1) * MISA_HEAD_DIM * sizeof(float));
    L.split = off;   // bf16 hi and lo rows of the pooled keys, for the router
    off += align_up(2 * (size_t)s.n_seq * (size_t)(n_full > 0 ? n_full : 1) * MISA_HEAD_DIM * sizeof(uint16_t));
  }
  L.tail = off;
  off += align_up((size_t)rows * MISA_HEAD_DIM * sizeof(float));
  L.heads = off;
  off += align_up((size_t)rows * h * sizeof(int32_t));
  const int n_parts = misa::route_parts(s);
  L.rpart = n_parts > 1 ? off : SIZE_MAX;   // the router's partial block sums (few queries)
  if (n_parts > 1) off += align_up((size_t)rows * (n_parts + 1) * s.n_heads * sizeof(float));
  if (quant_q) {   // fp8 queries and their scales (misa_indexer_q8)
    L.q8 = off;
    off += align_up((size_t)rows * s.n_heads * MISA_HEAD_DIM);
    L.qscale = off;
    off += align_up((size_t)rows * s.n_heads * sizeof(float));
  }
  if (k_prime > 0) {
    L.cand = off;
    off += align_up((size_t)rows * k_prime * sizeof(int32_t));
    L.dlog = off;
    off += align_up((size_t)rows * (size_t)L.ld_d * sizeof(float));
    L.ftopk = off;   // the final top-k of MISA-dagger runs over k' candidate columns
    L.ftopk_bytes = align_up(misa::topk_workspace_bytes(s, k_prime, topk));
    off += L.ftopk_bytes;
  }
  // last: the selection takes what the workspace has left
  L.sel = select_layout(s, h, k_prime > 0 ? k_prime : topk, off, kdtype == MISA_K_FP8_E4M3 && !quant_q, end_limit,
                        paged);
  L.total = L.sel.end;
  return L;
}

// pool (from block n_cached on) -> route -> select (-> MISA-dagger re-rank)
// quant_q: the routed scoring runs on fp8 queries (quantised into the
// workspace after routing); routing and the MISA-dagger re-rank keep bf16 q
misa_status run_indexer(const misa_shape& s, const IndexerLayout& L, char* base, const uint16_t* q, const float* w,
                        const void* k, int kdtype, const float* k_scale, int h, int topk, int k_prime,
                        float* pooled, uint16_t* split, int64_t n_cached, int64_t ld_blk, int32_t* idx,
                        float* vals, hipStream_t st, bool quant_q = false, const misa::KeyPages* pages = nullptr) {
  float* tail = reinterpret_cast<float*>(base + L.tail);
  int32_t* heads = reinterpret_cast<int32_t*>(base + L.heads);
  MISA_TRY(stage_begin(MISA_STAGE_POOL, st));
  MISA_TRY(from_hip(launch_pool(s, k, kdtype, k_scale, pooled, tail, split, st, n_cached, ld_blk, pages)));
  MISA_TRY(stage_end(MISA_STAGE_POOL, st));
  float* rpart = L.rpart == SIZE_MAX ? nullptr : reinterpret_cast<float*>(base + L.rpart);
  MISA_TRY(stage_begin(MISA_STAGE_ROUTE, st));
  MISA_TRY(from_hip(launch_route(s, q, w, pooled, split, tail, h, heads, nullptr, st, ld_blk, rpart)));
  MISA_TRY(stage_end(MISA_STAGE_ROUTE, st));
  QuantQ qq{reinterpret_cast<uint8_t*>(base + L.q8), reinterpret_cast<float*>(base + L.qscale)};
  if (quant_q)
    MISA_TRY(from_hip(misa::launch_quant_q(s, q, const_cast<uint8_t*>(qq.q8), const_cast<float*>(qq.q_scale), st)));
  const QuantQ* qp = quant_q ? &qq : nullptr;
  if (k_prime == 0)
    return run_select(s, L.sel, base, q, w, k, kdtype, k_scale, heads, h, topk, true, idx, vals, st, qp, pages);
  // the k' candidates are a set: the re-rank and the final top-k do not depend on their order
  int32_t* cand = reinterpret_cast<int32_t*>(base + L.cand);
  float* dlog = reinterpret_cast<float*>(base + L.dlog);
  MISA_TRY(run_select(s, L.sel, base, q, w, k, kdtype, k_scale, heads, h, k_prime, false, cand, nullptr, st, qp));
  MISA_TRY(stage_begin(MISA_STAGE_RERANK, st));
  MISA_TRY(from_hip(launch_score_gather(s, q, w, k, kdtype, k_scale, cand, k_prime, dlog, L.ld_d, st)));
  MISA_TRY(stage_end(MISA_STAGE_RERANK, st));
  MISA_TRY(stage_begin(MISA_STAGE_FINAL_TOPK, st));
  MISA_TRY(from_hip(launch_topk(s, dlog, L.ld_d, cand, k_prime, topk, idx, vals, base + L.ftopk, L.ftopk_bytes,
                                st)));
  return stage_end(MISA_STAGE_FINAL_TOPK, st);
}

misa_status check_indexer_args(const misa_shape* shape, const uint16_t* q, const float* w, const void* k,
                               misa_kdtype kdtype, const float* k_scale, int32_t h, int32_t topk, int32_t k_prime,
                               const int32_t* idx) {
  MISA_TRY(check_shape(shape));
  MISA_TRY(check_keys(k, kdtype, k_scale));
  // (no queries: the call has nothing to read or write per query)
  if (shape->q_per_seq > 0 && (q == nullptr || !aligned16(q) || w == nullptr || idx == nullptr))
    return MISA_ERR_INVALID_ARG;
  if (h < 1 || h > shape->n_heads) return MISA_ERR_INVALID_ARG;
  if (topk < 1 || topk > MISA_MAX_TOPK) return MISA_ERR_INVALID_ARG;
  if (k_prime != 0 && (k_prime < topk || k_prime > MISA_MAX_TOPK)) return MISA_ERR_INVALID_ARG;
  return MISA_OK;
}

// the caller's pooled-key cache for a shape
misa_status check_cache(const misa_shape* shape, int64_t n_cached, const float* pooled, const uint16_t* split,
                        int64_t cap_blocks) {
  const int64_t n_full = shape->n_keys / shape->block;
  if (cap_blocks < n_full || cap_blocks < 1 || n_cached < 0 || n_cached > n_full) return MISA_ERR_INVALID_ARG;
  if (pooled == nullptr || !aligned16(pooled) || split == nullptr || !aligned16(split)) return MISA_ERR_INVALID_ARG;
  return MISA_OK;
}

// chunk c of a chunked prefill of sequence b: its queries, keys through its last query
misa_shape chunk_shape(const misa_shape& s, int c, int chunk) {
  misa_shape sc = s;
  sc.n_seq = 1;
  sc.q_pos0 = s.q_pos0 + (int64_t)c * chunk;
  sc.q_per_seq = (int32_t)std::min<int64_t>(chunk, s.q_per_seq - (int64_t)c * chunk);
  sc.n_keys = sc.q_pos0 + sc.q_per_seq;
  return sc;
}

// Per device: the address of its copy of `scratch`, looked up on the first
// misa_indexer_noalloc call with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

misa_status scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MISA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MISA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MISA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return MISA_OK;
}

struct PrefillLayout {
  size_t pooled, split, ixws, total;
  int64_t cap;
};

PrefillLayout prefill_layout(const misa_shape& s, int kdtype, int h, int topk, int k_prime, int chunk,
                             size_t end_limit = SIZE_MAX) {
  PrefillLayout L{};
  L.cap = std::max<int64_t>(1, (s.q_pos0 + s.q_per_seq) / s.block);
  size_t off = 0;
  L.pooled = off;
  off += align_up((size_t)L.cap * MISA_HEAD_DIM * sizeof(float));
  L.split = off;
  off += align_up(2 * (size_t)L.cap * MISA_HEAD_DIM * sizeof(uint16_t));
  L.ixws = off;
  size_t most = 0;
  const int n_chunks = (int)((s.q_per_seq + chunk - 1) / chunk);
  const size_t limit = end_limit == SIZE_MAX ? SIZE_MAX : (end_limit > off ? end_limit - off : 0);
  for (int c = 0; c < n_chunks; ++c)
    most = std::max(most,
                    indexer_layout(chunk_shape(s, c, chunk), kdtype, h, topk, k_prime, false, false, limit).total);
  L.total = off + most;
  return L;
}

}  // namespace

extern "C" {

const char* misa_status_str(misa_status s) {
  switch (s) {
    case MISA_OK: return "MISA_OK";
    case MISA_ERR_INVALID_ARG: return "MISA_ERR_INVALID_ARG: invalid argument";
    case MISA_ERR_UNSUPPORTED: return "MISA_ERR_UNSUPPORTED: request outside what is implemented";
    case MISA_ERR_WORKSPACE: return "MISA_ERR_WORKSPACE: workspace missing or too small";
    case MISA_ERR_HIP: return "MISA_ERR_HIP: HIP runtime error";
    case MISA_ERR_SCRATCH:
      return "MISA_ERR_SCRATCH: the request needs more scratch than the library's fixed device buffer "
             "(MISA_NOALLOC_SCRATCH_BYTES) holds";
  }
  return "MISA: unknown status";
}

misa_status misa_pool_keys(const misa_shape* shape, const void* k, misa_kdtype kdtype,
                           const float* k_scale, float* pooled, float* tail, void* stream) {
  MISA_TRY(check_shape(shape));
  MISA_TRY(check_keys(k, kdtype, k_scale));
  const int64_t n_full = shape->n_keys / shape->block;
  if ((n_full > 0 && (pooled == nullptr || !aligned16(pooled))) || tail == nullptr || !aligned16(tail))
    return MISA_ERR_INVALID_ARG;
  if (shape->q_per_seq == 0 && n_full == 0) return MISA_OK;
  return from_hip(launch_pool(*shape, k, kdtype, k_scale, pooled, tail, nullptr, (hipStream_t)stream));
}

misa_status misa_gather_keys_paged(const misa_shape* shape, const void* k_pages, misa_kdtype kdtype,
                                   const float* scale_pages, const int32_t* block_table, int64_t max_pages,
                                   int64_t n_pages, int32_t page_keys, void* k_out, float* scale_out, void* stream) {
  MISA_TRY(check_shape(shape));
  MISA_TRY(check_keys(k_pages, kdtype, scale_pages));
  if (block_table == nullptr || k_out == nullptr || !aligned16(k_out) || page_keys < 1 || n_pages < 1)
    return MISA_ERR_INVALID_ARG;
  if (kdtype == MISA_K_FP8_E4M3 && scale_out == nullptr) return MISA_ERR_INVALID_ARG;
  if (max_pages < (shape->n_keys + page_keys - 1) / page_keys) return MISA_ERR_INVALID_ARG;
  return from_hip(misa::launch_gather_pages(*shape, k_pages, kdtype, scale_pages, block_table, max_pages, n_pages,
                                            page_keys, k_out, scale_out, (hipStream_t)stream));
}

misa_status misa_quantize_q(const misa_shape* shape, const uint16_t* q, uint8_t* q8, float* q_scale,
                            void* stream) {
  MISA_TRY(check_shape(shape));
  if (q == nullptr || !aligned16(q) || q8 == nullptr || !aligned16(q8) || q_scale == nullptr)
    return MISA_ERR_INVALID_ARG;
  return from_hip(misa::launch_quant_q(*shape, q, q8, q_scale, (hipStream_t)stream));
}

misa_status misa_sparse_head_logits_q8(const misa_shape* shape, const uint8_t* q8, const float* q_scale,
                                       const float* w, const void* k, misa_kdtype kdtype, const float* k_scale,
                                       const int32_t* heads, int32_t h, float* logits, int64_t ld,
                                       void* stream) {
  MISA_TRY(check_shape(shape));
  MISA_TRY(check_keys(k, kdtype, k_scale));
  if (kdtype != MISA_K_FP8_E4M3) return MISA_ERR_UNSUPPORTED;   // the fp8 MFMA takes fp8 on both sides
  if (q8 == nullptr || !aligned16(q8) || q_scale == nullptr || w == nullptr || heads == nullptr ||
      logits == nullptr || !aligned16(logits))
    return MISA_ERR_INVALID_ARG;
  if (h < 1 || h > shape->n_heads) return MISA_ERR_INVALID_ARG;
  if (h > 8) return MISA_ERR_UNSUPPORTED;
  if (ld < shape->n_keys || ld % 4 != 0) return MISA_ERR_INVALID_ARG;
  if (ld > kMaxLogitLd) return MISA_ERR_UNSUPPORTED;
  if (shape->q_per_seq == 0) return MISA_OK;
  return from_hip(misa::launch_score_q8(*shape, q8, q_scale, w, static_cast<const uint8_t*>(k), k_scale, heads, h,
                                        logits, ld, (hipStream_t)stream));
}

misa_status dsa_dense_logits_q8(const misa_shape* shape, const uint8_t* q8, const float* q_scale, const float* w,
                                const void* k, misa_kdtype kdtype, const float* k_scale, float* logits, int64_t ld,
                                void* stream) {
  MISA_TRY(check_shape(shape));
  MISA_TRY(check_keys(k, kdtype, k_scale));
  if (kdtype != MISA_K_FP8_E4M3) return MISA_ERR_UNSUPPORTED;   // the fp8 MFMA takes fp8 on both sides
  if (q8 == nullptr || !aligned16(q8) || q_scale == nullptr || w == nullptr || logits == nullptr ||
      !aligned16(logits))
    return MISA_ERR_INVALID_ARG;
  if (ld < shape->n_keys || ld % 4 != 0) return MISA_ERR_INVALID_ARG;
  if (ld > kMaxLogitLd) return MISA_ERR_UNSUPPORTED;
  if (shape->q_per_seq == 0) return MISA_OK;
  return from_hip(misa::launch_dense_q8(*shape, q8, q_scale, w, static_cast<const uint8_t*>(k), k_scale, logits, ld,
                                        (hipStream_t)stream));
}

misa_status misa_route_heads(const misa_shape* shape, const uint16_t* q, const float* w,
                             const float* pooled, const float* tail, int32_t h, int32_t* heads,
                             float* scores, void* stream) {
  MISA_TRY(check_shape(shape));
  if (q == nullptr || !aligned16(q) || w == nullptr || tail == nullptr || !aligned16(tail) ||
      heads == nullptr)
    return MISA_ERR_INVALID_ARG;
  if (shape->n_keys / shape->block > 0 && (pooled == nullptr || !aligned16(pooled)))
    return MISA_ERR_INVALID_ARG;
  if (h < 1 || h > shape->n_heads) return MISA_ERR_INVALID_ARG;
  if (shape->q_per_seq == 0) return MISA_OK;
  return from_hip(launch_route(*shape, q, w, pooled, nullptr, tail, h, heads, scores, (hipStream_t)stream));
}

misa_status misa_sparse_head_logits(const misa_shape* shape, const uint16_t* q, const float* w,
                                    const void* k, misa_kdtype kdtype, const float* k_scale,
                                    const int32_t* heads, int32_t h, float* logits, int64_t ld,
                                    void* stream) {
  MISA_TRY(check_shape(shape));
  MISA_TRY(check_keys(k, kdtype, k_scale));
  if (q == nullptr || !aligned16(q) || w == nullptr || heads == nullptr || logits == nullptr ||
      !aligned16(logits))
    return MISA_ERR_INVALID_ARG;
  if (h < 1 || h > shape->n_heads) return MISA_ERR_INVALID_ARG;
  if (ld < shape->n_keys || (ld & 3) != 0) return MISA_ERR_INVALID_ARG;
  if (ld > kMaxLogitLd) return MISA_ERR_UNSUPPORTED;
  if (shape->q_per_seq == 0) return MISA_OK;
  return from_hip(launch_score(*shape, q, w, k, kdtype, k_scale, heads, h, logits, ld, (hipStream_t)stream));
}

misa_status dsa_dense_logits(const misa_shape* shape, const uint16_t* q, const float* w,
                             const void* k, misa_kdtype kdtype, const float* k_scale,
                             const int32_t* cand, int32_t n_cand, float* logits, int64_t ld,
                             void* stream) {
  MISA_TRY(check_shape(shape));
  MISA_TRY(check_keys(k, kdtype, k_scale));
  if (q == nullptr || !aligned16(q) || w == nullptr || logits == nullptr || !aligned16(logits))
    return MISA_ERR_INVALID_ARG;
  if ((ld & 3) != 0) return MISA_ERR_INVALID_ARG;
  if (cand == nullptr) {
    if (ld < shape->n_keys) return MISA_ERR_INVALID_ARG;
    if (ld > kMaxLogitLd) return MISA_ERR_UNSUPPORTED;
    if (shape->q_per_seq == 0) return MISA_OK;
    return from_hip(launch_score(*shape, q, w, k, kdtype, k_scale, nullptr, shape->n_heads, logits, ld,
                                 (hipStream_t)stream));
  }
  if (n_cand < 1 || ld < n_cand) return MISA_ERR_INVALID_ARG;
  if (shape->q_per_seq == 0) return MISA_OK;
  return from_hip(launch_score_gather(*shape, q, w, k, kdtype, k_scale, cand, n_cand, logits, ld,
                                      (hipStream_t)stream));
}

size_t misa_topk_workspace_bytes(const misa_shape* shape, int32_t n_cols, int32_t k) {
  if (check_shape(shape) != MISA_OK) return 0;
  return misa::topk_workspace_bytes(*shape, n_cols, k);
}

misa_status misa_topk(const misa_shape* shape, const float* logits, int64_t ld, const int32_t* cand,
                      int32_t n_cols, int32_t k, int32_t sorted, int32_t* idx, float* vals, void* ws,
                      size_t ws_bytes, void* stream) {
  MISA_TRY(check_shape(shape));
  if (logits == nullptr || !aligned16(logits) || idx == nullptr) return MISA_ERR_INVALID_ARG;
  if (k < 1 || k > MISA_MAX_TOPK) return MISA_ERR_INVALID_ARG;
  if (n_cols < 1 || ld < n_cols || (ld & 3) != 0) return MISA_ERR_INVALID_ARG;
  if (cand != nullptr && !aligned16(cand)) return MISA_ERR_INVALID_ARG;
  const size_t need = misa::topk_workspace_bytes(*shape, n_cols, k);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return MISA_ERR_WORKSPACE;
  if (shape->q_per_seq == 0) return MISA_OK;
  return from_hip(launch_topk(*shape, logits, ld, cand, n_cols, k, idx, vals, ws, ws_bytes,
                              (hipStream_t)stream, sorted != 0));
}

size_t misa_indexer_workspace_bytes(const misa_shape* shape, misa_kdtype kdtype, int32_t h, int32_t topk,
                                    int32_t k_prime) {
  if (check_shape(shape) != MISA_OK || h < 1 || topk < 1 || k_prime < 0) return 0;
  return indexer_layout(*shape, kdtype, h, topk, k_prime).total;
}

size_t misa_indexer_workspace_min_bytes(const misa_shape* shape, misa_kdtype kdtype, int32_t h, int32_t topk,
                                        int32_t k_prime) {
  if (check_shape(shape) != MISA_OK || h < 1 || topk < 1 || k_prime < 0) return 0;
  return indexer_layout(*shape, kdtype, h, topk, k_prime, true, false, 0).total;
}

misa_status misa_indexer(const misa_shape* shape, const uint16_t* q, const float* w, const void* k,
                         misa_kdtype kdtype, const float* k_scale, int32_t h, int32_t topk,
                         int32_t k_prime, int32_t* idx, float* vals, void* ws, size_t ws_bytes,
                         void* stream) {
  MISA_TRY(check_indexer_args(shape, q, w, k, kdtype, k_scale, h, topk, k_prime, idx));
  const IndexerLayout L = indexer_layout(*shape, kdtype, h, topk, k_prime, true, false, ws_bytes);
  if (ws == nullptr || !aligned16(ws) || ws_bytes < L.total) return MISA_ERR_WORKSPACE;
  if (shape->q_per_seq == 0) return MISA_OK;
  char* base = static_cast<char*>(ws);
  return run_indexer(*shape, L, base, q, w, k, kdtype, k_scale, h, topk, k_prime,
                     reinterpret_cast<float*>(base + L.pooled), reinterpret_cast<uint16_t*>(base + L.split), 0,
                     shape->n_keys / shape->block, idx, vals, (hipStream_t)stream);
}

misa_status misa_indexer_noalloc(const misa_shape* shape, const uint16_t* q, const float* w, const void* k,
                                 misa_kdtype kdtype, const float* k_scale, int32_t h, int32_t topk, int32_t k_prime,
                                 int32_t* idx, float* vals, void* stream) {
  MISA_TRY(check_indexer_args(shape, q, w, k, kdtype, k_scale, h, topk, k_prime, idx));
  const IndexerLayout L = indexer_layout(*shape, kdtype, h, topk, k_prime, true, false, MISA_NOALLOC_SCRATCH_BYTES);
  if (L.total > MISA_NOALLOC_SCRATCH_BYTES) return MISA_ERR_SCRATCH;
  if (shape->q_per_seq == 0) return MISA_OK;
  char* base = nullptr;
  MISA_TRY(scratch_of_current_device(&base));
  // every counter the kernels use is initialised by a kernel of the same call:
  // nothing in the scratch has to start at zero
  return run_indexer(*shape, L, base, q, w, k, kdtype, k_scale, h, topk, k_prime,
                     reinterpret_cast<float*>(base + L.pooled), reinterpret_cast<uint16_t*>(base + L.split), 0,
                     shape->n_keys / shape->block, idx, vals, (hipStream_t)stream);
}

size_t misa_indexer_q8_workspace_bytes(const misa_shape* shape, int32_t h, int32_t topk, int32_t k_prime) {
  if (check_shape(shape) != MISA_OK || h < 1 || topk < 1 || k_prime < 0) return 0;
  return indexer_layout(*shape, MISA_K_FP8_E4M3, h, topk, k_prime, true, true).total;
}

misa_status misa_indexer_q8(const misa_shape* shape, const uint16_t* q, const float* w, const void* k,
                            misa_kdtype kdtype, const float* k_scale, int32_t h, int32_t topk, int32_t k_prime,
                            int32_t* idx, float* vals, void* ws, size_t ws_bytes, void* stream) {
  MISA_TRY(check_indexer_args(shape, q, w, k, kdtype, k_scale, h, topk, k_prime, idx));
  if (kdtype != MISA_K_FP8_E4M3 || h > 8) return MISA_ERR_UNSUPPORTED;   // the fp8 x fp8 routed kernels
  const IndexerLayout L = indexer_layout(*shape, kdtype, h, topk, k_prime, true, true, ws_bytes);
  if (ws == nullptr || !aligned16(ws) || ws_bytes < L.total) return MISA_ERR_WORKSPACE;
  if (shape->q_per_seq == 0) return MISA_OK;
  char* base = static_cast<char*>(ws);
  return run_indexer(*shape, L, base, q, w, k, kdtype, k_scale, h, topk, k_prime,
                     reinterpret_cast<float*>(base + L.pooled), reinterpret_cast<uint16_t*>(base + L.split), 0,
                     shape->n_keys / shape->block, idx, vals, (hipStream_t)stream, true);
}

misa_status misa_pool_keys_cached(const misa_shape* shape, const void* k, misa_kdtype kdtype, const float* k_scale,
                                  int64_t n_cached, float* pooled, uint16_t* pooled_split, int64_t cap_blocks,
                                  float* tail, void* stream) {
  MISA_TRY(check_shape(shape));
  MISA_TRY(check_keys(k, kdtype, k_scale));
  MISA_TRY(check_cache(shape, n_cached, pooled, pooled_split, cap_blocks));
  if (shape->q_per_seq > 0 && (tail == nullptr || !aligned16(tail))) return MISA_ERR_INVALID_ARG;
  return from_hip(launch_pool(*shape, k, kdtype, k_scale, pooled, tail, pooled_split, (hipStream_t)stream,
                              n_cached, cap_blocks));
}

size_t misa_indexer_cached_workspace_bytes(const misa_shape* shape, misa_kdtype kdtype, int32_t h, int32_t topk,
                                           int32_t k_prime) {
  if (check_shape(shape) != MISA_OK || h < 1 || topk < 1 || k_prime < 0) return 0;
  return indexer_layout(*shape, kdtype, h, topk, k_prime, false).total;
}

misa_status misa_indexer_cached(const misa_shape* shape, const uint16_t* q, const float* w, const void* k,
                                misa_kdtype kdtype, const float* k_scale, int32_t h, int32_t topk, int32_t k_prime,
                                int64_t n_cached, float* pooled, uint16_t* pooled_split, int64_t cap_blocks,
                                int32_t* idx, float* vals, void* ws, size_t ws_bytes, void* stream) {
  MISA_TRY(check_indexer_args(shape, q, w, k, kdtype, k_scale, h, topk, k_prime, idx));
  MISA_TRY(check_cache(shape, n_cached, pooled, pooled_split, cap_blocks));
  const IndexerLayout L = indexer_layout(*shape, kdtype, h, topk, k_prime, false, false, ws_bytes);
  if (ws == nullptr || !aligned16(ws) || ws_bytes < L.total) return MISA_ERR_WORKSPACE;
  if (shape->q_per_seq == 0)   // no queries: only bring the cache up to date
    return from_hip(launch_pool(*shape, k, kdtype, k_scale, pooled, nullptr, pooled_split, (hipStream_t)stream,
                                n_cached, cap_blocks));
  return run_indexer(*shape, L, static_cast<char*>(ws), q, w, k, kdtype, k_scale, h, topk, k_prime, pooled,
                     pooled_split, n_cached, cap_blocks, idx, vals, (hipStream_t)stream);
}

size_t misa_indexer_paged_workspace_bytes(const misa_shape* shape, misa_kdtype kdtype, int32_t h, int32_t topk) {
  if (check_shape(shape) != MISA_OK || h < 1 || topk < 1) return 0;
  return indexer_layout(*shape, kdtype, h, topk, 0, false, false, SIZE_MAX, true).total;
}

misa_status misa_indexer_paged(const misa_shape* shape, const uint16_t* q, const float* w, const void* k_pages,
                               misa_kdtype kdtype, const float* scale_pages, const int32_t* block_table,
                               int64_t max_pages, int64_t n_pages, int32_t page_keys, int32_t h, int32_t topk,
                               int64_t n_cached, float* pooled, uint16_t* pooled_split, int64_t cap_blocks,
                               int32_t* idx, float* vals, void* ws, size_t ws_bytes, void* stream) {
  MISA_TRY(check_indexer_args(shape, q, w, k_pages, kdtype, scale_pages, h, topk, 0, idx));
  MISA_TRY(check_cache(shape, n_cached, pooled, pooled_split, cap_blocks));
  if (block_table == nullptr || n_pages < 1 || page_keys < 64 || page_keys % 64 != 0) return MISA_ERR_INVALID_ARG;
  if (max_pages < (shape->n_keys + page_keys - 1) / page_keys) return MISA_ERR_INVALID_ARG;
  if (!aligned16(k_pages)) return MISA_ERR_INVALID_ARG;
  if (h > 8) return MISA_ERR_UNSUPPORTED;   // the routed kernel of h <= 8 reads the pages
  const IndexerLayout L = indexer_layout(*shape, kdtype, h, topk, 0, false, false, ws_bytes, true);
  if (ws == nullptr || !aligned16(ws) || ws_bytes < L.total) return MISA_ERR_WORKSPACE;
  const misa::KeyPages pages{block_table, max_pages, n_pages, page_keys};
  if (shape->q_per_seq == 0)   // no queries: only bring the cache up to date
    return from_hip(launch_pool(*shape, k_pages, kdtype, scale_pages, pooled, nullptr, pooled_split,
                                (hipStream_t)stream, n_cached, cap_blocks, &pages));
  return run_indexer(*shape, L, static_cast<char*>(ws), q, w, k_pages, kdtype, scale_pages, h, topk, 0, pooled,
                     pooled_split, n_cached, cap_blocks, idx, vals, (hipStream_t)stream, false, &pages);
}

size_t misa_prefill_workspace_bytes(const misa_shape* shape, misa_kdtype kdtype, int32_t h, int32_t topk,
                                    int32_t k_prime, int32_t chunk) {
  if (check_shape(shape) != MISA_OK || h < 1 || topk < 1 || k_prime < 0 || chunk < 1) return 0;
  return prefill_layout(*shape, kdtype, h, topk, k_prime, chunk).total;
}

misa_status misa_prefill_chunked(const misa_shape* shape, const uint16_t* q, const float* w, const void* k,
                                 misa_kdtype kdtype, const float* k_scale, int32_t h, int32_t topk, int32_t k_prime,
                                 int32_t chunk, int32_t* idx, float* vals, void* ws, size_t ws_bytes, void* stream) {
  MISA_TRY(check_indexer_args(shape, q, w, k, kdtype, k_scale, h, topk, k_prime, idx));
  if (chunk < 1) return MISA_ERR_INVALID_ARG;
  const PrefillLayout P = prefill_layout(*shape, kdtype, h, topk, k_prime, chunk, ws_bytes);
  if (ws == nullptr || !aligned16(ws) || ws_bytes < P.total) return MISA_ERR_WORKSPACE;
  if (shape->q_per_seq == 0) return MISA_OK;
  char* base = static_cast<char*>(ws);
  float* pooled = reinterpret_cast<float*>(base + P.pooled);
  uint16_t* split = reinterpret_cast<uint16_t*>(base + P.split);
  const int64_t M = shape->q_per_seq, N = shape->n_keys, H = shape->n_heads;
  const size_t key_bytes = kdtype == MISA_K_BF16 ? MISA_HEAD_DIM * 2 : MISA_HEAD_DIM;
  const int n_chunks = (int)((M + chunk - 1) / chunk);
  // sequences one after another on the stream, each through its chunks in
  // order; the pooled-key cache (one sequence's) carries over between chunks
  for (int b = 0; b < shape->n_seq; ++b) {
    int64_t n_cached = 0;
    for (int c = 0; c < n_chunks; ++c) {
      const misa_shape sc = chunk_shape(*shape, c, chunk);
      const int64_t r0 = (int64_t)b * M + (int64_t)c * chunk;   // first query row of the chunk
      const IndexerLayout L = indexer_layout(sc, kdtype, h, topk, k_prime, false, false, ws_bytes - P.ixws);
      MISA_TRY(run_indexer(sc, L, base + P.ixws, q + r0 * H * MISA_HEAD_DIM, w + r0 * H,
                           static_cast<const char*>(k) + (size_t)b * N * key_bytes, kdtype,
                           k_scale != nullptr ? k_scale + (size_t)b * N : nullptr, h, topk, k_prime, pooled, split,
                           n_cached, P.cap, idx + r0 * topk, vals != nullptr ? vals + r0 * topk : nullptr,
                           (hipStream_t)stream));
      n_cached = sc.n_keys / sc.block;
    }
  }
  return MISA_OK;
}

misa_status misa_sparse_head_topk(const misa_shape* shape, const uint16_t* q, const float* w, const void* k,
                                  misa_kdtype kdtype, const float* k_scale, const int32_t* heads, int32_t h,
                                  int32_t topk, int32_t sorted, int32_t* idx, float* vals, void* ws,
                                  size_t ws_bytes, void* stream) {
  MISA_TRY(check_shape(shape));
  MISA_TRY(check_keys(k, kdtype, k_scale));
  if (q == nullptr || !aligned16(q) || w == nullptr || heads == nullptr || idx == nullptr)
    return MISA_ERR_INVALID_ARG;
  if (h < 1 || h > shape->n_heads) return MISA_ERR_INVALID_ARG;
  if (topk < 1 || topk > MISA_MAX_TOPK) return MISA_ERR_INVALID_ARG;
  const SelectLayout L = select_layout(*shape, h, topk, 0, kdtype == MISA_K_FP8_E4M3, ws_bytes);
  if (ws == nullptr || !aligned16(ws) || ws_bytes < L.end) return MISA_ERR_WORKSPACE;
  if (shape->q_per_seq == 0) return MISA_OK;
  return run_select(*shape, L, static_cast<char*>(ws), q, w, k, kdtype, k_scale, heads, h, topk, sorted != 0, idx,
                    vals, (hipStream_t)stream);
}

misa_status misa_sparse_head_topk_q8(const misa_shape* shape, const uint8_t* q8, const float* q_scale,
                                     const float* w, const void* k, misa_kdtype kdtype, const float* k_scale,
                                     const int32_t* heads, int32_t h, int32_t topk, int32_t sorted, int32_t* idx,
                                     float* vals, void* ws, size_t ws_bytes, void* stream) {
  MISA_TRY(check_shape(shape));
  MISA_TRY(check_keys(k, kdtype, k_scale));
  if (kdtype != MISA_K_FP8_E4M3) return MISA_ERR_UNSUPPORTED;   // the fp8 MFMA takes fp8 on both sides
  if (q8 == nullptr || !aligned16(q8) || q_scale == nullptr || w == nullptr || heads == nullptr || idx == nullptr)
    return MISA_ERR_INVALID_ARG;
  if (h < 1 || h > shape->n_heads) return MISA_ERR_INVALID_ARG;
  if (h > 8) return MISA_ERR_UNSUPPORTED;
  if (topk < 1 || topk > MISA_MAX_TOPK) return MISA_ERR_INVALID_ARG;
  // fp8 keys feed the fp8 MFMA as they are
  const SelectLayout L = select_layout(*shape, h, topk, 0, false, ws_bytes);
  if (ws == nullptr || !aligned16(ws) || ws_bytes < L.end) return MISA_ERR_WORKSPACE;
  if (shape->q_per_seq == 0) return MISA_OK;
  const QuantQ qq{q8, q_scale};
  return run_select(*shape, L, static_cast<char*>(ws), nullptr, w, k, kdtype, k_scale, heads, h, topk, sorted != 0,
                    idx, vals, (hipStream_t)stream, &qq);
}

misa_status misa_profile_stage(int32_t stage, void* start_event, void* stop_event) {
  if (stage == MISA_STAGE_NONE) {
    t_profile = ProfileHook{MISA_STAGE_NONE, nullptr, nullptr};
    return MISA_OK;
  }
  if (stage < MISA_STAGE_POOL || stage > MISA_STAGE_LOGITS_TOPK || start_event == nullptr || stop_event == nullptr)
    return MISA_ERR_INVALID_ARG;
  t_profile = ProfileHook{stage, static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  return MISA_OK;
}

size_t misa_sparse_head_topk_workspace_bytes(const misa_shape* shape, misa_kdtype kdtype, int32_t h, int32_t topk) {
  if (check_shape(shape) != MISA_OK || h < 1 || topk < 1) return 0;
  return select_layout(*shape, h, topk, 0, kdtype == MISA_K_FP8_E4M3).end;
}

}  // extern "C"
