// Block mean-pooling of the shared indexer keys, plus the partial-block
// ("tail") mean of every query's prefix.
//
// Method: the prefix is split into blocks of B keys and each block is
// summarised by the mean of its indexer keys (gist.science summary of MISA,
// "Metodologia: MISA" item 1; agents-report summary, method overview).
//
// One workgroup of kPoolWaves waves per (sequence, block m); wave w sums the
// w-th slice of the block's keys.  Lane l owns dims 2l, 2l+1, so a wave reads
// one 256-byte (bf16) or 128-byte (fp8) key row per load, 8 rows in flight.
// The block mean is the slices' sums added in order.  Blocks that hold
// queries walk their slice a second time (an L2 hit) with the running sum
// started at the sum of the slices before it: that running sum is the prefix
// sum the tails of those queries need.  HBM-bound: one pass over K.
//
// Incremental use (chunked prefill, decode): block rows [0, n_cached) of the
// caller's cache already hold the means of the same keys, so only blocks
// from min(n_cached, first query block) on are visited, and of those only
// the complete blocks at or past n_cached are pooled.  Cache rows are
// ld_blk blocks apart per sequence.
//
// PAGED: the keys are read in place from a page pool (KeyPages): a wave looks
// up the page of its slice's first key once and only looks again for a key
// on another page.
#include <algorithm>

#include "misa_common.h"
#include "misa_launch.h"

namespace misa {

constexpr int kPoolWaves = 8;

template <int KDT>
__device__ __forceinline__ f32x2 pool_load(const void* kptr, const float* kscale, int64_t row, int lane) {
  if (KDT == MISA_K_BF16) {
    const uint32_t two = reinterpret_cast<const uint32_t*>(kptr)[row * (kD / 2) + lane];
    return f32x2{bf16_bits_to_f32(two & 0xFFFFu), bf16_bits_to_f32(two >> 16)};
  } else {
    const uint32_t two = reinterpret_cast<const uint16_t*>(kptr)[row * (kD / 2) + lane];
    const float sc = kscale[row];
    const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)two, false);
    return f32x2{f.x * sc, f.y * sc};
  }
}

template <int KDT, bool PAGED = false>
__global__ void __launch_bounds__(kWave * kPoolWaves) k_pool(const void* __restrict__ kptr,
                                                             const float* __restrict__ kscale,
                                                             float* __restrict__ pooled, float* __restrict__ tail,
                                                             uint32_t* __restrict__ split,
                                                             int64_t N, int64_t q_pos0, int M, int B,
                                                             int64_t n_full, int64_t m_first, int64_t n_cached,
                                                             int64_t ld_blk, KeyPages pages) {
  __shared__ f32x2 s_part[kPoolWaves][kWave];
  const int64_t m = m_first + blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t s0 = m * B;
  const int64_t s1 = (s0 + B < N) ? s0 + B : N;
  // only blocks that are complete or hold a query need any work
  const int64_t q_lo = q_pos0, q_hi = q_pos0 + M;  // queries occupy [q_lo, q_hi)
  const bool full = (s0 + B <= N) && m >= n_cached;   // a complete block not pooled yet
  const bool has_query = (s1 > q_lo) && (s0 < q_hi);
  if (!full && !has_query) return;   // uniform over the workgroup
  const int64_t per = (s1 - s0 + kPoolWaves - 1) / kPoolWaves;
  const int64_t w0 = min(s0 + w * per, s1), w1 = min(w0 + per, s1);   // this wave's slice
  // the key row of key t of this sequence (t uniform over the wave)
  int64_t pg_first = 0, pg_row = 0;   // PAGED: first key of the page looked up last, and its row
  if (PAGED) {
    pg_first = w0 - w0 % pages.page_keys;
    pg_row = paged_row(pages, b, pg_first);
  }
  auto row_of = [&](int64_t t) -> int64_t {
    if (!PAGED) return (int64_t)b * N + t;
    if (t < pg_first || t >= pg_first + pages.page_keys) {
      pg_first = t - t % pages.page_keys;
      pg_row = paged_row(pages, b, pg_first);
    }
    return pg_row + (t - pg_first);
  };

  constexpr int U = 8;
  float a0 = 0.f, a1 = 0.f;
  for (int64_t s = w0; s < w1; s += U) {
    f32x2 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = (s + u < w1) ? pool_load<KDT>(kptr, kscale, row_of(s + u), lane) : f32x2{0.f, 0.f};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a0 += v[u].x;
      a1 += v[u].y;
    }
  }
  s_part[w][lane] = f32x2{a0, a1};
  __syncthreads();
  if (full && w == 0) {
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int v = 0; v < kPoolWaves; ++v) {
      t0 += s_part[v][lane].x;
      t1 += s_part[v][lane].y;
    }
    const float p0 = t0 / (float)B, p1 = t1 / (float)B;
    reinterpret_cast<float2*>(pooled)[((int64_t)b * ld_blk + m) * (kD / 2) + lane] = make_float2(p0, p1);
    if (split != nullptr) {   // per sequence: bf16 hi rows, then lo rows (p - hi is exact in fp32)
      const int64_t o = ((int64_t)b * 2 * ld_blk + m) * (kD / 2) + lane;
      const uint32_t h01 = pk_bf16(p0, p1);
      split[o] = h01;
      split[o + ld_blk * (kD / 2)] =
          pk_bf16(p0 - __uint_as_float(h01 << 16), p1 - __uint_as_float(h01 & 0xFFFF0000u));
    }
  }
  if (!has_query) return;
  // tails: running prefix from the sum of the slices before this one
  a0 = 0.f;
  a1 = 0.f;
  for (int v = 0; v < w; ++v) {
    a0 += s_part[v][lane].x;
    a1 += s_part[v][lane].y;
  }
  for (int64_t s = w0; s < w1; s += U) {
    f32x2 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = (s + u < w1) ? pool_load<KDT>(kptr, kscale, row_of(s + u), lane) : f32x2{0.f, 0.f};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t ss = s + u;
      a0 += v[u].x;
      a1 += v[u].y;
      if (ss < w1 && ss >= q_lo && ss < q_hi) {
        // query t = ss: its tail is keys [m*B, t] of this block, empty (zeros)
        // when its prefix ends on the block's end
        const bool empty = ((ss + 1) % B) == 0;
        const float len = (float)(ss - s0 + 1);
        const float2 o = empty ? make_float2(0.f, 0.f) : make_float2(a0 / len, a1 / len);
        reinterpret_cast<float2*>(tail)[((int64_t)b * M + (ss - q_lo)) * (kD / 2) + lane] = o;
      }
    }
  }
}

hipError_t launch_pool(const misa_shape& s, const void* k, int kdtype, const float* k_scale,
                       float* pooled, float* tail, uint16_t* split, hipStream_t st, int64_t n_cached,
                       int64_t ld_blk, const KeyPages* pages) {
  const int64_t N = s.n_keys;
  const int B = s.block;
  const int64_t n_blk_total = (N + B - 1) / B;
  const int64_t n_full = N / B;
  if (ld_blk < 0) ld_blk = n_full;
  // first block with work: the first one not pooled yet, or the first holding a query
  int64_t m_first = s.q_per_seq > 0 ? std::min(n_cached, s.q_pos0 / B) : n_cached;
  if (m_first >= n_blk_total) return hipSuccess;
  dim3 grid((unsigned)(n_blk_total - m_first), (unsigned)s.n_seq);
  const KeyPages pg = pages != nullptr ? *pages : KeyPages{nullptr, 0, 0, 1};
#define MISA_POOL(KDT_, PAGED_)                                                                              \
  hipLaunchKernelGGL((k_pool<KDT_, PAGED_>), grid, dim3(kWave * kPoolWaves), 0, st, k, k_scale, pooled, tail, \
                     reinterpret_cast<uint32_t*>(split), N, s.q_pos0, s.q_per_seq, B, n_full, m_first, n_cached, \
                     ld_blk, pg)
  if (kdtype == MISA_K_BF16) {
    if (pages != nullptr) MISA_POOL(MISA_K_BF16, true);
    else MISA_POOL(MISA_K_BF16, false);
  } else {
    if (pages != nullptr) MISA_POOL(MISA_K_FP8_E4M3, true);
    else MISA_POOL(MISA_K_FP8_E4M3, false);
  }
#undef MISA_POOL
  return hipGetLastError();
}

}  // namespace misa
