// Per-query top-k token selection.
//
// The indexer keeps, for every query, the k prefix tokens with the largest
// scores (abstract of arXiv 2605.07363; gist.science summary of MISA,
// "Metodologia: MISA" item 2).  Order: score descending, equal scores (with
// -0.0 == +0.0) -> lower token id.
//
// Every element has a unique 64-bit composite
//     (order-preserving uint32 of the score) << 32 | ~token_id
// so "larger composite first" is exactly the required order and no two
// elements tie.  The candidate buffer holds raw (token id, score bits) pairs;
// composites are formed only when candidates are ranked.
//
// Design: one workgroup per row, one read of the row from HBM.
//  1. Threshold from a sample: every 32nd 128-byte line of the row (1/32 of it)
//     is loaded and the score key of the k_s-th largest sampled element becomes
//     the threshold, with k_s = 1.5 k (sample size / row length) + 16, so about
//     1.5 k row elements are expected to pass.  (Rows that fit the buffer take
//     every element.)
//  2. Optimistic stream: the row is read in float4s with no workgroup barrier
//     (the next four loads per thread in flight while four are filtered); a float compare against the threshold
//     flags the candidates and a wave appends all of its candidates to the LDS
//     buffer with one atomic (positions from three ballots).
//  3. Only if that overflowed the buffer (then more than CAP >= k elements pass
//     the threshold, so it is a proven bound) or let fewer than k through (then
//     the threshold is dropped), the row is streamed again in lock-step:
//     whenever the buffer could overflow on the next step it is compacted: an
//     MSB-first radix select over the buffered composites finds a threshold
//     with at least k buffered elements at or above it, and the rest is
//     dropped.  At least k elements always sit at or above the threshold, so
//     nothing below it can belong to the top k.
//  4. The radix select cuts the buffer to exactly k candidates.  They are
//     ranked by a counting sort on the top 11 bits of their composite span
//     followed by a rank count inside each (small) bucket, and each is written
//     straight to its output position.  Buckets too large for that fall back
//     to a bitonic sort held in registers.  Candidate lists that only need the
//     set skip the ranking.
// Radix digits start at the highest bit in which the buffered composites
// differ, so the histogram bins spread over the values actually present.
// The result is exact for every input; the sample only decides how much
// buffering and compaction work is done.
#include <algorithm>

#include <type_traits>

#include "misa_common.h"
#include "misa_launch.h"

namespace misa {

constexpr int kDigit = 11;                 // radix digit width
constexpr int kHistBins = 1 << kDigit;
constexpr uint32_t kMaxRankBucket = 64;    // larger buckets -> bitonic fallback
constexpr int kDigitIdx = 12;              // the region select's rank buckets
constexpr int kHistBinsIdx = 1 << kDigitIdx;

__device__ __forceinline__ uint64_t pack_raw(float v, int32_t id) {
  return ((uint64_t)(uint32_t)id << 32) | (uint64_t)__float_as_uint(v);
}
__device__ __forceinline__ uint64_t raw_to_comp(uint64_t r) {
  return ((uint64_t)order_key(__uint_as_float((uint32_t)r)) << 32) | (uint64_t)(~(uint32_t)(r >> 32));
}
__device__ __forceinline__ int32_t comp_id(uint64_t c) { return (int32_t)(~(uint32_t)c); }
__device__ __forceinline__ float comp_val(uint64_t c) { return key_to_float((uint32_t)(c >> 32)); }


__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)x, m), hi = __shfl_xor((uint32_t)(x >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// Workgroup-wide exclusive scan of x; *total receives the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* s_wave, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) s_wave[wave] = v;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int wv = 0; wv < NT / 64; ++wv) {
    const uint32_t t = s_wave[wv];
    if (wv < wave) before += t;
    all += t;
  }
  *total = all;
  __syncthreads();
  return before + v - x;
}

// Workgroup min and max of the composites of buf[0, n).
template <int NT>
__device__ __forceinline__ void block_minmax(const uint64_t* buf, uint32_t n, uint64_t* s_red, uint64_t* mn, uint64_t* mx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t lo = ~0ull, hi = 0;
  for (uint32_t e = threadIdx.x; e < n; e += NT) {
    const uint64_t c = raw_to_comp(buf[e]);
    lo = c < lo ? c : lo;
    hi = c > hi ? c : hi;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t a = shfl_xor_u64(lo, o), b = shfl_xor_u64(hi, o);
    lo = a < lo ? a : lo;
    hi = b > hi ? b : hi;
  }
  if (lane == 0) {
    s_red[2 * wave] = lo;
    s_red[2 * wave + 1] = hi;
  }
  __syncthreads();
  lo = ~0ull;
  hi = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    lo = s_red[2 * w] < lo ? s_red[2 * w] : lo;
    hi = s_red[2 * w + 1] > hi ? s_red[2 * w + 1] : hi;
  }
  __syncthreads();
  *mn = lo;
  *mx = hi;
}

__device__ __forceinline__ int bit_width64(uint64_t x) { return x ? 64 - __clzll((long long)x) : 0; }

// Radix select over the composites of the n raw entries of buf: returns a
// threshold T with need <= #{c >= T} <= limit (the upper bound can only fail
// for duplicate entries); with limit == need it selects exactly the need
// largest.  Requires 1 <= need <= n.  Every thread of the workgroup must call it.
// have_mm: the caller already holds the composites' min and max.
template <int NT>
__device__ __forceinline__ uint64_t select_threshold(const uint64_t* buf, uint32_t n, uint32_t need, uint32_t limit,
                                     uint32_t* s_hist, uint32_t* s_wave, uint32_t* s_sel, uint64_t* s_red,
                                     bool have_mm = false, uint64_t mm_lo = 0, uint64_t mm_hi = 0) {
  const int tid = threadIdx.x;
  constexpr int BPT = kHistBins / NT;  // bins per thread
  uint64_t cmin = mm_lo, cmax = mm_hi;
  if (!have_mm) block_minmax<NT>(buf, n, s_red, &cmin, &cmax);
  const int nb = bit_width64(cmax - cmin);
  if (nb == 0) return cmin;
  // digits over x = c - cmin, from the highest bit in which the composites differ
  int shift = nb > kDigit ? nb - kDigit : 0;
  int width = nb - shift;
  uint64_t prefix = 0, pmask = 0;
  uint32_t above = 0;
  for (;;) {
    const uint32_t dmask = (1u << width) - 1u;
    for (int e = tid; e < kHistBins; e += NT) s_hist[e] = 0;
    __syncthreads();
    for (uint32_t e = tid; e < n; e += NT) {
      const uint64_t x = raw_to_comp(buf[e]) - cmin;
      if ((x & pmask) == prefix) atomicAdd(&s_hist[(uint32_t)(x >> shift) & dmask], 1u);
    }
    __syncthreads();
    // rank order r = 0 is the highest bin; thread owns r in [BPT*tid, BPT*tid+BPT)
    uint32_t hv[BPT], ls = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      hv[u] = s_hist[kHistBins - 1 - (BPT * tid + u)];
      ls += hv[u];
    }
    uint32_t total;
    const uint32_t excl = block_exclusive_scan<NT>(ls, s_wave, &total);
    const uint32_t need_here = need - above;   // >= 1, <= total
    if (excl < need_here && need_here <= excl + ls) {
      uint32_t c = excl;
#pragma unroll
      for (int u = 0; u < BPT; ++u) {
        if (c + hv[u] >= need_here) {
          s_sel[0] = kHistBins - 1 - (BPT * tid + u);
          s_sel[1] = c;
          s_sel[2] = hv[u];
          break;
        }
        c += hv[u];
      }
    }
    __syncthreads();
    const uint32_t bin = s_sel[0], cab = s_sel[1], cnt = s_sel[2];
    __syncthreads();
    above += cab;
    prefix |= (uint64_t)bin << shift;
    pmask |= (uint64_t)dmask << shift;
    if (above + cnt <= limit || shift == 0) return cmin + prefix;
    if (shift >= kDigit) {
      shift -= kDigit;
      width = kDigit;
    } else {
      width = shift;
      shift = 0;
    }
  }
}

// Keep the raw entries whose composite is >= T; returns the new count.  In
// place, in chunks of 4*NT entries: kept entries only move to lower positions,
// and each chunk is fully read (scan barrier) before any of it is written.
template <int NT>
__device__ __forceinline__ uint32_t compact(uint64_t* buf, uint32_t n, uint64_t T, uint32_t* s_wave) {
  const int tid = threadIdx.x;
  uint32_t base = 0;
  for (uint32_t c0 = 0; c0 < n; c0 += 4 * NT) {
    uint64_t v[4];
    bool keep[4];
    uint32_t nk = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t e = c0 + tid + u * NT;
      v[u] = (e < n) ? buf[e] : 0;
      keep[u] = (e < n) && raw_to_comp(v[u]) >= T;
      nk += keep[u];
    }
    uint32_t total;
    uint32_t pos = base + block_exclusive_scan<NT>(nk, s_wave, &total);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (keep[u]) buf[pos++] = v[u];
    base += total;
    __syncthreads();
  }
  return base;
}

// The entries of buf whose composite is >= T written straight to the row's
// outputs (a set: buffer order), at most k of them; returns how many.
template <int NT>
__device__ __forceinline__ uint32_t compact_write(const uint64_t* buf, uint32_t n, uint64_t T, uint32_t* s_wave,
                                                  int64_t row, int k, int32_t* idx_out, float* val_out) {
  const int tid = threadIdx.x;
  uint32_t base = 0;
  for (uint32_t c0 = 0; c0 < n; c0 += 4 * NT) {
    uint64_t c[4];
    bool keep[4];
    uint32_t nk = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t e = c0 + tid + u * NT;
      c[u] = (e < n) ? raw_to_comp(buf[e]) : 0;
      keep[u] = (e < n) && c[u] >= T;
      nk += keep[u];
    }
    uint32_t total;
    uint32_t pos = base + block_exclusive_scan<NT>(nk, s_wave, &total);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (keep[u]) {
        if (pos < (uint32_t)k) {
          idx_out[row * k + pos] = comp_id(c[u]);
          if (val_out) val_out[row * k + pos] = comp_val(c[u]);
        }
        ++pos;
      }
    base += total;
    __syncthreads();   // s_wave is reused by the next chunk's scan
  }
  return base < (uint32_t)k ? base : (uint32_t)k;
}

// the set of the top kk of buf's cnt entries (radix select, then written
// straight out), padded to k
template <int NT>
__device__ __forceinline__ void write_set(const uint64_t* buf, uint32_t cnt, int k, int64_t row, int32_t* idx_out,
                                          float* val_out, uint32_t* s_hist, uint32_t* s_wave, uint32_t* s_sel,
                                          uint64_t* s_red, bool have_mm, uint64_t mm_lo, uint64_t mm_hi) {
  const uint32_t kk = min((uint32_t)k, cnt);
  const uint64_t Tk =
      cnt > kk ? select_threshold<NT>(buf, cnt, kk, kk, s_hist, s_wave, s_sel, s_red, have_mm, mm_lo, mm_hi) : 0;
  const uint32_t w = compact_write<NT>(buf, cnt, Tk, s_wave, row, k, idx_out, val_out);
  for (uint32_t p = w + threadIdx.x; p < (uint32_t)k; p += NT) {
    idx_out[row * k + p] = -1;
    if (val_out) val_out[row * k + p] = -__builtin_inff();
  }
}

// Bitonic sort of the composites of the first cnt raw entries of buf held in
// registers (E consecutive network positions per thread; strides below E are
// in-thread, below 64E lane shuffles, wider ones go through LDS), then the
// top k are written.  Positions past cnt hold 0, below every composite.
template <int NT, int E>
__device__ __forceinline__ void bitonic_write(uint64_t* buf, uint32_t cnt, int k, int64_t row, int32_t* idx_out,
                              float* val_out) {
  const int tid = threadIdx.x;
  uint64_t v[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const uint32_t p = tid * E + j;
    v[j] = (p < cnt) ? raw_to_comp(buf[p]) : 0;
  }
  __syncthreads();
  constexpr uint32_t L = (uint32_t)NT * E;
  for (uint32_t size = 2; size <= L; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      uint64_t o[E];
      if (stride >= 64u * E) {
#pragma unroll
        for (int j = 0; j < E; ++j) buf[tid * E + j] = v[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < E; ++j) o[j] = buf[(tid * E + j) ^ stride];
        __syncthreads();
      } else if (stride >= (uint32_t)E) {
        const int lx = (int)(stride / E);
#pragma unroll
        for (int j = 0; j < E; ++j) o[j] = shfl_xor_u64(v[j], lx);
      } else {
#pragma unroll
        for (int j = 0; j < E; ++j) o[j] = v[j ^ stride];
      }
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const uint32_t p = tid * E + j;
        const bool take_max = ((p & size) == 0) == ((p & stride) == 0);
        const uint64_t hi = v[j] > o[j] ? v[j] : o[j];
        const uint64_t lo = v[j] > o[j] ? o[j] : v[j];
        v[j] = take_max ? hi : lo;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const uint32_t p = tid * E + j;
    if (p < (uint32_t)k && p < cnt) {
      idx_out[row * k + p] = comp_id(v[j]);
      if (val_out) val_out[row * k + p] = comp_val(v[j]);
    }
  }
}

// b0 + the number of composites in sorted[b0, b1) above c: four reads in
// flight at a time (the bucket's entries are read back to back)
__device__ __forceinline__ uint32_t bucket_rank(const uint64_t* sorted, uint32_t b0, uint32_t b1, uint64_t c) {
  uint32_t r = b0, q = b0;
  for (; q + 4 <= b1; q += 4) {
    const uint64_t a0 = sorted[q], a1 = sorted[q + 1], a2 = sorted[q + 2], a3 = sorted[q + 3];
    r += (uint32_t)(a0 > c) + (uint32_t)(a1 > c) + (uint32_t)(a2 > c) + (uint32_t)(a3 > c);
  }
  for (; q < b1; ++q) r += sorted[q] > c;
  return r;
}

// Order the first cnt (<= CAP/2) raw entries of buf by composite and write the
// top k of them, then the padding.  Counting sort into 2048 buckets of the
// composite span (stored in buf[CAP/2 ...]), then each candidate's rank inside
// its bucket by direct comparison (skipped for buckets that start at or past
// rank k).  have_mm: the caller already holds the composites' min and max.
template <int CAP, int NT>
__device__ __forceinline__ void rank_write(uint64_t* buf, uint32_t cnt, int k, int64_t row, int32_t* idx_out, float* val_out,
                           uint32_t* s_hist, uint32_t* s_wave, uint64_t* s_red, bool have_mm = false,
                           uint64_t mm_lo = 0, uint64_t mm_hi = 0) {
  const int tid = threadIdx.x;
  constexpr int BPT = kHistBins / NT;
  uint64_t* sorted = buf + CAP / 2;
  if (cnt > 0) {
    uint64_t cmin = mm_lo, cmax = mm_hi;
    if (!have_mm) block_minmax<NT>(buf, cnt, s_red, &cmin, &cmax);
    const int nb = bit_width64(cmax - cmin);
    const int shift = nb > kDigit ? nb - kDigit : 0;
    for (int e = tid; e < kHistBins; e += NT) s_hist[e] = 0;
    __syncthreads();
    for (uint32_t e = tid; e < cnt; e += NT)
      atomicAdd(&s_hist[(uint32_t)((raw_to_comp(buf[e]) - cmin) >> shift)], 1u);
    __syncthreads();
    // bucket starts, highest bucket first: thread owns buckets 2047-BPT*tid-u
    uint32_t hv[BPT], ls = 0, big = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      hv[u] = s_hist[kHistBins - 1 - (BPT * tid + u)];
      ls += hv[u];
      big = hv[u] > big ? hv[u] : big;
    }
    uint32_t total;
    uint32_t start = block_exclusive_scan<NT>(ls, s_wave, &total);
    const uint32_t n_big = __syncthreads_or(big > kMaxRankBucket);
    if (n_big) {
      constexpr int EMAX = CAP / (2 * NT);
      if (cnt <= (uint32_t)NT) bitonic_write<NT, 1>(buf, cnt, k, row, idx_out, val_out);
      else if (cnt <= 2u * NT) bitonic_write<NT, 2>(buf, cnt, k, row, idx_out, val_out);
      else if (cnt <= 4u * NT || EMAX <= 4) bitonic_write<NT, (EMAX < 4 ? EMAX : 4)>(buf, cnt, k, row, idx_out, val_out);
      else bitonic_write<NT, EMAX>(buf, cnt, k, row, idx_out, val_out);
    } else {
#pragma unroll
      for (int u = 0; u < BPT; ++u) {
        s_hist[kHistBins - 1 - (BPT * tid + u)] = start;   // cursor = bucket start
        start += hv[u];
      }
      __syncthreads();
      for (uint32_t e = tid; e < cnt; e += NT) {
        const uint64_t c = raw_to_comp(buf[e]);
        const uint32_t d = (uint32_t)((c - cmin) >> shift);
        sorted[atomicAdd(&s_hist[d], 1u)] = c;
      }
      __syncthreads();
      // s_hist[d] is now the end of bucket d; bucket d spans [end(d+1), end(d))
      for (uint32_t e = tid; e < cnt; e += NT) {
        const uint64_t c = sorted[e];
        const uint32_t d = (uint32_t)((c - cmin) >> shift);
        const uint32_t b0 = (d + 1 < (uint32_t)kHistBins) ? s_hist[d + 1] : 0;
        if (b0 >= (uint32_t)k) continue;   // every element of the bucket ranks at or past k
        const uint32_t b1 = s_hist[d];
        const uint32_t r = bucket_rank(sorted, b0, b1, c);
        if (r < (uint32_t)k) {
          idx_out[row * k + r] = comp_id(c);
          if (val_out) val_out[row * k + r] = comp_val(c);
        }
      }
    }
  }
  for (uint32_t p = cnt + tid; p < (uint32_t)k; p += NT) {
    idx_out[row * k + p] = -1;
    if (val_out) val_out[row * k + p] = -__builtin_inff();
  }
}

// LDS of one top-k workgroup
template <int CAP, int NT>
struct TopkShared {
  uint64_t buf[CAP];
  uint32_t hist[kHistBins];
  uint32_t wave[NT / 64];
  uint64_t red[2 * (NT / 64)];
  uint32_t sel[3];
  uint32_t count;
};

// LDS of the region select for lists of up to CAP candidates: one copy of
// the candidates, sorted by bucket in place (through registers), so three
// 512-thread workgroups fit per CU.
template <int CAP, int NT>
struct TopkSharedIdx {
  uint64_t buf[CAP];
  uint32_t hist[kHistBinsIdx];
  uint32_t wave[NT / 64];
  uint64_t red[2 * (NT / 64)];
  uint32_t sel[3];
  uint32_t count;
};

// rank_write over all cnt (<= CAP) raw entries of sh.buf, given their min and
// max composite: each thread holds its entries' composites in registers, the
// counting sort scatters them back into sh.buf (now bucket-sorted
// composites), and each candidate's rank inside its bucket is found by
// comparing with the bucket's other entries.  Returns false, writing nothing,
// for a list of more than 8 NT entries with a crowded bucket (the bitonic
// fallback holds 8 entries per thread): the caller flags the row.
template <int CAP, int NT>
__device__ __forceinline__ bool rank_write_idx(TopkSharedIdx<CAP, NT>& sh, uint32_t cnt, int k, int64_t row,
                                               int32_t* idx_out, float* val_out, uint32_t kmin, uint32_t kmax) {
  static_assert(CAP % NT == 0, "whole entries per thread");
  constexpr int EPT = CAP / NT;   // entries per thread
  const int tid = threadIdx.x;
  constexpr int HB = kHistBinsIdx;   // finer buckets than rank_write: fewer in-bucket comparisons
  constexpr int BPT = HB / NT;
  if (cnt > 0) {
    // buckets by the value's order key (the composite's high word), so
    // equal values share a bucket and are ranked there by id
    const int nb = kmax > kmin ? 32 - __clz((int)(kmax - kmin)) : 0;
    const int shift = nb > kDigitIdx ? nb - kDigitIdx : 0;
    auto bucket = [&](uint64_t c) -> uint32_t { return ((uint32_t)(c >> 32) - kmin) >> shift; };
    for (int e = tid; e < HB; e += NT) sh.hist[e] = 0;
    __syncthreads();
    for (uint32_t e = tid; e < cnt; e += NT) atomicAdd(&sh.hist[bucket(raw_to_comp(sh.buf[e]))], 1u);
    __syncthreads();
    // bucket starts, highest bucket first: thread owns buckets HB-1-BPT*tid-u
    uint32_t hv[BPT], ls = 0, big = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      hv[u] = sh.hist[HB - 1 - (BPT * tid + u)];
      ls += hv[u];
      big = hv[u] > big ? hv[u] : big;
    }
    uint32_t total;
    uint32_t start = block_exclusive_scan<NT>(ls, sh.wave, &total);
    const uint32_t n_big = __syncthreads_or(big > kMaxRankBucket);
    if (n_big && cnt > 8u * NT) return false;   // uniform over the workgroup
    if (n_big) {
      if (cnt <= (uint32_t)NT) bitonic_write<NT, 1>(sh.buf, cnt, k, row, idx_out, val_out);
      else if (cnt <= 2u * NT) bitonic_write<NT, 2>(sh.buf, cnt, k, row, idx_out, val_out);
      else if (cnt <= 4u * NT) bitonic_write<NT, 4>(sh.buf, cnt, k, row, idx_out, val_out);
      else bitonic_write<NT, 8>(sh.buf, cnt, k, row, idx_out, val_out);
    } else {
#pragma unroll
      for (int u = 0; u < BPT; ++u) {
        sh.hist[HB - 1 - (BPT * tid + u)] = start;   // cursor = bucket start
        start += hv[u];
      }
      uint64_t mine[EPT];   // this thread's entries, read before any is overwritten
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const uint32_t e = tid + j * NT;
        mine[j] = e < cnt ? raw_to_comp(sh.buf[e]) : 0;
      }
      __syncthreads();   // (the cursors, and every thread's reads of sh.buf)
#pragma unroll
      for (int j = 0; j < EPT; ++j)
        if (tid + j * NT < cnt) sh.buf[atomicAdd(&sh.hist[bucket(mine[j])], 1u)] = mine[j];
      __syncthreads();
      // sh.hist[d] is now the end of bucket d; bucket d spans [end(d+1), end(d))
      for (uint32_t e = tid; e < cnt; e += NT) {
        const uint64_t c = sh.buf[e];
        const uint32_t d = bucket(c);
        const uint32_t b0 = (d + 1 < (uint32_t)HB) ? sh.hist[d + 1] : 0;
        if (b0 >= (uint32_t)k) continue;   // every element of the bucket ranks at or past k
        const uint32_t b1 = sh.hist[d];
        const uint32_t r = bucket_rank(sh.buf, b0, b1, c);
        if (r < (uint32_t)k) {
          idx_out[row * k + r] = comp_id(c);
          if (val_out) val_out[row * k + r] = comp_val(c);
        }
      }
    }
  }
  for (uint32_t p = cnt + tid; p < (uint32_t)k; p += NT) {
    idx_out[row * k + p] = -1;
    if (val_out) val_out[row * k + p] = -__builtin_inff();
  }
  return true;
}

template <int CAP, int NT>
__device__ __forceinline__ void topk_row(TopkShared<CAP, NT>& sh, int i, int b, const float* __restrict__ logits,
                                         int64_t ld, const int32_t* __restrict__ cand, int n_cols, int k,
                                         int64_t q_pos0, int M, int32_t* __restrict__ idx_out,
                                         float* __restrict__ val_out, int sorted,
                                         const float* __restrict__ lrow_in = nullptr) {
  constexpr int VPT = 2;                  // float4s per thread per lock-step (robust) step
  constexpr int STEP = 4 * VPT * NT;      // elements per lock-step step
  static_assert(CAP / 2 >= STEP, "a lock-step step must fit the free half of the buffer");
  uint64_t* s_buf = sh.buf;
  uint32_t* s_hist = sh.hist;
  uint32_t* s_wave = sh.wave;
  uint64_t* s_red = sh.red;
  uint32_t* s_sel = sh.sel;
  uint32_t& s_count = sh.count;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t row = (int64_t)b * M + i;
  const int64_t t = q_pos0 + i;
  const int n = cand ? n_cols : (int)min((int64_t)n_cols, t + 1);
  const float* lrow = lrow_in != nullptr ? lrow_in : logits + row * ld;   // the row's logits
  const int32_t* crow = cand ? cand + row * (int64_t)n_cols : nullptr;
  // float4 / int4 loads need 16-byte aligned rows: ld % 4 == 0 always, and the
  // candidate rows when n_cols % 4 == 0; otherwise every element is read singly
  const bool vec = (crow == nullptr || (n_cols & 3) == 0);

  // the 4 elements starting at column e0 (id -1 = no candidate)
  auto fetch4 = [&](int e0, float4& v, int4& id) {
    if (vec && e0 + 3 < n) {
      const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(lrow) + (e0 >> 2));
      v = make_float4(x[0], x[1], x[2], x[3]);
      if (crow) id = reinterpret_cast<const int4*>(crow)[e0 >> 2];
      else id = make_int4(e0, e0 + 1, e0 + 2, e0 + 3);
    } else {
      float vv[4];
      int ii[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u;
        vv[u] = (e < n) ? lrow[e] : 0.f;
        ii[u] = (e < n) ? (crow ? crow[e] : e) : -1;
      }
      v = make_float4(vv[0], vv[1], vv[2], vv[3]);
      id = make_int4(ii[0], ii[1], ii[2], ii[3]);
    }
  };
  // append the flagged elements of the wave's float4s with one LDS atomic;
  // entries past CAP are counted but dropped
  auto append4 = [&](const float4& v, const int4& id, bool f0, bool f1, bool f2, bool f3) {
    const uint32_t c = (uint32_t)f0 + f1 + f2 + f3;
    const uint64_t m0 = __ballot(c & 1u), m1 = __ballot(c & 2u), m2 = __ballot(c & 4u);
    if ((m0 | m1 | m2) == 0) return;
    uint32_t pos = lanes_below(m0) + 2 * lanes_below(m1) + 4 * lanes_below(m2);
    uint32_t base = 0;
    if (lane == __ffsll((unsigned long long)__ballot(1)) - 1)   // first active lane
      base = atomicAdd(&s_count, (uint32_t)(__popcll(m0) + 2 * __popcll(m1) + 4 * __popcll(m2)));
    pos += __builtin_amdgcn_readfirstlane(base);
    if (f0) { if (pos < (uint32_t)CAP) s_buf[pos] = pack_raw(v.x, id.x); ++pos; }
    if (f1) { if (pos < (uint32_t)CAP) s_buf[pos] = pack_raw(v.y, id.y); ++pos; }
    if (f2) { if (pos < (uint32_t)CAP) s_buf[pos] = pack_raw(v.z, id.z); ++pos; }
    if (f3) { if (pos < (uint32_t)CAP) s_buf[pos] = pack_raw(v.w, id.w); }
  };
  auto append_ge = [&](const float4& v, const int4& id, uint64_t T) {   // exact composite test
    append4(v, id, id.x >= 0 && raw_to_comp(pack_raw(v.x, id.x)) >= T,
            id.y >= 0 && raw_to_comp(pack_raw(v.y, id.y)) >= T,
            id.z >= 0 && raw_to_comp(pack_raw(v.z, id.z)) >= T,
            id.w >= 0 && raw_to_comp(pack_raw(v.w, id.w)) >= T);
  };

  if (tid == 0) s_count = 0;
  __syncthreads();

  // 1. threshold key from a sample of every 32nd 128-byte line; rows that fit
  //    the buffer keep T0 = 0 (every element passes)
  uint64_t T0 = 0;
  const int n_samp = (n / 32) / 32;   // sampled lines
  if (n > CAP && n_samp > 0) {
    for (int e0 = 0; e0 < n_samp * 8; e0 += NT) {   // 8 float4 per line; every lane takes part
      const int e = e0 + tid;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      int4 id = make_int4(-1, -1, -1, -1);
      if (e < n_samp * 8) fetch4((e / 8) * 32 * 32 + (e % 8) * 4, v, id);
      append4(v, id, id.x >= 0, id.y >= 0, id.z >= 0, id.w >= 0);
    }
    __syncthreads();
    const uint32_t ns = min(s_count, (uint32_t)CAP);
    const uint64_t ks = (uint64_t)3 * k * ns / (2 * (uint64_t)n) + 16;
    if (ks < ns) {
      // keep only the score-key part: passing then depends on the score alone
      T0 = select_threshold<NT>(s_buf, ns, (uint32_t)ks, (uint32_t)ks, s_hist, s_wave, s_sel, s_red) &
           0xFFFFFFFF00000000ull;
    }
    if (tid == 0) s_count = 0;
    __syncthreads();
  }

  // 2. optimistic stream: v >= tf  <=>  composite >= T0 (T0 has a zero id part)
  {
    float tf = -__builtin_inff();
    if (T0 != 0) {
      tf = key_to_float((uint32_t)(T0 >> 32));
      if (tf != tf) tf = -__builtin_inff();   // a key prefix below every finite value
    }
    constexpr int U = 4;
    constexpr int SPAN = 4 * U * NT;
    float4 nv[U];
    int4 nid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) fetch4(4 * (tid + u * NT), nv[u], nid[u]);
    for (int base = 0; base < n; base += SPAN) {
      float4 v[U];
      int4 id[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        v[u] = nv[u];
        id[u] = nid[u];
      }
      if (base + SPAN < n) {   // next loads in flight while this batch is filtered
#pragma unroll
        for (int u = 0; u < U; ++u) fetch4(base + SPAN + 4 * (tid + u * NT), nv[u], nid[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        append4(v[u], id[u], id[u].x >= 0 && v[u].x >= tf, id[u].y >= 0 && v[u].y >= tf,
                id[u].z >= 0 && v[u].z >= tf, id[u].w >= 0 && v[u].w >= tf);
    }
  }
  __syncthreads();
  const uint32_t got = s_count;
  __syncthreads();

  // 3. lock-step stream with compaction when the optimistic pass overflowed
  //    (T0 is then a proven bound) or let fewer than k through while filtering
  if (got > (uint32_t)CAP || (got < (uint32_t)k && T0 != 0)) {
    uint64_t T = (got > (uint32_t)CAP) ? T0 : 0;
    if (tid == 0) s_count = 0;
    __syncthreads();
    const int n_steps = (n + STEP - 1) / STEP;
    float4 nv[VPT];
    int4 nid[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) fetch4(4 * (tid + u * NT), nv[u], nid[u]);
    for (int s = 0; s < n_steps; ++s) {
      float4 v[VPT];
      int4 id[VPT];
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        v[u] = nv[u];
        id[u] = nid[u];
      }
      if (s + 1 < n_steps) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) fetch4((s + 1) * STEP + 4 * (tid + u * NT), nv[u], nid[u]);
      }
#pragma unroll
      for (int u = 0; u < VPT; ++u) append_ge(v[u], id[u], T);
      __syncthreads();
      const uint32_t cnt = min(s_count, (uint32_t)CAP);
      if (cnt > (uint32_t)(CAP - STEP) && s + 1 < n_steps) {
        // make room: a threshold with at least k buffered elements above it
        T = select_threshold<NT>(s_buf, cnt, min((uint32_t)k, cnt), (uint32_t)((k + CAP / 2) / 2), s_hist,
                                 s_wave, s_sel, s_red);
        const uint32_t nc = compact<NT>(s_buf, cnt, T, s_wave);
        if (tid == 0) s_count = nc;
        __syncthreads();
      }
    }
  }

  // 4. exactly the top min(k, count)
  uint32_t cnt = min(s_count, (uint32_t)CAP);
  __syncthreads();
  const uint32_t kk = min((uint32_t)k, cnt);
  if (cnt > kk) {
    const uint64_t Tk = select_threshold<NT>(s_buf, cnt, kk, kk, s_hist, s_wave, s_sel, s_red);
    cnt = compact<NT>(s_buf, cnt, Tk, s_wave);
  }
  cnt = min(cnt, (uint32_t)(CAP / 2));   // more only with duplicate candidate ids
  if (!sorted) {   // the set only (any order): candidate lists
    for (int e = tid; e < k; e += NT) {
      int32_t id = -1;
      float v = -__builtin_inff();
      if ((uint32_t)e < cnt) {
        const uint64_t c = raw_to_comp(s_buf[e]);
        id = comp_id(c);
        v = comp_val(c);
      }
      idx_out[row * k + e] = id;
      if (val_out) val_out[row * k + e] = v;
    }
    return;
  }
  rank_write<CAP, NT>(s_buf, cnt, k, row, idx_out, val_out, s_hist, s_wave, s_red);
}

template <int CAP, int NT>
__global__ void __launch_bounds__(NT, 2) k_topk(const float* __restrict__ logits, int64_t ld,
                                                const int32_t* __restrict__ cand, int n_cols, int k,
                                                int64_t q_pos0, int M, int32_t* __restrict__ idx_out,
                                                float* __restrict__ val_out, int sorted) {
  __shared__ TopkShared<CAP, NT> sh;
  topk_row<CAP, NT>(sh, blockIdx.x, blockIdx.y, logits, ld, cand, n_cols, k, q_pos0, M, idx_out, val_out, sorted);
}

// ---------------------------------------------------------------------------
// Long rows: the threshold, the stream and the selection run as three kernels
// so that the stream fills the whole chip with row chunks while the select and
// rank work, which reads no logits, runs afterwards on short candidate lists.
// ---------------------------------------------------------------------------
constexpr int kSplitMinCols = 16384;   // rows at least this long take the split path
// k_topk_fused (one workgroup per row) when there are at least this many
// rows; fewer rows (decode) fill the chip better split into chunks
constexpr int64_t kFusedMinRows = 512;
constexpr int kChunkMax = 65536;       // elements per filter workgroup, at most (256 KB of logits)
constexpr int kChunkCap = 4096;        // candidates a filter workgroup (4 waves) can hold

// candidates kept per row (the LDS buffer of the select kernel)
inline int list_cap(int k) { return k <= 4096 ? 8192 : 16384; }

struct SplitWs {
  float* thr;
  uint32_t* count;
  uint32_t* flag;
  uint64_t* list;
  int capg;
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static size_t split_ws_bytes(int64_t rows, int k) {
  return 3 * align256((size_t)rows * 4) + align256((size_t)rows * list_cap(k) * sizeof(uint64_t));
}

static SplitWs split_ws(void* ws, int64_t rows, int k) {
  char* p = static_cast<char*>(ws);
  SplitWs w;
  w.capg = list_cap(k);
  w.thr = reinterpret_cast<float*>(p);
  p += align256((size_t)rows * 4);
  w.count = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)rows * 4);
  w.flag = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)rows * 4);
  w.list = reinterpret_cast<uint64_t*>(p);
  return w;
}

// Per-row threshold from a sample of whole 128-byte lines: 128 lines of 32
// scores at a regular stride over the row (4096 scores, 1/32 of a
// 131072-score row; a line costs one memory transaction whether one of its
// scores is read or all 32, so sampling single 16-byte pieces fetched 8 times
// the bytes it used).  A line's scores are neighbours and may be correlated
// (a block of related keys), so each line counts at most 16 of its scores: a
// cluster of large scores cannot take more than a bounded share of the
// sample.  The threshold is the lower edge of the 16-bit order-key bucket
// above which the capped count reaches k_s = target * 4096 / n + 2, so that
// about `target` row elements are expected at or above it; rows too short
// for the sample keep every element (-inf).  Computed by one wave: lane l
// reads lines 2l and 2l + 1.
__device__ __forceinline__ float row_threshold(const float* __restrict__ lrow, int n, int target) {
  constexpr int kLines = 128, kCap = 16;  // sampled lines, scores a line can count
  constexpr int ns = kLines * 32;         // 4096 sampled scores
  const int lane = threadIdx.x & 63;
  const uint64_t ks = (uint64_t)target * ns / (uint64_t)max(n, 1) + 2;
  if (!(n > target && n >= 2 * ns && ks < (uint64_t)(kLines * kCap))) return -__builtin_inff();
  const uint32_t stride = ((uint32_t)n / 32u) / (uint32_t)kLines;   // lines apart, >= 2 (n >= 2 ns)
  uint32_t key[2][32];
#pragma unroll
  for (int ln = 0; ln < 2; ++ln) {
    const f32x4* src = reinterpret_cast<const f32x4*>(lrow + (size_t)((2 * lane + ln) * stride) * 32u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4 v = src[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) key[ln][4 * j + e] = order_key(v[e]);
    }
  }
  // bits decided from the top: capped per-line counts, one wave sum per bit
  uint32_t T = 0;
  for (int bit = 31; bit >= 16; --bit) {
    const uint32_t c = T | (1u << bit);
    uint32_t cl = 0;
#pragma unroll
    for (int ln = 0; ln < 2; ++ln) {
      uint32_t cnt = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) cnt += (key[ln][j] >= c) ? 1u : 0u;
      cl += min(cnt, (uint32_t)kCap);
    }
    if (__reduce_add_sync(~0ull, cl) >= (uint32_t)ks) T = c;
  }
  const float tf = key_to_float(T);
  return (tf != tf) ? -__builtin_inff() : tf;
}

// One wave per row: the row's threshold (row_threshold), and the row's list
// count and overflow flag reset.
constexpr int kThreshWaves = 4;
__global__ void __launch_bounds__(64 * kThreshWaves) k_topk_thresh(const float* __restrict__ logits, int64_t ld,
                                                                   int n_cols, int target, int64_t q_pos0, int M,
                                                                   int64_t rows, float* __restrict__ thr,
                                                                   uint32_t* __restrict__ count,
                                                                   uint32_t* __restrict__ flag) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kThreshWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int i = (int)(row % M);
  const int n = (int)min((int64_t)n_cols, q_pos0 + i + 1);
  const float tf = row_threshold(logits + row * ld, n, target);
  if (lane == 0) {
    thr[row] = tf;
    count[row] = 0;
    flag[row] = 0;
  }
}

// Stream one chunk of a row and append every element >= the row's threshold
// to the row's candidate list.  Each wave filters its own share of the chunk
// into its own LDS region, its running count in a scalar register (positions
// from ballots of the lanes' per-batch counts, no atomics), and then appends
// the region to the row's list with one global atomic.  A wave region that
// fills up, or a list that would pass its capacity, flags the row for the
// exact whole-row path.
constexpr int kWaveCap = 1024;   // candidates a wave can hold
template <int NT>
__global__ void __launch_bounds__(NT) k_topk_filter(const float* __restrict__ logits, int64_t ld, int n_cols,
                                                    int chunk, int n_chunks, int64_t q_pos0, int M,
                                                    const float* __restrict__ thr, uint32_t* __restrict__ count,
                                                    uint32_t* __restrict__ flag, uint64_t* __restrict__ list,
                                                    int capg) {
  constexpr int NW = NT / 64;
  constexpr int U = 4;                      // float4s per lane per batch
  __shared__ uint64_t s_c[NW][kWaveCap];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = blockIdx.x / n_chunks, ch = blockIdx.x % n_chunks, b = blockIdx.y;
  const int64_t row = (int64_t)b * M + i;
  const int n = (int)min((int64_t)n_cols, q_pos0 + i + 1);
  const int c0 = ch * chunk;
  if (c0 >= n) return;
  const int c1 = min(n, c0 + chunk);
  const float* lrow = logits + row * ld;
  const float tf = thr[row];
  uint64_t* reg = s_c[wv];

  // float4s of the chunk (rows are 16-byte aligned: ld % 4 == 0, c0 % 4 == 0),
  // interleaved across the waves, non-temporal (each is read once), the next
  // batch always in flight (index clamped to the chunk: no branch)
  const f32x4* p4 = reinterpret_cast<const f32x4*>(lrow + c0);
  const int n4 = (c1 - c0 + 3) / 4;
  uint32_t run = 0;                         // candidates found by this wave (uniform)
  f32x4 nv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) nv[u] = __builtin_nontemporal_load(p4 + min(tid + u * NT, n4 - 1));
  for (int base4 = 0; base4 < n4; base4 += U * NT) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = nv[u];
#pragma unroll
    for (int u = 0; u < U; ++u)
      nv[u] = __builtin_nontemporal_load(p4 + min(base4 + U * NT + tid + u * NT, n4 - 1));
    uint32_t fl = 0;   // bit 4u+j: element j of float4 u passes
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e0 = c0 + 4 * (base4 + tid + u * NT);
#pragma unroll
      for (int j = 0; j < 4; ++j) fl |= (uint32_t)(e0 + j < c1 && v[u][j] >= tf) << (4 * u + j);
    }
    const uint32_t cnt = __popc(fl);           // 0..16
    const uint64_t m0 = __ballot(cnt & 1u), m1 = __ballot(cnt & 2u), m2 = __ballot(cnt & 4u),
                   m3 = __ballot(cnt & 8u), m4 = __ballot(cnt & 16u);
    if ((m0 | m1 | m2 | m3 | m4) == 0) continue;
    uint32_t pos = run + lanes_below(m0) + 2 * lanes_below(m1) + 4 * lanes_below(m2) + 8 * lanes_below(m3) +
                   16 * lanes_below(m4);
    run += __popcll(m0) + 2 * __popcll(m1) + 4 * __popcll(m2) + 8 * __popcll(m3) + 16 * __popcll(m4);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e0 = c0 + 4 * (base4 + tid + u * NT);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (fl & (1u << (4 * u + j))) {
          if (pos < (uint32_t)kWaveCap) reg[pos] = pack_raw(v[u][j], e0 + j);
          ++pos;
        }
    }
  }
  if (run == 0) return;
  if (run > (uint32_t)kWaveCap) {
    if (lane == 0) flag[row] = 1;
    return;
  }
  uint32_t base = 0;
  if (lane == 0) base = atomicAdd(&count[row], run);
  base = __builtin_amdgcn_readfirstlane(base);
  if (base + run > (uint32_t)capg) {
    if (lane == 0) flag[row] = 1;
    return;
  }
  uint64_t* dst = list + row * (int64_t)capg + base;
  for (uint32_t e = lane; e < run; e += 64) dst[e] = reg[e];
}

// Exact top-k (sorted, or the set in no order) of the cnt candidates held in
// sh.buf, written to the row's outputs.
template <int CAP, int NT>
__device__ __forceinline__ void finish_list(TopkShared<CAP, NT>& sh, uint32_t cnt, int k, int64_t row,
                                            int32_t* __restrict__ idx_out, float* __restrict__ val_out, int sorted,
                                            bool have_mm = false, uint64_t mm_lo = 0, uint64_t mm_hi = 0) {
  const int tid = threadIdx.x;
  if (sorted && cnt <= (uint32_t)(CAP / 2)) {   // rank every candidate; ranks >= k are not written
    rank_write<CAP, NT>(sh.buf, cnt, k, row, idx_out, val_out, sh.hist, sh.wave, sh.red, have_mm, mm_lo, mm_hi);
    return;
  }
  if (!sorted) {
    write_set<NT>(sh.buf, cnt, k, row, idx_out, val_out, sh.hist, sh.wave, sh.sel, sh.red, have_mm, mm_lo, mm_hi);
    return;
  }
  const uint32_t kk = min((uint32_t)k, cnt);
  if (cnt > kk) {
    const uint64_t Tk = select_threshold<NT>(sh.buf, cnt, kk, kk, sh.hist, sh.wave, sh.sel, sh.red, have_mm, mm_lo,
                                             mm_hi);
    cnt = compact<NT>(sh.buf, cnt, Tk, sh.wave);
  }
  cnt = min(cnt, (uint32_t)(CAP / 2));
  rank_write<CAP, NT>(sh.buf, cnt, k, row, idx_out, val_out, sh.hist, sh.wave, sh.red);
}

// finish_list for the compact LDS: sorted output ranks every candidate;
// the set alone is an exact select to k and a compaction.
// Returns false when the list could not be ranked (see rank_write_idx).
template <int CAP, int NT>
__device__ __forceinline__ bool finish_list_idx(TopkSharedIdx<CAP, NT>& sh, uint32_t cnt, int k, int64_t row,
                                                int32_t* __restrict__ idx_out, float* __restrict__ val_out,
                                                int sorted, uint32_t kmin, uint32_t kmax) {
  if (sorted) return rank_write_idx<CAP, NT>(sh, cnt, k, row, idx_out, val_out, kmin, kmax);
  write_set<NT>(sh.buf, cnt, k, row, idx_out, val_out, sh.hist, sh.wave, sh.sel, sh.red, false, 0, 0);
  return true;
}

// Exact top-k of a row's candidate list (every element at or above the row's
// threshold).  A row whose list overflowed or came up short of k is done by
// the whole-row path instead, in the same workgroup, so the result is exact
// for every input.
template <int CAP, int NT>
__global__ void __launch_bounds__(NT, 2) k_topk_list(const float* __restrict__ logits, int64_t ld, int n_cols,
                                                     int k, int64_t q_pos0, int M, int32_t* __restrict__ idx_out,
                                                     float* __restrict__ val_out, int sorted,
                                                     const uint64_t* __restrict__ list,
                                                     const uint32_t* __restrict__ count,
                                                     const uint32_t* __restrict__ flag, int capg) {
  __shared__ TopkShared<CAP, NT> sh;
  const int tid = threadIdx.x;
  const int i = blockIdx.x, b = blockIdx.y;
  const int64_t row = (int64_t)b * M + i;
  const int n = (int)min((int64_t)n_cols, q_pos0 + i + 1);
  const uint32_t c = count[row];
  if (flag[row] != 0 || c < (uint32_t)min(k, n) || c > (uint32_t)min(capg, CAP)) {
    topk_row<CAP, NT>(sh, i, b, logits, ld, nullptr, n_cols, k, q_pos0, M, idx_out, val_out, sorted);
    return;
  }
  // the list into LDS: every thread's loads issued together (c >= 1 here)
  const uint64_t* src = list + row * (int64_t)capg;
  constexpr int EPT = CAP / NT;
  uint64_t v[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) v[j] = src[min((uint32_t)(tid + j * NT), c - 1)];
#pragma unroll
  for (int j = 0; j < EPT; ++j)
    if ((uint32_t)(tid + j * NT) < c) sh.buf[tid + j * NT] = v[j];
  __syncthreads();
  finish_list<CAP, NT>(sh, c, k, row, idx_out, val_out, sorted);
}

// The long-row top-k (k <= 4096) in one kernel, one workgroup per row: wave 0
// takes the row's threshold from its sampled lines (row_threshold) while the
// other waves' first loads are in flight; the row is streamed once, each wave
// keeping every element at or above the threshold in its own LDS region (the
// float4s interleaved over the waves, positions from ballots of the lanes'
// per-batch counts); the regions are gathered into one list and the exact
// top-k is selected from it (finish_list).  A row whose regions overflow, or
// whose candidates come short of k, takes the whole-row path in the same
// workgroup, so the result is exact for every input.  The list never leaves
// LDS, and the select of one row overlaps the streaming of the other
// workgroup on the CU.
template <int CAP, int NT>
__global__ void __launch_bounds__(NT, 2) k_topk_fused(const float* __restrict__ logits, int64_t ld, int n_cols,
                                                      int k, int target, int64_t q_pos0, int M,
                                                      int32_t* __restrict__ idx_out, float* __restrict__ val_out,
                                                      int sorted) {
  constexpr int NW = NT / 64;
  constexpr int WCAP = CAP / NW;   // candidates a wave's region holds
  constexpr int U = 4;             // float4s per lane per batch (two batches in flight)
  __shared__ TopkShared<CAP, NT> sh;
  __shared__ float s_thr;
  __shared__ uint32_t s_run[NW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = blockIdx.x, b = blockIdx.y;
  const int64_t row = (int64_t)b * M + i;
  const int n = (int)min((int64_t)n_cols, q_pos0 + i + 1);
  const float* lrow = logits + row * ld;
  // float4s of the row (16-byte aligned: ld % 4 == 0), non-temporal (read
  // once), index clamped into the row (no branch)
  const f32x4* p4 = reinterpret_cast<const f32x4*>(lrow);
  const int n4 = (n + 3) / 4;
  f32x4 va[U], vb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    va[u] = __builtin_nontemporal_load(p4 + min(tid + u * NT, n4 - 1));
    vb[u] = __builtin_nontemporal_load(p4 + min(U * NT + tid + u * NT, n4 - 1));
  }
  if (wv == 0) {
    const float t = row_threshold(lrow, n, target);
    if (lane == 0) s_thr = t;
  }
  __syncthreads();
  const float tf = s_thr;
  uint64_t* reg = sh.buf + wv * WCAP;
  uint32_t run = 0;   // candidates found by this wave (uniform)
  for (int base4 = 0; base4 < n4; base4 += U * NT) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = va[u];
      va[u] = vb[u];
      vb[u] = __builtin_nontemporal_load(p4 + min(base4 + 2 * U * NT + tid + u * NT, n4 - 1));
    }
    uint32_t fl = 0;   // bit 4u+j: element j of float4 u passes
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e0 = 4 * (base4 + tid + u * NT);
#pragma unroll
      for (int j = 0; j < 4; ++j) fl |= (uint32_t)(e0 + j < n && v[u][j] >= tf) << (4 * u + j);
    }
    const uint32_t cnt = __popc(fl);   // 0..16
    const uint64_t m0 = __ballot(cnt & 1u), m1 = __ballot(cnt & 2u), m2 = __ballot(cnt & 4u),
                   m3 = __ballot(cnt & 8u), m4 = __ballot(cnt & 16u);
    if ((m0 | m1 | m2 | m3 | m4) == 0) continue;
    uint32_t pos = run + lanes_below(m0) + 2 * lanes_below(m1) + 4 * lanes_below(m2) + 8 * lanes_below(m3) +
                   16 * lanes_below(m4);
    run += __popcll(m0) + 2 * __popcll(m1) + 4 * __popcll(m2) + 8 * __popcll(m3) + 16 * __popcll(m4);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e0 = 4 * (base4 + tid + u * NT);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (fl & (1u << (4 * u + j))) {
          if (pos < (uint32_t)WCAP) reg[pos] = pack_raw(v[u][j], e0 + j);
          ++pos;
        }
    }
  }
  if (lane == 0) s_run[wv] = run;
  __syncthreads();
  uint32_t tot = 0, before = 0;
  bool over = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t c = s_run[w];
    over |= c > (uint32_t)WCAP;
    before += (w < wv) ? c : 0u;
    tot += c;
  }
  if (over || tot < (uint32_t)min(k, n)) {   // uniform over the workgroup
    topk_row<CAP, NT>(sh, i, b, logits, ld, nullptr, n_cols, k, q_pos0, M, idx_out, val_out, sorted);
    return;
  }
  // the regions gathered into sh.buf[0, tot): every thread holds its wave's
  // entries in registers before any is written
  {
    constexpr int PER = WCAP / 64;
    uint64_t e[PER];
    const uint32_t mine = run;
#pragma unroll
    for (int m = 0; m < PER; ++m) e[m] = reg[min((uint32_t)(lane + 64 * m), (uint32_t)WCAP - 1)];
    __syncthreads();
#pragma unroll
    for (int m = 0; m < PER; ++m)
      if ((uint32_t)(lane + 64 * m) < mine) sh.buf[before + lane + 64 * m] = e[m];
    __syncthreads();
  }
  finish_list<CAP, NT>(sh, tot, k, row, idx_out, val_out, sorted);
}

size_t topk_workspace_bytes(const misa_shape& s, int n_cols, int k) {
  const int64_t rows = (int64_t)s.n_seq * s.q_per_seq;
  // k <= 4096 over enough rows: k_topk_fused keeps its list in LDS
  if (n_cols < kSplitMinCols || (k <= 4096 && rows >= kFusedMinRows)) return 0;
  return split_ws_bytes(rows, k);
}

hipError_t launch_topk(const misa_shape& s, const float* logits, int64_t ld, const int32_t* cand,
                       int n_cols, int k, int32_t* idx, float* vals, void* ws, size_t ws_bytes, hipStream_t st,
                       bool sorted) {
  dim3 grid((unsigned)s.q_per_seq, (unsigned)s.n_seq);
  const int64_t rows = (int64_t)s.n_seq * s.q_per_seq;
  if (cand == nullptr && n_cols >= kSplitMinCols && k <= 4096 && rows >= kFusedMinRows) {
    const int target = min(3 * k / 2, (k + list_cap(k)) / 2);
    hipLaunchKernelGGL((k_topk_fused<8192, 512>), grid, dim3(512), 0, st, logits, ld, n_cols, k, target, s.q_pos0,
                       s.q_per_seq, idx, vals, (int)sorted);
    return hipGetLastError();
  }
  const bool split = cand == nullptr && n_cols >= kSplitMinCols && ws != nullptr &&
                     ws_bytes >= split_ws_bytes(rows, k);
  if (split) {
    const SplitWs w = split_ws(ws, rows, k);
    const int target = min(3 * k / 2, (k + w.capg) / 2);
    hipLaunchKernelGGL(k_topk_thresh, dim3((unsigned)((rows + kThreshWaves - 1) / kThreshWaves)),
                       dim3(64 * kThreshWaves), 0, st, logits, ld, n_cols, target, s.q_pos0, s.q_per_seq, rows,
                       w.thr, w.count, w.flag);
    // chunk length: about target / 2 candidates expected per chunk buffer
    // half, and with few rows short enough for about 2048 workgroups
    int64_t chunk = (int64_t)(kChunkCap / 2) * n_cols / target;
    chunk = std::min<int64_t>(chunk, n_cols / std::max<int64_t>(1, 2048 / rows));
    chunk = chunk >= kChunkMax ? kChunkMax : (chunk < 4096 ? 4096 : chunk / 4096 * 4096);
    const int n_chunks = (int)((n_cols + chunk - 1) / chunk);
    dim3 fgrid((unsigned)((int64_t)s.q_per_seq * n_chunks), (unsigned)s.n_seq);
    hipLaunchKernelGGL(k_topk_filter<256>, fgrid, dim3(256), 0, st, logits, ld, n_cols, (int)chunk, n_chunks,
                       s.q_pos0, s.q_per_seq, w.thr, w.count, w.flag, w.list, w.capg);
    if (k <= 4096)
      hipLaunchKernelGGL((k_topk_list<8192, 512>), grid, dim3(512), 0, st, logits, ld, n_cols, k, s.q_pos0,
                         s.q_per_seq, idx, vals, (int)sorted, w.list, w.count, w.flag, w.capg);
    else
      hipLaunchKernelGGL((k_topk_list<16384, 512>), grid, dim3(512), 0, st, logits, ld, n_cols, k, s.q_pos0,
                         s.q_per_seq, idx, vals, (int)sorted, w.list, w.count, w.flag, w.capg);
    return hipGetLastError();
  }
  // CAP/2 >= max(k, one lock-step step of 4096 elements)
  if (k <= 4096)
    hipLaunchKernelGGL((k_topk<8192, 512>), grid, dim3(512), 0, st, logits, ld, cand, n_cols, k, s.q_pos0,
                       s.q_per_seq, idx, vals, (int)sorted);
  else
    hipLaunchKernelGGL((k_topk<16384, 512>), grid, dim3(512), 0, st, logits, ld, cand, n_cols, k,
                       s.q_pos0, s.q_per_seq, idx, vals, (int)sorted);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused scoring -> top-k: the top-k side (see plan_fused)
// ---------------------------------------------------------------------------

// One wave per row: the threshold from the row's sampled scores (key indices
// u <= t / kstride of the sample logits), the lower edge of the 16-bit
// order-key bucket of the k_s-th largest sample, k_s chosen so that about
// `target` of the row's t + 1 scores are expected at or above it.  Every
// sampled key is one key, so a cluster of large scores takes only its share
// of the sample.  Also clears the row's flag.
// WPR waves per row (1, or kThreshWaves for calls with few rows: decode):
// each wave counts its share of the row's samples, the counts meet in LDS
// once per bit (two slots, so one barrier a bit).  The threshold is the same
// for every WPR.
template <int WPR>
__global__ void __launch_bounds__(64 * kThreshWaves) k_topk_sample_thresh(const float* __restrict__ sample,
                                                                          int64_t ld_s, int n_sample, int kstride,
                                                                          int target, int64_t q_pos0, int M,
                                                                          int64_t rows, float* __restrict__ thr,
                                                                          uint32_t* __restrict__ flag) {
  constexpr int L = 16 / WPR;   // float4 loads per lane: 4096 sampled scores at most per row
  __shared__ uint32_t s_cnt[2][kThreshWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = ((int64_t)blockIdx.x * kThreshWaves + wave) / WPR;
  const int part = wave % WPR;   // this wave's share of the row
  if (WPR == 1 && row >= rows) return;   // (WPR > 1: every wave reaches the barriers)
  const int64_t rowc = row < rows ? row : rows - 1;
  const int64_t t = q_pos0 + rowc % M;
  const int ns = (int)min((int64_t)n_sample, t / kstride + 1);   // sampled keys the query sees
  const uint64_t ks = (uint64_t)target * (uint64_t)ns / (uint64_t)(t + 1) + 2;
  float tf = -__builtin_inff();
  if (ks < (uint64_t)ns) {   // uniform over the row's waves
    const f32x4* src = reinterpret_cast<const f32x4*>(sample + rowc * ld_s);   // ld_s % 4 == 0
    const int n4 = (ns + 3) / 4;
    uint32_t key[4 * L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int f = (j * WPR + part) * 64 + lane;
      const f32x4 v = src[min(f, n4 - 1)];
#pragma unroll
      for (int e = 0; e < 4; ++e) key[4 * j + e] = (4 * f + e < ns) ? order_key(v[e]) : 0u;
    }
    uint32_t T = 0;
    for (int bit = 31; bit >= 16; --bit) {
      const uint32_t c = T | (1u << bit);
      uint32_t cl = 0;
#pragma unroll
      for (int j = 0; j < 4 * L; ++j) cl += (key[j] >= c) ? 1u : 0u;
      uint32_t tot = __reduce_add_sync(~0ull, cl);
      if (WPR > 1) {
        if (lane == 0) s_cnt[bit & 1][wave] = tot;
        __syncthreads();
        tot = 0;
#pragma unroll
        for (int w = 0; w < WPR; ++w) tot += s_cnt[bit & 1][wave - part + w];
      }
      if (tot >= (uint32_t)ks) T = c;
    }
    tf = key_to_float(T);
    if (tf != tf) tf = -__builtin_inff();
  }
  if (row < rows && part == 0 && lane == 0) {
    thr[row] = tf;
    flag[row] = 0;
  }
}

// Exact top-k of a row's candidates, gathered from its key-range regions:
// groups of 4 consecutive scores, of which the ones at or above the row's
// threshold (clamped finite, as the scoring pass used it) are kept.  A row
// with an overflowed region, more candidates than the buffer holds, or fewer
// than k is flagged (and left for the re-scoring path).
template <int CAP, int NT, bool IDX>
__global__ void __launch_bounds__(NT) k_topk_regions(int64_t n_keys, int k, int64_t q_pos0, int M, int n_splits,
                                                        int cap_region, int cap_list, const float* __restrict__ thr,
                                                        const f32x4* __restrict__ gvals,
                                                        const int32_t* __restrict__ gkeys,
                                                        const uint32_t* __restrict__ rcount,
                                                        uint32_t* __restrict__ flag, int32_t* __restrict__ idx_out,
                                                        float* __restrict__ val_out, int sorted) {
  __shared__ std::conditional_t<IDX, TopkSharedIdx<CAP, NT>, TopkShared<CAP, NT>> sh;
  // first flat group of each region.  The compact variant keeps it in the
  // rank histogram, which is not used before the gather has finished: the
  // 4 KB go to the candidate list instead
  __shared__ uint32_t s_start_own[IDX ? 1 : kMaxRegionSplits + 1];
  static_assert(!IDX || kHistBinsIdx >= kMaxRegionSplits + 1, "the region starts fit in the histogram");
  uint32_t* const s_start = IDX ? sh.hist : s_start_own;
  __shared__ uint32_t s_bad;
  const int tid = threadIdx.x, lane = tid & 63;
  const int i = blockIdx.x, b = blockIdx.y;
  const int64_t row = (int64_t)b * M + i;
  const int n = (int)min(n_keys, q_pos0 + i + 1);
  const float tf = __builtin_fmaxf(thr[row], -__FLT_MAX__);
  if (tid < 64) {   // the regions' counts and their prefix, one wave
    uint32_t run = 0, bad = 0;
    for (int s0 = 0; s0 < n_splits; s0 += 64) {
      const int sp = s0 + lane;
      const uint32_t c = (sp < n_splits) ? rcount[row * n_splits + sp] : 0u;
      bad |= c > (uint32_t)cap_region;
      uint32_t x = c;   // inclusive scan over the wave
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d);
        if (lane >= d) x += y;
      }
      if (sp < n_splits) s_start[sp] = run + x - c;
      run += __shfl(x, 63);
    }
    if (lane == 0) {
      s_start[n_splits] = run;
      sh.count = 0;
    }
    bad = __ballot(bad != 0) != 0;
    if (lane == 0) s_bad = bad;
  }
  __syncthreads();
  if (s_bad != 0) {
    if (tid == 0) flag[row] = 1;
    return;
  }
  // every group of every region, flat: U groups per thread loaded together.
  // A thread's candidates of a batch are written one after another from its
  // position (the wave-exclusive sum of the threads' counts, one LDS atomic
  // per wave); the largest value seen bounds the rank's buckets from above,
  // the threshold from below
  constexpr int U = 8;
  const uint32_t total = s_start[n_splits];
  float gmax = -__builtin_inff();
  for (uint32_t e0 = 0; e0 < total; e0 += U * NT) {
    // slots past the last group are skipped by the whole workgroup (a row
    // holds ~2,000 groups: 4 or 5 of the 8 slots of 512 threads)
    const int nu = (int)min((uint32_t)U, (total - e0 + NT - 1) / NT);
    f32x4 v[U];
    int32_t key[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u >= nu) break;   // uniform
      const uint32_t e = e0 + u * NT + tid;
      v[u] = f32x4{-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
      key[u] = 0;
      if (e < total) {
        int lo = 0, hi = n_splits;   // region: the last one starting at or before e
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_start[mid] <= e) lo = mid;
          else hi = mid;
        }
        const int64_t g = (row * n_splits + lo) * (int64_t)cap_region + (e - s_start[lo]);
        v[u] = gvals[g];
        key[u] = gkeys[g];
      }
    }
    uint32_t fl = 0;   // bit 4u + j: element j of group u is a candidate
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u >= nu) break;   // uniform
#pragma unroll
      for (int j = 0; j < 4; ++j) fl |= (uint32_t)(v[u][j] >= tf) << (4 * u + j);
      const float m01 = __builtin_fmaxf(v[u][0], v[u][1]), m23 = __builtin_fmaxf(v[u][2], v[u][3]);
      gmax = __builtin_fmaxf(gmax, __builtin_fmaxf(m01, m23));
    }
    const uint32_t cnt = __popc(fl);   // 0..32
    const uint64_t b0 = __ballot(cnt & 1u), b1 = __ballot(cnt & 2u), b2 = __ballot(cnt & 4u), b3 = __ballot(cnt & 8u),
                   b4 = __ballot(cnt & 16u), b5 = __ballot(cnt & 32u);
    if ((b0 | b1 | b2 | b3 | b4 | b5) == 0) continue;   // uniform over the wave
    uint32_t pos = lanes_below(b0) + 2 * lanes_below(b1) + 4 * lanes_below(b2) + 8 * lanes_below(b3) +
                   16 * lanes_below(b4) + 32 * lanes_below(b5);
    const uint32_t wtot = __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2) + 8 * __popcll(b3) +
                          16 * __popcll(b4) + 32 * __popcll(b5);
    uint32_t wbase = 0;
    if (lane == 0) wbase = atomicAdd(&sh.count, wtot);
    pos += __builtin_amdgcn_readfirstlane(wbase);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u >= nu) break;   // uniform
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (fl & (1u << (4 * u + j))) {
          if (pos < (uint32_t)CAP) sh.buf[pos] = pack_raw(v[u][j], key[u] + j);
          ++pos;
        }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) gmax = __builtin_fmaxf(gmax, __shfl_xor(gmax, o));
  if (lane == 0) sh.red[tid >> 6] = __float_as_uint(gmax);
  __syncthreads();
  const uint32_t tot = sh.count;
  if (tot > (uint32_t)min(cap_list, CAP) || tot < (uint32_t)min(k, n)) {
    if (tid == 0) flag[row] = 1;
    return;
  }
  for (int wv = 0; wv < NT / 64; ++wv) gmax = __builtin_fmaxf(gmax, __uint_as_float((uint32_t)sh.red[wv]));
  __syncthreads();   // sh.red is reused by the select
  if constexpr (IDX) {
    if (!finish_list_idx<CAP, NT>(sh, tot, k, row, idx_out, val_out, sorted, order_key(tf), order_key(gmax)) &&
        tid == 0)
      flag[row] = 1;
  } else
    finish_list<CAP, NT>(sh, tot, k, row, idx_out, val_out, sorted);
}

// Whole-row top-k of the flagged rows from a logits slab: slab_tiles query
// tiles (32 queries each) of the flattened (sequence, query tile) order from
// tile slab_first on, query qi of the tile in slot s in slab row
// s * slab_tr + (qi - first query of the tile).  A fixed grid walks the slab
// rows, so the (rare) flagged rows cost one cheap flag check each.
// the row (b * M + i) of slab row r of a batch (see k_topk_flagged), or -1
__device__ __forceinline__ int64_t slab_row(int64_t r, int64_t slab_first, int slab_tr, int n_qtiles, int64_t n_flat,
                                            int M) {
  const int64_t flat = slab_first + r / slab_tr;
  const int i = (int)(flat % n_qtiles) * 32 + (int)(r % slab_tr);
  return (flat < n_flat && i < M) ? (flat / n_qtiles) * M + i : -1;
}

template <int CAP, int NT>
__global__ void __launch_bounds__(NT, 2) k_topk_flagged(const float* __restrict__ slab, int64_t ld,
                                                        int64_t n_keys, int k, int64_t q_pos0, int M,
                                                        int n_qtiles, int64_t n_flat, int64_t slab_first,
                                                        int slab_tiles, int slab_tr,
                                                        const uint32_t* __restrict__ flag,
                                                        int32_t* __restrict__ idx_out, float* __restrict__ val_out,
                                                        int sorted) {
  __shared__ TopkShared<CAP, NT> sh;
  const int64_t n_rows = (int64_t)slab_tiles * slab_tr;
  {   // the workgroup's flags loaded together: most calls have none
    uint32_t mine = 0;
    for (int64_t r = blockIdx.x + (int64_t)threadIdx.x * gridDim.x; r < n_rows; r += (int64_t)NT * gridDim.x) {
      const int64_t row = slab_row(r, slab_first, slab_tr, n_qtiles, n_flat, M);
      if (row >= 0) mine |= flag[row];
    }
    if (!__syncthreads_or(mine != 0)) return;   // uniform over the workgroup
  }
  for (int64_t r = blockIdx.x; r < n_rows; r += gridDim.x) {
    const int64_t row = slab_row(r, slab_first, slab_tr, n_qtiles, n_flat, M);
    if (row < 0 || flag[row] == 0) continue;   // uniform over the workgroup
    topk_row<CAP, NT>(sh, (int)(row % M), (int)(row / M), slab, ld, nullptr, (int)n_keys, k, q_pos0, M, idx_out,
                      val_out, sorted, slab + r * ld);
    __syncthreads();
  }
}

hipError_t launch_topk_sample_thresh(const misa_shape& s, const FusedPlan& p, const float* sample_logits,
                                     float* thr, uint32_t* row_flag, hipStream_t st) {
  const int64_t rows = (int64_t)s.n_seq * s.q_per_seq;
  if (rows < 1024) {   // few rows (decode): a workgroup per row, so the chip is not left idle
    hipLaunchKernelGGL(k_topk_sample_thresh<kThreshWaves>, dim3((unsigned)rows), dim3(64 * kThreshWaves), 0, st,
                       sample_logits, p.ld_sample, (int)p.n_sample, p.kstride, p.target, s.q_pos0, s.q_per_seq, rows,
                       thr, row_flag);
  } else {
    hipLaunchKernelGGL(k_topk_sample_thresh<1>, dim3((unsigned)((rows + kThreshWaves - 1) / kThreshWaves)),
                       dim3(64 * kThreshWaves), 0, st, sample_logits, p.ld_sample, (int)p.n_sample, p.kstride,
                       p.target, s.q_pos0, s.q_per_seq, rows, thr, row_flag);
  }
  return hipGetLastError();
}

hipError_t launch_topk_regions(const misa_shape& s, const FusedPlan& p, int k, const float* thr,
                               const float* gvals, const int32_t* gkeys, const uint32_t* rcount, uint32_t* row_flag,
                               int32_t* idx, float* vals, bool sorted, hipStream_t st) {
  dim3 grid((unsigned)s.q_per_seq, (unsigned)s.n_seq);
  const f32x4* gv = reinterpret_cast<const f32x4*>(gvals);
#define MISA_REGIONS_LAUNCH(CAP_, IDX_)                                                                      \
  hipLaunchKernelGGL((k_topk_regions<CAP_, 512, IDX_>), grid, dim3(512), 0, st, s.n_keys, k, s.q_pos0,       \
                     s.q_per_seq, p.n_splits, p.cap_region, p.cap_list, thr, gv, gkeys, rcount, row_flag, idx, \
                     vals, (int)sorted)
  if (p.cap_list <= 4608 && (int64_t)s.n_seq * s.q_per_seq < 1024)
    // few rows (decode): twice the threads per row, so each row's chain of
    // gather, counting sort and ranks is shorter while most CUs are idle
    hipLaunchKernelGGL((k_topk_regions<4096, 1024, true>), grid, dim3(1024), 0, st, s.n_keys, k, s.q_pos0,
                       s.q_per_seq, p.n_splits, p.cap_region, p.cap_list, thr, gv, gkeys, rcount, row_flag, idx,
                       vals, (int)sorted);
  else if (p.cap_list <= 4608)
    MISA_REGIONS_LAUNCH(4608, true);
  else if (p.cap_list <= 8192)
    MISA_REGIONS_LAUNCH(8192, false);
  else {
    hipLaunchKernelGGL((k_topk_regions<16384, 1024, false>), grid, dim3(1024), 0, st, s.n_keys, k, s.q_pos0,
                       s.q_per_seq, p.n_splits, p.cap_region, p.cap_list, thr, gv, gkeys, rcount, row_flag, idx,
                       vals, (int)sorted);
  }
#undef MISA_REGIONS_LAUNCH
  return hipGetLastError();
}

hipError_t launch_topk_flagged(const misa_shape& s, int k, const float* slab, int64_t ld, const SlabBatch& sb,
                               const uint32_t* row_flag, int32_t* idx, float* vals, bool sorted, hipStream_t st) {
  const int64_t slab_first = sb.first;
  const int slab_tiles = sb.tiles, slab_tr = sb.tr;
  const int n_qtiles = (s.q_per_seq + 31) / 32;
  const int64_t n_flat = (int64_t)s.n_seq * n_qtiles;
  const unsigned g = (unsigned)std::min<int64_t>((int64_t)slab_tiles * slab_tr, 512);
  if (k <= 4096)
    hipLaunchKernelGGL((k_topk_flagged<8192, 512>), dim3(g), dim3(512), 0, st, slab, ld, s.n_keys, k, s.q_pos0,
                       s.q_per_seq, n_qtiles, n_flat, slab_first, slab_tiles, slab_tr, row_flag, idx, vals,
                       (int)sorted);
  else
    hipLaunchKernelGGL((k_topk_flagged<16384, 512>), dim3(g), dim3(512), 0, st, slab, ld, s.n_keys, k, s.q_pos0,
                       s.q_per_seq, n_qtiles, n_flat, slab_first, slab_tiles, slab_tr, row_flag, idx, vals,
                       (int)sorted);
  return hipGetLastError();
}

}  // namespace misa
