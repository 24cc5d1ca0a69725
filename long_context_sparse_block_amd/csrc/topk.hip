// Per-query top-k token selection.
//
// The indexer keeps, for every query, the k prefix tokens with the largest
// scores (abstract of arXiv 2605.07363; gist.science summary of MISA,
// "Metodologia: MISA" item 2).  Order: score descending, equal scores (with
// -0.0 == +0.0) -> lower token id.
//
// Design: exact MSB-first radix select, one workgroup (8 waves) per row.
// Every element becomes a unique 64-bit composite
//     (order-preserving uint32 of the score) << 32 | ~token_id
// so "larger composite first" is exactly the required order and ties are
// impossible.  Each pass streams the row (float4 loads) and builds an LDS
// histogram of the next 12-bit digit among elements still matching the
// selected prefix; a block scan from the top bin finds the bin holding the
// k-th element.  As soon as the elements above that bin plus the bin itself
// fit the LDS buffer, one more pass collects them, a bitonic sort in LDS
// orders them, and the first k are written.  Usually one histogram pass
// suffices, so a row is read twice (the second read mostly from cache).
#include "misa_common.h"
#include "misa_launch.h"

namespace misa {

constexpr int kTopkThreads = 512;
constexpr int kHistBins = 4096;

__device__ __forceinline__ uint64_t composite(float v, int32_t id) {
  return ((uint64_t)order_key(v) << 32) | (uint64_t)(~(uint32_t)id);
}

// inclusive scan over the workgroup; returns the exclusive prefix of `x`
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
  for (int wv = 0; wv < kTopkThreads / 64; ++wv) {
    const uint32_t t = s_wave[wv];
    if (wv < wave) before += t;
    all += t;
  }
  *total = all;
  __syncthreads();
  return before + v - x;
}

template <int CAP>
__global__ void __launch_bounds__(kTopkThreads) k_topk(const float* __restrict__ logits, int64_t ld,
                                                       const int32_t* __restrict__ cand, int n_cols,
                                                       int k, int64_t q_pos0, int M,
                                                       int32_t* __restrict__ idx_out,
                                                       float* __restrict__ val_out) {
  __shared__ uint32_t s_hist[kHistBins];
  __shared__ uint64_t s_buf[CAP];
  __shared__ uint32_t s_wave[kTopkThreads / 64];
  __shared__ uint32_t s_count;
  __shared__ uint32_t s_sel_bin, s_sel_above;

  const int tid = threadIdx.x;
  const int i = blockIdx.x, b = blockIdx.y;
  const int64_t row = (int64_t)b * M + i;
  const int64_t t = q_pos0 + i;
  const int n = cand ? n_cols : (int)min((int64_t)n_cols, t + 1);
  const float* lrow = logits + row * ld;
  const int32_t* crow = cand ? cand + row * (int64_t)n_cols : nullptr;
  // float4 / int4 loads need 16-byte aligned rows: ld % 4 == 0 always, and the
  // candidate rows when n_cols % 4 == 0; otherwise every element is read singly
  const int n4 = (crow == nullptr || (n_cols & 3) == 0) ? (n >> 2) : 0;

  // visit every candidate element: f(composite)
  auto visit = [&](auto&& f) {
    for (int e = tid; e < n4; e += kTopkThreads) {
      const float4 v = reinterpret_cast<const float4*>(lrow)[e];
      int4 id;
      if (crow) id = reinterpret_cast<const int4*>(crow)[e];
      else id = make_int4(4 * e, 4 * e + 1, 4 * e + 2, 4 * e + 3);
      if (id.x >= 0) f(composite(v.x, id.x));
      if (id.y >= 0) f(composite(v.y, id.y));
      if (id.z >= 0) f(composite(v.z, id.z));
      if (id.w >= 0) f(composite(v.w, id.w));
    }
    for (int c = 4 * n4 + tid; c < n; c += kTopkThreads) {
      const int id = crow ? crow[c] : c;
      if (id >= 0) f(composite(lrow[c], id));
    }
  };

  uint64_t prefix = 0, pmask = 0;
  uint32_t above = 0, need = 0;
  bool take_all = false;
  int shift = 52;
  for (int pass = 0;; ++pass) {
    const uint32_t dmask = (shift >= 4) ? 0xFFFu : 0xFu;
    for (int e = tid; e < kHistBins; e += kTopkThreads) s_hist[e] = 0;
    __syncthreads();
    visit([&](uint64_t c) {
      if ((c & pmask) == prefix) atomicAdd(&s_hist[(uint32_t)(c >> shift) & dmask], 1u);
    });
    __syncthreads();
    // rank order r = 0 is the highest bin; thread owns r in [8*tid, 8*tid+8)
    uint32_t h8[8], ls = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      h8[u] = s_hist[kHistBins - 1 - (8 * tid + u)];
      ls += h8[u];
    }
    uint32_t total;
    const uint32_t excl = block_exclusive_scan(ls, s_wave, &total);
    if (pass == 0) {
      const uint32_t n_valid = total;
      need = min((uint32_t)k, n_valid);
      if (n_valid <= (uint32_t)CAP) {
        take_all = true;
        break;
      }
    }
    if (excl < need && need <= excl + ls) {
      uint32_t c = excl;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (c + h8[u] >= need) {
          s_sel_bin = kHistBins - 1 - (8 * tid + u);
          s_sel_above = c;
          break;
        }
        c += h8[u];
      }
    }
    __syncthreads();
    const uint32_t bin = s_sel_bin, cab = s_sel_above;
    const uint32_t bin_count = s_hist[bin];
    above += cab;
    need -= cab;
    prefix |= (uint64_t)bin << shift;
    pmask |= (uint64_t)dmask << shift;
    __syncthreads();
    if (above + bin_count <= (uint32_t)CAP || shift == 0) break;
    shift = (shift >= 16) ? shift - 12 : (shift == 4 ? 0 : 4);
  }

  // collect the elements above the threshold bin and the bin itself
  if (tid == 0) s_count = 0;
  __syncthreads();
  visit([&](uint64_t c) {
    const uint64_t top = c & pmask;
    if (take_all || top >= prefix) {
      const uint32_t pos = atomicAdd(&s_count, 1u);
      if (pos < (uint32_t)CAP) s_buf[pos] = c;   // can only overflow on duplicate candidate ids
    }
  });
  __syncthreads();
  const uint32_t cnt = min(s_count, (uint32_t)CAP);
  // sort only the smallest power of two holding cnt entries
  uint32_t len = 2;
  while (len < cnt) len <<= 1;
  for (uint32_t e = cnt + tid; e < len; e += kTopkThreads) s_buf[e] = 0;
  __syncthreads();
  for (uint32_t size = 2; size <= len; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (uint32_t e = tid; e < len / 2; e += kTopkThreads) {
        const uint32_t a = (e / stride) * 2 * stride + (e % stride);
        const uint32_t c = a + stride;
        const uint64_t x = s_buf[a], y = s_buf[c];
        const bool desc = (a & size) == 0;
        if (desc ? (x < y) : (x > y)) {
          s_buf[a] = y;
          s_buf[c] = x;
        }
      }
      __syncthreads();
    }
  }
  const uint32_t n_out = min((uint32_t)k, cnt);
  for (int e = tid; e < k; e += kTopkThreads) {
    int32_t id = -1;
    float v = -__builtin_inff();
    if ((uint32_t)e < n_out) {
      const uint64_t c = s_buf[e];
      id = (int32_t)(~(uint32_t)c);
      v = key_to_float((uint32_t)(c >> 32));
    }
    idx_out[row * k + e] = id;
    if (val_out) val_out[row * k + e] = v;
  }
}

size_t topk_workspace_bytes(const misa_shape&, int, int) { return 0; }

hipError_t launch_topk(const misa_shape& s, const float* logits, int64_t ld, const int32_t* cand,
                       int n_cols, int k, int32_t* idx, float* vals, void*, size_t, hipStream_t st) {
  dim3 grid((unsigned)s.q_per_seq, (unsigned)s.n_seq);
  dim3 block(kTopkThreads);
  if (k <= 512)
    hipLaunchKernelGGL(k_topk<1024>, grid, block, 0, st, logits, ld, cand, n_cols, k, s.q_pos0,
                       s.q_per_seq, idx, vals);
  else if (k <= 2048)
    hipLaunchKernelGGL(k_topk<4096>, grid, block, 0, st, logits, ld, cand, n_cols, k, s.q_pos0,
                       s.q_per_seq, idx, vals);
  else
    hipLaunchKernelGGL(k_topk<16384>, grid, block, 0, st, logits, ld, cand, n_cols, k, s.q_pos0,
                       s.q_per_seq, idx, vals);
  return hipGetLastError();
}

}  // namespace misa
