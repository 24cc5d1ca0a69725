// Block mean-pooling of the shared indexer keys, plus the partial-block
// ("tail") mean of every query's prefix.
//
// Method: the prefix is split into blocks of B keys and each block is
// summarised by the mean of its indexer keys (gist.science summary of MISA,
// "Metodologia: MISA" item 1; agents-report summary, method overview).
//
// One workgroup (one wave) per (sequence, block m).  Lane l owns dims 2l, 2l+1
// and walks the block's keys in order, so a wave reads one 256-byte (bf16) or
// 128-byte (fp8) key row per step: fully coalesced, one pass over K.  The
// running fp32 sum is also the prefix sum that the tails of queries inside
// this block need, so tails cost no extra traffic.  HBM-bound.
#include "misa_common.h"
#include "misa_launch.h"

namespace misa {

template <int KDT>
__global__ void __launch_bounds__(kWave) k_pool(const void* __restrict__ kptr,
                                                const float* __restrict__ kscale,
                                                float* __restrict__ pooled, float* __restrict__ tail,
                                                int64_t N, int64_t q_pos0, int M, int B,
                                                int64_t n_blk_total, int64_t n_full) {
  const int64_t m = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int64_t s0 = m * B;
  const int64_t s1 = (s0 + B < N) ? s0 + B : N;
  // only blocks that are complete or hold a query need any work
  const int64_t q_lo = q_pos0, q_hi = q_pos0 + M;  // queries occupy [q_lo, q_hi)
  const bool full = (s0 + B <= N);
  const bool has_query = (s1 > q_lo) && (s0 < q_hi);
  if (!full && !has_query) return;

  float a0 = 0.f, a1 = 0.f;
  constexpr int U = 8;
  for (int64_t s = s0; s < s1; s += U) {
    float v0[U], v1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t ss = s + u;
      v0[u] = 0.f;
      v1[u] = 0.f;
      if (ss < s1) {
        int64_t row = (int64_t)b * N + ss;
        if (KDT == MISA_K_BF16) {
          uint32_t two = reinterpret_cast<const uint32_t*>(kptr)[row * (kD / 2) + lane];
          v0[u] = bf16_bits_to_f32(two & 0xFFFFu);
          v1[u] = bf16_bits_to_f32(two >> 16);
        } else {
          uint32_t two = reinterpret_cast<const uint16_t*>(kptr)[row * (kD / 2) + lane];
          float sc = kscale[row];
          f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)two, false);
          v0[u] = f.x * sc;
          v1[u] = f.y * sc;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t ss = s + u;
      if (ss < s1) {
        a0 += v0[u];
        a1 += v1[u];
        // query t = ss has a partial block iff (t+1) % B != 0; its tail is
        // keys [m*B, t] of this block
        if (ss >= q_lo && ss < q_hi && ((ss + 1) % B) != 0) {
          float len = (float)(ss - s0 + 1);
          float2 o = make_float2(a0 / len, a1 / len);
          reinterpret_cast<float2*>(tail)[((int64_t)b * M + (ss - q_lo)) * (kD / 2) + lane] = o;
        }
      }
    }
  }
  if (full && m < n_full) {
    float2 o = make_float2(a0 / (float)B, a1 / (float)B);
    reinterpret_cast<float2*>(pooled)[((int64_t)b * n_full + m) * (kD / 2) + lane] = o;
  }
  // queries whose prefix ends exactly on this block's end have no tail: zeros
  if (full) {
    int64_t t = s0 + B - 1;
    if (t >= q_lo && t < q_hi)
      reinterpret_cast<float2*>(tail)[((int64_t)b * M + (t - q_lo)) * (kD / 2) + lane] =
          make_float2(0.f, 0.f);
  }
}

hipError_t launch_pool(const misa_shape& s, const void* k, int kdtype, const float* k_scale,
                       float* pooled, float* tail, hipStream_t st) {
  const int64_t N = s.n_keys;
  const int B = s.block;
  const int64_t n_blk_total = (N + B - 1) / B;
  const int64_t n_full = N / B;
  dim3 grid((unsigned)n_blk_total, (unsigned)s.n_seq);
  if (kdtype == MISA_K_BF16)
    hipLaunchKernelGGL(k_pool<MISA_K_BF16>, grid, dim3(kWave), 0, st, k, k_scale, pooled, tail, N,
                       s.q_pos0, s.q_per_seq, B, n_blk_total, n_full);
  else
    hipLaunchKernelGGL(k_pool<MISA_K_FP8_E4M3>, grid, dim3(kWave), 0, st, k, k_scale, pooled, tail,
                       N, s.q_pos0, s.q_per_seq, B, n_blk_total, n_full);
  return hipGetLastError();
}

}  // namespace misa
