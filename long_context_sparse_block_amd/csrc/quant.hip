// Per-row fp8 quantisation of the indexer queries, for the fp8 scoring path.
//
// The pages' own indexer runs in fp8 and the GitHub issue on the vLLM kernel
// asks for an fp8 MISA path that avoids widening fp8 to bf16 (issue
// "Clarification on the Figure 3 baseline and plans for an optimized vLLM MISA
// kernel", second question).  Each (query, head) row of 128 bf16 values gets
// its own scale:
//   s = fp32(amax / 448), amax = max |q| over the row (s = 1 for a zero row)
//   code = e4m3fn round-to-nearest-even of fp32(q / s)
// with both divisions correctly rounded, so the codes are a fixed function of
// the input (448 is e4m3fn's largest finite value: the row maximum lands on it).
//
// 16 lanes per row, 8 values (16 bytes of bf16) per lane; a 16-lane max, one
// division for the scale and one per value, gfx950's packed fp32 -> e4m3fn
// convert (round to nearest even).  HBM-bound: 256 bytes in, 132 out per row.
#include "misa_common.h"
#include "misa_launch.h"

namespace misa {

__global__ void __launch_bounds__(256) k_quant_q(const uint4* __restrict__ q, uint2* __restrict__ codes,
                                                 float* __restrict__ scales, int64_t rows) {
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 16;
  const int p = threadIdx.x & 15;
  const bool live = row < rows;   // uniform over each 16-lane group
  const uint4 v = live ? q[row * 16 + p] : make_uint4(0, 0, 0, 0);
  const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(wd[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_bits_to_f32(wd[i] >> 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, o, 16));
  const float s = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  uint32_t c[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int r = 0;
    r = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(x[4 * h], s), __fdiv_rn(x[4 * h + 1], s), r, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(x[4 * h + 2], s), __fdiv_rn(x[4 * h + 3], s), r, true);
    c[h] = (uint32_t)r;
  }
  if (live) {
    codes[row * 16 + p] = make_uint2(c[0], c[1]);
    if (p == 0) scales[row] = s;
  }
}

hipError_t launch_quant_q(const misa_shape& s, const uint16_t* q, uint8_t* q8, float* q_scale, hipStream_t st) {
  const int64_t rows = (int64_t)s.n_seq * s.q_per_seq * s.n_heads;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quant_q, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(q), reinterpret_cast<uint2*>(q8), q_scale, rows);
  return hipGetLastError();
}

}  // namespace misa
