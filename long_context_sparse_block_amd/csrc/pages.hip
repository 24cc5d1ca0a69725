// Paged key cache -> contiguous keys.
//
// Serving engines keep the indexer's key cache in fixed-size pages named by
// a per-sequence block table (the GitHub issue measures the indexer inside
// vLLM, whose per-layer boundary includes this cache handling).  The kernels
// of this library read keys as one contiguous [n_seq][N][128] array, so a
// paged cache is first gathered into that layout: key s of sequence b is row
// s % P of page block_table[b][s / P] (P keys per page).  One thread moves 16
// bytes of a key row; HBM-bound (the keys read once and written once).  Page
// ids outside [0, n_pages) are a precondition violation: their keys are
// written as zeros (with scale 1) instead of being read.
#include "misa_common.h"
#include "misa_launch.h"

namespace misa {

template <int ROW_BYTES>
__global__ void __launch_bounds__(256) k_gather_pages(const uint4* __restrict__ pages,
                                                      const float* __restrict__ page_scales,
                                                      const int32_t* __restrict__ table, int64_t max_pages,
                                                      int64_t n_pages, int page_keys, int64_t N,
                                                      uint4* __restrict__ out, float* __restrict__ out_scale) {
  constexpr int kChunks = ROW_BYTES / 16;   // 16-byte pieces per key row
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // piece of sequence b
  const int b = blockIdx.y;
  if (i >= N * kChunks) return;
  const int64_t s = i / kChunks;
  const int c = (int)(i % kChunks);
  const int64_t page = table[(int64_t)b * max_pages + s / page_keys];
  const bool ok = page >= 0 && page < n_pages;
  const int64_t src_row = page * page_keys + s % page_keys;
  out[((int64_t)b * N + s) * kChunks + c] = ok ? pages[src_row * kChunks + c] : make_uint4(0, 0, 0, 0);
  if (out_scale != nullptr && c == 0) out_scale[(int64_t)b * N + s] = ok ? page_scales[src_row] : 1.f;
}

hipError_t launch_gather_pages(const misa_shape& s, const void* pages, int kdtype, const float* page_scales,
                               const int32_t* table, int64_t max_pages, int64_t n_pages, int page_keys, void* out,
                               float* out_scale, hipStream_t st) {
  const int64_t N = s.n_keys;
  const int chunks = kdtype == MISA_K_BF16 ? kD * 2 / 16 : kD / 16;
  dim3 grid((unsigned)((N * chunks + 255) / 256), (unsigned)s.n_seq);
  if (kdtype == MISA_K_BF16)
    hipLaunchKernelGGL(k_gather_pages<kD * 2>, grid, dim3(256), 0, st, static_cast<const uint4*>(pages), nullptr,
                       table, max_pages, n_pages, page_keys, N, static_cast<uint4*>(out), nullptr);
  else
    hipLaunchKernelGGL(k_gather_pages<kD>, grid, dim3(256), 0, st, static_cast<const uint4*>(pages), page_scales,
                       table, max_pages, n_pages, page_keys, N, static_cast<uint4*>(out), out_scale);
  return hipGetLastError();
}

}  // namespace misa
