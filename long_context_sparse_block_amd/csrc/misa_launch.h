// Host-side launchers of the MISA kernels (internal; the public ABI is misa.h).
// Each returns hipSuccess or the error of the launch.  Arguments have been
// validated by the caller (misa_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "misa.h"

namespace misa {

hipError_t launch_pool(const misa_shape& s, const void* k, int kdtype, const float* k_scale,
                       float* pooled, float* tail, hipStream_t st);

hipError_t launch_route(const misa_shape& s, const uint16_t* q, const float* w, const float* pooled,
                        const float* tail, int h, int32_t* heads, float* scores, hipStream_t st);

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

}  // namespace misa
