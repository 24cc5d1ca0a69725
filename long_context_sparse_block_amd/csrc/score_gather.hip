// All-head DSA re-rank of per-query candidate tokens (MISA-dagger).
//
// MISA-dagger keeps an enlarged candidate set from the routed pass and lets
// the original all-head DSA indexer re-score only those candidates; the final
// top-k comes from that re-ranking (gist.science summary of MISA, "Variante
// Hierárquica (MISA†)"; agents-report summary, section on MISA†).
//
//   D[t,c] = sum_{j<H} w[t,j] * ReLU(q[t,j] . k[cand[t,c]]) * sigma[cand[t,c]]
//
// Each query has its own candidate keys, so nothing is shared across queries:
// one wave owns one query and a run of 512 of its candidates.  Its 64 head
// rows stay in registers as four 16x16x32 MFMA row blocks (row r = head
// 16*grp + r); candidate keys are gathered straight from memory (K is small
// enough to stay in the last-level cache) as the B operand, one 16-candidate
// group ahead of the one being scored, with the run's ids read once into LDS.  The D layout gives lane group
// g = l/16 the head quad g of each 16-head group, so the quad partials are
// lane-local and the group sum (P0+P1)+(P2+P3) is two butterfly adds across
// lane groups.  The summation order is the one of k_score_q64, so every D is
// bitwise equal to the all-keys dense logit of the same (query, token).
#include "misa_common.h"
#include "misa_launch.h"

namespace misa {

constexpr int kGatherCands = 512;  // candidates per wave

// A run's 16-candidate group as loaded (codes or bf16 bits; fp8 uses x, y)
struct GatherRaw {
  uint4 r[kKSteps];
  float sc;
};

template <int KDT>
__global__ void __launch_bounds__(256) k_score_gather(const uint16_t* __restrict__ q,
                                                      const float* __restrict__ w,
                                                      const void* __restrict__ kptr,
                                                      const float* __restrict__ kscale,
                                                      const int32_t* __restrict__ cand, int n_cand,
                                                      float* __restrict__ logits, int64_t ld, int64_t N,
                                                      int M, int H, int chunks_per_query) {
  __shared__ int32_t s_id[4][kGatherCands];   // each wave's candidate ids
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, p16 = lane & 15;
  const int b = blockIdx.y;
  const int64_t unit = (int64_t)blockIdx.x * 4 + wave;   // (query, candidate run)
  const int qi = (int)(unit / chunks_per_query);
  const int run = (int)(unit % chunks_per_query);
  if (qi >= M) return;
  const int c_begin = run * kGatherCands;
  const int c_end = min(c_begin + kGatherCands, n_cand);
  if (c_begin >= c_end) return;
  const int64_t row = (int64_t)b * M + qi;
  const int n_grp = (H + 15) / 16;

  // the run's ids, once (a wave's own LDS writes and reads happen in order)
  const int32_t* crow = cand + row * (int64_t)n_cand;
  int32_t* sid = s_id[wave];
  for (int e = lane; e < kGatherCands; e += 64) {
    const int c = c_begin + e;
    sid[e] = (c < c_end) ? crow[c] : -1;
  }

  // A: row block grp, row r -> head 16*grp + r
  bf16x8 afr[4][kKSteps];
  float wq[4][4];
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    const int j = grp * 16 + p16;
    const bool ok = (grp < n_grp) && (j < H);
    const uint4* src = reinterpret_cast<const uint4*>(q + (row * H + (ok ? j : 0)) * kD);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) afr[grp][ks] = as_bf16x8(ok ? src[ks * 4 + g] : make_uint4(0, 0, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jj = grp * 16 + 4 * g + i;     // head of output row 4g+i
      wq[grp][i] = (grp < n_grp && jj < H) ? w[row * H + jj] : 0.f;
    }
  }

  // group it's key rows: ids are a documented precondition (in [0, t]);
  // clamped so a bad one cannot fault.  Loads are unconditional, so waiting
  // for one group never waits for the next group's loads.
  auto load_group = [&](int it, GatherRaw& o) {
    const int id = sid[16 * it + p16];
    const int64_t kid = (id >= 0) ? (id < N ? id : N - 1) : 0;
    if (KDT == MISA_K_BF16) {
      const uint4* kr = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(kptr) +
                                                       ((int64_t)b * N + kid) * kD);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) o.r[ks] = kr[ks * 4 + g];
      o.sc = 1.f;
    } else {
      const uint2* kr = reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(kptr) +
                                                       ((int64_t)b * N + kid) * kD);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const uint2 cv = kr[ks * 4 + g];     // 8 codes: d = 32*ks + 8*g .. +7
        o.r[ks] = make_uint4(cv.x, cv.y, 0u, 0u);
      }
      o.sc = kscale[(int64_t)b * N + kid];
    }
  };
  // the run's scores through a descriptor ending at the run's end (stores of
  // candidates past it are dropped)
  const __amdgpu_buffer_rsrc_t orsrc = uniform_rsrc(logits + row * ld, (uint32_t)c_end * 4u);

  const float ninf = -__builtin_inff();
  const int n_it = (c_end - c_begin + 15) / 16;
  GatherRaw cur, nxt;
  load_group(0, cur);
  for (int it = 0; it < n_it; ++it) {
    load_group(min(it + 1, n_it - 1), nxt);
    const int c = c_begin + 16 * it + p16;
    const int id = sid[16 * it + p16];
    bf16x8 bfr[kKSteps];
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (KDT == MISA_K_BF16) {
        bfr[ks] = as_bf16x8(cur.r[ks]);
      } else {
        const uint2 lo = e4m3x4_to_bf16x4(cur.r[ks].x), hi = e4m3x4_to_bf16x4(cur.r[ks].y);
        bfr[ks] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
    }
    float s = 0.f;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      if (grp >= n_grp) break;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) acc = mfma16(afr[grp][ks], bfr[ks], acc);
      const float P = quad_chain(acc, wq[grp][0], wq[grp][1], wq[grp][2], wq[grp][3]);
      const float v = P + __shfl_xor(P, 16);       // P0+P1 on groups 0/1, P2+P3 on 2/3
      const float T = v + __shfl_xor(v, 32);       // (P0+P1)+(P2+P3)
      s = s + T;
    }
    if (KDT == MISA_K_FP8_E4M3) s *= cur.sc;
    if (id < 0) s = ninf;
    // the 4 lane groups hold the same score: every lane stores it
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(s), orsrc, (int)((uint32_t)c * 4u), 0, 0);
    cur = nxt;
  }
}

hipError_t launch_score_gather(const misa_shape& s, const uint16_t* q, const float* w, const void* k,
                               int kdtype, const float* k_scale, const int32_t* cand, int n_cand,
                               float* logits, int64_t ld, hipStream_t st) {
  const int M = s.q_per_seq;
  const int cpq = (n_cand + kGatherCands - 1) / kGatherCands;
  const int64_t units = (int64_t)M * cpq;
  dim3 grid((unsigned)((units + 3) / 4), (unsigned)s.n_seq);
  if (kdtype == MISA_K_BF16)
    hipLaunchKernelGGL(k_score_gather<MISA_K_BF16>, grid, dim3(256), 0, st, q, w, k, k_scale, cand,
                       n_cand, logits, ld, s.n_keys, M, s.n_heads, cpq);
  else
    hipLaunchKernelGGL(k_score_gather<MISA_K_FP8_E4M3>, grid, dim3(256), 0, st, q, w, k, k_scale,
                       cand, n_cand, logits, ld, s.n_keys, M, s.n_heads, cpq);
  return hipGetLastError();
}

}  // namespace misa
