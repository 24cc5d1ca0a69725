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

// (waves_per_eu(2): at most 256 registers, so the MFMA accumulators stay in
// VGPRs instead of AGPRs read back one v_accvgpr_read per value)
template <int KDT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
k_score_gather(const uint16_t* __restrict__ q,
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
      const float T = sum_rows(P);   // (P0+P1)+(P2+P3) on every lane
      s = s + T;
    }
    if (KDT == MISA_K_FP8_E4M3) s *= cur.sc;
    if (id < 0) s = ninf;
    // the 4 lane groups hold the same score: every lane stores it
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(s), orsrc, (int)((uint32_t)c * 4u), 0, 0);
    cur = nxt;
  }
}

// The same re-rank with each wave's candidate key rows staged by direct
// global -> LDS loads into a ring of 4 wave-private slots (16 rows each, fp8
// scales after them), three groups ahead of the one being scored: no
// registers hold loads in flight, so three times as many gathers are
// outstanding per wave.  Chunk c (16 bytes) of a slot's row j sits at
// position c ^ (j mod CPR) of the row (CPR = chunks per row), which keeps the
// B-fragment reads within two lanes per bank.
//
// Waiting.  The compiler cannot tell which slot a direct load writes, so any
// LDS read it sees after one would wait for all of them.  After the first
// load every LDS read here is therefore an asm block that waits for its own
// results (lds_read_*), and each step waits explicitly for its slot: per step
// a wave issues one slot's loads (kStageOps) and one store, and a slot is
// read three steps after its loads, so vmcnt(3 (kStageOps + 1)) leaves
// exactly the later operations in flight.  The prologue issues a dropped
// store after each of its three loads to keep that count from the start.
// Needs the sequence's K below 2^31 bytes (one descriptor); k_score_gather
// otherwise.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
__device__ __forceinline__ int32_t lds_read_i32(const void* p) {
  int32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}

template <int KDT, int NG>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
k_score_gather_lds(const uint16_t* __restrict__ q,
                   const float* __restrict__ w,
                   const void* __restrict__ kptr,
                   const float* __restrict__ kscale,
                   const int32_t* __restrict__ cand, int n_cand,
                   float* __restrict__ logits, int64_t ld, int64_t N,
                   int M, int H, int chunks_per_query) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  constexpr bool kFp8 = KDT == MISA_K_FP8_E4M3;
  constexpr int RB = kFp8 ? kD : 2 * kD;     // bytes per key row
  constexpr int CPR = RB / 16;               // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;              // rows per 64-lane load
  constexpr int SLOT = 16 * RB + (kFp8 ? 256 : 0);
  constexpr int kStageOps = 16 / RPI + (kFp8 ? 1 : 0);
  __shared__ int32_t s_id[4 * kGatherCands];
  __shared__ __attribute__((aligned(16))) unsigned char s_ring[4 * 4 * SLOT];   // [wave][slot]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  const int32_t* crow = cand + row * (int64_t)n_cand;
  int32_t* sid = s_id + wave * kGatherCands;
  for (int e = lane; e < kGatherCands; e += 64) {
    const int c = c_begin + e;
    sid[e] = (c < c_end) ? crow[c] : -1;
  }
  unsigned char* ring = s_ring + wave * 4 * SLOT;

  bf16x8 afr[NG][kKSteps];
  float wq[NG][4];
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    const int j = grp * 16 + p16;
    const bool ok = j < H;
    const uint4* src = reinterpret_cast<const uint4*>(q + (row * H + (ok ? j : 0)) * kD);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) afr[grp][ks] = as_bf16x8(ok ? src[ks * 4 + g] : make_uint4(0, 0, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jj = grp * 16 + 4 * g + i;
      wq[grp][i] = (jj < H) ? w[row * H + jj] : 0.f;
    }
  }

  const __amdgpu_buffer_rsrc_t krsrc =
      uniform_rsrc(static_cast<const unsigned char*>(kptr) + (int64_t)b * N * RB, (uint32_t)(N * RB));
  const __amdgpu_buffer_rsrc_t srsrc = uniform_rsrc(kFp8 ? kscale + (int64_t)b * N : kscale, kFp8 ? (uint32_t)N * 4u : 0u);
  const __amdgpu_buffer_rsrc_t orsrc = uniform_rsrc(logits + row * ld, (uint32_t)c_end * 4u);
  constexpr uint32_t kDrop = 0x80000000u;
  const int last = (c_end - c_begin + 15) / 16 - 1;   // last real group
  const int n_it = (last + 1 + 3) / 4 * 4;            // groups, padded to the ring

  // the key id of candidate e of the run, clamped into range (ids are a
  // documented precondition, in [0, t]; -1 marks padding)
  auto kid_of = [&](int id) -> uint32_t { return (uint32_t)((id >= 0) ? (id < N ? id : N - 1) : 0); };
  // stage group it (clamped to a real one, so every load is issued) into slot r
  auto stage = [&](int it, int r) {
    const int gi = min(it, last);
    unsigned char* slot = ring + r * SLOT;
#pragma unroll
    for (int u = 0; u < 16 / RPI; ++u) {
      const int j = u * RPI + lane / CPR;   // row of the slot this lane fills
      const int c = (lane % CPR) ^ (j % CPR);
      const uint32_t kid = kid_of(lds_read_i32(sid + 16 * gi + j));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_ptr)(slot + u * RPI * RB), 16, kid * RB + c * 16, 0, 0, 0);
    }
    if (kFp8) {
      const uint32_t kid = kid_of(lds_read_i32(sid + 16 * gi + p16));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srsrc, (lds_ptr)(slot + 16 * RB), 4, kid * 4u, 0, 0, 0);
    }
  };
  const float ninf = -__builtin_inff();
  auto score = [&](int it, int r) {
    const unsigned char* slot = ring + r * SLOT;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * (kStageOps + 1)));   // this slot's loads have landed
    const int c = c_begin + 16 * it + p16;
    const int id = lds_read_i32(sid + min(16 * it + p16, kGatherCands - 1));
    bf16x8 bfr[kKSteps];
    float sc = 1.f;
    uint32_t a[kKSteps];
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const int off = kFp8 ? 32 * ks + 8 * g : 64 * ks + 16 * g;   // this lane's bytes of row p16
      a[ks] = lds_addr(slot + p16 * RB + ((((off >> 4) ^ (p16 % CPR))) << 4) + (off & 15));
    }
    if (kFp8) {
      uint64_t v0, v1, v2, v3;
      uint32_t scb;
      asm volatile(
          "ds_read_b64 %0, %5\n\t"
          "ds_read_b64 %1, %6\n\t"
          "ds_read_b64 %2, %7\n\t"
          "ds_read_b64 %3, %8\n\t"
          "ds_read_b32 %4, %9\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(scb)
          : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(lds_addr(slot + 16 * RB + 4 * p16))
          : "memory");
      const uint64_t v[4] = {v0, v1, v2, v3};
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {   // 8 codes: d = 32*ks + 8*g .. +7
        const uint2 lo = e4m3x4_to_bf16x4((uint32_t)v[ks]), hi = e4m3x4_to_bf16x4((uint32_t)(v[ks] >> 32));
        bfr[ks] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
      sc = __uint_as_float(scb);
    } else {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      u32x4 v0, v1, v2, v3;
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %5\n\t"
          "ds_read_b128 %2, %6\n\t"
          "ds_read_b128 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3)
          : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
          : "memory");
      bfr[0] = __builtin_bit_cast(bf16x8, v0);
      bfr[1] = __builtin_bit_cast(bf16x8, v1);
      bfr[2] = __builtin_bit_cast(bf16x8, v2);
      bfr[3] = __builtin_bit_cast(bf16x8, v3);
    }
    float s = 0.f;
#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) acc = mfma16(afr[grp][ks], bfr[ks], acc);
      const float P = quad_chain(acc, wq[grp][0], wq[grp][1], wq[grp][2], wq[grp][3]);
      const float T = sum_rows(P);   // (P0+P1)+(P2+P3) on every lane
      s = s + T;
    }
    if (kFp8) s *= sc;
    if (id < 0) s = ninf;
    // the 4 lane groups hold the same score: every lane stores it (past the
    // run's end, or in a padding group, the store is dropped)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(s), orsrc, (int)((c < c_end) ? (uint32_t)c * 4u : kDrop), 0, 0);
  };

  for (int r = 0; r < 3; ++r) {
    stage(r, r);
    __builtin_amdgcn_raw_buffer_store_b32(0, orsrc, (int)kDrop, 0, 0);   // keeps the per-step count
  }
  for (int it = 0; it < n_it; it += 4) {
    stage(it + 3, 3);
    score(it, 0);
    stage(it + 4, 0);
    score(it + 1, 1);
    stage(it + 5, 1);
    score(it + 2, 2);
    stage(it + 6, 2);
    score(it + 3, 3);
  }
}

hipError_t launch_score_gather(const misa_shape& s, const uint16_t* q, const float* w, const void* k,
                               int kdtype, const float* k_scale, const int32_t* cand, int n_cand,
                               float* logits, int64_t ld, hipStream_t st) {
  const int M = s.q_per_seq;
  const int cpq = (n_cand + kGatherCands - 1) / kGatherCands;
  const int64_t units = (int64_t)M * cpq;
  dim3 grid((unsigned)((units + 3) / 4), (unsigned)s.n_seq);
  const int64_t row_bytes = (kdtype == MISA_K_BF16) ? 2 * kD : kD;
  const bool lds = s.n_keys * row_bytes < ((int64_t)1 << 31);   // one descriptor over the sequence's K
  const int ng = (s.n_heads + 15) / 16;
#define MISA_GATHER(KERNEL_)                                                                             \
  hipLaunchKernelGGL(KERNEL_, grid, dim3(256), 0, st, q, w, k, k_scale, cand, n_cand, logits, ld, s.n_keys, \
                     M, s.n_heads, cpq)
#define MISA_GATHER_LDS(KDT_)                                                   \
  switch (ng) {                                                                 \
    case 1: MISA_GATHER((k_score_gather_lds<KDT_, 1>)); break;                  \
    case 2: MISA_GATHER((k_score_gather_lds<KDT_, 2>)); break;                  \
    case 3: MISA_GATHER((k_score_gather_lds<KDT_, 3>)); break;                  \
    default: MISA_GATHER((k_score_gather_lds<KDT_, 4>)); break;                 \
  }
  if (kdtype == MISA_K_BF16) {
    if (lds) { MISA_GATHER_LDS(MISA_K_BF16) } else { MISA_GATHER(k_score_gather<MISA_K_BF16>); }
  } else {
    if (lds) { MISA_GATHER_LDS(MISA_K_FP8_E4M3) } else { MISA_GATHER(k_score_gather<MISA_K_FP8_E4M3>); }
  }
#undef MISA_GATHER_LDS
#undef MISA_GATHER
  return hipGetLastError();
}

}  // namespace misa
