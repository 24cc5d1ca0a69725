// Routed-head token scoring with fp8 queries and fp8 keys (h <= 8).
//
//   I[t,s] = sum_{j in heads(t)} w[t,j] * ReLU(sq[t,j] qc[t,j] . kc[s]) * sigma[s]
//          = sigma[s] * sum_j (w[t,j] sq[t,j]) * ReLU(qc[t,j] . kc[s])      (sq, sigma > 0)
// with qc / sq the e4m3fn codes and scale of misa_quantize_q and kc / sigma
// those of the fp8 key cache: the MISA scoring of item 2 of "Metodologia:
// MISA" (gist.science summary) on the fp8 inputs the pages' indexer uses, as
// the GitHub issue on the vLLM kernel asks (no fp8 -> bf16 widening).
//
// Design (gfx950): v_mfma_f32_16x16x128_f8f6f4 takes a whole 128-long dot
// product in one instruction (lane l holds bytes 32 (l/16) .. +31 of row
// l % 16 of A, and of column l % 16 of B).  As in k_score_h8, a 16-row block
// is 4 queries x 4 head slots, so all heads of one (query, key) land in one
// lane and the epilogue is lane-local; a wave owns 8 queries (2 groups x 2
// head quads), a workgroup 32 queries, and 64-key tiles pass through LDS
// (double buffered) in the column order of k_score_h8, so a lane ends a tile
// with 4 consecutive logits.  The tiles are the fp8 codes themselves (128-byte
// rows), staged by direct global -> LDS loads; chunk c (16 bytes) of row j
// sits at slot c ^ (((j >> 1) & 1) | (j & 4)), which makes the B-fragment
// reads (2 x 16 bytes per lane) free of bank conflicts on gfx950.  The query
// scale is folded into the head weight.  This MFMA accumulates at slightly
// less than fp32 precision (about 2^-14 of the sum of |products| measured),
// well inside the scoring tolerance.
#include <type_traits>

#include "misa_common.h"
#include "misa_launch.h"
#include "score_shared.h"

namespace misa {

namespace {

constexpr int kQ8KT = 64;          // keys per tile
constexpr int kQ8Row = kD;         // bytes per fp8 key row
constexpr int kQ8Tile = kQ8KT * kQ8Row;

__device__ __forceinline__ int q8_tile_key(int j) { return (j & 15) * 4 + (j >> 4); }
__device__ __forceinline__ int q8_swz(int j) { return ((j >> 1) & 1) | (j & 4); }

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_f8(const i32x8& a, const i32x8& b) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// tile keys [key0, key0+64) of the sequence 0, ks, 2ks, ... into LDS (rows past
// N read as zeros); every wave also loads the tile's 64 scales (same data)
__device__ __forceinline__ void q8_stage(const uint8_t* kbase, const float* sbase, int key0, int N, int ks,
                                         int lane, int wave, unsigned char* s_dst, float* s_sc) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  // 32-bit scalar arithmetic: N < 2^26 keys (the ABI checks it)
  const int first = key0 * ks;
  const int rem = max(0, min(kQ8KT * ks, N - first));
  const __amdgpu_buffer_rsrc_t kr = uniform_rsrc(kbase + (int64_t)first * kQ8Row, (uint32_t)rem * kQ8Row);
#pragma unroll
  for (int u = 0; u < 2; ++u) {   // 8 loads of 8 rows (1 KB) per tile, 2 per wave
    const int r0 = (u * 4 + wave) * 8;
    const int j = r0 + (lane >> 3);
    const int c = (lane & 7) ^ q8_swz(j);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_ptr)(s_dst + r0 * kQ8Row), 16,
                                             (uint32_t)(q8_tile_key(j) * ks) * kQ8Row + c * 16, 0, 0, 0);
  }
  const __amdgpu_buffer_rsrc_t sr = uniform_rsrc(sbase + first, (uint32_t)rem * 4u);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_ptr)s_sc, 4, (uint32_t)(q8_tile_key(lane) * ks) * 4u, 0, 0, 0);
}

}  // namespace

// One scoring pass over the key sequence 0, ks, 2ks, ... (key index u is
// key u ks); MODE and out_spec as for k_score_h8 (score_shared.h):
//   kLogits: logits[row][u], -inf past each query's prefix (columns N ..
//   roundup4(N)-1 may be set to -inf); full rows (ks = 1) stream out
//   non-temporally, sampled rows stay cacheable (they are read at once);
//   kCands: groups of 4 consecutive scores with one at or above the row's
//   threshold appended to the (row, key range) regions, no logits.
// (the occupancy hints of this file keep the MFMA accumulators in VGPRs, as
// for k_score_h8: with room for more than 256 registers they go to AGPRs and
// every result costs a v_accvgpr_read)
template <int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
k_score_q8(const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
           const float* __restrict__ w, const uint8_t* __restrict__ kptr,
           const float* __restrict__ kscale,
           const int32_t* __restrict__ heads, int h, ScoreOut out_spec,
           int64_t N64, int kstride, int64_t q_pos0_64, int M, int H,
           int n_qtiles, int n_ksplits, int64_t KR) {
  constexpr int KT = kQ8KT, QT = 32;
  __shared__ __attribute__((aligned(16))) unsigned char s_k0[kQ8Tile], s_k1[kQ8Tile];
  __shared__ float s_sc0[KT], s_sc1[KT];

  const int Nk = (int)N64, q_pos0 = (int)q_pos0_64;
  const int N = (Nk + kstride - 1) / kstride;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, p16 = lane & 15;
  const WgTile tc = wg_tile<QT, MODE == kLogits>(out_spec, M, n_qtiles, n_ksplits, KR, N);
  if (!tc.valid) return;   // uniform over the workgroup
  const int b = tc.b;
  const int k0 = (int)tc.k0, k1 = (int)tc.k1;
  const int qa = tc.qt * QT, qb = min(qa + QT, M);
  const int64_t qrow0 = (int64_t)b * M;
  if (out_spec.row_flag != nullptr) {   // one flag per thread (QT <= 256), loaded together
    const bool mine = tid < qb - qa && out_spec.row_flag[qrow0 + qa + tid] != 0;
    if (!__syncthreads_or(mine)) return;   // uniform over the workgroup
  }
  const int t_last = (q_pos0 + qb - 1) / kstride;
  const int kend = min(k1, t_last + 1);
  const int n_tiles = kend > k0 ? (kend - k0 + KT - 1) / KT : 0;
  const int q0w = qa + wave * 8;
  const int t_lo = (q_pos0 + q0w) / kstride;
  const int t_hi = (q0w < qb) ? (q_pos0 + min(q0w + 8, qb) - 1) / kstride : -1;
  const int split = (int)(k0 / KR);

  // A fragments: block 2G+qd, row r -> query q0w + 4G + r/4, head slot 4qd + r%4;
  // lane (g, p16) holds bytes 32g .. 32g+31 of its row
  i32x8 afr[4];
  float wv[2][8];
  int tq[2];
  __amdgpu_buffer_rsrc_t orsrc[2];   // kLogits: the two groups' rows; kCands: gvals, gkeys
  float thr[2];
  uint32_t reg[2];
  const uint32_t row_bytes = (uint32_t)out_spec.ld * 4u;
  const uint32_t lane_row_off = (uint32_t)g * row_bytes;
  if (MODE == kCands) cand_rsrc(out_spec, qrow0, qa, qb, n_ksplits, split, orsrc);
#pragma unroll
  for (int G = 0; G < 2; ++G) {
    const int qg0 = q0w + 4 * G;
    const int nrows = max(0, min(4, qb - qg0));
    const int qo = qg0 + g;
    tq[G] = (qo < qb) ? (q_pos0 + qo) / kstride : -1;
    const int qoc = min(qo, M - 1);
    if (MODE == kLogits)
      orsrc[G] = uniform_rsrc(out_spec.logits + (tc.orow0 + min(qg0, M - 1)) * out_spec.ld, (uint32_t)nrows * row_bytes);
    else
      cand_lane(out_spec, qrow0, qa, qb, qo, qoc, n_ksplits, thr[G], reg[G]);
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const int j = clamp_head(heads[(qrow0 + qoc) * h + min(sl, h - 1)], H);
      const int64_t r = (qrow0 + qoc) * H + j;
      wv[G][sl] = w[r] * q_scale[r] * ((qo < qb && sl < h) ? 1.f : 0.f);
    }
    const int qi = qg0 + (p16 >> 2);
    const int qic = min(qi, M - 1);
#pragma unroll
    for (int qd = 0; qd < 2; ++qd) {
      const int sl = 4 * qd + (p16 & 3);
      const bool ok = (qi < qb) && (sl < h);
      const int j = clamp_head(heads[(qrow0 + qic) * h + min(sl, h - 1)], H);
      const uint4* src = reinterpret_cast<const uint4*>(q8 + ((qrow0 + qic) * H + j) * kD + 32 * g);
      const uint4 v0 = src[0], v1 = src[1];
      const int keep = ok ? -1 : 0;
      afr[2 * G + qd] = i32x8{(int)v0.x & keep, (int)v0.y & keep, (int)v0.z & keep, (int)v0.w & keep,
                              (int)v1.x & keep, (int)v1.y & keep, (int)v1.z & keep, (int)v1.w & keep};
    }
  }

  const uint8_t* kb_ptr = kptr + (int64_t)b * Nk * kD;
  const float* sc_ptr = kscale + (int64_t)b * Nk;
  // lane's B-fragment byte offsets inside a column block: chunks 2g, 2g+1 of row p16
  const uint32_t rd0 = (uint32_t)p16 * kQ8Row + (uint32_t)(((2 * g) ^ q8_swz(p16)) << 4);
  const uint32_t rd1 = (uint32_t)p16 * kQ8Row + (uint32_t)(((2 * g + 1) ^ q8_swz(p16)) << 4);

  q8_stage(kb_ptr, sc_ptr, k0, Nk, kstride, lane, wave, s_k0, s_sc0);
  __builtin_amdgcn_s_waitcnt(0);   // prologue loads (q, w, heads) and the first tile
  __syncthreads();
  const float ninf = -__builtin_inff();
  const int pol = kstride == 1 ? kStream : 0;
  uint32_t run[2] = {0u, 0u};   // kCands: groups found for the lane's query so far
  const uint64_t gmask = 0xFFFFull << (16 * g);
  // stores a wave issues per tile (issued after the next tile's loads, which
  // the wait before each barrier must cover)
  constexpr int kTileStores = MODE == kLogits ? 2 : 4;

  auto tile = [&](auto buf_tag, int key0) {
    constexpr int BUF = decltype(buf_tag)::value;
    const unsigned char* sk = BUF ? s_k1 : s_k0;
    const float* ssc = BUF ? s_sc1 : s_sc0;
    const int kg = key0 + 4 * p16;
    f32x4 out[2];
    if (key0 > t_hi) {
      out[0] = f32x4{ninf, ninf, ninf, ninf};
      out[1] = out[0];
    } else {
      // DIAG: some key of the tile may lie after some query of the wave; only
      // those tiles pay for the causal mask
      auto scores = [&](auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;
#pragma unroll
        for (int kb = 0; kb < KT / 16; ++kb) {
          const uint4 b0 = *reinterpret_cast<const uint4*>(sk + kb * 16 * kQ8Row + rd0);
          const uint4 b1 = *reinterpret_cast<const uint4*>(sk + kb * 16 * kQ8Row + rd1);
          const i32x8 bf = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          const float sc = ssc[kb * 16 + p16];
#pragma unroll
          for (int G = 0; G < 2; ++G) {
            const f32x4 a0 = mfma_f8(afr[2 * G], bf);
            const f32x4 a1 = mfma_f8(afr[2 * G + 1], bf);
            const float P0 = quad_chain(a0, wv[G][0], wv[G][1], wv[G][2], wv[G][3]);
            const float P1 = quad_chain(a1, wv[G][4], wv[G][5], wv[G][6], wv[G][7]);
            float s = (P0 + P1) * sc;
            if (DIAG && kg + kb > tq[G]) s = ninf;
            out[G][kb] = s;
          }
        }
      };
      if (key0 + KT - 1 > t_lo)
        scores(std::true_type{});
      else
        scores(std::false_type{});
    }
    if (MODE == kLogits) {
      const uint32_t off = (kg < N) ? lane_row_off + (uint32_t)kg * 4u : kDrop;
      store_f32x4(orsrc[0], off, out[0], pol);
      store_f32x4(orsrc[1], off, out[1], pol);
    } else {
#pragma unroll
      for (int G = 0; G < 2; ++G) append_group(orsrc, out[G], thr[G], gmask, run[G], reg[G], out_spec.cap, kg);
    }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  for (int jt = 0; jt < n_tiles; jt += 2) {
    const int key0 = k0 + jt * KT;
    q8_stage(kb_ptr, sc_ptr, key0 + KT, Nk, kstride, lane, wave, s_k1, s_sc1);   // tile jt+1
    tile(B0{}, key0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kTileStores));   // this wave's loads of tile jt+1 (its stores may fly)
    __syncthreads();
    if (jt + 1 < n_tiles) {
      q8_stage(kb_ptr, sc_ptr, key0 + 2 * KT, Nk, kstride, lane, wave, s_k0, s_sc0);   // tile jt+2
      tile(B1{}, key0 + KT);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kTileStores));
      __syncthreads();
    }
  }
  if (MODE == kLogits) {
    // keys of this range after the last computed tile: -inf for every query
    fill_neg_inf(out_spec.logits, out_spec.ld, tc.orow0, qa, qb, k0 + (int64_t)n_tiles * KT, k1, tid, 256);
  } else {
#pragma unroll
    for (int G = 0; G < 2; ++G) {
      const int qo = q0w + 4 * G + g;
      if (qo < qb && p16 == 0) out_spec.rcount[(qrow0 + qo) * n_ksplits + split] = run[G];
    }
  }
}

// Dense (all-head) fp8 scoring, the fp8-query DSA comparator:
//   D[t,s] = sigma[s] * sum_{j < H} w[t,j] q_scale[t,j] ReLU(q8[t,j] . k8[s]),
// -inf after t.  One query per wave with its H head rows resident in
// registers as NG row blocks of 16 heads (8 VGPRs each: a whole 128-byte
// row per MFMA), 4 queries per workgroup, the 64-key fp8 tiles of
// k_score_q8.  In the D layout lane group g holds head quad g of each block,
// so a quad's terms are lane-local and the block sum (P0+P1)+(P2+P3) is two
// butterfly adds; blocks add in order (the head order of the bf16 dense
// kernel).  Lane group 0 stores a tile's 4 consecutive logits per lane.
template <int NG>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
k_score_dense_q8(const uint8_t* __restrict__ q8,
                 const float* __restrict__ q_scale,
                 const float* __restrict__ w, const uint8_t* __restrict__ kptr,
                 const float* __restrict__ kscale, float* __restrict__ logits,
                 int64_t ld, int64_t N64, int64_t q_pos0_64, int M, int H,
                 int n_qtiles, int n_ksplits, int64_t KR) {
  constexpr int KT = kQ8KT, QT = 4;
  __shared__ __attribute__((aligned(16))) unsigned char s_k0[kQ8Tile], s_k1[kQ8Tile];
  __shared__ float s_sc0[KT], s_sc1[KT];

  const int Nk = (int)N64, q_pos0 = (int)q_pos0_64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, p16 = lane & 15;
  const int b = blockIdx.y;
  const TileCoords tc = tile_coords(n_qtiles, n_ksplits, KR, Nk);
  const int k0 = (int)tc.k0, k1 = (int)tc.k1;
  const int qa = tc.qt * QT, qb = min(qa + QT, M);
  const int64_t qrow0 = (int64_t)b * M;
  const int t_last = q_pos0 + qb - 1;
  const int kend = min(k1, t_last + 1);
  const int n_tiles = kend > k0 ? (kend - k0 + KT - 1) / KT : 0;
  const int qi = qa + wave;   // this wave's query
  const bool qok = qi < qb;
  const int qic = min(qi, M - 1);
  const int tq = qok ? q_pos0 + qi : -1;

  i32x8 afr[NG];
  float wq[NG][4];
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    const int j = 16 * grp + p16;   // A row p16 of block grp
    const int jc = min(j, H - 1);
    const uint4* src = reinterpret_cast<const uint4*>(q8 + ((qrow0 + qic) * H + jc) * kD + 32 * g);
    const uint4 v0 = src[0], v1 = src[1];
    const int keep = (qok && j < H) ? -1 : 0;
    afr[grp] = i32x8{(int)v0.x & keep, (int)v0.y & keep, (int)v0.z & keep, (int)v0.w & keep,
                     (int)v1.x & keep, (int)v1.y & keep, (int)v1.z & keep, (int)v1.w & keep};
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // D rows 4g + i of block grp
      const int jd = 16 * grp + 4 * g + i;
      const int64_t r = (qrow0 + qic) * H + min(jd, H - 1);
      wq[grp][i] = w[r] * q_scale[r] * ((qok && jd < H) ? 1.f : 0.f);
    }
  }
  const __amdgpu_buffer_rsrc_t orsrc = uniform_rsrc(logits + (qrow0 + qic) * ld, qok ? (uint32_t)ld * 4u : 0u);

  const uint8_t* kb_ptr = kptr + (int64_t)b * Nk * kD;
  const float* sc_ptr = kscale + (int64_t)b * Nk;
  const uint32_t rd0 = (uint32_t)p16 * kQ8Row + (uint32_t)(((2 * g) ^ q8_swz(p16)) << 4);
  const uint32_t rd1 = (uint32_t)p16 * kQ8Row + (uint32_t)(((2 * g + 1) ^ q8_swz(p16)) << 4);

  q8_stage(kb_ptr, sc_ptr, k0, Nk, 1, lane, wave, s_k0, s_sc0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const float ninf = -__builtin_inff();

  auto tile = [&](auto buf_tag, int key0) {
    constexpr int BUF = decltype(buf_tag)::value;
    const unsigned char* sk = BUF ? s_k1 : s_k0;
    const float* ssc = BUF ? s_sc1 : s_sc0;
    const int kg = key0 + 4 * p16;
    f32x4 out = {ninf, ninf, ninf, ninf};
    if (key0 <= tq) {
      const bool diag = key0 + KT - 1 > tq;
#pragma unroll
      for (int kb = 0; kb < KT / 16; ++kb) {
        const uint4 b0 = *reinterpret_cast<const uint4*>(sk + kb * 16 * kQ8Row + rd0);
        const uint4 b1 = *reinterpret_cast<const uint4*>(sk + kb * 16 * kQ8Row + rd1);
        const i32x8 bf = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        float s = 0.f;
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) {
          const f32x4 acc = mfma_f8(afr[grp], bf);
          const float P = quad_chain(acc, wq[grp][0], wq[grp][1], wq[grp][2], wq[grp][3]);
          const float T = sum_rows(P);   // (P0+P1)+(P2+P3) on every lane
          s = s + T;
        }
        s *= ssc[kb * 16 + p16];
        if (diag && kg + kb > tq) s = ninf;
        out[kb] = s;
      }
    }
    store_f32x4(orsrc, (g == 0 && kg < Nk) ? (uint32_t)kg * 4u : kDrop, out, kStream);
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  for (int jt = 0; jt < n_tiles; jt += 2) {
    const int key0 = k0 + jt * KT;
    q8_stage(kb_ptr, sc_ptr, key0 + KT, Nk, 1, lane, wave, s_k1, s_sc1);   // tile jt+1
    tile(B0{}, key0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(1));   // this wave's loads of tile jt+1 (its store may fly)
    __syncthreads();
    if (jt + 1 < n_tiles) {
      q8_stage(kb_ptr, sc_ptr, key0 + 2 * KT, Nk, 1, lane, wave, s_k0, s_sc0);   // tile jt+2
      tile(B1{}, key0 + KT);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(1));
      __syncthreads();
    }
  }
  fill_neg_inf(logits, ld, (int64_t)b * M, qa, qb, k0 + (int64_t)n_tiles * KT, k1, tid, 256);
}

hipError_t launch_dense_q8(const misa_shape& s, const uint8_t* q8, const float* q_scale, const float* w,
                           const uint8_t* k, const float* k_scale, float* logits, int64_t ld, hipStream_t st) {
  const int M = s.q_per_seq;
  const int n_qtiles = (M + 3) / 4;
  int nks;
  int64_t KR;
  plan_split(s.n_keys, s.n_seq, n_qtiles, kQ8KT, &nks, &KR);
  dim3 grid((unsigned)((int64_t)n_qtiles * nks), (unsigned)s.n_seq);
  const int ng = (s.n_heads + 15) / 16;
#define MISA_DQ8(NG_)                                                                                       \
  hipLaunchKernelGGL(k_score_dense_q8<NG_>, grid, dim3(256), 0, st, q8, q_scale, w, k, k_scale, logits, ld, \
                     s.n_keys, s.q_pos0, M, s.n_heads, n_qtiles, nks, KR)
  switch (ng) {
    case 1: MISA_DQ8(1); break;
    case 2: MISA_DQ8(2); break;
    case 3: MISA_DQ8(3); break;
    default: MISA_DQ8(4); break;
  }
#undef MISA_DQ8
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_q8(const misa_shape& s, const uint8_t* q8, const float* q_scale, const float* w,
                            const uint8_t* k, const float* k_scale, const int32_t* heads, int h, const ScoreOut& o,
                            int kstride, int nks, int64_t KR, hipStream_t st) {
  const int M = s.q_per_seq;
  const int n_qtiles = (M + 31) / 32;
  dim3 grid((unsigned)((int64_t)n_qtiles * nks), (unsigned)s.n_seq);
  if (o.slab_tiles > 0) grid = dim3((unsigned)((int64_t)o.slab_tiles * nks), 1);
  hipLaunchKernelGGL(k_score_q8<MODE>, grid, dim3(256), 0, st, q8, q_scale, w, k, k_scale, heads, h, o, s.n_keys,
                     kstride, s.q_pos0, M, s.n_heads, n_qtiles, nks, KR);
  return hipGetLastError();
}

hipError_t launch_score_q8(const misa_shape& s, const uint8_t* q8, const float* q_scale, const float* w,
                          const uint8_t* k, const float* k_scale, const int32_t* heads, int h, float* logits,
                          int64_t ld, hipStream_t st, const uint32_t* row_flag, const SlabBatch* slab) {
  int nks;
  int64_t KR;
  const int n_qtiles = (s.q_per_seq + 31) / 32;
  plan_split(s.n_keys, s.n_seq, n_qtiles, kQ8KT, &nks, &KR);
  ScoreOut o{logits, ld, nullptr, nullptr, nullptr, nullptr, 0, row_flag};
  if (slab != nullptr) {
    o.slab_tiles = slab->tiles;
    o.slab_first = (int)slab->first;
    o.slab_tr = slab->tr;
    o.n_flat = s.n_seq * n_qtiles;
  }
  return launch_q8<kLogits>(s, q8, q_scale, w, k, k_scale, heads, h, o, 1, nks, KR, st);
}

hipError_t launch_score_q8_sampled(const misa_shape& s, const uint8_t* q8, const float* q_scale, const float* w,
                                   const uint8_t* k, const float* k_scale, const int32_t* heads, int h,
                                   const FusedPlan& p, float* sample_logits, hipStream_t st) {
  int nks;
  int64_t KR;
  plan_split(p.n_sample, s.n_seq, (s.q_per_seq + 31) / 32, kQ8KT, &nks, &KR);
  const ScoreOut o{sample_logits, p.ld_sample, nullptr, nullptr, nullptr, nullptr, 0, nullptr};
  return launch_q8<kLogits>(s, q8, q_scale, w, k, k_scale, heads, h, o, p.kstride, nks, KR, st);
}

hipError_t launch_score_q8_cands(const misa_shape& s, const uint8_t* q8, const float* q_scale, const float* w,
                                 const uint8_t* k, const float* k_scale, const int32_t* heads, int h,
                                 const FusedPlan& p, const float* thr, float* gvals, int32_t* gkeys, uint32_t* rcount,
                                 hipStream_t st) {
  static_assert(kQ8KT == 64, "the fused plan's key ranges are multiples of 64 keys");
  const ScoreOut o{nullptr, 0, thr, reinterpret_cast<f32x4*>(gvals), gkeys, rcount, p.cap_region, nullptr};
  return launch_q8<kCands>(s, q8, q_scale, w, k, k_scale, heads, h, o, 1, p.n_splits, p.key_range, st);
}

}  // namespace misa
