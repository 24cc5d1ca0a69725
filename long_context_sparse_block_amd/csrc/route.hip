// Block-summary head router.
//
// Method (gist.science summary of MISA, "Metodologia: MISA" item 1;
// agents-report summary, method overview and the HISA comparison): every
// indexer head is scored against the mean-pooled block keys, the per-block
// affinities are aggregated along the blocks into one importance per head,
// and the top-h heads are kept for the query.  Reading taken here:
//   S[t,j] = sum_{complete blocks m of t's prefix} ReLU(q[t,j] . pooled[m])
//            + ReLU(q[t,j] . tail[t])      (partial block, when non-empty)
//   r[t,j] = w[t,j] * S[t,j];  heads(t) = top-h of r, equal r -> lower j.
//
// Design.  The (query, head) x (block) products are a dense contraction, so
// they run on bf16 MFMA: q is bf16 already, and each fp32 pooled key is split
// into hi + lo bf16 parts when it is staged (p - hi is exact in fp32;
// |p - hi - lo| <= 2^-16 |p|), so q.p = q.hi + q.lo is accumulated by two
// MFMAs into the same fp32 accumulator (bf16 pooled keys alone are not
// accurate enough where a block's dot product cancels).  A wave owns
// 4 queries x 16 heads (four 16x16 row blocks: row r = query r/4, head
// 4*rb + r%4), keeps its q fragments in registers and streams 64-block chunks
// of pooled keys staged once per workgroup in LDS (XOR-swizzled 256-byte rows,
// as in the scoring kernel, so the fragment reads are free of bank conflicts);
// a workgroup serves 4 (H = 64) to 16 (H <= 16) queries.  ReLU, the causal
// block mask and the block sum stay in registers; the partial block's term
// runs on the same resident q fragments (the wave's 4 tails as B columns, hi
// + lo), so q is read once; the top-h selection is a rank count over <= 64
// values, one wave per query.
#include <algorithm>
#include <type_traits>

#include "misa_common.h"
#include "misa_launch.h"

namespace misa {

constexpr int kRouteChunk = 64;            // pooled rows staged per step (register staging)
constexpr int kPreChunk = 32;              // rows per buffer of the direct-load staging
constexpr int kRowBytes = kD * 2;           // bf16 LDS row (256 bytes), 16-byte chunks XOR-swizzled

// byte offset of 16-byte chunk c of staged row j
__device__ __forceinline__ uint32_t rt_off(int j, int c) { return (uint32_t)j * kRowBytes + (uint32_t)((c ^ (j & 15)) << 4); }


// top-h of one query's r (lane j holds r_j, the wave's LDS row sr holds all
// of them) by rank counting, ties -> lower head id, stored ascending
__device__ __forceinline__ void select_heads(const float* sr, int H, int h, int64_t row, int32_t* heads,
                                             float* scores) {
  const int j = threadIdx.x & 63;
  const float rj = (j < H) ? sr[j] : 0.f;
  int cnt = 0;
  for (int jj = 0; jj < H; ++jj) {
    const float rv = sr[jj];
    cnt += (rv > rj) || (rv == rj && jj < j);
  }
  const bool sel = (j < H) && (cnt < h);
  const uint64_t mask = __ballot(sel);
  const int pos = __popcll(mask & ((1ull << j) - 1ull));
  if (sel) heads[row * h + pos] = j;
  if (scores != nullptr && j < H) scores[row * H + j] = rj;
}

// NHC: 16-head chunks per query group (= ceil(H/16)).  PRESPLIT: the pooled
// keys' bf16 hi and lo rows come precomputed (`split`: per sequence, ld_blk
// hi rows then ld_blk lo rows; the pooling kernel writes them with the same
// conversion) and are staged by direct global -> LDS loads.  Pooled rows are
// ld_blk blocks apart per sequence (a cache may hold more than this call's
// complete blocks).
template <int NHC, bool PRESPLIT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) k_route(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                               const float* __restrict__ pooled,
                                               const uint16_t* __restrict__ split,
                                               const float* __restrict__ tail,
                                               int32_t* __restrict__ heads, float* __restrict__ scores,
                                               int64_t q_pos0, int M, int H, int B, int h,
                                               int64_t ld_blk, int n_parts, float* __restrict__ part_out,
                                               int seq_parts) {
  constexpr int QG = (NHC == 1) ? 4 : (NHC == 2 ? 2 : 1);  // query groups per workgroup
  constexpr int NW = NHC * QG;                              // waves per workgroup
  constexpr int QWG = 4 * QG;                               // queries per workgroup
  // register staging: one 64-row chunk; direct loads (PRESPLIT): two buffers
  // of 32 rows, separate arrays so the compiler sees that loads into one never
  // alias reads of the other
  __shared__ __attribute__((aligned(16))) unsigned char s_hi[PRESPLIT ? 1 : kRouteChunk * kRowBytes];
  __shared__ __attribute__((aligned(16))) unsigned char s_lo[PRESPLIT ? 1 : kRouteChunk * kRowBytes];
  __shared__ __attribute__((aligned(16))) unsigned char s_h0[PRESPLIT ? kPreChunk * kRowBytes : 1];
  __shared__ __attribute__((aligned(16))) unsigned char s_l0[PRESPLIT ? kPreChunk * kRowBytes : 1];
  __shared__ __attribute__((aligned(16))) unsigned char s_h1[PRESPLIT ? kPreChunk * kRowBytes : 1];
  __shared__ __attribute__((aligned(16))) unsigned char s_l1[PRESPLIT ? kPreChunk * kRowBytes : 1];
  __shared__ float s_r[QWG][64];
  __shared__ float s_t[QWG][64];   // the partial blocks' terms

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qg = wave / NHC;
  const int hc = wave % NHC;
  const int b = blockIdx.y;
  const int q0_wg = blockIdx.x * QWG;
  const int q0w = q0_wg + qg * 4;
  const int g = lane >> 4;     // output row group -> query q0w + g
  const int p16 = lane & 15;

  // n_full of the last valid query of the workgroup bounds the chunk loop
  const int q_last = min(q0_wg + QWG, M) - 1;
  const int64_t nfull_wg = (q_pos0 + q_last + 1) / B;
  const int qi_out = q0w + g;
  const int64_t nfull_g = (qi_out < M) ? (q_pos0 + qi_out + 1) / B : 0;
  const int q_last_w = min(q0w + 4, M) - 1;
  const int64_t nfull_w = (q0w < M) ? (q_pos0 + q_last_w + 1) / B : 0;
  const int64_t nfull_lo = (q0w < M) ? (q_pos0 + q0w + 1) / B : 0;   // fewest complete blocks in the wave

  // q fragments: row r = lane%16 -> query q0w + r/4, head hc*16 + 4*rb + r%4
  bf16x8 afr[4][kKSteps];
  {
    const int qi = q0w + (p16 >> 2);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int j = hc * 16 + rb * 4 + (p16 & 3);
      const bool ok = (qi < M) && (j < H);
      const uint4* src = reinterpret_cast<const uint4*>(q + (((int64_t)b * M + (ok ? qi : 0)) * H + (ok ? j : 0)) * kD);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        uint4 v = ok ? src[ks * 4 + g] : make_uint4(0, 0, 0, 0);
        afr[rb][ks] = as_bf16x8(v);
      }
    }
  }

  float S[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) S[rb][i] = 0.f;

  // the block sum so far over the 16 block columns held by the 16 lanes of a
  // row group; lane (g, p16) keeps head hc*16 + p16 of query q0w + g.  The
  // lanes' running sums restart from 0.
  auto fold = [&]() -> float {
    float sel = 0.f;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = S[rb][i];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        if (p16 == rb * 4 + i) sel = v;
        S[rb][i] = 0.f;
      }
    return sel;
  };
  // A block sum split into parts (part z of n covers blocks [z per, (z+1) per),
  // per a multiple of 64) is added part by part: over workgroups (blockIdx.z,
  // n_parts > 1, finished by k_route_finish) or here in order (seq_parts > 1),
  // so that both give the same sum bit for bit.
  const int n_split = n_parts > 1 ? n_parts : seq_parts;
  const int64_t per = ((nfull_wg + n_split - 1) / n_split + 2 * kPreChunk - 1) / (2 * kPreChunk) * (2 * kPreChunk);
  float s_acc = 0.f;   // seq_parts > 1: the parts folded so far

  // column block cb (16 pooled rows from row cbase + 16 cb of the chunk) of a
  // staged chunk: hi/lo fragments from LDS, 8 MFMAs per row block, ReLU and
  // the block sum in registers
  auto block = [&](const unsigned char* sh, const unsigned char* sl, int cb, int64_t col0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    bf16x8 bh[kKSteps], bl[kKSteps];
    const int row = cb * 16 + p16;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      bh[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(&sh[rt_off(row, ks * 4 + g)]));
      bl[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(&sl[rt_off(row, ks * 4 + g)]));
    }
    const bool valid = !MASK || (col0 + p16) < nfull_g;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        acc = mfma16(afr[rb][ks], bh[ks], acc);
        acc = mfma16(afr[rb][ks], bl[ks], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) S[rb][i] += (MASK && !valid) ? 0.f : relu(acc[i]);
    }
  };
  auto chunk_blocks = [&](const unsigned char* sh, const unsigned char* sl, int64_t cbase, int ncb) {
    if (cbase + 16 * ncb <= nfull_lo) {
      // every block of the chunk is complete for every query of the wave: no
      // branch between the column blocks, so their MFMAs and epilogues overlap
#pragma unroll
      for (int cb = 0; cb < ncb; ++cb) block(sh, sl, cb, cbase + cb * 16, std::false_type{});
      return;
    }
#pragma unroll
    for (int cb = 0; cb < ncb; ++cb) {
      const int64_t col0 = cbase + cb * 16;
      if (col0 < nfull_w) {
        // only column blocks reaching past the wave's first query's complete
        // blocks need the per-lane mask
        if (col0 + 16 <= nfull_lo)
          block(sh, sl, cb, col0, std::false_type{});
        else
          block(sh, sl, cb, col0, std::true_type{});
      }
    }
  };

  if (PRESPLIT) {
    // 32-row chunks of the hi/lo rows by direct global -> LDS loads, the next
    // chunk in flight while this one is scored: load u of a chunk's 16 (8 of
    // hi rows, 8 of lo rows) fills rows r0 .. r0+3, lane l writing slot l % 16
    // of row r0 + l / 16, i.e. chunk (l % 16) ^ (row % 16) of that row (the
    // rt_off layout)
    typedef __attribute__((address_space(3))) void* lds_ptr;
    const uint16_t* hb0 = split + (int64_t)b * 2 * ld_blk * kD;
    const int64_t lo_off = ld_blk * kD;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    // part blockIdx.z of n_parts covers the blocks [c_lo, c_hi)
    const int64_t c_lo = n_parts > 1 ? (int64_t)blockIdx.z * per : 0;
    const int64_t c_hi = n_parts > 1 ? min(nfull_wg, c_lo + per) : nfull_wg;
    auto stage = [&](int64_t cbase, unsigned char* sh, unsigned char* sl) {
      const int64_t nrows = max((int64_t)0, min((int64_t)kPreChunk, c_hi - cbase));   // zeros past it
      const __amdgpu_buffer_rsrc_t rh = uniform_rsrc(hb0 + cbase * kD, (uint32_t)nrows * kRowBytes);
      const __amdgpu_buffer_rsrc_t rl = uniform_rsrc(hb0 + lo_off + cbase * kD, (uint32_t)nrows * kRowBytes);
      for (int u = wv; u < 2 * (kPreChunk / 4); u += NW) {
        const int part = u / (kPreChunk / 4), r0 = (u % (kPreChunk / 4)) * 4;
        const int j = r0 + (lane >> 4);
        const int c = (lane & 15) ^ (j & 15);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(part ? rl : rh, (lds_ptr)((part ? sl : sh) + r0 * kRowBytes), 16,
                                                 (uint32_t)(j * kRowBytes + c * 16), 0, 0, 0);
      }
    };
    stage(c_lo, s_h0, s_l0);
    __builtin_amdgcn_s_waitcnt(0);   // (also the q fragments)
    __syncthreads();
    for (int64_t cbase = c_lo; cbase < c_hi; cbase += 2 * kPreChunk) {
      if (seq_parts > 1 && cbase > 0 && cbase % per == 0) s_acc += fold();
      stage(cbase + kPreChunk, s_h1, s_l1);   // rows past c_hi: an empty range, no data
      chunk_blocks(s_h0, s_l0, cbase, kPreChunk / 16);
      __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of the next chunk (no other memory ops in flight)
      __syncthreads();
      if (cbase + kPreChunk < c_hi) {
        stage(cbase + 2 * kPreChunk, s_h0, s_l0);
        chunk_blocks(s_h1, s_l1, cbase + kPreChunk, kPreChunk / 16);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
  } else {
  const float* pool_b = pooled + (int64_t)b * ld_blk * kD;
  for (int64_t cbase = 0; cbase < nfull_wg; cbase += kRouteChunk) {
    if (seq_parts > 1 && cbase > 0 && cbase % per == 0) s_acc += fold();
    // stage pooled rows [cbase, cbase+64) as bf16 hi/lo
    constexpr int kTotal = kRouteChunk * (kD / 4);                 // float4 of a chunk
    constexpr int kPer = (kTotal + NW * 64 - 1) / (NW * 64);       // per thread (3 waves: ragged)
    constexpr int kBatch = NW == 4 ? 4 : 2;   // loads in flight per batch (3 waves: ragged, fewer registers)
#pragma unroll 1   // (unrolled, the compiler keeps both batches live and spills)
    for (int u0 = 0; u0 < kPer; u0 += kBatch) {
      float4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int e = tid + (u0 + u) * NW * 64;
        const int row = e / (kD / 4);
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (u0 + u < kPer && e < kTotal && cbase + row < nfull_wg) v[u] = reinterpret_cast<const float4*>(pool_b + (cbase + row) * kD)[e % (kD / 4)];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int e = tid + (u0 + u) * NW * 64;
        const int row = e / (kD / 4);
        const int c4 = e % (kD / 4);
        if (u0 + u >= kPer || e >= kTotal) break;
        const uint32_t h01 = pk_bf16(v[u].x, v[u].y), h23 = pk_bf16(v[u].z, v[u].w);
        // f - hi is exact in fp32
        const uint32_t l01 = pk_bf16(v[u].x - __uint_as_float(h01 << 16), v[u].y - __uint_as_float(h01 & 0xFFFF0000u));
        const uint32_t l23 = pk_bf16(v[u].z - __uint_as_float(h23 << 16), v[u].w - __uint_as_float(h23 & 0xFFFF0000u));
        const uint32_t o = rt_off(row, c4 >> 1) + (c4 & 1) * 8;
        *reinterpret_cast<uint2*>(&s_hi[o]) = make_uint2(h01, h23);
        *reinterpret_cast<uint2*>(&s_lo[o]) = make_uint2(l01, l23);
      }
    }
    __syncthreads();
    chunk_blocks(s_hi, s_lo, cbase, kRouteChunk / 16);
    __syncthreads();
  }
  }

  // lane (g, p16) handles head hc*16 + p16 of query q0w + g
  float s_sel = fold();
  if (seq_parts > 1) s_sel = s_acc + s_sel;
  const int qi_o = q0w + g;
  const int j_o = hc * 16 + p16;
  const bool own = qi_o < M && j_o < H;
  if (n_parts > 1) {
    // one part of the block sum: k_route_finish adds the parts (in order), then
    // the partial block's term, which part 0 also writes (slot n_parts)
    if (own) part_out[(((int64_t)b * M + qi_o) * (n_parts + 1) + blockIdx.z) * H + j_o] = s_sel;
    if (blockIdx.z != 0) return;   // uniform over the workgroup
  }
  // The partial block's term ReLU(q . tail) on the resident q fragments: the
  // wave's 4 tails (fp32, split into bf16 hi + lo like the pooled keys) are
  // the B columns 0..3, so the product of query g's rows with column g sits in
  // lane (g, g); it reaches the lanes that own the heads through LDS.  A query
  // whose prefix ends on a block boundary has a zero tail: a zero term.
  {
    bf16x8 th[kKSteps], tl[kKSteps];
    const int qc = q0w + p16;
    const bool col_ok = p16 < 4 && qc < M;
    const float4* tr = reinterpret_cast<const float4*>(tail + ((int64_t)b * M + (col_ok ? qc : 0)) * kD);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      float4 v0 = col_ok ? tr[(ks * 32 + 8 * g) / 4] : make_float4(0.f, 0.f, 0.f, 0.f);
      float4 v1 = col_ok ? tr[(ks * 32 + 8 * g) / 4 + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
      const uint32_t h01 = pk_bf16(v0.x, v0.y), h23 = pk_bf16(v0.z, v0.w);
      const uint32_t h45 = pk_bf16(v1.x, v1.y), h67 = pk_bf16(v1.z, v1.w);
      // f - hi is exact in fp32
      const uint32_t l01 = pk_bf16(v0.x - __uint_as_float(h01 << 16), v0.y - __uint_as_float(h01 & 0xFFFF0000u));
      const uint32_t l23 = pk_bf16(v0.z - __uint_as_float(h23 << 16), v0.w - __uint_as_float(h23 & 0xFFFF0000u));
      const uint32_t l45 = pk_bf16(v1.x - __uint_as_float(h45 << 16), v1.y - __uint_as_float(h45 & 0xFFFF0000u));
      const uint32_t l67 = pk_bf16(v1.z - __uint_as_float(h67 << 16), v1.w - __uint_as_float(h67 & 0xFFFF0000u));
      th[ks] = as_bf16x8(make_uint4(h01, h23, h45, h67));
      tl[ks] = as_bf16x8(make_uint4(l01, l23, l45, l67));
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        acc = mfma16(afr[rb][ks], th[ks], acc);
        acc = mfma16(afr[rb][ks], tl[ks], acc);
      }
      if (p16 == g) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s_t[qg * 4 + g][hc * 16 + rb * 4 + i] = relu(acc[i]);
      }
    }
  }
  __syncthreads();
  {
    const float tterm = own ? s_t[qg * 4 + g][j_o] : 0.f;
    if (n_parts > 1) {
      if (own) part_out[(((int64_t)b * M + qi_o) * (n_parts + 1) + n_parts) * H + j_o] = tterm;
      return;   // uniform over the workgroup (part 0)
    }
    if (own) {
      const int64_t row = (int64_t)b * M + qi_o;
      s_r[qg * 4 + g][j_o] = w[row * H + j_o] * (s_sel + tterm);
    }
  }
  __syncthreads();

  // top-h per query by rank counting (ties -> lower head id), stored ascending
  for (int ql = wave; ql < QWG; ql += NW) {
    const int qi = q0_wg + ql;
    if (qi >= M) continue;
    select_heads(s_r[ql], H, h, (int64_t)b * M + qi, heads, scores);
  }
}

// Parts of a split block sum (few queries: decode) -> S, r and the top-h: one
// wave per query, lane j the head; the parts are added in order, then the
// partial block's term (slot n_parts, written by part 0), as the unsplit
// kernel adds its running sum and then that term.
__global__ void __launch_bounds__(256) k_route_finish(const float* __restrict__ w, const float* __restrict__ part,
                                                      int n_parts, int32_t* __restrict__ heads,
                                                      float* __restrict__ scores, int H, int h, int64_t rows) {
  __shared__ float s_r[4][64];
  const int wave = threadIdx.x >> 6, j = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= rows) return;   // uniform over the wave; no workgroup barrier below
  float r = 0.f;
  if (j < H) {
    float S = 0.f;
    for (int p = 0; p < n_parts; ++p) S += part[(row * (n_parts + 1) + p) * H + j];
    S += part[(row * (n_parts + 1) + n_parts) * H + j];   // the partial block's term
    r = w[row * H + j] * S;
  }
  s_r[wave][j] = r;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  select_heads(s_r[wave], H, h, row, heads, scores);
}

int route_parts(const misa_shape& s) {
  const int nhc = (s.n_heads + 15) / 16;
  const int qwg = 4 * ((nhc == 1) ? 4 : (nhc == 2 ? 2 : 1));
  const int64_t wgs = (int64_t)((s.q_per_seq + qwg - 1) / qwg) * s.n_seq;
  const int64_t nfull_max = (s.q_pos0 + s.q_per_seq) / s.block;
  if (wgs == 0 || wgs >= 256 || nfull_max < 256) return 1;   // (no queries: nothing to split)
  return (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)kMaxRouteParts, (512 + wgs - 1) / wgs, nfull_max / 128}));
}

hipError_t launch_route(const misa_shape& s, const uint16_t* q, const float* w, const float* pooled,
                        const uint16_t* split, const float* tail, int h, int32_t* heads, float* scores,
                        hipStream_t st, int64_t ld_blk, float* part_ws) {
  const int H = s.n_heads;
  const int nhc = (H + 15) / 16;
  const int qg = (nhc == 1) ? 4 : (nhc == 2 ? 2 : 1);
  const int qwg = 4 * qg;
  const int64_t n_full_total = ld_blk < 0 ? s.n_keys / s.block : ld_blk;
  // few workgroups (decode) and long prefixes: split each workgroup's block
  // sum into parts over more workgroups, then a finishing kernel
  const int n_parts = (part_ws != nullptr && split != nullptr) ? route_parts(s) : 1;
  // without the part workspace, the same parts are added in order in-kernel
  const int seq_parts = n_parts > 1 ? 1 : route_parts(s);
  dim3 grid((unsigned)((s.q_per_seq + qwg - 1) / qwg), (unsigned)s.n_seq, (unsigned)n_parts);
  dim3 block((unsigned)(64 * nhc * qg));
#define MISA_ROUTE_LAUNCH(NHC_)                                                                          \
  if (split != nullptr)                                                                                   \
    hipLaunchKernelGGL((k_route<NHC_, true>), grid, block, 0, st, q, w, pooled, split, tail, heads, scores, \
                       s.q_pos0, s.q_per_seq, H, s.block, h, n_full_total, n_parts, part_ws, seq_parts); \
  else                                                                                                    \
    hipLaunchKernelGGL((k_route<NHC_, false>), grid, block, 0, st, q, w, pooled, split, tail, heads,      \
                       scores, s.q_pos0, s.q_per_seq, H, s.block, h, n_full_total, 1, nullptr, seq_parts)
  switch (nhc) {
    case 1: MISA_ROUTE_LAUNCH(1); break;
    case 2: MISA_ROUTE_LAUNCH(2); break;
    case 3: MISA_ROUTE_LAUNCH(3); break;
    default: MISA_ROUTE_LAUNCH(4); break;
  }
#undef MISA_ROUTE_LAUNCH
  if (n_parts > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)s.n_seq * s.q_per_seq;
    hipLaunchKernelGGL(k_route_finish, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, w, part_ws, n_parts,
                       heads, scores, H, h, rows);
  }
  return hipGetLastError();
}

}  // namespace misa
