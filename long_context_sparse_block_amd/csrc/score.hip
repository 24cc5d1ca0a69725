// Token scoring: routed heads (MISA) and all heads (the dense DSA indexer).
//
//   I[t,s] = sum_{j in heads(t)} w[t,j] * ReLU(q[t,j] . k[s]) * sigma[s],  s <= t
//   I[t,s] = -inf,                                                          t < s < N
// (DSA indexer score; MISA scores every prefix token with the h routed heads
// only: gist.science summary of MISA, "Metodologia: MISA" item 2.  The
// fp8 scale sigma > 0 commutes with ReLU, so it is applied once after the
// head sum.)
//
// Design (gfx950).  The (query, head) x key products are a dense contraction
// on v_mfma_f32_16x16x32_bf16.  K tiles of 64 keys are staged in LDS once per
// workgroup in a swizzled layout (fp8 codes widened to bf16 on the way in:
// exact), double buffered, and shared by the workgroup's waves; q fragments
// sit in registers for the whole key range.  Workgroups are (query tile x key
// range); the key-range split is mapped so that each XCD sweeps one key range,
// keeping that slice of K resident in the XCD's L2.
//   k_score_h8 (h <= 8): a 16-row MFMA block holds 4 queries x 4 heads, so
//     each lane gets all four heads of one (query, key) and the epilogue is
//     lane-local with no shuffles.
//   k_score_q64 (h > 8, and the dense indexer's H heads): one query per wave,
//     all its head rows resident as 16-head row blocks.
//
// Summation order (fixed; every kernel that must agree bitwise uses it):
//   quad partial  P = fma chain over the quad's 4 heads in ascending order, from 0
//   16-head group T = (P0 + P1) + (P2 + P3)
//   total         s = (((0 + T_0) + T_1) + ...) over 16-head groups ascending
//   then s *= sigma (fp8).
// k_score_q64 and the re-rank gather follow it exactly; k_score_h8 (h <= 8)
// uses s = P0 + P1, which is the same value (the missing quads are exact zeros).
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "misa_common.h"
#include "misa_launch.h"
#include "score_shared.h"

namespace misa {

// ---------------------------------------------------------------------------
// Swizzled K tile for k_score_h8 (64 keys, bf16 rows of 256 bytes).
//
// Column order.  LDS row j holds tile key 4*(j % 16) + j / 16, so MFMA column
// block kb (rows 16*kb .. 16*kb+15) gives lane column c the key 4*c + kb: over
// the four blocks of a tile a lane collects 4 consecutive keys and stores them
// with one 16-byte write.
//
// Bank layout.  gfx950 LDS has 64 four-byte banks; a ds_read_b128 is served in
// passes of 16 lanes, a pass being the lanes with equal bit 5 and equal parity
// of bits 2..4 of the lane id (measured with two-lane bank-conflict probes).
// Chunk c (16 bytes) of row j is stored at slot c ^ (j % 16) of the row, so
// for the B-fragment read (lane = 16*g + col reads chunk 4*ks + g of row
// 16*kb + col) every pass touches 16 distinct slots, and so does every staging
// write (16 consecutive lanes write 16 distinct slots).  No padding.
// ---------------------------------------------------------------------------
constexpr int kSwKT = 64;                       // keys per tile
constexpr int kSwRowBytes = kD * 2;             // 256
constexpr int kSwTileBytes = kSwKT * kSwRowBytes;

__device__ __forceinline__ int sw_tile_key(int j) { return (j & 15) * 4 + (j >> 4); }
__device__ __forceinline__ uint32_t sw_off(int j, int chunk) {
  return (uint32_t)j * kSwRowBytes + (uint32_t)((chunk ^ (j & 15)) << 4);
}

template <int KDT, int NT>
struct KStageSw {
  static constexpr int kVecPerKey = (KDT == MISA_K_BF16) ? 16 : 8;   // 16-byte global chunks per key
  static constexpr int kRowBytes = kVecPerKey * 16;
  static constexpr int kPerThread = kSwKT * kVecPerKey / NT;
  static_assert(kSwKT * kVecPerKey % NT == 0, "tile not divisible");
  uint4 r[kPerThread];
  float sc;

  // Tile keys [key0, key0 + 64) of the key sequence 0, ks, 2 ks, ... (ks = 1:
  // every key) through descriptors based at the tile and bounded by the N
  // keys (rows past N read as zeros; their logits are never kept).  Thread
  // chunk e fills LDS row e / kVecPerKey, i.e. tile key sw_tile_key(row).
  // pages != nullptr: kbase / sbase are page pools, the tile's rows found
  // through sequence b's block table (ks == 1; the tile lies in one page)
  __device__ __forceinline__ void load(const void* kbase, const float* sbase, int key0, int N, int ks, int tid,
                                       const KeyPages* pages = nullptr, int b = 0) {
    const int64_t first = (int64_t)key0 * ks;   // position of the tile's first key
    if (pages != nullptr && ks > 1) {
      // sampled keys lie on different pages: each key row is looked up
      // through the block table (rows past N read as zeros)
#pragma unroll
      for (int u = 0; u < kPerThread; ++u) {
        const int e = tid + u * NT;
        const int j = e / kVecPerKey, c = e % kVecPerKey;
        const int64_t key = first + (int64_t)sw_tile_key(j) * ks;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (key < N)
          v = *reinterpret_cast<const uint4*>(static_cast<const char*>(kbase) + paged_row(*pages, b, key) * kRowBytes +
                                              c * 16);
        r[u] = v;
      }
      if (KDT == MISA_K_FP8_E4M3) {
        const int64_t key = first + (int64_t)sw_tile_key(tid % kSwKT) * ks;
        sc = key < N ? sbase[paged_row(*pages, b, key)] : 0.f;
      }
      return;
    }
    const int rem = (int)max((int64_t)0, min((int64_t)kSwKT * ks, (int64_t)N - first));   // keys in range
    const int64_t row0 = pages != nullptr ? paged_row(*pages, b, first) : first;
    const __amdgpu_buffer_rsrc_t kr =
        uniform_rsrc(static_cast<const char*>(kbase) + row0 * kRowBytes, (uint32_t)rem * kRowBytes);
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int e = tid + u * NT;
      const int j = e / kVecPerKey, c = e % kVecPerKey;
      r[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           kr, (uint32_t)(sw_tile_key(j) * ks) * kRowBytes + c * 16, 0, 0));
    }
    if (KDT == MISA_K_FP8_E4M3) {
      const __amdgpu_buffer_rsrc_t sr = uniform_rsrc(sbase + row0, (uint32_t)rem * 4u);
      sc = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(sr, (uint32_t)(sw_tile_key(tid % kSwKT) * ks) * 4u, 0, 0));
    }
  }

  __device__ __forceinline__ void store(unsigned char* s_k, float* s_sc, int tid) const {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int e = tid + u * NT;
      const int j = e / kVecPerKey, c = e % kVecPerKey;
      if (KDT == MISA_K_BF16) {
        *reinterpret_cast<uint4*>(s_k + sw_off(j, c)) = r[u];
      } else {
        const uint2 a = e4m3x4_to_bf16x4(r[u].x), b2 = e4m3x4_to_bf16x4(r[u].y);
        const uint2 c2 = e4m3x4_to_bf16x4(r[u].z), d2 = e4m3x4_to_bf16x4(r[u].w);
        *reinterpret_cast<uint4*>(s_k + sw_off(j, 2 * c)) = make_uint4(a.x, a.y, b2.x, b2.y);
        *reinterpret_cast<uint4*>(s_k + sw_off(j, 2 * c + 1)) = make_uint4(c2.x, c2.y, d2.x, d2.y);
      }
    }
    if (KDT == MISA_K_FP8_E4M3 && tid < kSwKT) s_sc[tid] = sc;
  }
};

// Tile staging straight from global memory into LDS (buffer loads with the
// LDS flag: no registers, no VALU), for bf16 keys in global memory (the
// input's, or fp8 keys widened once by k_widen_fp8).  A wave-wide load writes
// 16 bytes per lane to consecutive LDS slots from the address in M0, so wave
// v's load u fills LDS rows r0 .. r0+3, r0 = 4 (u NT/64 + v): lane l fills
// slot l % 16 of row r0 + l / 16, which holds chunk (l % 16) ^ (row % 16) of
// tile key sw_tile_key(row) -- the layout KStageSw writes.  With fp8 scales,
// every wave loads the tile's 64 scales (256 bytes) into the same LDS floats
// (identical data).  Rows past N read as zeros.
// AUX: cache policy of the loads (kStream when each key is read by one
// workgroup only: decode, one query tile per sequence)
template <int KDT, int NT, int AUX = 0>
__device__ __forceinline__ void dma_tile(const uint16_t* kbase, const float* sbase, int key0, int N, int ks,
                                         int lane, int wave, unsigned char* s_dst, float* s_sc_dst,
                                         const KeyPages* pages = nullptr, int b = 0) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  // 32-bit scalar arithmetic: N < 2^26 keys (the ABI checks it)
  const int first = key0 * ks;
  const int rem = max(0, min(kSwKT * ks, N - first));
  // pages: kbase / sbase are page pools (ks == 1; the tile lies in one page)
  const int64_t row0 = pages != nullptr ? paged_row(*pages, b, first) : (int64_t)first;
  const __amdgpu_buffer_rsrc_t kr = uniform_rsrc(kbase + row0 * kD, (uint32_t)rem * kSwRowBytes);
  constexpr int kLoads = kSwKT / 4 / (NT / 64);
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int r0 = (u * (NT / 64) + wave) * 4;
    const int j = r0 + (lane >> 4);
    const int c = (lane & 15) ^ (j & 15);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_ptr)(s_dst + r0 * kSwRowBytes), 16,
                                             (uint32_t)(sw_tile_key(j) * ks) * kSwRowBytes + c * 16, 0, 0, AUX);
  }
  if (KDT == MISA_K_FP8_E4M3) {
    const __amdgpu_buffer_rsrc_t sr = uniform_rsrc(sbase + row0, (uint32_t)rem * 4u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_ptr)s_sc_dst, 4, (uint32_t)(sw_tile_key(lane) * ks) * 4u, 0,
                                             0, AUX);
  }
}


// ---------------------------------------------------------------------------
// h <= 8: 8 queries per wave (2 groups x 2 head quads = 4 MFMA row blocks),
// 32 queries per workgroup, 64-key tiles in the swizzled layout above.  The B
// fragments of the next column block are read from LDS while the current
// block's 16 MFMAs and epilogue run.  After a tile each lane holds 4
// consecutive scores of 2 queries.
//   kLogits: each group is written with one 16-byte buffer store (rows past M
//   and key groups past N fall outside the store descriptor and are dropped; a
//   group straddling N also writes -inf into columns N .. roundup4(N)-1,
//   which lie inside the row).
//   kCands: a lane's group of 4 scores with one at or above the row
//   threshold is appended whole (a float4 and its first key) to the row's
//   region (positions from a ballot within the 16 lanes that hold one
//   query), through buffer stores that every lane issues (the others' are
//   dropped by the descriptor bounds).
// All loads are unconditional, so the compiler never waits on the stores.
// The tile loop is unrolled by two so both LDS buffers are addressed by
// immediates.  Keys are scored along the sequence 0, ks, 2 ks, ... (ks = 1:
// every key; a stride samples the keys): key index u < ceil(N / ks) is the key
// at position u ks, and query t sees indices u <= t / ks.  N is 32-bit here.
// ---------------------------------------------------------------------------
// Registers: the occupancy hint (at least 3 waves per SIMD: at most 168
// registers; 2 for the register-staged paged variants, which need a few more)
// keeps the MFMA accumulators in ordinary VGPRs.  Given room for more than 256
// registers the compiler accumulates in AGPRs and copies every result out with
// a v_accvgpr_read, 64 more VALU instructions per tile.
// NW: waves per workgroup (8 NW queries a query tile).  One wave (NW = 1)
// serves calls with at most 8 queries per sequence (decode): there the key
// stream is the whole cost, and four-wave workgroups would leave three waves
// without queries while each workgroup holds one tile in flight; one-wave
// workgroups take a quarter of the registers and the same LDS, so more of
// them, and more tiles in flight, fit on a CU.
template <int KDT, int MODE, bool DMA, bool PAGED = false, int NW = 4>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 1 ? 1 : (PAGED && !DMA ? 2 : 3))))
k_score_h8(const uint16_t* __restrict__ q,
           const float* __restrict__ w,
           const void* __restrict__ kptr,
           const float* __restrict__ kscale,
           const int32_t* __restrict__ heads, int h, ScoreOut out_spec,
           int64_t N64, int kstride, int64_t q_pos0_64, int M, int H,
           int n_qtiles, int n_ksplits, int64_t KR, KeyPages pages) {
  constexpr int NT = 64 * NW, KT = kSwKT, QT = 8 * NW;
  // B fragments read one column block ahead where the registers allow it
  // (16 more VGPRs; the other variants would drop to 2 waves per SIMD)
  constexpr bool kPrefetchB = MODE == kLogits && KDT == MISA_K_FP8_E4M3;
  // with direct loads the two tile buffers are separate arrays, so the
  // compiler can see that loads into one never alias reads of the other (one
  // array otherwise: the register-staged variants allocate better with it)
  __shared__ __attribute__((aligned(16))) unsigned char s_kk[DMA ? 1 : 2 * kSwTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char s_kd0[DMA ? kSwTileBytes : 1], s_kd1[DMA ? kSwTileBytes : 1];
  __shared__ float s_scc[DMA ? 1 : 2 * KT];
  __shared__ float s_scd0[DMA ? KT : 1], s_scd1[DMA ? KT : 1];
  unsigned char* const s_k0 = DMA ? s_kd0 : s_kk;
  unsigned char* const s_k1 = DMA ? s_kd1 : s_kk + kSwTileBytes;
  float* const s_sc0 = DMA ? s_scd0 : s_scc;
  float* const s_sc1 = DMA ? s_scd1 : s_scc + KT;

  const int Nk = (int)N64, q_pos0 = (int)q_pos0_64;   // keys; position of query 0
  const int N = (Nk + kstride - 1) / kstride;          // scored key indices
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) index
  const int g = lane >> 4, p16 = lane & 15;
  const WgTile tc = wg_tile<QT, MODE == kLogits>(out_spec, M, n_qtiles, n_ksplits, KR, N);
  if (!tc.valid) return;   // uniform over the workgroup
  const int b = tc.b;
  const int k0 = (int)tc.k0, k1 = (int)tc.k1;
  const int qa = tc.qt * QT;
  const int qb = min(qa + QT, M);
  const int64_t qrow0 = (int64_t)b * M;
  if (out_spec.row_flag != nullptr) {   // one flag per thread (QT <= 256), loaded together
    const bool mine = tid < qb - qa && out_spec.row_flag[qrow0 + qa + tid] != 0;
    if (!__syncthreads_or(mine)) return;   // uniform over the workgroup
  }
  const int t_last = (q_pos0 + qb - 1) / kstride;
  const int kend = min(k1, t_last + 1);   // key indices past kend are masked for every query
  const int n_tiles = kend > k0 ? (kend - k0 + KT - 1) / KT : 0;

  const int q0w = qa + wave * 8;
  const int t_lo = (q_pos0 + q0w) / kstride;                                   // first query of the wave
  const int t_hi = (q0w < qb) ? (q_pos0 + min(q0w + 8, qb) - 1) / kstride : -1;   // last one (-1: none)
  // A fragments: row block rb = 2*G + qd; row r -> query q0w + 4G + r/4, slot 4*qd + r%4
  // (all prologue loads are unconditional, clamped in range, so they issue in
  //  two dependent batches: head ids, then weights and q rows)
  bf16x8 afr[4][kKSteps];
  float wv[2][8];
  int tq[2];
  __amdgpu_buffer_rsrc_t orsrc[2];   // kLogits: the two groups' rows; kCands: gvals, gkeys of the workgroup
  float thr[2];
  uint32_t reg[2];   // kCands: group offset of the lane's region from the workgroup's first
  const uint32_t row_bytes = (uint32_t)out_spec.ld * 4u;
  const uint32_t lane_row_off = (uint32_t)g * row_bytes;
  const int split = (int)(k0 / KR);
  if (MODE == kCands) cand_rsrc(out_spec, qrow0, qa, qb, n_ksplits, split, orsrc);
  int hw[2][8], ha[2][2];
#pragma unroll
  for (int G = 0; G < 2; ++G) {
    const int qg0 = q0w + 4 * G;                      // first query of group G
    const int nrows = max(0, min(4, qb - qg0));       // its queries inside the tile
    const int qo = qg0 + g;                           // query of this lane's output rows
    tq[G] = (qo < qb) ? (q_pos0 + qo) / kstride : -1;
    const int qoc = min(qo, M - 1);
    if (MODE == kLogits) {
      orsrc[G] = uniform_rsrc(out_spec.logits + (tc.orow0 + min(qg0, M - 1)) * out_spec.ld,
                              (uint32_t)nrows * row_bytes);
    } else {
      cand_lane(out_spec, qrow0, qa, qb, qo, qoc, n_ksplits, thr[G], reg[G]);
    }
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) hw[G][sl] = heads[(qrow0 + qoc) * h + min(sl, h - 1)];
    const int qic = min(qg0 + (p16 >> 2), M - 1);
#pragma unroll
    for (int qd = 0; qd < 2; ++qd) ha[G][qd] = heads[(qrow0 + qic) * h + min(4 * qd + (p16 & 3), h - 1)];
  }
#pragma unroll
  for (int G = 0; G < 2; ++G) {
    const int qg0 = q0w + 4 * G;
    const int qo = qg0 + g;
    const int qoc = min(qo, M - 1);
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const float wj = w[(qrow0 + qoc) * H + clamp_head(hw[G][sl], H)];
      wv[G][sl] = wj * ((qo < qb && sl < h) ? 1.f : 0.f);   // (a select would sink the load into a branch)
    }
    const int qi = qg0 + (p16 >> 2);
    const int qic = min(qi, M - 1);
#pragma unroll
    for (int qd = 0; qd < 2; ++qd) {
      const bool ok = (qi < qb) && (4 * qd + (p16 & 3) < h);
      const uint4* src = reinterpret_cast<const uint4*>(q + ((qrow0 + qic) * H + clamp_head(ha[G][qd], H)) * kD);
      const uint32_t keep = ok ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const uint4 v = src[ks * 4 + g];
        afr[2 * G + qd][ks] = as_bf16x8(make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep));
      }
    }
  }

  // DMA: kptr holds bf16 keys whatever KDT is (KDT then only says whether the
  // fp8 scales apply)
  // PAGED: kptr / kscale are page pools (rows found per tile through b's table)
  const int64_t seq_rows = PAGED ? 0 : (int64_t)b * Nk;
  const void* kb_ptr = (KDT == MISA_K_BF16 || DMA)
                           ? (const void*)(reinterpret_cast<const uint16_t*>(kptr) + seq_rows * kD)
                           : (const void*)(reinterpret_cast<const uint8_t*>(kptr) + seq_rows * kD);
  const float* sc_ptr = (KDT == MISA_K_FP8_E4M3) ? kscale + seq_rows : nullptr;
  const KeyPages* pg = PAGED ? &pages : nullptr;

  // lane's B-fragment byte offsets inside a tile (column block 0), one per k-step
  uint32_t rd[kKSteps];
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) rd[ks] = sw_off(p16, 4 * ks + g);

  // staging of tile `key` into LDS buffer `buf`: issued before the current
  // tile's compute, completed (stage_done) after it, before the barrier
  KStageSw<KDT, NT> stg;
  // with one query tile per sequence (decode) every key is read once: the
  // key tiles stream past the caches (same-box: 392 -> 337 us for 64
  // sequences x 131072 keys; with many query tiles the keys are re-read and
  // must stay cached)
  const bool stream_keys = n_qtiles == 1;
  auto kbuf = [&](int buf) { return buf ? s_k1 : s_k0; };
  auto scbuf = [&](int buf) { return buf ? s_sc1 : s_sc0; };
  auto stage_issue = [&](int key, int buf) {
    if (DMA) {
      if (stream_keys)
        dma_tile<KDT, NT, kStream>(reinterpret_cast<const uint16_t*>(kb_ptr), sc_ptr, key, Nk, kstride, lane, wave,
                                   kbuf(buf), scbuf(buf), pg, b);
      else
        dma_tile<KDT, NT>(reinterpret_cast<const uint16_t*>(kb_ptr), sc_ptr, key, Nk, kstride, lane, wave,
                          kbuf(buf), scbuf(buf), pg, b);
    }
    else
      stg.load(kb_ptr, sc_ptr, key, Nk, kstride, tid, pg, b);
  };
  auto stage_done = [&](int buf) {
    if (DMA)   // the stores issued after the loads (2 per tile, or 4 with candidates) may stay in flight
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(MODE == kLogits ? 2 : 4));
    else
      stg.store(buf ? s_k1 : s_k0, buf ? s_sc1 : s_sc0, tid);
  };
  stage_issue(k0, 0);
  if (!DMA) stage_done(0);
  // every load issued so far (q fragments, weights) has landed: without this the
  // compiler cannot prove it inside the loop and waits for all memory traffic
  // (the next tile's prefetch included) before each block's first MFMA
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const float ninf = -__builtin_inff();

  uint32_t run[2] = {0u, 0u};   // kCands: groups found for the lane's query so far
  const uint64_t gmask = 0xFFFFull << (16 * g);

  // one tile from LDS buffer BUF
  // a tile's scores; kCands keeps the previous tile's in a tile that lies
  // after every query of the wave (its appends then use an infinite
  // threshold: nothing qualifies), so no registers are filled for it
  f32x4 out[2] = {f32x4{ninf, ninf, ninf, ninf}, f32x4{ninf, ninf, ninf, ninf}};
  auto tile = [&](auto buf_tag, int key0) {
    constexpr int BUF = decltype(buf_tag)::value;
    const unsigned char* sk = BUF ? s_k1 : s_k0;
    const float* ssc = BUF ? s_sc1 : s_sc0;
    const int kg = key0 + 4 * p16;   // this lane's first key index
    const bool dead = key0 > t_hi;   // the whole tile lies after every query of the wave
    if (dead) {
      if (MODE == kLogits) {
        out[0] = f32x4{ninf, ninf, ninf, ninf};
        out[1] = out[0];
      }
    } else {
      // DIAG: some key of the tile may lie after some query of the wave.  In
      // kCands only those tiles pay for the causal mask (the logits variants
      // have no registers to spare for a second copy of the tile)
      const bool diag = key0 + KT - 1 > t_lo;
      auto scores = [&](auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        bf16x8 bcur[kKSteps], bnxt[kKSteps];
        if (kPrefetchB) {
#pragma unroll
          for (int ks = 0; ks < kKSteps; ++ks) bcur[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(sk + rd[ks]));
        }
#pragma unroll
        for (int kb = 0; kb < KT / 16; ++kb) {
          if (!kPrefetchB) {
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks)
              bcur[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(sk + kb * 16 * kSwRowBytes + rd[ks]));
          } else if (kb + 1 < KT / 16) {
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks)
              bnxt[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(sk + (kb + 1) * 16 * kSwRowBytes + rd[ks]));
          }
          const float sc = (KDT == MISA_K_FP8_E4M3) ? ssc[kb * 16 + p16] : 1.f;
          f32x4 acc[2][2];
#pragma unroll
          for (int G = 0; G < 2; ++G)
#pragma unroll
            for (int qd = 0; qd < 2; ++qd) acc[G][qd] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < kKSteps; ++ks)
#pragma unroll
            for (int G = 0; G < 2; ++G)
#pragma unroll
              for (int qd = 0; qd < 2; ++qd) acc[G][qd] = mfma16(afr[2 * G + qd][ks], bcur[ks], acc[G][qd]);
#pragma unroll
          for (int G = 0; G < 2; ++G) {
            const float P0 = quad_chain(acc[G][0], wv[G][0], wv[G][1], wv[G][2], wv[G][3]);
            const float P1 = quad_chain(acc[G][1], wv[G][4], wv[G][5], wv[G][6], wv[G][7]);
            float s = P0 + P1;
            if (KDT == MISA_K_FP8_E4M3) s *= sc;
            if (DIAG && diag && kg + kb > tq[G]) s = ninf;
            out[G][kb] = s;
          }
          if (kPrefetchB && kb + 1 < KT / 16) {
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) bcur[ks] = bnxt[ks];
          }
        }
      };
      if (MODE == kLogits || diag)
        scores(std::true_type{});
      else
        scores(std::false_type{});
    }
    if (MODE == kLogits) {
      const uint32_t off = (kg < N) ? lane_row_off + (uint32_t)kg * 4u : kDrop;
      // full rows stream out; the sampled pass's rows are re-read at once
      const int pol = kstride == 1 ? kStream : 0;
      store_f32x4(orsrc[0], off, out[0], pol);
      store_f32x4(orsrc[1], off, out[1], pol);
    } else {
      // every lane issues its stores, so the wait for the next tile's
      // prefetch, issued before them, is a fixed count
#pragma unroll
      for (int G = 0; G < 2; ++G)
        append_group(orsrc, out[G], dead ? __builtin_inff() : thr[G], gmask, run[G], reg[G], out_spec.cap, kg);
    }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  for (int jt = 0; jt < n_tiles; jt += 2) {
    const int key0 = k0 + jt * KT;
    stage_issue(key0 + KT, 1);   // tile jt+1 (zeros past N)
    tile(B0{}, key0);
    stage_done(1);
    __syncthreads();
    if (jt + 1 < n_tiles) {
      stage_issue(key0 + 2 * KT, 0);   // tile jt+2
      tile(B1{}, key0 + KT);
      stage_done(0);
      __syncthreads();
    }
  }
  if (MODE == kLogits) {
    // keys of this range after the last computed tile: -inf for every query
    fill_neg_inf(out_spec.logits, out_spec.ld, tc.orow0, qa, qb, k0 + (int64_t)n_tiles * KT, k1, tid, NT);
  } else {
#pragma unroll
    for (int G = 0; G < 2; ++G) {
      const int qo = q0w + 4 * G + g;
      if (qo < qb && p16 == 0) out_spec.rcount[(qrow0 + qo) * n_ksplits + split] = run[G];
    }
  }
}

// ---------------------------------------------------------------------------
// Any head count up to 64 (routed h > 8, or the dense indexer's H heads):
// one query per wave with every head row resident in registers, as NG row
// blocks of 16 heads (row r of block grp = head slot 16 grp + r), so the A
// operand is read once per query.  A workgroup is 8 waves = 8 queries over
// one key range (NT = 512; 4 with NT = 256), with the 64-key swizzled
// tiles of k_score_h8 (register
// staging, fp8 widened exactly on the way in).  In the D layout lane group g
// holds head quad g of each block, so a quad's terms are lane-local and the
// group sum (P0+P1)+(P2+P3) is two butterfly adds; groups are added in order:
// the canonical head order of every scoring kernel here.  After a tile each
// lane holds 4 consecutive logits (keys 4 p16 .. +3); lane group 0 stores them.
// ---------------------------------------------------------------------------
constexpr int kQ64Threads = 256;   // 4 queries per workgroup, 3 workgroups per CU

template <int KDT, bool HEADS, int NG, int NT>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT == 256 ? 3 : 2)))
k_score_q64(const uint16_t* __restrict__ q, const float* __restrict__ w, const void* __restrict__ kptr,
            const float* __restrict__ kscale, const int32_t* __restrict__ heads, int h,
            float* __restrict__ logits, int64_t ld, int64_t N64, int64_t q_pos0_64, int M, int H, int n_qtiles,
            int n_ksplits, int64_t KR) {
  constexpr int KT = kSwKT, QT = NT / 64;
  __shared__ __attribute__((aligned(16))) unsigned char s_k[2 * kSwTileBytes];
  __shared__ float s_sc[2][KT];

  const int Nk = (int)N64, q_pos0 = (int)q_pos0_64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, p16 = lane & 15;
  const int b = blockIdx.y;
  const TileCoords tc = tile_coords(n_qtiles, n_ksplits, KR, Nk);
  const int k0 = (int)tc.k0, k1 = (int)tc.k1;
  const int qa = tc.qt * QT;
  const int qb = min(qa + QT, M);
  const int t_last = q_pos0 + qb - 1;
  const int kend = min(k1, t_last + 1);   // keys past kend are masked for every query
  const int n_tiles = kend > k0 ? (kend - k0 + KT - 1) / KT : 0;

  const int qi = qa + wave;
  const bool live = qi < qb;                      // wave-uniform
  const int tq = live ? q_pos0 + qi : -1;
  const int64_t row = (int64_t)b * M + min(qi, M - 1);

  // A fragments and the weights of the D rows each lane holds; every load is
  // unconditional (clamped in range) and masked afterwards
  bf16x8 afr[NG][kKSteps];
  float wq[NG][4];
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    const int sl = grp * 16 + p16;
    const bool ok = live && sl < h;
    const int j = HEADS ? clamp_head(heads[row * h + min(sl, h - 1)], H) : min(sl, H - 1);
    const uint4* src = reinterpret_cast<const uint4*>(q + (row * H + j) * kD);
    const uint32_t keep = ok ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const uint4 v = src[ks * 4 + g];
      afr[grp][ks] = as_bf16x8(make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sl2 = grp * 16 + 4 * g + i;
      const int j2 = HEADS ? clamp_head(heads[row * h + min(sl2, h - 1)], H) : min(sl2, H - 1);
      wq[grp][i] = w[row * H + j2] * ((live && sl2 < h) ? 1.f : 0.f);
    }
  }

  const void* kb_ptr = (KDT == MISA_K_BF16)
                           ? (const void*)(reinterpret_cast<const uint16_t*>(kptr) + (int64_t)b * Nk * kD)
                           : (const void*)(reinterpret_cast<const uint8_t*>(kptr) + (int64_t)b * Nk * kD);
  const float* sc_ptr = (KDT == MISA_K_FP8_E4M3) ? kscale + (int64_t)b * Nk : nullptr;
  const __amdgpu_buffer_rsrc_t orsrc = uniform_rsrc(logits + row * ld, live ? (uint32_t)ld * 4u : 0u);
  uint32_t rd[kKSteps];
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) rd[ks] = sw_off(p16, 4 * ks + g);

  KStageSw<KDT, NT> stg;
  stg.load(kb_ptr, sc_ptr, k0, Nk, 1, tid);
  stg.store(s_k, s_sc[0], tid);
  __builtin_amdgcn_s_waitcnt(0);   // as in k_score_h8
  __syncthreads();
  const float ninf = -__builtin_inff();

  auto tile = [&](auto buf_tag, int key0) {
    constexpr int BUF = decltype(buf_tag)::value;
    const unsigned char* sk = s_k + BUF * kSwTileBytes;
    const int kg = key0 + 4 * p16;
    f32x4 out = {ninf, ninf, ninf, ninf};
    if (key0 <= tq) {   // wave-uniform
      const bool diag = key0 + KT - 1 > tq;
#pragma unroll
      for (int kb = 0; kb < KT / 16; ++kb) {
        f32x4 acc[NG];
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) acc[grp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
          const bf16x8 bf = as_bf16x8(*reinterpret_cast<const uint4*>(sk + kb * 16 * kSwRowBytes + rd[ks]));
#pragma unroll
          for (int grp = 0; grp < NG; ++grp) acc[grp] = mfma16(afr[grp][ks], bf, acc[grp]);
        }
        float s = 0.f;
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) {
          const float P = quad_chain(acc[grp], wq[grp][0], wq[grp][1], wq[grp][2], wq[grp][3]);
          const float T = sum_rows(P);   // (P0+P1)+(P2+P3) on every lane
          s = s + T;
        }
        if (KDT == MISA_K_FP8_E4M3) s *= s_sc[BUF][kb * 16 + p16];
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
    stg.load(kb_ptr, sc_ptr, key0 + KT, Nk, 1, tid);   // tile jt+1 (zeros past N)
    tile(B0{}, key0);
    stg.store(s_k + kSwTileBytes, s_sc[1], tid);
    __syncthreads();
    if (jt + 1 < n_tiles) {
      stg.load(kb_ptr, sc_ptr, key0 + 2 * KT, Nk, 1, tid);   // tile jt+2
      tile(B1{}, key0 + KT);
      stg.store(s_k, s_sc[0], tid);
      __syncthreads();
    }
  }
  // keys of this range after the last computed tile: -inf for every query
  fill_neg_inf(logits, ld, (int64_t)b * M, qa, qb, k0 + (int64_t)n_tiles * KT, k1, tid, NT);
}

// ---------------------------------------------------------------------------
// Launch: pick the kernel, the key-range split and the grid.
// ---------------------------------------------------------------------------
void plan_split(int64_t N, int n_seq, int n_qtiles, int KT, int* n_ksplits, int64_t* KR, int64_t target) {
  const int64_t n_ktiles = (N + KT - 1) / KT;
  int64_t ns = (target + (int64_t)n_seq * n_qtiles - 1) / ((int64_t)n_seq * n_qtiles);
  if (ns < 1) ns = 1;
  if (ns > n_ktiles) ns = n_ktiles;
  int64_t kr = ((n_ktiles + ns - 1) / ns) * KT;
  ns = (N + kr - 1) / kr;
  *n_ksplits = (int)ns;
  *KR = kr;
}

// DMA: k holds bf16 keys (for kdtype fp8: the widened copy; k_scale still
// applies), staged by direct loads into LDS
template <int MODE, bool DMA = false, bool PAGED = false, int NW = 4>
static hipError_t launch_h8(const misa_shape& s, const uint16_t* q, const float* w, const void* k, int kdtype,
                            const float* k_scale, const int32_t* heads, int h, const ScoreOut& o, int kstride,
                            int nks, int64_t KR, hipStream_t st, const KeyPages* pages = nullptr) {
  const int M = s.q_per_seq;
  const int n_qtiles = (M + 8 * NW - 1) / (8 * NW);
  dim3 grid((unsigned)((int64_t)n_qtiles * nks), (unsigned)s.n_seq);
  if (o.slab_tiles > 0) grid = dim3((unsigned)((int64_t)o.slab_tiles * nks), 1);
  const KeyPages pg = pages != nullptr ? *pages : KeyPages{nullptr, 0, 0, 1};
  if (kdtype == MISA_K_BF16)
    hipLaunchKernelGGL((k_score_h8<MISA_K_BF16, MODE, DMA, PAGED, NW>), grid, dim3(64 * NW), 0, st, q, w, k, k_scale,
                       heads, h, o, s.n_keys, kstride, s.q_pos0, M, s.n_heads, n_qtiles, nks, KR, pg);
  else
    hipLaunchKernelGGL((k_score_h8<MISA_K_FP8_E4M3, MODE, DMA, PAGED, NW>), grid, dim3(64 * NW), 0, st, q, w, k,
                       k_scale,
                       heads, h, o, s.n_keys, kstride, s.q_pos0, M, s.n_heads, n_qtiles, nks, KR, pg);
  return hipGetLastError();
}

hipError_t launch_score_paged(const misa_shape& s, const uint16_t* q, const float* w, const void* k_pages,
                              int kdtype, const float* scale_pages, const int32_t* heads, int h, float* logits,
                              int64_t ld, const KeyPages& pages, hipStream_t st) {
  int nks;
  int64_t KR;
  plan_split(s.n_keys, s.n_seq, (s.q_per_seq + 31) / 32, 64, &nks, &KR);
  const ScoreOut o{logits, ld, nullptr, nullptr, nullptr, nullptr, 0, nullptr};
  if (kdtype == MISA_K_BF16)
    return launch_h8<kLogits, true, true>(s, q, w, k_pages, kdtype, scale_pages, heads, h, o, 1, nks, KR, st,
                                          &pages);
  return launch_h8<kLogits, false, true>(s, q, w, k_pages, kdtype, scale_pages, heads, h, o, 1, nks, KR, st,
                                         &pages);
}

hipError_t launch_score(const misa_shape& s, const uint16_t* q, const float* w, const void* k,
                        int kdtype, const float* k_scale, const int32_t* heads, int h,
                        float* logits, int64_t ld, hipStream_t st) {
  const int M = s.q_per_seq, H = s.n_heads;
  const int64_t N = s.n_keys;
  if (heads != nullptr && h <= 8) {
    int nks;
    int64_t KR;
    plan_split(N, s.n_seq, (M + 31) / 32, 64, &nks, &KR);
    const ScoreOut o{logits, ld, nullptr, nullptr, nullptr, nullptr, 0, nullptr};
    // bf16 keys are staged by direct loads into LDS; fp8 keys through
    // registers, where they are widened (the same bf16 tiles either way)
    if (kdtype == MISA_K_BF16)
      return launch_h8<kLogits, true>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st);
    return launch_h8<kLogits>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st);
  }
  const int hh = heads ? h : H;
  constexpr int kQT = kQ64Threads / 64;   // queries per workgroup
  const int n_qtiles = (M + kQT - 1) / kQT;
  int nks;
  int64_t KR;
  plan_split(N, s.n_seq, n_qtiles, 64, &nks, &KR);
  dim3 grid((unsigned)((int64_t)n_qtiles * nks), (unsigned)s.n_seq);
  const int ng = (hh + 15) / 16;
#define MISA_Q64(KDT_, HEADS_, NG_)                                                                          \
  hipLaunchKernelGGL((k_score_q64<KDT_, HEADS_, NG_, kQ64Threads>), grid, dim3(kQ64Threads), 0, st, q, w, k,  \
                     k_scale, heads, hh, logits, ld, N, s.q_pos0, M, H, n_qtiles, nks, KR)
#define MISA_Q64_NG(KDT_, HEADS_)   \
  switch (ng) {                     \
    case 1: MISA_Q64(KDT_, HEADS_, 1); break; \
    case 2: MISA_Q64(KDT_, HEADS_, 2); break; \
    case 3: MISA_Q64(KDT_, HEADS_, 3); break; \
    default: MISA_Q64(KDT_, HEADS_, 4); break; \
  }
  if (kdtype == MISA_K_BF16) {
    if (heads) { MISA_Q64_NG(MISA_K_BF16, true) } else { MISA_Q64_NG(MISA_K_BF16, false) }
  } else {
    if (heads) { MISA_Q64_NG(MISA_K_FP8_E4M3, true) } else { MISA_Q64_NG(MISA_K_FP8_E4M3, false) }
  }
#undef MISA_Q64_NG
#undef MISA_Q64
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused scoring -> top-k (the indexer's path for h <= 8 and long prefixes)
// ---------------------------------------------------------------------------
FusedPlan plan_fused(const misa_shape& s, int h, int k) {
  FusedPlan p{};
  const int64_t N = s.n_keys;
  const int64_t n_min = s.q_pos0 + 1;   // shortest prefix of the chunk
  // prefixes long enough that the candidates are a small share of each row
  // (k at most a quarter of the shortest prefix; below 16384 keys the
  // materialised logits are cheap anyway)
  p.ok = h <= 8 && k <= 8192 && n_min >= std::max<int64_t>(16384, 4 * (int64_t)k) && s.q_per_seq > 0;
  if (!p.ok) return p;
  p.kstride = (int)std::max<int64_t>(32, (N + 4095) / 4096);   // <= 4096 sampled keys per row
  p.n_sample = (N + p.kstride - 1) / p.kstride;
  p.ld_sample = (p.n_sample + 3) / 4 * 4;
  // the region select's list capacity (its LDS variant: 4608 in the compact
  // one that fits three workgroups per CU, 4096 in its few-row variant).  A
  // row with more candidates is re-scored whole: at k = 2048 the list holds
  // 1.5 times the target (4096 held 1.33 times, and 4 of the 8192 rows of a
  // 32K-key chunk overflowed it, each costing the slow path about 0.15 ms)
  p.cap_list = k <= 2048 ? 4608 : (k <= 4096 ? 8192 : 16384);
  // candidates aimed for: k plus a margin of 4 standard deviations of the
  // sampled threshold's error (about k / kstride sampled keys lie above it,
  // relative spread 1/sqrt of that), at most k/2
  const double margin = std::min(0.5, 4.0 / std::sqrt(std::max(1.0, (double)k / p.kstride)));
  p.target = std::min((int)(k * (1.0 + margin)), (k + p.cap_list) / 2);
  int nks;
  int64_t KR;
  // with at most 8 queries per sequence (decode) the candidate pass runs
  // one-wave workgroups, four per CU: 1024 of them are one resident round.
  // Same-box, 64 sequences x 131072 bf16 keys: 333 -> 323 us (2048 of them:
  // 2 rounds), 335 us at 4096, 348 us at 8192; paged keys 325 -> 318 us
  plan_split(N, s.n_seq, (s.q_per_seq + 31) / 32, 64, &nks, &KR, s.q_per_seq <= 8 ? 1024 : 2048);
  p.n_splits = nks;
  p.key_range = KR;
  if (nks > kMaxRegionSplits) {
    p.ok = false;
    return p;
  }
  // expected candidate groups of 4 keys per (row, key range) (at most the
  // expected candidates), doubled, plus room for a few clusters of large scores
  const int64_t expect = (int64_t)p.target * KR / n_min + 1;
  p.cap_region = (int)((2 * expect + 512 + 255) / 256 * 256);
  // a key range of KR keys holds at most KR / 4 groups: short ranges (few
  // queries spread over many ranges) never need more
  p.cap_region = (int)std::min<int64_t>(p.cap_region, (KR + 3) / 4);
  // a workgroup's 32 rows of regions are addressed with byte offsets below 2^31
  if ((int64_t)32 * p.n_splits * p.cap_region * 16 >= ((int64_t)1 << 31)) p.ok = false;
  return p;
}

FusedPlan lean_plan(const FusedPlan& fast, const misa_shape& s) {
  FusedPlan p = fast;
  if (!p.ok) return p;
  // the expected groups per region with a quarter more and room for one
  // cluster of large scores: a region that overflows flags its row for the
  // exact re-scoring, so a tighter region costs time, never results
  const int64_t n_min = s.q_pos0 + 1;
  const int64_t expect = (int64_t)p.target * p.key_range / n_min + 1;
  p.cap_region = (int)std::min<int64_t>(fast.cap_region, (expect + expect / 4 + 128 + 63) / 64 * 64);
  return p;
}

hipError_t launch_score_sampled(const misa_shape& s, const uint16_t* q, const float* w, const void* k, int kdtype,
                                const float* k_scale, const int32_t* heads, int h, const FusedPlan& p,
                                float* sample_logits, hipStream_t st, bool direct, const KeyPages* pages) {
  int nks;
  int64_t KR;
  // fewer, longer workgroups than the full passes (one resident round: 3
  // per CU): a sampled key range is short, so each workgroup's fixed cost
  // (head ids, then weights and q rows, the first tile) weighs more.
  // Same-box: 82 -> 76 us for the 8192 x 131072 chunk, 31 -> 23 us for 64
  // decode rows (2048 workgroups before)
  const ScoreOut o{sample_logits, p.ld_sample, nullptr, nullptr, nullptr, nullptr, 0, nullptr};
  // at most 8 queries per sequence (decode), contiguous keys: one-wave
  // workgroups, 512 of them (same-box, 64 sequences x 131072 keys: 22.7 ->
  // 19.7 us; 2048 of them 23.2 us).  Paged keys keep four-wave workgroups:
  // their per-key block-table lookups ran 42 -> 95 us in one-wave ones
  if (s.q_per_seq <= 8 && pages == nullptr) {
    plan_split(p.n_sample, s.n_seq, 1, 64, &nks, &KR, 512);
    if (!direct)
      return launch_h8<kLogits, false, false, 1>(s, q, w, k, kdtype, k_scale, heads, h, o, p.kstride, nks, KR, st);
    return launch_h8<kLogits, true, false, 1>(s, q, w, k, kdtype, k_scale, heads, h, o, p.kstride, nks, KR, st);
  }
  plan_split(p.n_sample, s.n_seq, (s.q_per_seq + 31) / 32, 64, &nks, &KR, 768);
  if (pages != nullptr)   // the sampled keys' rows are looked up one by one: staged through registers
    return launch_h8<kLogits, false, true>(s, q, w, k, kdtype, k_scale, heads, h, o, p.kstride, nks, KR, st, pages);
  if (!direct) return launch_h8<kLogits, false>(s, q, w, k, kdtype, k_scale, heads, h, o, p.kstride, nks, KR, st);
  return launch_h8<kLogits, true>(s, q, w, k, kdtype, k_scale, heads, h, o, p.kstride, nks, KR, st);
}

hipError_t launch_score_cands(const misa_shape& s, const uint16_t* q, const float* w, const void* k, int kdtype,
                              const float* k_scale, const int32_t* heads, int h, const FusedPlan& p,
                              const float* thr, float* gvals, int32_t* gkeys, uint32_t* rcount, hipStream_t st,
                              bool direct, const KeyPages* pages) {
  const ScoreOut o{nullptr, 0, thr, reinterpret_cast<f32x4*>(gvals), gkeys, rcount, p.cap_region, nullptr};
  const int nks = p.n_splits;
  const int64_t KR = p.key_range;
  // at most 8 queries per sequence (decode): one-wave workgroups (one query
  // tile per sequence either way).  Same-box, 64 sequences x 131072 bf16
  // keys, against four-wave workgroups: 338 -> 334 us, paged keys 368 -> 325 us
  if (s.q_per_seq <= 8) {
    if (pages != nullptr) {
      if (direct)
        return launch_h8<kCands, true, true, 1>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st, pages);
      return launch_h8<kCands, false, true, 1>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st, pages);
    }
    if (!direct) return launch_h8<kCands, false, false, 1>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st);
    return launch_h8<kCands, true, false, 1>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st);
  }
  if (pages != nullptr) {
    if (direct) return launch_h8<kCands, true, true>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st, pages);
    return launch_h8<kCands, false, true>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st, pages);
  }
  if (!direct) return launch_h8<kCands, false>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st);
  return launch_h8<kCands, true>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st);
}

hipError_t launch_score_rescore(const misa_shape& s, const uint16_t* q, const float* w, const void* k,
                                int kdtype, const float* k_scale, const int32_t* heads, int h,
                                const uint32_t* row_flag, float* slab, int64_t ld, const SlabBatch& sb,
                                hipStream_t st, bool direct, const KeyPages* pages) {
  int nks;
  int64_t KR;
  const int n_qtiles = (s.q_per_seq + 31) / 32;
  // any key split gives the same logits rows; with few queries per sequence
  // (decode) a small grid, since the workgroups of unflagged rows only check
  // their flags and leave (8.6 -> 8.2 us at 64 decode rows)
  plan_split(s.n_keys, s.n_seq, n_qtiles, 64, &nks, &KR, s.q_per_seq <= 8 ? 256 : 2048);
  ScoreOut o{slab, ld, nullptr, nullptr, nullptr, nullptr, 0, row_flag};
  o.slab_tiles = sb.tiles;
  o.slab_first = (int)sb.first;
  o.slab_tr = sb.tr;
  o.n_flat = s.n_seq * n_qtiles;
  if (pages != nullptr) {
    if (direct) return launch_h8<kLogits, true, true>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st, pages);
    return launch_h8<kLogits, false, true>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st, pages);
  }
  if (!direct) return launch_h8<kLogits, false>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st);
  return launch_h8<kLogits, true>(s, q, w, k, kdtype, k_scale, heads, h, o, 1, nks, KR, st);
}

// fp8 keys widened to bf16 (exactly: every e4m3 value is a bf16 value) for the
// direct-load staging; 16 codes per thread, the same decoder as the
// register staging, so both stagings put identical bits in LDS
__global__ void __launch_bounds__(256) k_widen_fp8(const uint4* __restrict__ codes, uint4* __restrict__ out,
                                                   int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const uint4 v = codes[i];
  const uint2 a = e4m3x4_to_bf16x4(v.x), b2 = e4m3x4_to_bf16x4(v.y);
  const uint2 c2 = e4m3x4_to_bf16x4(v.z), d2 = e4m3x4_to_bf16x4(v.w);
  out[2 * i] = make_uint4(a.x, a.y, b2.x, b2.y);
  out[2 * i + 1] = make_uint4(c2.x, c2.y, d2.x, d2.y);
}

hipError_t launch_widen_fp8(const misa_shape& s, const void* k, uint16_t* out, hipStream_t st) {
  const int64_t n16 = (int64_t)s.n_seq * s.n_keys * kD / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_widen_fp8, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(k), reinterpret_cast<uint4*>(out), n16);
  return hipGetLastError();
}

}  // namespace misa
