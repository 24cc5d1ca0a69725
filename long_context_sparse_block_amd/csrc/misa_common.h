// Device-side building blocks shared by the MISA kernels (gfx950 / CDNA4).
//
// Wavefronts are 64 lanes.  Matrix work uses v_mfma_f32_16x16x32_bf16, whose
// operand layout (per lane l of the wave) is:
//   A (16 rows x 32 k):  lane l supplies row l%16, k = 8*(l/16) .. 8*(l/16)+7
//   B (32 k x 16 cols):  lane l supplies col l%16, k = 8*(l/16) .. 8*(l/16)+7
//   D (16 x 16, fp32):   lane l holds rows 4*(l/16)+i (i = 0..3) of col l%16
// so one MFMA consumes 16 bytes of A and 16 bytes of B per lane, and a full
// 128-wide dot product is 4 MFMAs ("k-steps") accumulated in order 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "misa_launch.h"

namespace misa {

constexpr int kWave = 64;
constexpr int kD = 128;          // indexer head dim
constexpr int kKSteps = kD / 32;  // MFMA k-steps per dot product

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// OCP e4m3fn -> bf16 is exact (3-bit mantissa inside bf16's 7 bits, exponent
// range inside bf16's; e4m3 subnormals are bf16 normals).  gfx950 converts two
// codes to a packed bf16 pair in one instruction; a scale of 1.0 leaves the
// value unchanged.  Four codes (one dword) -> four bf16 (two dwords).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t codes) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);   // codes 0, 1
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true);    // codes 2, 3
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false);
  return v.x;
}

// ReLU as an integer max on the bit pattern: non-negative floats are
// non-negative integers and negative floats negative ones, so max(bits, 0)
// keeps x >= 0 and gives +0.0 otherwise.  One VALU op, and unlike fmaxf no
// NaN canonicalisation (inputs are finite).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Canonical per-(query, key) reduction of one quad of four head terms:
//   p = fma(w3, relu(x3), fma(w2, relu(x2), fma(w1, relu(x1), fma(w0, relu(x0), 0))))
// Every kernel that must agree bitwise with another uses exactly this chain.
__device__ __forceinline__ float quad_chain(const f32x4 x, float w0, float w1, float w2, float w3) {
  float p = 0.0f;
  p = __builtin_fmaf(w0, relu(x[0]), p);
  p = __builtin_fmaf(w1, relu(x[1]), p);
  p = __builtin_fmaf(w2, relu(x[2]), p);
  p = __builtin_fmaf(w3, relu(x[3]), p);
  return p;
}

// Two fp32 -> packed bf16 (element 0 in the low half), round to nearest even
// (gfx950's packed converter).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2_t));
}

// Cache-policy operand of a buffer store: non-temporal (gfx950's nt bit), for
// data written once and not read again while it could still be cached.
constexpr int kStream = 2;

// s_waitcnt immediate: wait until at most n vector-memory operations of the
// wave are outstanding (the export and LDS/scalar counters are not waited on)
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

// Number of set bits of m below the calling lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Order-preserving map float -> uint32 (larger float <=> larger key), with
// The page-pool row of key t of sequence b (KeyPages).  Table entries are a
// documented precondition (in [0, n_pages)); they are clamped so that a bad
// one cannot fault.
__device__ __forceinline__ int64_t paged_row(const KeyPages& pg, int b, int64_t t) {
  const uint32_t p = (uint32_t)t / (uint32_t)pg.page_keys;   // t < 2^31 (the ABI bounds N)
  int64_t e = pg.table[(int64_t)b * pg.max_pages + min((int64_t)p, pg.max_pages - 1)];
  e = e < 0 ? 0 : (e >= pg.n_pages ? pg.n_pages - 1 : e);
  return e * pg.page_keys + (t - (int64_t)p * pg.page_keys);
}

// (P0 + P1) + (P2 + P3) of a value P held on the four 16-lane rows of a wave,
// on every lane: the xor-16 and xor-32 butterflies done by gfx950's
// v_permlane16_swap / v_permlane32_swap (VALU, no LDS round trip).  The
// 16-swap of P with itself leaves rows (0, 0, 2, 2) in one register and (1, 1,
// 3, 3) in the other, so their sum is P0 + P1 on rows 0 and 1 and P2 + P3 on
// rows 2 and 3; the 32-swap does the same across the two halves.  Each add
// has the same two operands as P + shfl_xor(P, 16) and v + shfl_xor(v, 32)
// (in some order, and float addition is commutative), so the result is
// bitwise the same.
__device__ __forceinline__ float sum_rows(float P) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(P), __float_as_uint(P), false, false);
  const float v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// -0.0 folded onto +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t key) {
  uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

// Raw buffer descriptor over [base, base + bytes).  Its fields are read from
// the first lane, so the compiler knows the descriptor is wave-uniform and
// emits plain buffer instructions (no per-lane descriptor loop); callers pass
// values that are uniform anyway.  With stride 0 the hardware range check
// (gfx9-family descriptor word 3) drops stores and zero-fills loads whose byte
// offset is at or past `bytes`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  void* pu = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(pu, (short)0, n, 0x00020000);
}

// Hardware dispatches workgroup i of a launch to XCD (i mod 8).  Remap the
// linear id so that each XCD walks a contiguous range of logical tiles (tiles
// that share key data then share that XCD's L2).
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t total) {
  constexpr int64_t kXcds = 8;
  int64_t per = total / kXcds;
  if (i < per * kXcds) return (i % kXcds) * per + i / kXcds;
  return i;
}

}  // namespace misa
