// kda_chunk_common.h - device helpers of the bf16 chunked KDA kernels
// (fused forward, and the two passes of the split forward) on gfx950:
// matrix-core wrappers, 16-lane DPP scans and sums, bf16/fp16 packing, and
// LDS/global access helpers.
#pragma once

#include "kda_device.h"

namespace kda {
namespace {

constexpr int kC = 32;          // chunk length (tokens)
// Word 3 of a raw (unformatted, unswizzled) buffer resource on gfx950.
constexpr int kBufferRsrcFlags = 0x00020000;
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;

__device__ __forceinline__ f32x4_t mma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma_f16(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// (ah + al)(bh + bl) ~ ah bh + ah bl + al bh
__device__ __forceinline__ f32x4_t mma_x3(bf16x8_t ah, bf16x8_t al, bf16x8_t bh, bf16x8_t bl,
                                          f32x4_t c) {
  c = mma_bf16(al, bh, c);
  c = mma_bf16(ah, bl, c);
  return mma_bf16(ah, bh, c);
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcpf_fast(float x) { return __builtin_amdgcn_rcpf(x); }
// Log-decay in log2 units from the decay logit: g log2(e) = -5 log2(e)
// sigmoid(a) = 1 / ((1 + e^-a) / (-5 log2(e))), the scale folded into one fma
// before the reciprocal.
__device__ __forceinline__ float log2_decay(float a) {
  constexpr float kInv = 1.f / (kGMin * kLog2e);
  return rcpf_fast(__builtin_fmaf(exp2f_fast(-kLog2e * a), kInv, kInv));
}
// acc + the squares of the two bf16 halves of w (one dot-product instruction;
// the bf16 products are exact in fp32).
__device__ __forceinline__ float sq2_bf16(uint32_t w, float acc) {
  typedef __attribute__((ext_vector_type(2))) __bf16 b2_t;
  const b2_t x = __builtin_bit_cast(b2_t, w);
  return __builtin_amdgcn_fdot2_f32_bf16(x, x, acc, false);
}

// Data-parallel primitives within a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp0(float x) {  // lanes whose source is outside the row read 0
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ void scan_step_x8(float (&x)[2][4]) {
  float y[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) y[t][j] = dpp0<CTRL>(x[t][j]);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) x[t][j] += y[t][j];
}
// Inclusive prefix sums over the 16 lanes of each row, for eight independent
// values, step by step (row_shr 1, 2, 4, 8; lanes whose source is outside the
// row add 0).
__device__ __forceinline__ void scan16_x8(float (&x)[2][4]) {
  scan_step_x8<0x111>(x);
  scan_step_x8<0x112>(x);
  scan_step_x8<0x114>(x);
  scan_step_x8<0x118>(x);
}
// Sum over the 16 lanes of each row, in every lane of the row.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp0<0x128>(x);  // row_ror:8
  x += dpp0<0x124>(x);  // row_ror:4
  x += dpp0<0x122>(x);  // row_ror:2
  x += dpp0<0x121>(x);  // row_ror:1
  return x;
}
// Value held by lane S of each quad of lanes, in all four lanes of the quad.
template <int S>
__device__ __forceinline__ float quad_bcast_t(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                            S | (S << 2) | (S << 4) | (S << 6), 0xf,
                                                            0xf, false));
}
__device__ __forceinline__ float quad_bcast(float x, int s) {  // s: compile-time after unrolling
  return s == 0 ? quad_bcast_t<0>(x) : s == 1 ? quad_bcast_t<1>(x) : s == 2 ? quad_bcast_t<2>(x)
                                                                            : quad_bcast_t<3>(x);
}
// Value of lane 15 of each row of 16 lanes, in every lane of the row: DPP
// row_newbcast:15 (a vector ALU move; the same lanes as the ds_swizzle
// broadcast it replaces, without the LDS crossbar).
__device__ __forceinline__ float row_last16(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x15F, 0xf, 0xf, false));
}

// ---- fp16 range of the state-chain operands ---------------------------------
// The state S and the pseudo-values U enter the W S, Qbar S and Kend^T U
// products as fp16, whose largest value is 65504, while the state itself is
// fp32 and unbounded (a caller's initial state, large values).  Each state
// column j is therefore carried as S_j 2^(esc_j - 127) with a per-column
// power of two (exact): when the column's largest magnitude leaves
// [2^-8, 2^10) it is brought back to [2^6, 2^7), which keeps the fp16 copy of
// S in range and its entries above fp16's subnormals.  U (U0 and every
// product with U carry the same column scale) is checked where its fp16 copy
// is formed: if a column of it would reach 2^15 it is scaled down by another
// power of two f for the Kend^T U product, whose result is scaled back by
// 1/f.  Both checks are lane-local in the common case (each lane tests its
// own entries, then one wave vote); only when some lane is out of range does
// the wave form the exact column maxima over the column's four lanes.

// 2^(e - 127) for a biased exponent e in [1, 254].
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)e << 23); }
// Biased exponent of |x| (0 for zero and subnormals, 255 for inf and NaN).
__device__ __forceinline__ int bexp(float x) { return (int)((__float_as_uint(x) >> 23) & 0xffu); }
// Largest value over the four lanes (li, li + 16, li + 32, li + 48) that
// hold one column of a 16x16 accumulator tile.
__device__ __forceinline__ float col_max4(float m) { return rows4_max(m); }
// Largest magnitude of this lane's part of a state column.
template <int N>
__device__ __forceinline__ float abs_max(const f32x4_t (&S)[N]) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(S[i][j]));
  return m;
}
// Keeps the lane's part of a state column in range (see above); esc is the
// column's biased scale exponent, kept in [4, 250].
template <int N>
__device__ __forceinline__ void rescale_state(f32x4_t (&S)[N], int& esc) {
  const float ml = abs_max(S);
  if (__any(ml >= 1024.f || (ml < 0x1p-8f && ml > 0.f))) {  // wave-uniform, rare
    const int E = bexp(col_max4(ml));
    const bool need = E != 0 && E != 255 && (E < 127 - 8 || E >= 127 + 10);
    const int en = need ? min(250, max(4, esc + (127 + 6) - E)) : esc;
    const int d = en - esc;  // |d| <= 246: applied as two factors of at most 2^123
    const float r1 = pow2f(127 + d / 2), r2 = pow2f(127 + d - d / 2);
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[i][j] = S[i][j] * r1 * r2;
    esc = en;
  }
}
// For 8 entries x of a column of U (in place): scales them by f = 2^(141 - E)
// when the column's largest magnitude (biased exponent E) reaches 2^15, so
// that the column lies in [2^14, 2^15), and returns 1/f (1 otherwise).  The
// wave takes the exact column maxima only when some lane has an entry at or
// above 2^15; *any_big tells whether it did.
__device__ __forceinline__ float u_range(float (&x)[8], bool& any_big) {
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
  any_big = __any(m >= 32768.f);
  float finv = 1.f;
  if (any_big) {  // wave-uniform, rare
    const int E = bexp(col_max4(m));
    const bool big = E >= 127 + 15 && E != 255;
    const float f = big ? pow2f(268 - E) : 1.f;
    finv = big ? pow2f(E - 14) : 1.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] *= f;
  }
  return finv;
}

__device__ __forceinline__ f16x8_t pack_f16x8(const float (&x)[8]) {
  f16x8_t r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (_Float16)x[j];
  return r;
}
// fp16 hi + lo parts of 8 values (hi = fp16(x), lo = fp16(x - hi)).
__device__ __forceinline__ void split_f16x8(const float (&x)[8], f16x8_t& hi, f16x8_t& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const _Float16 hv = (_Float16)x[j];
    hi[j] = hv;
    lo[j] = (_Float16)(x[j] - (float)hv);
  }
}
// Two values rounded to nearest-even bf16 in one packed conversion (a in the
// low half), and the bf16 hi + lo parts of two values from it.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
__device__ __forceinline__ void split_pk_bf16(float a, float b, uint32_t& h, uint32_t& l) {
  h = pk_bf16(a, b);
  l = pk_bf16(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xFFFF0000u));
}
// 4 values as bf16 (and as bf16 hi + lo), two per packed conversion.
__device__ __forceinline__ bf16x4_t pack_bf16x4(const float (&x)[4]) {
  const u32x2_t w = {pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3])};
  return __builtin_bit_cast(bf16x4_t, w);
}
__device__ __forceinline__ void split_bf16x4(const float (&x)[4], bf16x4_t& hi, bf16x4_t& lo) {
  uint32_t h0, l0, h1, l1;
  split_pk_bf16(x[0], x[1], h0, l0);
  split_pk_bf16(x[2], x[3], h1, l1);
  hi = __builtin_bit_cast(bf16x4_t, u32x2_t{h0, h1});
  lo = __builtin_bit_cast(bf16x4_t, u32x2_t{l0, l1});
}
// bf16 hi + lo parts of 8 values, two at a time through the packed
// conversion; hi is read back from its packed bits.
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8_t& hi, bf16x8_t& lo) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  u32x4_t hv, lv;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t hw = __builtin_bit_cast(
        uint32_t, __builtin_convertvector((f32x2_t){x[2 * p], x[2 * p + 1]}, bf16x2_t));
    hv[p] = hw;
    const f32x2_t r = {x[2 * p] - __uint_as_float(hw << 16),
                       x[2 * p + 1] - __uint_as_float(hw & 0xFFFF0000u)};
    lv[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
  }
  hi = __builtin_bit_cast(bf16x8_t, hv);
  lo = __builtin_bit_cast(bf16x8_t, lv);
}

// 8 consecutive 16-bit values from LDS (16-byte aligned).
template <typename V>
__device__ __forceinline__ V lds8(const uint16_t* p) {
  return __builtin_bit_cast(V, *reinterpret_cast<const u32x4_t*>(p));
}
// 4 + 4 16-bit values at p and p + 16 (8-byte aligned each): the permuted k
// order that matches a B operand made of two stacked accumulator tiles.
template <typename V>
__device__ __forceinline__ V lds4x2(const uint16_t* p) {
  const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(p);
  const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(p + 16);
  const u32x4_t v = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(V, v);
}
__device__ __forceinline__ void lds_f32x8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
// 4 + 4 floats at p and p + 16 (permuted k order).
__device__ __forceinline__ void lds_f32x4x2(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 16);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
// Pins a wave-uniform pointer in scalar registers and hides its provenance
// from the optimiser, so `p + lane_offset` is addressed as SGPR base + 32-bit
// VGPR offset instead of a hoisted 64-bit address per access.
template <typename T>
using gptr = __attribute__((address_space(1))) T*;  // global memory
template <typename T>
__device__ __forceinline__ gptr<T> sbase(T* p) {
  gptr<T> gp = (gptr<T>)p;
  __asm__ volatile("" : "+s"(gp));
  return gp;
}
// Element i of a scalar-based array as a T pointer, the byte offset formed in
// 32 bits: `base[i]` would scale the zero-extended index in 64-bit vector
// arithmetic, this is the access's 32-bit vector offset.
template <typename T, typename B>
__device__ __forceinline__ gptr<T> gat(gptr<B> base, uint32_t i) {
  return (gptr<T>)((__attribute__((address_space(1))) const char*)base + i * (uint32_t)sizeof(B));
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

}  // namespace
}  // namespace kda
