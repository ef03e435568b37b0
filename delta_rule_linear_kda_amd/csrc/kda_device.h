// kda_device.h - device helpers shared by the libkda kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// g_min of the lower-bounded scaled-sigmoid log-decay (page "[Paper Review]
// Kimi K3...", section "Kimi Delta Attention (KDA)", "Lower-bounded decay").
constexpr float kGMin = -5.0f;
// epsilon inside the L2 normalisation root of q and k.
constexpr float kNormEps = 1e-6f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Element i of an input tensor as fp32 (fp32 or bf16 storage).
template <typename T>
__device__ __forceinline__ float ld_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

// 8 consecutive elements (16-byte aligned start for bf16, 32-byte for fp32).
template <typename T>
__device__ __forceinline__ void ld8(const T* p, float (&x)[8]);
template <>
__device__ __forceinline__ void ld8<float>(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <>
__device__ __forceinline__ void ld8<uint16_t>(const uint16_t* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// 4 consecutive elements (8-byte aligned for bf16, 16-byte for fp32).
template <typename T>
__device__ __forceinline__ void ld4(const T* p, float (&x)[4]);
template <>
__device__ __forceinline__ void ld4<float>(const float* p, float (&x)[4]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
template <>
__device__ __forceinline__ void ld4<uint16_t>(const uint16_t* p, float (&x)[4]) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  x[0] = __uint_as_float(u.x << 16);
  x[1] = __uint_as_float(u.x & 0xFFFF0000u);
  x[2] = __uint_as_float(u.y << 16);
  x[3] = __uint_as_float(u.y & 0xFFFF0000u);
}

// exp(x) via the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

// Logistic function; sigmoid(-inf) = 0, sigmoid(+inf) = 1 (no NaN for +-inf).
__device__ __forceinline__ float sigmoidf(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, then synchronises the workgroup.  Unlike __syncthreads() it does
// not wait for outstanding global loads/stores, so register prefetches and
// output stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Same ordering within one wavefront (LDS written by other lanes of this wave).
__device__ __forceinline__ void lds_wave_fence() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Sum over the 64 lanes of a wavefront (every lane gets the total).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Sum over aligned groups of `W` consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = W / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Sum and maximum over the four 16-lane rows of a wave, lane position by lane
// position (the lanes l, l ^ 16, l ^ 32, l ^ 48), through gfx950's cross-row
// swaps: v_permlane16_swap(x, x) returns rows (0, 0, 2, 2) and (1, 1, 3, 3),
// v_permlane32_swap(x, x) the lower and the upper half twice.  Vector ALU
// only, no LDS traffic; the additions are those of an xor butterfly over
// 16 and 32, so every lane gets the same bits.
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

}  // namespace kda
