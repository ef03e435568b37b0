// kda_bwd_chunk.hip - chunked backward of the KDA recurrence on gfx950:
// gradients of L = sum_t <dy_t, y_t> + <dS_final, S_final> with respect to q,
// k, v, a, b, gate and the initial state, on bf16x3 matrix-core products
// (fp32 accuracy to about 2^-16 per product).
//
// The recurrence is the one of page "[Paper Review] Kimi K3...", section
// "Kimi Delta Attention (KDA)", in its chunkwise form (same section: the
// recurrence is parallelisable per chunk).  The pages give no backward; it is
// reverse mode through the chunk form.  Per chunk of n <= 32 tokens with
// start state S (b = chunk-local cumulative log-decay, Gamma = exp(b),
// Qbar = qh Gamma, Kbar = kh Gamma, Kend = kh exp(b_end - b),
// Mkk = strict_lower(kh exp(b) (kh exp(-b))^T), P = lower(qh exp(b) (kh exp(-b))^T),
// X = (I + diag(beta) Mkk)^-1):
//   Vt = V - Kbar S,  U = X diag(beta) Vt,  O = Qbar S + P U,
//   S_end = diag(Gamma_end) S + Kend^T U.
// With dO = dy sigmoid(gate) and dS_end the adjoint of S_end:
//   dU = P^T dO + Kend dS_end,   Z = X^T dU,   dV = diag(beta) Z
//   dS = diag(Gamma_end) dS_end + Qbar^T dO - Kbar^T diag(beta) Z   (chunk start)
//   dbeta_r = sum_j Z_rj Vt_rj - sum_i (Z U^T)_ri Mkk_ri
//   dMkk = -diag(beta) (Z U^T) (strict lower),  dP = dO U^T (lower)
//   dQbar = dO S^T,  dKbar = -diag(beta) Z S^T,  dKend = U dS_end^T,
//   dGamma_end = rowsum(dS_end * S)
// then through the pairwise decays of Mkk and P (left factor exp(b_r), right
// exp(-b_i), each taken against the 16-token tile references as in the
// forward, so that every factor stays finite: the lower bound g_min = -5 of
// the "Lower-bounded decay" paragraph keeps a tile's cumulative decay in
// [-80, 0]) to dqh, dkh and the gradient of b, whose suffix sums over the
// chunk give the gradient of g = -5 sigmoid(a); last the input maps (L2 norm,
// sigmoid).
//
// Kernels:
//   bwd_plan_kernel       per-sequence chunk and recorded-state offsets
//   bwd_chainprep_kernel  one workgroup per (chunk, head), all in parallel:
//                         the adjoint chain's chunk-local operands (Qbar^T -
//                         W P^T and -W with W = (beta Kbar)^T X^T, Kend,
//                         Gamma_end) as a record, with P^T, X^T and Mkk for
//                         the chunk kernel
//   bwd_chain_kernel      the adjoint chain: one workgroup per (sequence,
//                         head) walks the chunks last to first over the
//                         records and stores dS_end of every chunk
//   bwd_chunk_kernel      one workgroup per (chunk, head), all in parallel:
//                         every gradient of the chunk's tokens from its start
//                         state (recorded by the forward every 32 tokens) and
//                         dS_end
// The first three need no forward state: the chain runs on the device's
// second stream beside the forward recomputation.
#include <mutex>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kCB = 32;      // chunk length (tokens)
constexpr int kTl = 16;      // tile length (tokens)
constexpr int kL32 = kCB + 4;  // padded row stride of [32][32] tiles
constexpr int kPlanThr = 256;

__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
// A wave-uniform pointer pinned in scalar registers (and hidden from the
// optimiser), so that p[lane_offset] with a 32-bit offset is addressed as
// scalar base + 32-bit vector offset instead of 64-bit vector arithmetic.
template <typename T>
using gptr = __attribute__((address_space(1))) T*;
template <typename T>
__device__ __forceinline__ gptr<T> sbase(T* p) {
  gptr<T> gp = (gptr<T>)p;
  __asm__ volatile("" : "+s"(gp));
  return gp;
}
// Element i of a scalar-based array, as a T pointer whose byte offset is
// formed in 32 bits (the access's 32-bit vector offset).
template <typename T, typename B>
__device__ __forceinline__ gptr<T> gat(gptr<B> base, uint32_t i) {
  return (gptr<T>)((__attribute__((address_space(1))) const char*)base + i * (uint32_t)sizeof(B));
}
// A bf16 input element loaded ahead of its use as the aligned 32-bit word that
// holds it (element i of a row-major tensor with even rows), converted where
// it is used: the empty asm keeps the compiler from moving the conversion (and
// with it the wait for the load, which also covers every earlier request) up
// to the load.
__device__ __forceinline__ uint32_t word_of(gptr<const uint16_t> p, uint32_t i) {
  return *gat<const uint32_t>(p, i & ~1u);
}
__device__ __forceinline__ float late_f32(uint32_t u, bool high) {
  asm volatile("" : "+v"(u));
  return __uint_as_float(high ? (u & 0xFFFF0000u) : (u << 16));
}

// Matrix-core products over one 32-wide block of the contraction index: lane
// l supplies 8 values of row m = l % 16 of A and 8 of column n = l % 16 of B;
// slot j of lane group g = l / 16 stands for one contraction index (any
// bijection onto the block, the same for A and B).  The 16x16 fp32 result
// tile: lane l holds rows 4 (l / 16) + 0..3 of column l % 16.
//
// Each fp32 operand is split into bf16 hi + lo (hi = x rounded to bf16, lo =
// x - hi, exact in fp32, rounded to bf16; gfx950's packed fp32 -> bf16
// conversion does both roundings) and the block is three bf16 MFMAs
// (v_mfma_f32_16x16x32_bf16), hi*hi + hi*lo + lo*hi with fp32 accumulation:
// the "bf16x3" method (Henry, Tang & Heinecke, 2019), about 2^-16 relative
// error per product, with fp32's exponent range (the tile factors reach e^80).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
struct F8 {
  bf16x8_t h, l;
};
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
// Two fp32 values rounded to nearest-even bf16, packed (a in the low half).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
__device__ __forceinline__ F8 split8(const float (&x)[8]) {
  u32x4_t hv, lv;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t hw = pk_bf16(x[2 * p], x[2 * p + 1]);
    hv[p] = hw;
    lv[p] = pk_bf16(x[2 * p] - __uint_as_float(hw << 16),
                    x[2 * p + 1] - __uint_as_float(hw & 0xFFFF0000u));
  }
  return {__builtin_bit_cast(bf16x8_t, hv), __builtin_bit_cast(bf16x8_t, lv)};
}
__device__ __forceinline__ void mma3(f32x4_t& acc, const F8& a, const F8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.l, b.h, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.h, b.l, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.h, b.h, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma3(f32x4_t& acc, const float (&a)[8], const F8& b) {
  mma3(acc, split8(a), b);
}
__device__ __forceinline__ void mma3(f32x4_t& acc, const float (&a)[8], const float (&b)[8]) {
  mma3(acc, split8(a), split8(b));
}

// Contraction index of slot j for lane group g when the B operand is formed
// from two stacked 16-row result tiles held in registers (rows 0-15 then 16-31).
__device__ __forceinline__ int kperm(int g, int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); }

// Sum over the 16 lanes of each row of 16 (lanes 16 q .. 16 q + 15), in every
// lane of the row: rotations within the row by 8, 4, 2 and 1 lanes (DPP).
template <int CTRL>
__device__ __forceinline__ float dpp_ror(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_ror<0x128>(x);  // row_ror:8
  x += dpp_ror<0x124>(x);  // row_ror:4
  x += dpp_ror<0x122>(x);  // row_ror:2
  return x + dpp_ror<0x121>(x);  // row_ror:1
}

// 8 consecutive floats from LDS (16-byte aligned), and 4 + 4 floats at p and
// p + 16 (the contraction order of a B operand formed from two stacked result
// tiles: slot j < 4 is index 4 g + j, slot j >= 4 is index 16 + 4 g + j - 4).
__device__ __forceinline__ void lds8f(const float* p, float (&x)[8]) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  const float4 w = *reinterpret_cast<const float4*>(p + 4);
  x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
  x[4] = w.x; x[5] = w.y; x[6] = w.z; x[7] = w.w;
}
__device__ __forceinline__ void st8f(float* p, const float (&x)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void lds44f(const float* p, float (&x)[8]) {
  const float4 u = *reinterpret_cast<const float4*>(p);
  const float4 w = *reinterpret_cast<const float4*>(p + 16);
  x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
  x[4] = w.x; x[5] = w.y; x[6] = w.z; x[7] = w.w;
}

// Operands kept in LDS already split: a bf16 hi plane and a lo plane of the
// same shape (u16 elements, row stride ld).  8 consecutive elements of a row
// as the F8 of a matrix-core operand (16-byte aligned), a split row segment
// written, and one element written.
__device__ __forceinline__ F8 ld8h(const uint16_t* hp, const uint16_t* lp, int off) {
  return {__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(hp + off)),
          __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(lp + off))};
}
__device__ __forceinline__ void st8h(uint16_t* hp, uint16_t* lp, int off, const float (&x)[8]) {
  const F8 f = split8(x);
  *reinterpret_cast<u32x4_t*>(hp + off) = __builtin_bit_cast(u32x4_t, f.h);
  *reinterpret_cast<u32x4_t*>(lp + off) = __builtin_bit_cast(u32x4_t, f.l);
}
__device__ __forceinline__ void st1h(uint16_t* hp, uint16_t* lp, int off, float x) {
  const __bf16 h = (__bf16)x;
  hp[off] = __builtin_bit_cast(uint16_t, h);
  lp[off] = __builtin_bit_cast(uint16_t, (__bf16)(x - (float)h));
}
// 8 elements of a column (rows r0 + 0..7, row stride ld) as an F8.
__device__ __forceinline__ F8 col8h(const uint16_t* hp, const uint16_t* lp, int off, int ld) {
  u32x4_t hv, lv;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    hv[q] = (uint32_t)hp[off + 2 * q * ld] | ((uint32_t)hp[off + (2 * q + 1) * ld] << 16);
    lv[q] = (uint32_t)lp[off + 2 * q * ld] | ((uint32_t)lp[off + (2 * q + 1) * ld] << 16);
  }
  return {__builtin_bit_cast(bf16x8_t, hv), __builtin_bit_cast(bf16x8_t, lv)};
}

// Element offset of the 4-row run (rows 16 ct + 4 (l / 16) + 0..3, column
// 16 w + l % 16) in the tile layout of a [DK][DV] adjoint state: runs ordered
// by row tile ct, then column tile w, then lane l, so that a wave storing its
// result tiles writes 1 KB contiguous per tile.
__device__ __forceinline__ int64_t dse_tile(int ct, int w, int l, int DV) {
  return ((int64_t)(ct * (DV / 16) + w) * 64 + l) * 4;
}

// Chunk offsets per sequence: cbase[n] = sum over m < n of ceil(L_m / 32)
// (the chunks), kbase[n] = sum of floor(L_m / 32) (the forward's states
// recorded every 32 tokens); cbase[N], kbase[N] are the totals.
__global__ void __launch_bounds__(kPlanThr)
    bwd_plan_kernel(const int32_t* __restrict__ cu_seqlens, int N, int32_t* __restrict__ cbase,
                    int32_t* __restrict__ kbase) {
  __shared__ int sc[kPlanThr], sk[kPlanThr];
  const int t = threadIdx.x;
  const int per = (N + kPlanThr - 1) / kPlanThr;
  const int n0 = min(N, t * per), n1 = min(N, n0 + per);
  int mc = 0, mk = 0;
  for (int n = n0; n < n1; ++n) {
    const int L = cu_seqlens[n + 1] - cu_seqlens[n];
    mc += (L + kCB - 1) / kCB;
    mk += L / kCB;
  }
  sc[t] = mc;
  sk[t] = mk;
  __syncthreads();
  for (int d = 1; d < kPlanThr; d <<= 1) {  // inclusive scans
    const int xc = t >= d ? sc[t - d] : 0, xk = t >= d ? sk[t - d] : 0;
    __syncthreads();
    sc[t] += xc;
    sk[t] += xk;
    __syncthreads();
  }
  int oc = sc[t] - mc, ok = sk[t] - mk;
  for (int n = n0; n < n1; ++n) {
    const int L = cu_seqlens[n + 1] - cu_seqlens[n];
    cbase[n] = oc;
    kbase[n] = ok;
    oc += (L + kCB - 1) / kCB;
    ok += L / kCB;
  }
  if (t == kPlanThr - 1) {
    cbase[N] = sc[t];
    kbase[N] = sk[t];
  }
}

// ---------------------------------------------------------------------------
// Chunk-local preparation shared by both kernels: the rows of the chunk's q,
// k, a (rows past the end are zero, so they add nothing and keep b flat),
// their L2 norms, g = -5 sigmoid(a) and its chunk-local inclusive cumsum b
// (into sB), the per-tile factors, and the scaled operands
//   Qt = qh exp(b - p), Kt = kh exp(b - p), Kh = kh exp(p - b)
// with p the cumulative decay before the row's 16-token tile (0 or b_15).
// Factor tables (DK each): sE[tt] = exp(p_tt), sF[tt] = exp(e_tt - p_tt)
// (e_tt = b at the tile's last row), sF2[tt] = exp(b_end - e_tt),
// sD = exp(p_1 - p_0), sGe = exp(b_end).
// ---------------------------------------------------------------------------
// The chunk's q, k, a rows as bf16 words (8 channels per thread and round),
// requested ahead of the rest of the preparation so that their wait can be
// shared with other requests; rows past the sequence's end read its last row
// and are masked in chunk_prep.
template <int DK, int NTHR>
struct PrepRows {
  static constexpr int NSEG = DK / 8;
  static constexpr int NIT = (kCB * NSEG + NTHR - 1) / NTHR;
  u32x4_t q[NIT], k[NIT], a[NIT];
};
template <int DK, int NTHR>
__device__ __forceinline__ void prep_rows(const uint16_t* __restrict__ q,
                                          const uint16_t* __restrict__ k,
                                          const uint16_t* __restrict__ a, int64_t c0, int nrows,
                                          int H, int h, int t, PrepRows<DK, NTHR>& in) {
  using PR = PrepRows<DK, NTHR>;
  const int64_t rb = (c0 * H + h) * (int64_t)DK;  // row 0 of the chunk, head h
  const gptr<const uint16_t> qb = sbase(q + rb), kb = sbase(k + rb), ab = sbase(a + rb);
#pragma unroll
  for (int it = 0; it < PR::NIT; ++it) {
    const int idx = t + NTHR * it, row = idx / PR::NSEG, seg = idx % PR::NSEG;
    if (idx < kCB * PR::NSEG) {  // uniform per wave: kCB * NSEG is a multiple of 64
      const int rr = row < nrows ? row : nrows - 1;
      const uint32_t off = (uint32_t)(rr * H * DK + seg * 8);
      in.q[it] = *gat<const u32x4_t>(qb, off);
      in.k[it] = *gat<const u32x4_t>(kb, off);
      in.a[it] = *gat<const u32x4_t>(ab, off);
    }
  }
}
__device__ __forceinline__ void unpack8(const u32x4_t& w, bool valid, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = valid ? __uint_as_float(w[i] << 16) : 0.f;
    x[2 * i + 1] = valid ? __uint_as_float(w[i] & 0xFFFF0000u) : 0.f;
  }
}

template <int DK, int NTHR>
__device__ __forceinline__ void chunk_prep(const PrepRows<DK, NTHR>& in, int nrows, int t,
                                           float* sB, float* sQt, float* sKt, float* sKh,
                                           float* sE, float* sF, float* sF2, float* sD,
                                           float* sGe) {
  constexpr int LDK = DK + 4;
  constexpr int NSEG = DK / 8;
  constexpr int NIT = PrepRows<DK, NTHR>::NIT;
  float qh[NIT][8], kh[NIT][8];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int idx = t + NTHR * it, row = idx / NSEG, seg = idx % NSEG;
    if (idx < kCB * NSEG) {  // uniform per wave: kCB * NSEG is a multiple of 64
      float qx[8], kx[8], ax[8];
      const bool valid = row < nrows;
      unpack8(in.q[it], valid, qx);
      unpack8(in.k[it], valid, kx);
      unpack8(in.a[it], valid, ax);
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sq += qx[j] * qx[j];
        sk += kx[j] * kx[j];
      }
      sq = group_sum<NSEG>(sq);
      sk = group_sum<NSEG>(sk);
      const float rq = rsqrtf(sq + kNormEps), rk = rsqrtf(sk + kNormEps);
      float g8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        qh[it][j] = qx[j] * rq;
        kh[it][j] = kx[j] * rk;
        g8[j] = valid ? kGMin * sigm(ax[j]) : 0.f;
      }
      st8f(sB + row * LDK + seg * 8, g8);
    }
  }
  lds_barrier();
  {  // cumsum along the chunk, then the factors of each channel
    // TPC neighbouring lanes share a channel, each with RPT consecutive rows:
    // a prefix over its rows, then over the lanes before it (shuffles).
    constexpr int TPC = NTHR / DK, RPT = kCB / TPC;
    static_assert(TPC * DK == NTHR && RPT * TPC == kCB && (TPC & (TPC - 1)) == 0, "scan split");
    const int c = t / TPC, qq = t % TPC;
    float x[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) x[i] = sB[(qq * RPT + i) * LDK + c];
#pragma unroll
    for (int i = 1; i < RPT; ++i) x[i] += x[i - 1];
    float incl = x[RPT - 1];  // inclusive over the lanes qq' <= qq
#pragma unroll
    for (int d = 1; d < TPC; d <<= 1) {
      const float y = __shfl_up(incl, d, TPC);
      if (qq >= d) incl += y;
    }
    const float before = incl - x[RPT - 1];
#pragma unroll
    for (int i = 0; i < RPT; ++i) sB[(qq * RPT + i) * LDK + c] = x[i] + before;
    const float p1 = __shfl(incl, (t & 63 & ~(TPC - 1)) + (kTl / RPT - 1), 64);
    const float be = __shfl(incl, (t & 63) | (TPC - 1), 64);
    if (qq == 0) {
      sE[c] = 1.f;
      sE[DK + c] = __expf(p1);
      sF[c] = __expf(p1);            // e_0 = p_1, p_0 = 0
      sF[DK + c] = __expf(be - p1);  // e_1 = b_end
      sF2[c] = __expf(be - p1);
      sF2[DK + c] = 1.f;
      sD[c] = __expf(p1);
      sGe[c] = __expf(be);
    }
  }
  lds_barrier();
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int idx = t + NTHR * it, row = idx / NSEG, seg = idx % NSEG;
    if (idx < kCB * NSEG) {
      float b8[8], p8[8], q8[8], k8[8], h8[8];
      lds8f(sB + row * LDK + seg * 8, b8);
      if (row < kTl) {
#pragma unroll
        for (int j = 0; j < 8; ++j) p8[j] = 0.f;
      } else {
        lds8f(sB + (kTl - 1) * LDK + seg * 8, p8);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = b8[j] - p8[j];  // in [-80, 0]
        const float er = __expf(x);
        q8[j] = qh[it][j] * er;
        k8[j] = kh[it][j] * er;
        h8[j] = kh[it][j] * __expf(-x);
      }
      st8f(sQt + row * LDK + seg * 8, q8);
      st8f(sKt + row * LDK + seg * 8, k8);
      st8f(sKh + row * LDK + seg * 8, h8);
    }
  }
  lds_barrier();
}

// Mkk and P tiles of the chunk (six 16x16 jobs: Mkk (0,0), (1,0), (1,1) and P
// the same, contraction over the DK channels), job j on wave j % nwaves:
// Mkk_ri = sum_c Kt_rc Kh_ic [exp(p_1 - p_0) when i is in tile 0 and r in
// tile 1], strictly lower; P likewise from Qt, lower with the diagonal.  Mkk
// goes to sM (scaled by beta_r when `scale_beta`: the A = diag(beta) Mkk of
// X), P to sP and its transpose to sPT.  The upper tiles are the caller's.
template <int DK>
__device__ __forceinline__ void key_products(int wave, int nwaves, int g, int li,
                                             const float* sQt, const float* sKt,
                                             const float* sKh, const float* sD,
                                             const float* sBeta, bool scale_beta, float* sM,
                                             float* sP, float* sPT) {
  constexpr int LDK = DK + 4;
  for (int job = wave; job < 6; job += nwaves) {
    const bool isP = job >= 3;
    const int jb = job % 3;
    const int tr = jb == 0 ? 0 : 1, ti = jb == 2 ? 1 : 0;
    const float* rows = isP ? sQt : sKt;
    const bool dsc = ti < tr;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      float av[8], bv[8];
      const int cb = 32 * kb + 8 * g;
      lds8f(rows + (16 * tr + li) * LDK + cb, av);
      lds8f(sKh + (16 * ti + li) * LDK + cb, bv);
      if (dsc) {
        float dv8[8];
        lds8f(sD + cb, dv8);
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[j] *= dv8[j];
      }
      mma3(acc, av, bv);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * tr + 4 * g + jj, i = 16 * ti + li;
      if (isP) {
        const float pv = i <= r ? acc[jj] : 0.f;
        sP[r * kL32 + i] = pv;
        sPT[i * kL32 + r] = pv;
      } else {
        sM[r * kL32 + i] = i < r ? (scale_beta ? acc[jj] * sBeta[r] : acc[jj]) : 0.f;
      }
    }
  }
}

// Zero of the upper 16x16 tile (rows 0-15, columns 16-31) of a [32][32] tile
// set, and of the lower-left tile of its transpose, by one wave.
__device__ __forceinline__ void zero_upper(int lane, float* M, float* MT) {
#pragma unroll
  for (int e = lane; e < 256; e += 64) {
    M[(e / 16) * kL32 + 16 + e % 16] = 0.f;
    if (MT) MT[(16 + e / 16) * kL32 + e % 16] = 0.f;
  }
}
// Element (r, i) of a split [32][32] plane: rows of 32 u16 (64 bytes) whose
// 16-byte groups are permuted by row (group i / 8 stored at (i / 8) xor
// ((r / 2) % 4)), so that sixteen rows' reads of one group hit the banks as a
// padded layout would, in 2 KB per plane.
__device__ __forceinline__ int sw32(int r, int i) {
  return r * 32 + ((((i >> 3) ^ (r >> 1)) & 3) << 3) + (i & 7);
}
// The upper tile of split [32][32] planes (hi and lo of M and of M^T) zeroed.
__device__ __forceinline__ void zero_upper_h(int lane, uint16_t* Mh, uint16_t* Ml, uint16_t* MTh,
                                             uint16_t* MTl) {
#pragma unroll
  for (int e = lane; e < 256; e += 64) {
    const int o = sw32(e / 16, 16 + e % 16), oT = sw32(16 + e / 16, e % 16);
    Mh[o] = 0;
    Ml[o] = 0;
    MTh[oT] = 0;
    MTl[oT] = 0;
  }
}

// X = (I + diag(beta) Mkk)^-1 (unit lower triangular, 32 x 32) by wave 0,
// into sX and its transpose sXT: the two diagonal 16x16 blocks by forward
// substitution (one lane per block column), then X_10 = -X_11 A_10 X_00
// through the scratch tile sT.  `betaM` says whether sM already holds
// diag(beta) Mkk.
__device__ __forceinline__ void solve_x(int wave, int lane, int g, int li, const float* sM,
                                        const float* sBeta, bool betaM, float* sX, float* sXT,
                                        float* sT) {
  if (wave != 0) return;
  if (lane < 32) {
    const int tb = lane / 16, jc = lane % 16;
    const float* blk = sM + (16 * tb) * kL32 + 16 * tb;
    float x[16];
    // row r of the block is read (4 x 16 bytes) while row r - 1 is solved
    float4 cur[4], nxt[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) cur[q4] = *reinterpret_cast<const float4*>(blk + 4 * q4);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r < 15) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          nxt[q4] = *reinterpret_cast<const float4*>(blk + (r + 1) * kL32 + 4 * q4);
      }
      const float arow[16] = {cur[0].x, cur[0].y, cur[0].z, cur[0].w, cur[1].x, cur[1].y,
                              cur[1].z, cur[1].w, cur[2].x, cur[2].y, cur[2].z, cur[2].w,
                              cur[3].x, cur[3].y, cur[3].z, cur[3].w};
      const float br = betaM ? 1.f : sBeta[16 * tb + r];
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc += arow[i] * x[i];
      x[r] = (r == jc ? 1.f : 0.f) - br * acc;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) cur[q4] = nxt[q4];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sX[(16 * tb + r) * kL32 + 16 * tb + jc] = x[r];
      sXT[(16 * tb + jc) * kL32 + 16 * tb + r] = x[r];
    }
  }
  zero_upper(lane, sX, sXT);
  lds_wave_fence();
  // sT = A_10 X_00, rows 4g + jj, column li
  float y[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int r = 4 * g + jj;
    const float br = betaM ? 1.f : sBeta[16 + r];
    float s = 0.f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) s += sM[(16 + r) * kL32 + kk] * sX[kk * kL32 + li];
    y[jj] = br * s;
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) sT[(4 * g + jj) * 16 + li] = y[jj];
  lds_wave_fence();
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int r = 4 * g + jj;
    float s = 0.f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) s += sX[(16 + r) * kL32 + 16 + kk] * sT[kk * 16 + li];
    sX[(16 + r) * kL32 + li] = -s;
    sXT[li * kL32 + 16 + r] = -s;
  }
}

// ---------------------------------------------------------------------------
// The adjoint chain, in two kernels.  Per chunk,
//   dS <- diag(Gamma_end) dS + Qbar^T dO - (beta Kbar)^T X^T (P^T dO + Kend dS)
//       = diag(Gamma_end) dS + Qc dO + Wn (Kend dS),
// with the chunk-local Wn = -(beta Kbar)^T X^T and Qc = Qbar^T + Wn P^T, so
// bwd_chainprep_kernel forms Qc, Wn, Kend and Gamma_end for every (chunk,
// head) in parallel and stores them as a chain record, and bwd_chain_kernel
// walks each head's chunks last to first reading the records (the next
// chunk's record and dO are fetched while the current chunk is processed):
// two dependent products per chunk (Kend dS, then Wn times it).
// Record, fp32 (the operands read along the chunk's rows transposed, so that
// every matrix-core operand is a contiguous read):
//   Qc [DK][32] | Wn [DK][32] | Kend [32][DK] | Gamma_end [DK] | P^T [32][32] |
//   X^T [32][32] | Mkk [32][32]
// ---------------------------------------------------------------------------
template <int DK>
struct ChainRec {
  // the chain's operands (it reads the first `chain` floats), then P^T, X^T
  // and Mkk for the chunk kernel; `floats` is the record's stride
  static constexpr int oQc = 0, oWn = DK * kCB, oKe = 2 * DK * kCB, oGe = 3 * DK * kCB,
                       chain = oGe + DK, oPT = chain, oXT = oPT + kCB * kCB,
                       oM = oXT + kCB * kCB, floats = oM + kCB * kCB;
  static_assert(chain % 4 == 0 && floats % 4 == 0, "float4 copies");
};

template <int DK>
struct PrepLayout {
  static constexpr int LDK = DK + 4;
  // The chunk-local cumsum b during the preparation; once the scaled operands
  // are formed, Mkk, P, P^T and the solve's 16 x 16 scratch in its place.
  static constexpr int oB = 0;
  static constexpr int oM = 0, oP = oM + kCB * kL32, oPT = oP + kCB * kL32, oT = oPT + kCB * kL32;
  static constexpr int r0 = kCB * LDK > oT + 256 ? kCB * LDK : oT + 256;
  static constexpr int oQt = oB + r0;
  static constexpr int oKt = oQt + kCB * LDK;
  static constexpr int oKh = oKt + kCB * LDK;    // Kh, then Kend
  static constexpr int oX = oKh + kCB * LDK;
  static constexpr int oXT = oX + kCB * kL32;
  // Factor tables: exp(p_0) (tile 0 of E) and exp(b_end - e_1) (tile 1 of
  // F2) are both all ones and share storage: [F2 tile 0 | ones | E tile 1].
  static constexpr int oF2 = oXT + kCB * kL32;
  static constexpr int oE = oF2 + DK;
  static constexpr int oF = oE + 2 * DK;
  static constexpr int oD = oF + 2 * DK;
  static constexpr int oGe = oD + DK;
  static constexpr int oBeta = oGe + DK;
  static constexpr int total = oBeta + kCB;
  static_assert(total * 4 <= 80 * 1024, "LDS budget: two workgroups per CU");
};

constexpr int kPrepThr = 512;

// Chain records of every (chunk, head): workgroup (chunk, head), 8 waves.
template <typename TI, int DK>
__global__ void __launch_bounds__(kPrepThr, 2)
    bwd_chainprep_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                         const TI* __restrict__ a, const TI* __restrict__ bl,
                         const int32_t* __restrict__ cu_seqlens,
                         const int32_t* __restrict__ cbase, float* __restrict__ crec, int N,
                         int H) {
  using Ly = PrepLayout<DK>;
  using R = ChainRec<DK>;
  constexpr int LDK = Ly::LDK;
  extern __shared__ float smem[];
  float* sB = smem + Ly::oB;
  float* sQt = smem + Ly::oQt;
  float* sKt = smem + Ly::oKt;
  float* sKh = smem + Ly::oKh;
  float* sM = smem + Ly::oM;
  float* sP = smem + Ly::oP;
  float* sPT = smem + Ly::oPT;
  float* sX = smem + Ly::oX;
  float* sXT = smem + Ly::oXT;
  float* sT = smem + Ly::oT;
  float* sE = smem + Ly::oE;
  float* sF = smem + Ly::oF;
  float* sF2 = smem + Ly::oF2;
  float* sD = smem + Ly::oD;
  float* sGe = smem + Ly::oGe;
  float* sBeta = smem + Ly::oBeta;

  const int ci = blockIdx.x / H, h = blockIdx.x % H;
  if (ci >= cbase[N]) return;  // the grid covers an upper bound of the chunk count
  int lo = 0, hi = N;          // the sequence n with cbase[n] <= ci < cbase[n + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (cbase[mid] <= ci) lo = mid; else hi = mid;
  }
  const int n = lo;
  const int m = ci - cbase[n];
  const int t = threadIdx.x, wave = t / 64, lane = t % 64, g = lane / 16, li = lane % 16;
  const int64_t tok_beg = cu_seqlens[n], tok_end = cu_seqlens[n + 1];
  const int64_t c0 = tok_beg + (int64_t)kCB * m;
  const int nrows = (int)(tok_end - c0 < kCB ? tok_end - c0 : kCB);

  PrepRows<DK, kPrepThr> rows;
  prep_rows<DK, kPrepThr>(q, k, a, c0, nrows, H, h, t, rows);
  // b of row t (a valid row), from an even base so that words stay aligned
  const int64_t b0 = c0 * H + h;
  const uint32_t eb = (uint32_t)((b0 & 1) + (t < nrows ? t : nrows - 1) * H);
  const uint32_t bw = word_of(sbase(bl + (b0 & ~(int64_t)1)), eb);
  if (t < kCB) sBeta[t] = t < nrows ? sigm(late_f32(bw, eb & 1)) : 0.f;
  chunk_prep<DK, kPrepThr>(rows, nrows, t, sB, sQt, sKt, sKh, sE, sF, sF2, sD, sGe);
  key_products<DK>(wave, kPrepThr / 64, g, li, sQt, sKt, sKh, sD, sBeta, false, sM, sP, sPT);
  if (wave == 6) zero_upper(lane, sP, sPT);
  if (wave == 7) zero_upper(lane, sM, nullptr);
  lds_barrier();
  solve_x(wave, lane, g, li, sM, sBeta, false, sX, sXT, sT);
  // Kend in place
  for (int idx = t; idx < kCB * DK / 4; idx += kPrepThr) {
    const int row = idx % kCB, c = 4 * (idx / kCB), tt = row / kTl;
    const float4 f = *reinterpret_cast<const float4*>(sF + tt * DK + c);
    const float4 f2 = *reinterpret_cast<const float4*>(sF2 + tt * DK + c);
    float4* kh = reinterpret_cast<float4*>(sKh + row * LDK + c);
    const float4 hv = *kh;
    *kh = make_float4(hv.x * f.x * f2.x, hv.y * f.y * f2.y, hv.z * f.z * f2.z, hv.w * f.w * f2.w);
  }
  lds_barrier();  // X, X^T and Kend
  float* dst = crec + (((int64_t)cbase[n] + m) * H + h) * (int64_t)R::floats;
  // Wn and Qc on the matrix cores (bf16x3): wave w, key channels
  // i = 16 w + li.  Wn^T = -X (beta Kbar) leaves lane (li, g) holding Wn[i][u]
  // at u = kperm(g, j), which is the B operand of Qc^T = Qbar + P Wn^T over
  // that u order (the A operand P[r][u] = (P^T)[u][r] is read in it).
  if (16 * wave < DK) {
    const int i = 16 * wave + li;
    float kb[8];  // -(beta Kbar)[s][i] at s = 8 g + 0..7
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sr = 8 * g + j;
      kb[j] = -sBeta[sr] * sKt[sr * LDK + i] * sE[(sr / kTl) * DK + i];
    }
    const F8 kbf = split8(kb);
    f32x4_t wt[2];  // wt[rt][j] = Wn[i][16 rt + 4 g + j]
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      wt[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      float av[8];
      lds8f(sX + (16 * rt + li) * kL32 + 8 * g, av);
      mma3(wt[rt], av, kbf);
      *reinterpret_cast<f32x4_t*>(dst + R::oWn + i * kCB + 16 * rt + 4 * g) = wt[rt];
    }
    F8 wf;
    {
      float wv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[j] = wt[j >> 2][j & 3];
      wf = split8(wv);
    }
#pragma unroll
    for (int ot = 0; ot < 2; ++ot) {  // Qc^T rows r = 16 ot + 4 g + j, column i
      f32x4_t acc;
      float av[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = sQt[(16 * ot + 4 * g + j) * LDK + i] * sE[ot * DK + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) av[j] = sPT[kperm(g, j) * kL32 + 16 * ot + li];
      mma3(acc, av, wf);
      *reinterpret_cast<f32x4_t*>(dst + R::oQc + i * kCB + 16 * ot + 4 * g) = acc;
    }
  }
  // Kend, Gamma_end, P^T, X^T, Mkk
  for (int i4 = t + R::oKe / 4; i4 < R::floats / 4; i4 += kPrepThr) {
    const int e = 4 * i4;
    const float* src;
    if (e < R::oGe) {
      src = sKh + ((e - R::oKe) / DK) * LDK + (e - R::oKe) % DK;
    } else if (e < R::oPT) {
      src = sGe + (e - R::oGe);
    } else if (e < R::oXT) {
      src = sPT + ((e - R::oPT) / kCB) * kL32 + (e - R::oPT) % kCB;
    } else if (e < R::oM) {
      src = sXT + ((e - R::oXT) / kCB) * kL32 + (e - R::oXT) % kCB;
    } else {
      src = sM + ((e - R::oM) / kCB) * kL32 + (e - R::oM) % kCB;
    }
    *reinterpret_cast<float4*>(dst + e) = *reinterpret_cast<const float4*>(src);
  }
}

// The chain: workgroup (sequence, head), one wave per 16 columns of d_v; wave
// w holds columns 16 w .. 16 w + 15 of dS (d_k rows) in matrix-core result
// tiles: dS[ct] = rows 16 ct + 4 g + 0..3, column 16 w + li.  Two LDS buffers
// of [record | dO^T]; per chunk, last first: store dS (= dS_end of the
// chunk), request the next chunk's record and dO, run the chain on this
// chunk's buffer, then write the requested data to the other buffer.
template <int DK, int DV>
struct ChainLayout {
  static constexpr int LDK = DK + 4;
  static constexpr int oQc = 0;                  // [DK][36]
  static constexpr int oWn = oQc + DK * kL32;    // [DK][36]
  static constexpr int oKe = oWn + DK * kL32;    // [32][LDK]
  static constexpr int oGe = oKe + kCB * LDK;    // [DK]
  static constexpr int oDOT = oGe + DK;          // dO^T [DV][36]
  static constexpr int buf = oDOT + DV * kL32;   // floats per buffer
  static constexpr int total = 2 * buf;
  static_assert(total * 4 <= 160 * 1024, "LDS budget");
};

template <typename TI, int DK, int DV>
__device__ __forceinline__ void chain_fetch(const float* __restrict__ src,
                                            const TI* __restrict__ gate,
                                            const float* __restrict__ dy, int64_t tok_beg,
                                            int64_t tok_end, int m, int H, int h, int t,
                                            f32x4_t (&rv)[(ChainRec<DK>::chain / 4 + 4 * DV - 1) / (4 * DV)],
                                            float (&d8)[8], u32x4_t& g8, bool& have_row) {
  using R = ChainRec<DK>;
  static_assert(sizeof(TI) == 2, "bf16 gate: 8 values in 16 bytes");
  constexpr int NTHR = 4 * DV;
  constexpr int NR4 = (R::chain / 4 + NTHR - 1) / NTHR;
#pragma unroll
  for (int i = 0; i < NR4; ++i) {
    const int i4 = t + NTHR * i;
    if (NTHR * (i + 1) <= R::chain / 4 || i4 < R::chain / 4)
      rv[i] = *reinterpret_cast<const f32x4_t*>(src + 4 * i4);
  }
  const int64_t c0 = tok_beg + (int64_t)kCB * m;
  const int nrows = (int)(tok_end - c0 < kCB ? tok_end - c0 : kCB);
  const int row = t % kCB, seg = t / kCB;
  have_row = row < nrows;
  if (have_row) {
    const int64_t off = ((c0 + row) * H + h) * (int64_t)DV + seg * 8;
    ld8(dy + off, d8);
    // the gate's raw 16-byte row piece: unpacked in chain_stash, so that no
    // wait for the loads (and the stores before them) lands here
    if (gate) g8 = *reinterpret_cast<const u32x4_t*>(gate + off);
  }
}

template <int DK, int DV>
__device__ __forceinline__ void chain_stash(float* b, int t, bool gated,
                                            const f32x4_t (&rv)[(ChainRec<DK>::chain / 4 + 4 * DV - 1) / (4 * DV)],
                                            const float (&d8)[8], const u32x4_t& g8,
                                            bool have_row) {
  using R = ChainRec<DK>;
  using Ly = ChainLayout<DK, DV>;
  constexpr int NTHR = 4 * DV;
  constexpr int NR4 = (R::chain / 4 + NTHR - 1) / NTHR;
  constexpr int LDK = Ly::LDK;
#pragma unroll
  for (int i = 0; i < NR4; ++i) {
    const int i4 = t + NTHR * i;
    if (NTHR * (i + 1) <= R::chain / 4 || i4 < R::chain / 4) {
      const int e = 4 * i4;
      float* d;
      if (e < R::oWn) {
        d = b + Ly::oQc + (e / kCB) * kL32 + e % kCB;
      } else if (e < R::oKe) {
        d = b + Ly::oWn + ((e - R::oWn) / kCB) * kL32 + (e - R::oWn) % kCB;
      } else if (e < R::oGe) {
        d = b + Ly::oKe + ((e - R::oKe) / DK) * LDK + (e - R::oKe) % DK;
      } else {
        d = b + Ly::oGe + (e - R::oGe);
      }
      *reinterpret_cast<f32x4_t*>(d) = rv[i];
    }
  }
  const int row = t % kCB, seg = t / kCB;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float gv = __uint_as_float(j % 2 ? (g8[j / 2] & 0xFFFF0000u) : (g8[j / 2] << 16));
    b[Ly::oDOT + (seg * 8 + j) * kL32 + row] = have_row ? (gated ? d8[j] * sigm(gv) : d8[j]) : 0.f;
  }
}

template <typename TI, int DK, int DV>
__global__ void __launch_bounds__(4 * DV)
    bwd_chain_kernel(const TI* __restrict__ gate, const float* __restrict__ dy,
                     const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cbase,
                     const float* __restrict__ crec, const float* __restrict__ d_sfinal,
                     float* __restrict__ dse, float* __restrict__ d_s0, int H) {
  using Ly = ChainLayout<DK, DV>;
  using R = ChainRec<DK>;
  constexpr int NTHR = 4 * DV;  // 64 lanes per 16 columns
  constexpr int LDK = Ly::LDK;
  constexpr int NCT = DK / 16, NKB = DK / 32;
  constexpr int NR4 = (R::chain / 4 + NTHR - 1) / NTHR;  // record float4 per thread
  extern __shared__ float smem[];

  const int item = blockIdx.x;
  const int n = item / H, h = item % H;
  const int t = threadIdx.x, wave = t / 64, lane = t % 64, g = lane / 16, li = lane % 16;
  const int jl = 16 * wave + li;  // this lane's column
  const int64_t tok_beg = cu_seqlens[n], tok_end = cu_seqlens[n + 1];
  const int64_t st_off = (int64_t)item * DK * DV;
  const int nch = (int)((tok_end - tok_beg + kCB - 1) / kCB);
  const int64_t cb0 = cbase[n];

  // The data of chunk m in registers: its record and this thread's 8 values
  // of dy and gate (row t % 32, columns 8 (t / 32) + 0..7), requested by
  // chain_fetch() and used only in chain_stash() (dO = dy sigmoid(gate) formed
  // there), so the loads stay in flight during the chain.
  f32x4_t rv[NR4];  // (native vectors: an array of HIP's float4 class stays in scratch)
  float d8[8];
  u32x4_t g8 = {0u, 0u, 0u, 0u};
  bool have_row = false;
  f32x4_t dS[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      dS[ct][jj] = d_sfinal ? d_sfinal[st_off + (int64_t)(16 * ct + 4 * g + jj) * DV + jl] : 0.f;

  if (nch > 0) {
    chain_fetch<TI, DK, DV>(crec + ((cb0 + nch - 1) * H + h) * (int64_t)R::floats, gate, dy,
                            tok_beg, tok_end, nch - 1, H, h, t, rv, d8, g8, have_row);
    chain_stash<DK, DV>(smem + ((nch - 1) & 1) * Ly::buf, t, gate != nullptr, rv, d8, g8, have_row);
    lds_barrier();
  }
  for (int m = nch - 1; m >= 0; --m) {
    const float* b = smem + (m & 1) * Ly::buf;
    const float* sQc = b + Ly::oQc;
    const float* sWn = b + Ly::oWn;
    const float* sKe = b + Ly::oKe;
    const float* sGe = b + Ly::oGe;
    const float* sDOT = b + Ly::oDOT;
    // dS_end of this chunk, in the tile layout (each wave writes 1 KB runs)
    {
      float* dst = dse + ((cb0 + m) * H + h) * (int64_t)DK * DV;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        *reinterpret_cast<f32x4_t*>(dst + dse_tile(ct, wave, lane, DV)) = dS[ct];
    }
    if (m > 0)
      chain_fetch<TI, DK, DV>(crec + ((cb0 + m - 1) * H + h) * (int64_t)R::floats, gate, dy,
                              tok_beg, tok_end, m - 1, H, h, t, rv, d8, g8, have_row);

    F8 dOf;  // column jl of dO, rows 8 g + 0..7
    {
      float dOv[8];
      lds8f(sDOT + jl * kL32 + 8 * g, dOv);
      dOf = split8(dOv);
    }
    F8 dSf[NKB];  // dS as B operand (rows 32 kb + kperm(g, j))
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float bv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) bv[j] = dS[2 * kb + (j >> 2)][j & 3];
      dSf[kb] = split8(bv);
    }
    // Y = Kend dS (rows 16 tt + 4 g + jj, column jl)
    f32x4_t Y[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      Y[tt] = {0.f, 0.f, 0.f, 0.f};
      float av[8];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        lds44f(sKe + (16 * tt + li) * LDK + 32 * kb + 4 * g, av);
        mma3(Y[tt], av, dSf[kb]);
      }
    }
    // dS <- diag(Gamma_end) dS + Qc dO + Wn Y
    F8 yf;
    {
      float yv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) yv[j] = Y[j >> 2][j & 3];
      yf = split8(yv);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4_t acc;
      const float4 ge = *reinterpret_cast<const float4*>(sGe + 16 * ct + 4 * g);
      acc[0] = ge.x * dS[ct][0]; acc[1] = ge.y * dS[ct][1];
      acc[2] = ge.z * dS[ct][2]; acc[3] = ge.w * dS[ct][3];
      const int c = 16 * ct + li;
      float av[8];
      lds8f(sQc + c * kL32 + 8 * g, av);
      mma3(acc, av, dOf);
      lds44f(sWn + c * kL32 + 4 * g, av);
      mma3(acc, av, yf);
      dS[ct] = acc;
    }
    if (m > 0)
      chain_stash<DK, DV>(smem + ((m - 1) & 1) * Ly::buf, t, gate != nullptr, rv, d8, g8,
                          have_row);
    lds_barrier();  // the next chunk's buffer is complete; this one is free
  }
  if (d_s0) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        d_s0[st_off + (int64_t)(16 * ct + 4 * g + jj) * DV + jl] = dS[ct][jj];
  }
}

// ---------------------------------------------------------------------------
// Gradients of one chunk.  Workgroup (chunk, head), 8 waves.  In the
// column-owning stages wave w owns column tile w (16 columns of d_v, later 16
// channels of d_k) over both 16-row tiles of the chunk.
// ---------------------------------------------------------------------------
constexpr int kGrThr = 512;

template <int DK, int DV>
struct GrLayout {
  static constexpr int LDK = DK + 4;
  static constexpr int LDH = DV + 8;           // row stride of the split [32][DV] planes (u16)
  static constexpr int oB = 0;                 // cumsum b
  static constexpr int oQt = oB + kCB * LDK;   // Qt, later dqh
  static constexpr int oKt = oQt + kCB * LDK;  // Kt, later dkh
  static constexpr int oKh = oKt + kCB * LDK;  // Kh, later the gradient of b
  static constexpr int oM = oKh + kCB * LDK;   // Mkk (without beta)
  // P, P^T, X, X^T (fp32), later dP, dP^T, dMkk, dMkk^T (split: a hi and a lo
  // [32][32] u16 plane each, in the same space)
  static constexpr int oP = oM + kCB * kL32;
  static constexpr int oPT = oP + kCB * kL32;
  static constexpr int oX = oPT + kCB * kL32;
  static constexpr int oXT = oX + kCB * kL32;
  // dO, U, Z [32][DV], split: hi plane then lo plane (kCB * LDH u16 each)
  static constexpr int oDO = oXT + kCB * kL32;
  static constexpr int oU = oDO + kCB * LDH;
  static constexpr int oZ = oU + kCB * LDH;
  static constexpr int oE = oZ + kCB * LDH;
  static constexpr int oF = oE + 2 * DK;
  static constexpr int oF2 = oF + 2 * DK;
  static constexpr int oD = oF2 + 2 * DK;
  static constexpr int oGe = oD + DK;
  static constexpr int oBeta = oGe + DK;
  static constexpr int oRed = oBeta + kCB;     // [16][32] partial row sums of dbeta
  static constexpr int total = oRed + 16 * kCB;
  static_assert(total * 4 <= 160 * 1024, "LDS budget");
};

// A (chunk, head) item of the chunk kernel: ci = chunk over all sequences,
// n = its sequence, m = its index there, c0 = its first token, nrows = its
// tokens (1..32).
struct BwdItem {
  int ci, h, n, m, nrows;
  int64_t c0;
};
__device__ __forceinline__ BwdItem bwd_item(int w, int H, int N, const int32_t* cbase,
                                            const int32_t* cu_seqlens) {
  BwdItem it;
  it.ci = w / H;
  it.h = w % H;
  int lo = 0, hi = N;  // the sequence n with cbase[n] <= ci < cbase[n + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (cbase[mid] <= it.ci) lo = mid; else hi = mid;
  }
  it.n = lo;
  it.m = it.ci - cbase[lo];
  const int64_t te = cu_seqlens[lo + 1];
  it.c0 = cu_seqlens[lo] + (int64_t)kCB * it.m;
  it.nrows = (int)(te - it.c0 < kCB ? te - it.c0 : kCB);
  return it;
}
// An item's prologue inputs, in registers: its q, k, a rows, the b word of
// row t, dO, gate and o of one 8-column segment, and the record's P^T, X^T
// (rpx) and Mkk (rmk) pieces.
template <int DK>
struct BwdPro {
  PrepRows<DK, kGrThr> rows;
  uint32_t bw;
  f32x4_t d0, d1, o0, o1, rpx, rmk;
  u32x4_t gw;
};
template <int DK, int DV, bool GATED>
__device__ __forceinline__ void bwd_request(const BwdItem& it, const uint16_t* __restrict__ q,
                                            const uint16_t* __restrict__ k,
                                            const uint16_t* __restrict__ a,
                                            const uint16_t* __restrict__ bl,
                                            const float* __restrict__ dy,
                                            const uint16_t* __restrict__ gate,
                                            const float* __restrict__ o_raw,
                                            const float* __restrict__ crec, int H, int t,
                                            BwdPro<DK>& p) {
  using R = ChainRec<DK>;
  prep_rows<DK, kGrThr>(q, k, a, it.c0, it.nrows, H, it.h, t, p.rows);
  // b of row t (a valid row), from an even base so that words stay aligned
  const int64_t b0 = it.c0 * H + it.h;
  const uint32_t eb = (uint32_t)((b0 & 1) + (t < it.nrows ? t : it.nrows - 1) * H);
  p.bw = word_of(sbase(bl + (b0 & ~(int64_t)1)), eb);
  constexpr int NDO = kCB * (DV / 8);
  const int drow = t / (DV / 8), dseg = t % (DV / 8);
  const int64_t rbv = (it.c0 * H + it.h) * (int64_t)DV;
  const uint32_t doff = (uint32_t)((drow < it.nrows ? drow : it.nrows - 1) * H * DV + dseg * 8);
  if (NDO == kGrThr || t < NDO) {
    const gptr<const f32x4_t> dp = gat<const f32x4_t>(sbase(dy + rbv), doff);
    p.d0 = dp[0];
    p.d1 = dp[1];
    if constexpr (GATED) {
      p.gw = *gat<const u32x4_t>(sbase(gate + rbv), doff);
      const gptr<const f32x4_t> op = gat<const f32x4_t>(sbase(o_raw + rbv), doff);
      p.o0 = op[0];
      p.o1 = op[1];
    }
  }
  const gptr<const float> rec = sbase(crec + ((int64_t)it.ci * H + it.h) * (int64_t)R::floats);
  p.rpx = *gat<const f32x4_t>(rec, R::oPT + 4 * t);
  p.rmk = *gat<const f32x4_t>(rec, R::oM + 4 * (t < kCB * kCB / 4 ? t : 0));
}

template <typename TI, int DK, int DV, bool GATED>
__global__ void __launch_bounds__(kGrThr)
    bwd_chunk_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                     const TI* __restrict__ v, const TI* __restrict__ a,
                     const TI* __restrict__ bl, const TI* __restrict__ gate,
                     const float* __restrict__ dy, const float* __restrict__ o_raw,
                     const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cbase,
                     const int32_t* __restrict__ kbase, const float* __restrict__ s_init,
                     const float* __restrict__ ckpt, const float* __restrict__ dse,
                     const float* __restrict__ crec, float* __restrict__ dq_out,
                     float* __restrict__ dk_out, float* __restrict__ dv_out,
                     float* __restrict__ da_out, float* __restrict__ db_out,
                     float* __restrict__ dgate_out, int N, int H) {
  using Ly = GrLayout<DK, DV>;
  using R = ChainRec<DK>;
  constexpr int LDK = Ly::LDK, LDH = Ly::LDH;
  constexpr int NKB = DK / 32, NVB = DV / 32;
  extern __shared__ float smem[];
  float* sB = smem + Ly::oB;
  float* sQt = smem + Ly::oQt;
  float* sKt = smem + Ly::oKt;
  float* sKh = smem + Ly::oKh;
  float* sM = smem + Ly::oM;
  float* sPT = smem + Ly::oPT;
  float* sX = smem + Ly::oX;
  float* sXT = smem + Ly::oXT;
  uint16_t* sDOh = reinterpret_cast<uint16_t*>(smem + Ly::oDO);
  uint16_t* sDOl = sDOh + kCB * LDH;
  uint16_t* sUh = reinterpret_cast<uint16_t*>(smem + Ly::oU);
  uint16_t* sUl = sUh + kCB * LDH;
  uint16_t* sZh = reinterpret_cast<uint16_t*>(smem + Ly::oZ);
  uint16_t* sZl = sZh + kCB * LDH;
  // the split dP, dP^T, dMkk, dMkk^T of stage E (over P, P^T, X, X^T)
  uint16_t* sdPh = reinterpret_cast<uint16_t*>(smem + Ly::oP);
  uint16_t* sdPl = sdPh + kCB * kCB;
  uint16_t* sdPTh = reinterpret_cast<uint16_t*>(smem + Ly::oPT);
  uint16_t* sdPTl = sdPTh + kCB * kCB;
  uint16_t* sdMh = reinterpret_cast<uint16_t*>(smem + Ly::oX);
  uint16_t* sdMl = sdMh + kCB * kCB;
  uint16_t* sdMTh = reinterpret_cast<uint16_t*>(smem + Ly::oXT);
  uint16_t* sdMTl = sdMTh + kCB * kCB;
  float* sE = smem + Ly::oE;
  float* sF = smem + Ly::oF;
  float* sF2 = smem + Ly::oF2;
  float* sD = smem + Ly::oD;
  float* sGe = smem + Ly::oGe;
  float* sBeta = smem + Ly::oBeta;
  float* sRed = smem + Ly::oRed;

  // One workgroup per CU walks the (chunk, head) items w = blockIdx.x +
  // k gridDim.x.  An item's prologue inputs (its q, k, a, b rows, dO, gate,
  // o and record tiles, about 77 KB) are requested during the previous item,
  // after that item's last loads: requested at the start of each item, as
  // every CU did at once, they made a burst that kept HBM busy while the
  // compute units waited (about 9K cycles per item).
  constexpr int NDO = kCB * (DV / 8);
  static_assert(NDO <= kGrThr, "one dO segment per thread");
  static_assert(R::oXT == R::oPT + kCB * kCB && 2 * kCB * kCB == 4 * kGrThr, "record split");
  const int total = cbase[N] * H;
  int w = blockIdx.x;
  if (w >= total) return;
  BwdItem it = bwd_item(w, H, N, cbase, cu_seqlens);
  BwdPro<DK> pro;
  bwd_request<DK, DV, GATED>(it, q, k, a, bl, dy, gate, o_raw, crec, H, (int)threadIdx.x, pro);
  for (;;) {
  // Lane indices re-derived from an opaque copy each item (keeps the
  // optimiser from hoisting every lane-dependent address out of the loop and
  // holding them all in registers).
  int t_ = threadIdx.x;
  __asm__ volatile("" : "+v"(t_));
  const int t = t_, wave = t / 64, lane = t % 64, g = lane / 16, li = lane % 16;
  // owns a column tile of d_v (of d_k): every wave when there are as many tiles
  const bool vwave = DV / 16 >= kGrThr / 64 || wave < DV / 16;
  const bool kwave = DK / 16 >= kGrThr / 64 || wave < DK / 16;
  const int jc = 16 * wave + li;      // this lane's column (d_v or d_k)
  const int drow = t / (DV / 8), dseg = t % (DV / 8);
  const bool dthr = NDO == kGrThr || t < NDO;  // (a branch only when d_v < 128)
  const int ci = it.ci, h = it.h, n = it.n, m = it.m, nrows = it.nrows;
  const int64_t c0 = it.c0;
  const int64_t item = (int64_t)n * H + h;
  // start state (null: zero) and dS_end of the chunk, [DK][DV] each
  const float* S = m == 0 ? (s_init ? s_init + item * DK * DV : nullptr)
                          : ckpt + (((int64_t)kbase[n] + m - 1) * H + h) * DK * DV;
  const float* dSe = dse + (((int64_t)cbase[n] + m) * H + h) * DK * DV;
  const int64_t b0 = c0 * H + h;
  const uint32_t eb = (uint32_t)((b0 & 1) + (t < nrows ? t : nrows - 1) * H);
  const uint32_t bw = pro.bw;
  const bool dvalid = dthr && drow < nrows;
  const int64_t rbv = (c0 * H + h) * (int64_t)DV;  // row 0 of the chunk, head h
  const uint32_t doff = (uint32_t)((drow < nrows ? drow : nrows - 1) * H * DV + dseg * 8);
  const f32x4_t rpx = pro.rpx, rmk = pro.rmk;
  float d8[8] = {}, g8[8] = {}, o8[8] = {};
  if (dthr) {
#pragma unroll
    for (int j = 0; j < 4; ++j) d8[j] = pro.d0[j], d8[4 + j] = pro.d1[j];
    if constexpr (GATED) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        g8[2 * j] = __uint_as_float(pro.gw[j] << 16);
        g8[2 * j + 1] = __uint_as_float(pro.gw[j] & 0xFFFF0000u);
        o8[j] = pro.o0[j];
        o8[4 + j] = pro.o1[j];
      }
    }
  }
  if (t < kCB) sBeta[t] = t < nrows ? sigm(late_f32(bw, eb & 1)) : 0.f;
  float dg8[8] = {};
  if (dthr) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (GATED) {
        const float sg = sigm(g8[j]);
        dg8[j] = d8[j] * o8[j] * sg * (1.f - sg);
        d8[j] *= sg;
      }
      if (!dvalid) d8[j] = 0.f;
    }
    st8h(sDOh, sDOl, drow * LDH + dseg * 8, d8);
  }
  {  // the record's tiles into LDS: P^T, X^T and X (transposed), Mkk
    const int e = 4 * t, row = (e % (kCB * kCB)) / kCB, col = e % kCB;
    if (e < kCB * kCB) {
      *reinterpret_cast<f32x4_t*>(sPT + row * kL32 + col) = rpx;
    } else {
      *reinterpret_cast<f32x4_t*>(sXT + row * kL32 + col) = rpx;
#pragma unroll
      for (int j = 0; j < 4; ++j) sX[(col + j) * kL32 + row] = rpx[j];
    }
    if (e < kCB * kCB) *reinterpret_cast<f32x4_t*>(sM + row * kL32 + col) = rmk;
  }
  if (GATED && dvalid) {
    const gptr<f32x4_t> gp = gat<f32x4_t>(sbase(dgate_out + rbv), doff);
    gp[0] = f32x4_t{dg8[0], dg8[1], dg8[2], dg8[3]};
    gp[1] = f32x4_t{dg8[4], dg8[5], dg8[6], dg8[7]};
  }
  // q, k words of this thread's output row (row t / 16, channels CPL (t % 16)
  // + 0..CPL-1 with CPL = d_k / 16): kept from the prologue, whose layout is
  // the same at d_k = 128, else requested before the next item's inputs
  constexpr int CPL = DK / 16;
  static_assert(CPL == 8 || CPL == 4, "d_k of 128 or 64");
  u32x4_t oq4 = {}, ok4 = {};
  if constexpr (DK == 128) {
    static_assert(PrepRows<DK, kGrThr>::NIT == 1 && PrepRows<DK, kGrThr>::NSEG == 16, "layout");
    oq4 = pro.rows.q[0];
    ok4 = pro.rows.k[0];
  }
  chunk_prep<DK, kGrThr>(pro.rows, nrows, t, sB, sQt, sKt, sKh, sE, sF, sF2, sD, sGe);
  // The value-side B operands, requested before the key products and the
  // solve for X: column jc of S and of dS_end, rows 32 kb + 8 g + 0..7.
  float Sv[NKB][8] = {}, Ev[NKB][8] = {};
  // v of this lane's rows r = 16 tt + 4 g + jj (clamped to the last row of the
  // chunk, masked where used): unconditional, so the eight requests share one
  // wait instead of one each.
  static_assert(sizeof(TI) == 2, "bf16 inputs");
  uint32_t vraw[2][4] = {};  // bf16 bits
  const gptr<const float> Sb = sbase(S), Eb = sbase(dSe);
  if (vwave) {
    const gptr<const uint16_t> vb = sbase(v + rbv);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * tt + 4 * g + jj, rr = r < nrows ? r : nrows - 1;
        vraw[tt][jj] = word_of(vb, (uint32_t)(rr * H * DV + jc));
      }
    if (S) {  // (uniform)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) Sv[kb][j] = *gat<const float>(Sb, (32 * kb + 8 * g + j) * DV + jc);
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) Sv[kb][j] = 0.f;
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      // rows 32 kb + 8 g + 0..7 of column jc: two runs of 4 in the tile layout
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const f32x4_t v4 = *gat<const f32x4_t>(
            Eb, (uint32_t)dse_tile(2 * kb + g / 2, wave, 16 * (2 * (g % 2) + hf) + li, DV));
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) Ev[kb][4 * hf + jj] = v4[jj];
      }
    }
  }

  // ---- value side, columns of wave w: Vt = V - Kbar S, dU = P^T dO + Kend
  // dS_end, then U = X diag(beta) Vt, Z = X^T dU, dV = diag(beta) Z, dbeta
  // partial sum_j Z Vt.
  f32x4_t Vt[2] = {}, dU[2] = {};
  if (vwave) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * tt + 4 * g + jj;
        Vt[tt][jj] = r < nrows ? late_f32(vraw[tt][jj], jc & 1) : 0.f;
        dU[tt][jj] = 0.f;
      }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int cb = 32 * kb + 8 * g;
      float kf[8], f2[8];
      const F8 sf = split8(Sv[kb]), ef = split8(Ev[kb]);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float ek[8], av[8];
        lds8f(sE + tt * DK + cb, ek);
        lds8f(sKt + (16 * tt + li) * LDK + cb, av);
#pragma unroll
        for (int j = 0; j < 8; ++j) av[j] = -av[j] * ek[j];
        if (S) mma3(Vt[tt], av, sf);
        lds8f(sF + tt * DK + cb, kf);
        lds8f(sF2 + tt * DK + cb, f2);
        lds8f(sKh + (16 * tt + li) * LDK + cb, av);
#pragma unroll
        for (int j = 0; j < 8; ++j) av[j] *= kf[j] * f2[j];
        mma3(dU[tt], av, ef);
      }
    }
    const F8 dof = col8h(sDOh, sDOl, 8 * g * LDH + jc, LDH);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float av[8];
      lds8f(sPT + (16 * tt + li) * kL32 + 8 * g, av);
      mma3(dU[tt], av, dof);
    }
  }
  // The d_k-side B operands of the next stage, requested now: row jc of S and
  // of dS_end, columns 32 kb + 8 g + 0..7.
  float Sr[NVB][8] = {}, Er[NVB][8] = {};
  uint32_t araw[2][4] = {};  // bf16 bits of the decay logits of this lane's elements (rows as vraw, channel jc)
  if (kwave) {
    const gptr<const uint16_t> ab = sbase(a + (c0 * H + h) * (int64_t)DK);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * tt + 4 * g + jj, rr = r < nrows ? r : nrows - 1;
        araw[tt][jj] = word_of(ab, (uint32_t)(rr * H * DK + jc));
      }
    if (S) {  // (uniform)
#pragma unroll
      for (int kb = 0; kb < NVB; ++kb) {
        const gptr<const f32x4_t> sp = gat<const f32x4_t>(Sb, jc * DV + 32 * kb + 8 * g);
        const f32x4_t s0 = sp[0], s1 = sp[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) Sr[kb][j] = s0[j], Sr[kb][4 + j] = s1[j];
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < NVB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) Sr[kb][j] = 0.f;
    }
#pragma unroll
    for (int kb = 0; kb < NVB; ++kb)
      // row jc, columns 32 kb + 8 g + 0..7 (tile layout: one element per run)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        Er[kb][j] = *gat<const float>(
            Eb, (uint32_t)(dse_tile(wave, 2 * kb + g / 2, 16 * (li / 4) + 8 * (g % 2) + j, DV) +
                           li % 4));
  }
  if (vwave) {
    f32x4_t U[2], Z[2];
    const gptr<float> dvp = sbase(dv_out + rbv);
    float bu[8], bz[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bu[j] = sBeta[kperm(g, j)] * Vt[j >> 2][j & 3];
      bz[j] = dU[j >> 2][j & 3];
    }
    const F8 buf = split8(bu), bzf = split8(bz);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      U[tt] = Z[tt] = {0.f, 0.f, 0.f, 0.f};
      float av[8];
      lds44f(sX + (16 * tt + li) * kL32 + 4 * g, av);
      mma3(U[tt], av, buf);
      lds44f(sXT + (16 * tt + li) * kL32 + 4 * g, av);
      mma3(Z[tt], av, bzf);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * tt + 4 * g + jj;
        st1h(sUh, sUl, r * LDH + jc, U[tt][jj]);
        st1h(sZh, sZl, r * LDH + jc, Z[tt][jj]);
        if (r < nrows) *gat<float>(dvp, r * H * DV + jc) = sBeta[r] * Z[tt][jj];
        const float part = row16_sum(Z[tt][jj] * Vt[tt][jj]);
        if (li == 0) sRed[wave * kCB + r] = part;
      }
  }
  lds_barrier();

  // ---- dP = dO U^T, Z U^T (waves 0-5); dQbar, dKbar, dKend (d_k waves) ----
  if (wave < 6) {
    const bool isZ = wave >= 3;
    const int jb = wave % 3;
    const int tr = jb == 0 ? 0 : 1, ti = jb == 2 ? 1 : 0;
    const uint16_t* rh = isZ ? sZh : sDOh;
    const uint16_t* rl = isZ ? sZl : sDOl;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NVB; ++kb) {
      const int cb = 32 * kb + 8 * g;
      mma3(acc, ld8h(rh, rl, (16 * tr + li) * LDH + cb), ld8h(sUh, sUl, (16 * ti + li) * LDH + cb));
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * tr + 4 * g + jj, i = 16 * ti + li;
      if (!isZ) {
        const float dp = i <= r ? acc[jj] : 0.f;
        st1h(sdPh, sdPl, sw32(r, i), dp);
        st1h(sdPTh, sdPTl, sw32(i, r), dp);
      } else {
        const float zu = i < r ? acc[jj] : 0.f;
        // dbeta_r -= sum_i (Z U^T)_ri Mkk_ri;  dMkk = -beta_r (Z U^T)
        const float part = row16_sum(zu * sM[r * kL32 + i]);
        if (li == 0) sRed[(8 + jb) * kCB + r] = -part;
        const float dm = -sBeta[r] * zu;
        st1h(sdMh, sdMl, sw32(r, i), dm);
        st1h(sdMTh, sdMTl, sw32(i, r), dm);
      }
    }
  } else if (wave == 6) {
    zero_upper_h(lane, sdPh, sdPl, sdPTh, sdPTl);
  } else {
    zero_upper_h(lane, sdMh, sdMl, sdMTh, sdMTl);
  }
  f32x4_t dQb[2] = {}, dKb[2] = {}, dKe[2] = {};
  float dge = 0.f;  // dGamma_end of channel jc (partial over this lane group's columns)
  if (kwave) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) dQb[tt] = dKb[tt] = dKe[tt] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NVB; ++kb) {
      const int jb0 = 32 * kb + 8 * g;
#pragma unroll
      for (int j = 0; j < 8; ++j) dge += Sr[kb][j] * Er[kb][j];
      const F8 srf = split8(Sr[kb]), erf = split8(Er[kb]);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int o = (16 * tt + li) * LDH + jb0;
        mma3(dQb[tt], ld8h(sDOh, sDOl, o), srf);
        mma3(dKb[tt], ld8h(sZh, sZl, o), srf);
        mma3(dKe[tt], ld8h(sUh, sUl, o), erf);
      }
    }
    // dKbar = -diag(beta) Z S^T: the row scale after the product
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) dKb[tt][jj] *= -sBeta[16 * tt + 4 * g + jj];
    dge = rows4_sum(dge);
  }
  lds_barrier();

  // ---- through the pairwise decays, then per element ----------------------
  // accLk = dMkk (Kh D), accLq = dP (Kh D) (rows r), accR = dMkk^T (Kt D) +
  // dP^T (Qt D) (rows i); D = exp(p_1 - p_0) between a row in tile 1 and a
  // column in tile 0.
  // decay logits of this lane's elements, for dg/da (this item's last loads)
  float av_[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * tt + 4 * g + jj;
      av_[tt][jj] = kwave && r < nrows ? late_f32(araw[tt][jj], jc & 1) : 0.f;
    }
  if constexpr (DK != 128) {
    const int r = t / 16, rr = r < nrows ? r : nrows - 1;
    const int64_t rb = (c0 * H + h) * (int64_t)DK;
    const uint32_t off = (uint32_t)(rr * H * DK + CPL * (t % 16));
    const u32x2_t a2 = *gat<const u32x2_t>(sbase(q + rb), off);
    const u32x2_t b2 = *gat<const u32x2_t>(sbase(k + rb), off);
    oq4 = u32x4_t{a2[0], a2[1], 0u, 0u};
    ok4 = u32x4_t{b2[0], b2[1], 0u, 0u};
  }
  // The next item's prologue inputs, requested after this item's last loads
  // (the memory counter completes in order); after the last item the same
  // requests are made for it again, so that every iteration issues the same
  // memory operations and the compiler's wait counts hold on every path.
  const int wn = w + gridDim.x;
  const bool more = wn < total;  // (uniform)
  const BwdItem nx = more ? bwd_item(wn, H, N, cbase, cu_seqlens) : it;
  bwd_request<DK, DV, GATED>(nx, q, k, a, bl, dy, gate, o_raw, crec, H, t, pro);
  if (kwave) {
    const int c = jc;
    const float dc = sD[c];
    f32x4_t accLk[2], accLq[2], accR[2];
    float bk[8], bkd[8], bkt[8], bqt[8], bktd[8], bqtd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = 8 * g + j;
      bk[j] = sKh[i * LDK + c];
      bkd[j] = i < kTl ? bk[j] * dc : bk[j];
      bkt[j] = sKt[i * LDK + c];
      bqt[j] = sQt[i * LDK + c];
      bktd[j] = i >= kTl ? bkt[j] * dc : bkt[j];
      bqtd[j] = i >= kTl ? bqt[j] * dc : bqt[j];
    }
    const F8 fbk = split8(bk), fbkd = split8(bkd), fbkt = split8(bkt), fbqt = split8(bqt),
             fbktd = split8(bktd), fbqtd = split8(bqtd);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      accLk[tt] = accLq[tt] = accR[tt] = {0.f, 0.f, 0.f, 0.f};
      const int o = sw32(16 * tt + li, 8 * g);
      mma3(accLk[tt], ld8h(sdMh, sdMl, o), tt == 1 ? fbkd : fbk);
      mma3(accLq[tt], ld8h(sdPh, sdPl, o), tt == 1 ? fbkd : fbk);
      mma3(accR[tt], ld8h(sdMTh, sdMTl, o), tt == 0 ? fbktd : fbkt);
      mma3(accR[tt], ld8h(sdPTh, sdPTl, o), tt == 0 ? fbqtd : fbqt);
    }
    // per element (r = 16 tt + 4 g + jj, channel c)
    float dbv[2][4], dqv[2][4], dkv[2][4];
    float colsum = 0.f;  // sum over rows of dKend Kend
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const float et = sE[tt * DK + c];
      const float kf = sF[tt * DK + c] * sF2[tt * DK + c];
      const float p = tt == 0 ? 0.f : sB[(kTl - 1) * LDK + c];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * tt + 4 * g + jj;
        const float x = sB[r * LDK + c] - p;
        const float fr = __expf(x), gr = __expf(-x);
        const float qt = sQt[r * LDK + c], kt = sKt[r * LDK + c], khv = sKh[r * LDK + c];
        const float ke = dKe[tt][jj] * khv * kf;
        colsum += ke;
        dqv[tt][jj] = dQb[tt][jj] * fr * et + fr * accLq[tt][jj];
        dkv[tt][jj] = dKb[tt][jj] * fr * et + dKe[tt][jj] * gr * kf + fr * accLk[tt][jj] +
                      gr * accR[tt][jj];
        dbv[tt][jj] = dQb[tt][jj] * qt * et + dKb[tt][jj] * kt * et - ke + qt * accLq[tt][jj] +
                      kt * accLk[tt][jj] - khv * accR[tt][jj];
      }
    }
    colsum = rows4_sum(colsum);
    // b_end = b at row 31 (rows past the end keep b flat): its gradient goes to row 31
    if (g == 3) dbv[1][3] += colsum + dge * sGe[c];
    // Only this wave reads or writes channel c of these rows in this stage.
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * tt + 4 * g + jj;
        sQt[r * LDK + c] = dqv[tt][jj];
        sKt[r * LDK + c] = dkv[tt][jj];
      }
    // da: the suffix sums of the b-gradient over the chunk (row r: rows >= r)
    // times dg/da = -5 sigmoid(a) sigmoid(-a) (no cancellation as
    // sigmoid(a) -> 1).  This lane holds rows 4 g + 0..3 of each tile; the
    // later rows of its tile are in lane groups g + 1..3.
    float suf[2][4], later[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      suf[tt][3] = dbv[tt][3];
#pragma unroll
      for (int jj = 2; jj >= 0; --jj) suf[tt][jj] = dbv[tt][jj] + suf[tt][jj + 1];
      // the sums of the lane groups after g: the next group's (g even) plus
      // the upper pair's (g < 2), from the cross-row swaps (rows of 16 lanes)
      const float x = suf[tt][0];
      const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      const float pair = __uint_as_float(a[0]) + __uint_as_float(a[1]);
      const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
      later[tt] = (g % 2 == 0 ? __uint_as_float(a[1]) : 0.f) + (g < 2 ? __uint_as_float(b[1]) : 0.f);
    }
    const float tile1 = rows4_sum(suf[1][0]);  // all of tile 1
    later[0] += tile1;
    const gptr<float> dap = sbase(da_out + (c0 * H + h) * (int64_t)DK);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * tt + 4 * g + jj;
        const float dgda = kGMin * sigm(av_[tt][jj]) * sigm(-av_[tt][jj]);
        if (r < nrows) *gat<float>(dap, r * H * DK + c) = (suf[tt][jj] + later[tt]) * dgda;
      }
  }
  lds_barrier();

  // ---- outputs ------------------------------------------------------------
  // dq, dk through the L2 norms: 16 lanes per row.
  {
    const int r = t / 16, l16 = t % 16;
    if (r < nrows) {
      const int64_t rb = (c0 * H + h) * (int64_t)DK;  // row 0 of the chunk, head h
      const uint32_t off = (uint32_t)(r * H * DK + CPL * l16);
      float qv[CPL], kv[CPL], dqh[CPL], dkh[CPL], sq = 0.f, sk = 0.f, qd = 0.f, kd = 0.f;
      uint32_t qw[CPL / 2], kw[CPL / 2];
#pragma unroll
      for (int i = 0; i < CPL / 2; ++i) qw[i] = oq4[i], kw[i] = ok4[i];
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
        qv[cc] = __uint_as_float(cc % 2 ? (qw[cc / 2] & 0xFFFF0000u) : (qw[cc / 2] << 16));
        kv[cc] = __uint_as_float(cc % 2 ? (kw[cc / 2] & 0xFFFF0000u) : (kw[cc / 2] << 16));
        dqh[cc] = sQt[r * LDK + CPL * l16 + cc];
        dkh[cc] = sKt[r * LDK + CPL * l16 + cc];
        sq += qv[cc] * qv[cc];
        sk += kv[cc] * kv[cc];
        qd += qv[cc] * dqh[cc];
        kd += kv[cc] * dkh[cc];
      }
      sq = group_sum<16>(sq);
      sk = group_sum<16>(sk);
      qd = group_sum<16>(qd);
      kd = group_sum<16>(kd);
      const float rq = rsqrtf(sq + kNormEps), rk = rsqrtf(sk + kNormEps);
      const gptr<f32x4_t> dqp = gat<f32x4_t>(sbase(dq_out + rb), off);
      const gptr<f32x4_t> dkp = gat<f32x4_t>(sbase(dk_out + rb), off);
#pragma unroll
      for (int c4 = 0; c4 < CPL / 4; ++c4) {
        f32x4_t oq, ok;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cc = 4 * c4 + i;
          oq[i] = rq * dqh[cc] - rq * rq * rq * qd * qv[cc];
          ok[i] = rk * dkh[cc] - rk * rk * rk * kd * kv[cc];
        }
        dqp[c4] = oq;
        dkp[c4] = ok;
      }
      if (l16 == 0) {
        float dbeta = 0.f;
        for (int w = 0; w < DV / 16; ++w) dbeta += sRed[w * kCB + r];
        if (r >= kTl) {
          dbeta += sRed[(8 + 1) * kCB + r] + sRed[(8 + 2) * kCB + r];
        } else {
          dbeta += sRed[8 * kCB + r];
        }
        const float beta = sBeta[r];
        *gat<float>(sbase(db_out + (c0 * H + h)), r * H) = dbeta * beta * (1.f - beta);
      }
    }
  }
  if (!more) break;
  w = wn;
  it = nx;
  lds_barrier();  // this item's outputs stage is done with LDS
  }
  __builtin_amdgcn_s_waitcnt(0);  // the last item's repeated requests
}

template <typename TI, int DK, int DV>
hipError_t launch_grad(const BwdChunkArgs& p, int64_t items, hipStream_t stream) {
  const size_t lds = sizeof(float) * GrLayout<DK, DV>::total;
  auto kern = p.gate ? bwd_chunk_kernel<TI, DK, DV, true> : bwd_chunk_kernel<TI, DK, DV, false>;
  // one workgroup per compute unit (139+ KB of LDS each), looping over items
  const int64_t cus = device_cus();
  const int64_t grid = items < cus ? items : cus;
  // Dynamic LDS above the default limit: set on every call (the attribute is
  // the device's, and a process may drive several devices or threads).
  {
    const hipError_t e =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kGrThr), lds, stream, (const TI*)p.q,
                     (const TI*)p.k, (const TI*)p.v, (const TI*)p.a, (const TI*)p.b,
                     (const TI*)p.gate, p.dy, p.o_raw, p.cu_seqlens, p.cbase, p.kbase,
                     p.initial_state, p.ckpt, p.dse, p.crec, p.dq_out, p.dk_out, p.dv_out,
                     p.da_out, p.db_out, p.dgate_out, p.num_seqs, p.num_heads);
  return hipGetLastError();
}

template <typename TI, int DK>
hipError_t launch_chainprep(const BwdChunkArgs& p, int64_t grid, hipStream_t stream) {
  const size_t lds = sizeof(float) * PrepLayout<DK>::total;
  auto kern = bwd_chainprep_kernel<TI, DK>;
  // Dynamic LDS above the default limit: set on every call (the attribute is
  // the device's, and a process may drive several devices or threads).
  {
    const hipError_t e =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kPrepThr), lds, stream, (const TI*)p.q,
                     (const TI*)p.k, (const TI*)p.a, (const TI*)p.b, p.cu_seqlens, p.cbase,
                     p.crec, p.num_seqs, p.num_heads);
  return hipGetLastError();
}

template <typename TI, int DK, int DV>
hipError_t launch_chain(const BwdChunkArgs& p, hipStream_t stream) {
  const size_t lds = sizeof(float) * ChainLayout<DK, DV>::total;
  auto kern = bwd_chain_kernel<TI, DK, DV>;
  {
    const hipError_t e =
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t grid = (int64_t)p.num_seqs * p.num_heads;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(4 * DV), lds, stream, (const TI*)p.gate,
                     p.dy, p.cu_seqlens, p.cbase, p.crec, p.d_final_state, p.dse, p.d_s0,
                     p.num_heads);
  return hipGetLastError();
}

// Per device: the events that fork the adjoint chain onto the second stream
// and join it back, created on first use (on the device of the caller's
// stream) and kept for the process; one mutex serialises the enqueueing.
struct BwdEvents {
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_bwd_mu;
BwdEvents g_bwd_ev[64];

hipError_t bwd_events(hipStream_t stream, BwdEvents** out) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  BwdEvents& be = g_bwd_ev[dev];
  if (!be.fork) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    BwdEvents made;
    e = hipEventCreateWithFlags(&made.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&made.join, hipEventDisableTiming);
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    be = made;
  }
  *out = &be;
  return hipSuccess;
}

template <typename TI>
hipError_t launch_t(const BwdChunkArgs& p, const FwdArgs& f, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_plan_kernel, dim3(1), dim3(kPlanThr), 0, stream, p.cu_seqlens,
                     p.num_seqs, p.cbase, p.kbase);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The chain's operand records first, alone on the caller's stream (a
  // parallel pass over every chunk); then the serial chain (one workgroup per
  // head) on the second stream while the forward records the states on the
  // caller's stream with one workgroup per head as well: split into d_v
  // slices it would take every compute unit for its whole run (a workgroup
  // per unit) and hold most of the chain's workgroups back until it ends.
  const int64_t cgrid = (p.total_tokens / kCB + p.num_seqs) * p.num_heads;
  if (cgrid > 0) {
    e = p.dk == 128 ? launch_chainprep<TI, 128>(p, cgrid, stream)
                    : launch_chainprep<TI, 64>(p, cgrid, stream);
    if (e != hipSuccess) return e;
  }
  {
    std::lock_guard<std::mutex> lock(g_bwd_mu);
    BwdEvents* ev = nullptr;
    hipStream_t s2 = nullptr;
    if ((e = bwd_events(stream, &ev)) != hipSuccess) return e;
    if ((e = device_side_stream(stream, &s2)) != hipSuccess) return e;
    if ((e = hipEventRecord(ev->fork, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(s2, ev->fork, 0)) != hipSuccess) return e;
    if (p.dk == 128)
      e = p.dv == 128 ? launch_chain<TI, 128, 128>(p, s2) : launch_chain<TI, 128, 64>(p, s2);
    else
      e = p.dv == 128 ? launch_chain<TI, 64, 128>(p, s2) : launch_chain<TI, 64, 64>(p, s2);
    if (e != hipSuccess) return e;
    if ((e = hipEventRecord(ev->join, s2)) != hipSuccess) return e;
    FwdArgs fw = f;
    fw.whole_items = true;
    if ((e = launch_fwd_chunked(fw, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(stream, ev->join, 0)) != hipSuccess) return e;
  }
  if (cgrid == 0) return hipSuccess;
  const int64_t grid = cgrid;
  if (p.dk == 128)
    return p.dv == 128 ? launch_grad<TI, 128, 128>(p, grid, stream)
                       : launch_grad<TI, 128, 64>(p, grid, stream);
  return p.dv == 128 ? launch_grad<TI, 64, 128>(p, grid, stream)
                     : launch_grad<TI, 64, 64>(p, grid, stream);
}

}  // namespace

int bwd_chunk_len() { return kCB; }
int bwd_chain_record_floats(int dk) {
  return dk == 128 ? ChainRec<128>::floats : ChainRec<64>::floats;
}

hipError_t launch_bwd_chunked(const BwdChunkArgs& p, const FwdArgs& f, hipStream_t stream) {
  if ((int64_t)p.num_seqs * p.num_heads == 0) return launch_fwd_chunked(f, stream);
  // bf16 inputs only (fp32 inputs run the token form, kda_bwd.hip)
  if (!p.in_bf16) return hipErrorInvalidValue;
  return launch_t<uint16_t>(p, f, stream);
}

}  // namespace kda
