// kda_chunk_bf16.hip - chunked KDA forward for bf16 inputs on gfx950 (MI355X).
//
// The KDA recurrence (page "[Paper Review] Kimi K3...", section "Kimi Delta
// Attention (KDA)") in its chunkwise-parallel form (same section: recurrent
// but parallelisable per chunk), on 32-token chunks of two 16-token tiles.
// The log-decay is bounded below by g_min = -5 ("Lower-bounded decay"
// paragraph), so the cumulative log-decay of a 16-token tile lies in [-80, 0]
// and every pairwise decay exp(b_r - b_i) splits into a row factor
// exp(b_r - p) <= 1 and a column factor exp(p - b_i) <= e^80 (p = cumulative
// decay before row r's tile): both finite in bf16, so every intra-chunk tile,
// diagonal or not, is a dense matrix-core product.
//
// Per chunk (rows r < 32, start state S, b = chunk-local cumsum of g):
//   A      = diag(beta) strict_lower(Kt Kh^T)   bf16 operands
//   P      = lower(Qt Kh^T)                      bf16 hi/lo split (3 products)
//   X      = (I + A)^-1                          fp32, vector ALU
//   W      = X diag(beta) Kbar                   fp16 (computed as W^T)
//   U0     = X diag(beta) V                      bf16 hi/lo
//   U      = U0 - W S                            fp16
//   O      = Qbar S + P U,  y = sigmoid(gate) O  fp16 / bf16 hi/lo
//   S     <- diag(Gamma_end) S + Kend^T U        fp16
// Kt = kh exp(b-p), Kh = kh exp(p-b) (the off-diagonal tile's column operand
// is rescaled by exp(p_1) <= 1), Qt = qh exp(b-p), Qbar = qh exp(b),
// Kbar = kh exp(b), Kend = kh exp(b_end - b).  Accumulation is fp32 and the
// state is fp32 throughout.  bf16 (not fp16) is used wherever the e^80 column
// factors appear; the hi/lo splits (Henry, Tang & Heinecke, ARITH 2019) are
// where the 2e-2 accuracy budget needs more than one 16-bit product.
//
// One workgroup of NW = dv/16 wavefronts per (sequence, head); wave w owns
// state columns [16w, 16w+16) for the whole sequence, in MFMA accumulator
// registers.  The dk-side work of a chunk (elementwise, A, P, X, W) is shared
// by all waves through LDS; an MFMA accumulator tile feeds the next product's
// B operand directly (its row index is the B operand's k index up to a fixed
// permutation of k, matched on the A side), so S and U stay in registers.
//   S1  norms, g, in-register cumulative sum; per-row-group totals to LDS
//   S2  prefix of the totals; every scaled operand written once, in the
//       layout its product reads; the next chunk's inputs are requested
//   S3  A (waves 0-2) | P; then X (wave 0) | P; then O = Qbar S (all)
//   S4  W^T = (beta Kbar)^T X^T (all waves), U0 (own columns)
//   S5  the state chain and the gated output
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 32;          // chunk length (tokens)
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
// (ah + al)(bh + bl) ~ ah bh + ah bl + al bh
__device__ __forceinline__ f32x4_t mma_x3(bf16x8_t ah, bf16x8_t al, bf16x8_t bh, bf16x8_t bl,
                                          f32x4_t c) {
  c = mma_bf16(al, bh, c);
  c = mma_bf16(ah, bl, c);
  return mma_bf16(ah, bh, c);
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcpf_fast(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ bf16x8_t pack_bf16x8(const float (&x)[8]) {
  bf16x8_t r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
  return r;
}
__device__ __forceinline__ f16x8_t pack_f16x8(const float (&x)[8]) {
  f16x8_t r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (_Float16)x[j];
  return r;
}
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 hv = (__bf16)x[j];
    hi[j] = hv;
    lo[j] = (__bf16)(x[j] - (float)hv);
  }
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
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int DK, int NW>
struct Cfg {
  static constexpr int NT = 64 * NW;        // threads
  static constexpr int LPR = DK / 4;        // lanes per row in the elementwise mapping
  static constexpr int NRG = NT / LPR;      // row groups
  static constexpr int RPT = kC / NRG;      // consecutive rows per thread
  static_assert(RPT >= 1 && RPT * NRG == kC, "row split");
  // LDS strides (elements)
  static constexpr int LB = DK + 8;         // 16-bit [32][DK]
  static constexpr int LT = kC + 8;         // 16-bit [DK][32] and [32][32]
  static constexpr int LX = kC + 4;         // fp32 [32][32]
  // byte offsets: the small regions with many access sites first, so their
  // addresses fit the 16-bit immediate offset of LDS instructions
  static constexpr int oA = 0;                           // A fp32 [32][LX]
  static constexpr int oX = oA + kC * LX * 4;            // X fp32 [32][LX]
  static constexpr int oPH = oX + kC * LX * 4;           // P hi bf16 [32][LT]
  static constexpr int oPL = oPH + kC * LT * 2;          // P lo bf16 [32][LT]
  static constexpr int oE1 = oPL + kC * LT * 2;          // exp(p_1) [DK]
  static constexpr int oGE = oE1 + DK * 4;               // exp(b_end) [DK]
  static constexpr int oBeta = oGE + DK * 4;             // beta [32]
  static constexpr int oKE = oBeta + kC * 4;             // Kend^T fp16 [DK][LT]
  static constexpr int oKB = oKE + DK * LT * 2;          // (beta Kbar)^T fp16 [DK][LT]
  static constexpr int oKT = oKB + DK * LT * 2;          // Kt bf16 [32][LB]
  static constexpr int oQH = oKT + kC * LB * 2;          // Qt hi bf16; -W fp16 from S4
  static constexpr int oQL = oQH + kC * LB * 2;          // Qt lo bf16
  static constexpr int oQB = oQL + kC * LB * 2;          // Qbar fp16
  static constexpr int oKHH = oQB + kC * LB * 2;         // Kh hi bf16 [32][LB]
  static constexpr int oKHL = oKHH + kC * LB * 2;        // Kh lo bf16 [32][LB]
  static constexpr int oK1H = oKHL + kC * LB * 2;        // Kh exp(p_1) hi, rows 0-15
  static constexpr int oK1L = oK1H + 16 * LB * 2;        // Kh exp(p_1) lo, rows 0-15
  static constexpr int bytes = oK1L + 16 * LB * 2;
  // per-wave cumulative totals [NW][DK] fp32 overlay A, X, P (dead in S1-S2)
  static constexpr int oTOT = oA;
  static_assert(NW * DK * 4 <= oE1 - oA, "totals overlay");
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

template <int DK, int NW>
__global__ void __launch_bounds__(64 * NW)
    chunk_fwd_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                          const uint16_t* __restrict__ v, const uint16_t* __restrict__ a,
                          const uint16_t* __restrict__ bl, const uint16_t* __restrict__ gate,
                          const int32_t* __restrict__ cu_seqlens, const float* __restrict__ s_init,
                          float* __restrict__ o, float* __restrict__ s_final, int H) {
  using L = Cfg<DK, NW>;
  constexpr int DV = 16 * NW;
  constexpr int LPR = L::LPR, NRG = L::NRG, RPT = L::RPT;
  constexpr int LB = L::LB, LT = L::LT, LX = L::LX;
  constexpr int NCT = DK / 16, NKB = DK / 32;

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::bytes];
  uint16_t* sKT = reinterpret_cast<uint16_t*>(smem + L::oKT);
  uint16_t* sQH = reinterpret_cast<uint16_t*>(smem + L::oQH);
  uint16_t* sW = sQH;
  uint16_t* sQL = reinterpret_cast<uint16_t*>(smem + L::oQL);
  uint16_t* sQB = reinterpret_cast<uint16_t*>(smem + L::oQB);
  uint16_t* sKHH = reinterpret_cast<uint16_t*>(smem + L::oKHH);
  uint16_t* sKHL = reinterpret_cast<uint16_t*>(smem + L::oKHL);
  uint16_t* sK1H = reinterpret_cast<uint16_t*>(smem + L::oK1H);
  uint16_t* sK1L = reinterpret_cast<uint16_t*>(smem + L::oK1L);
  uint16_t* sKE = reinterpret_cast<uint16_t*>(smem + L::oKE);
  uint16_t* sKB = reinterpret_cast<uint16_t*>(smem + L::oKB);
  float* sA = reinterpret_cast<float*>(smem + L::oA);
  float* sX = reinterpret_cast<float*>(smem + L::oX);
  uint16_t* sPH = reinterpret_cast<uint16_t*>(smem + L::oPH);
  uint16_t* sPL = reinterpret_cast<uint16_t*>(smem + L::oPL);
  float* sE1 = reinterpret_cast<float*>(smem + L::oE1);
  float* sGE = reinterpret_cast<float*>(smem + L::oGE);
  float* sBeta = reinterpret_cast<float*>(smem + L::oBeta);
  float* sTOT = reinterpret_cast<float*>(smem + L::oTOT);

  const int item = blockIdx.x;  // sequence * H + head
  const int n = item / H, h = item % H;
  const int t = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(t / 64), lane = t % 64, g = lane / 16, li = lane % 16;
  const int cq = t % LPR, rg = t / LPR;  // elementwise: channels 4cq.., rows RPT*rg..
  const int64_t tok_beg = cu_seqlens[n], tok_end = cu_seqlens[n + 1];
  const int64_t st_off = (int64_t)item * DK * DV;
  const int jcol = 16 * wave + li;

  // Global addressing: a wave-uniform base pointer plus a small 32-bit lane
  // offset (keeps 64-bit per-access addresses out of the register file).
  const uint32_t st_lane = 4 * g * DV + jcol;  // state element (row 4g, column jcol)
  f32x4_t S[NCT];
  if (s_init) {
    const auto sp = sbase(s_init + st_off);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) S[ct][jj] = sp[st_lane + (16 * ct + jj) * DV];
  } else {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) S[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Registers holding one chunk's raw inputs (requested one stage ahead).
  u32x2_t rq_[RPT], rk_[RPT], ra_[RPT];  // 4 bf16 each: rows RPT*rg + i, channels 4cq..4cq+3
  uint32_t rb_[RPT];                     // b of those rows
  uint32_t rv_[8], rgt_[8];              // v, gate at rows 16*(i/4) + 4g + i%4, column jcol
  auto load_qka = [&](int64_t c0, int cq, int rg) {
    const int nr = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
    const int64_t tb = c0 * H + h;  // token-head index of row 0 of the chunk
    const auto qb_ = sbase(q + tb * DK);
    const auto kb_ = sbase(k + tb * DK);
    const auto ab_ = sbase(a + tb * DK);
    const auto bb_ = sbase(bl + tb);
    // Rows past the end of the sequence re-load its last row (always in
    // bounds, finite).  They need no zeroing here: S1 gives them g = 0 and
    // beta = 0, which removes every contribution they could make (their rows
    // of A, beta*Kbar and beta*V vanish, hence their rows of X, W, U0 and U
    // are those of the identity / zero), and their outputs are never stored.
    // Consuming the loaded values only at use keeps the loads in flight.
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = RPT * rg + i;
      const int rr = r < nr ? r : nr - 1;
      const uint32_t off = (uint32_t)(rr * H * DK) + 4 * cq;
      rq_[i] = *reinterpret_cast<const __attribute__((address_space(1))) u32x2_t*>(qb_ + off);
      rk_[i] = *reinterpret_cast<const __attribute__((address_space(1))) u32x2_t*>(kb_ + off);
      ra_[i] = *reinterpret_cast<const __attribute__((address_space(1))) u32x2_t*>(ab_ + off);
      rb_[i] = bb_[(uint32_t)(rr * H)];
    }
  };
  auto load_vg = [&](int64_t c0, int g, int jcol) {
    const int nr = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
    const int64_t tb = c0 * H + h;
    const auto vb_ = sbase(v + tb * DV);
    const auto gb_ = sbase(gate ? gate + tb * DV : v + tb * DV);
    // Rows past the end re-load the last row: beta = 0 there removes their v,
    // and their gated outputs are not stored.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 16 * (i / 4) + 4 * g + (i % 4);
      const int rr = r < nr ? r : nr - 1;
      const uint32_t off = (uint32_t)(rr * H * DV) + jcol;
      rv_[i] = vb_[off];
      rgt_[i] = gb_[off];
    }
  };
  if (tok_beg < tok_end) {
    load_qka(tok_beg, cq, rg);
    load_vg(tok_beg, g, jcol);
  }

  for (int64_t c0 = tok_beg; c0 < tok_end; c0 += kC) {
    const int nrows = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
    // Lane-derived indices are re-derived from an opaque copy of the thread
    // index every chunk: recomputing them costs a few ALU operations, while
    // letting the compiler hoist every lane-dependent address and constant out
    // of the loop would hold them in registers for the whole sequence.
    int t_ = t;
    __asm__ volatile("" : "+v"(t_));
    const int lane = t_ % 64, g = lane / 16, li = lane % 16;
    const int cq = t_ % LPR, rg = t_ / LPR;
    const int jcol = 16 * wave + li;
    const uint32_t vo_lane = (4 * g) * H * DV + jcol;

    // ---- S1: norms, g (log2 units), in-register cumulative sum ---------------
    float qv[RPT][4], kv[RPT][4], cum[RPT][4];
    float betar[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const u32x2_t uq = rq_[i], uk = rk_[i], ua = ra_[i];
      qv[i][0] = bf16lo(uq[0]); qv[i][1] = bf16hi(uq[0]); qv[i][2] = bf16lo(uq[1]); qv[i][3] = bf16hi(uq[1]);
      kv[i][0] = bf16lo(uk[0]); kv[i][1] = bf16hi(uk[0]); kv[i][2] = bf16lo(uk[1]); kv[i][3] = bf16hi(uk[1]);
      const float av[4] = {bf16lo(ua[0]), bf16hi(ua[0]), bf16lo(ua[1]), bf16hi(ua[1])};
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sq += qv[i][j] * qv[i][j];
        sk += kv[i][j] * kv[i][j];
      }
      sq = group_sum<LPR>(sq);
      sk = group_sum<LPR>(sk);
      const float nq = rsqrtf(sq + kNormEps), nk = rsqrtf(sk + kNormEps);
      const bool valid = RPT * rg + i < nrows;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qv[i][j] *= nq;
        kv[i][j] *= nk;
        // g in log2 units: -5 log2(e) sigmoid(a)
        const float gl =
            valid ? (kGMin * kLog2e) * rcpf_fast(1.f + exp2f_fast(-kLog2e * av[j])) : 0.f;
        cum[i][j] = i == 0 ? gl : cum[i - 1][j] + gl;
      }
      betar[i] = valid ? rcpf_fast(1.f + exp2f_fast(-kLog2e * bf16lo(rb_[i]))) : 0.f;
    }
    // Inclusive scan of the row-group totals across the row groups of this
    // wave (lane blocks of LPR), then the wave totals to LDS.
    float inw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x = cum[RPT - 1][j];
#pragma unroll
      for (int d = LPR; d < 64; d *= 2) {
        const float y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
      }
      inw[j] = x - cum[RPT - 1][j];  // exclusive: row groups of this wave before mine
      if (lane >= 64 - LPR) sTOT[wave * DK + 4 * cq + j] = x;
    }
    lds_barrier();

    // ---- S2: prefix over row groups; scaled operands --------------------------
    // pre: decay accumulated before this thread's rows; p1: before row 16
    // (rows 0-15 belong to waves < NW/2); be: over the whole chunk.
    float pre[4] = {inw[0], inw[1], inw[2], inw[3]}, p1[4] = {0.f, 0.f, 0.f, 0.f};
    for (int w2 = 0; w2 < wave; ++w2) {  // wave-uniform trip count
      const float4 tv = *reinterpret_cast<const float4*>(sTOT + w2 * DK + 4 * cq);
      pre[0] += tv.x; pre[1] += tv.y; pre[2] += tv.z; pre[3] += tv.w;
    }
#pragma unroll
    for (int w2 = 0; w2 < NW / 2; ++w2) {
      const float4 tv = *reinterpret_cast<const float4*>(sTOT + w2 * DK + 4 * cq);
      p1[0] += tv.x; p1[1] += tv.y; p1[2] += tv.z; p1[3] += tv.w;
    }
    float be[4] = {p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
    for (int w2 = NW / 2; w2 < NW; ++w2) {
      const float4 tv = *reinterpret_cast<const float4*>(sTOT + w2 * DK + 4 * cq);
      be[0] += tv.x; be[1] += tv.y; be[2] += tv.z; be[3] += tv.w;
    }
    float e1[4], f0[4], f1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e1[j] = exp2f_fast(p1[j]);          // exp(p_1): decay accumulated over tile 0
      f0[j] = exp2f_fast(be[j]);          // exp(b_end - p_0) = Gamma_end
      f1[j] = exp2f_fast(be[j] - p1[j]);  // exp(b_end - p_1)
    }
    if (rg == 0) {
      *reinterpret_cast<float4*>(sE1 + 4 * cq) = make_float4(e1[0], e1[1], e1[2], e1[3]);
      *reinterpret_cast<float4*>(sGE + 4 * cq) = make_float4(f0[0], f0[1], f0[2], f0[3]);
    }
    _Float16 ke16[4][RPT], kb16[4][RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = RPT * rg + i;
      const bool t1 = r >= 16;
      float kt[4], qt[4], kh[4], qb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = pre[j] + cum[i][j] - (t1 ? p1[j] : 0.f);  // log2(e) (b - p) <= 0
        const float er = exp2f_fast(x), ir = exp2f_fast(-x);
        kt[j] = kv[i][j] * er;
        qt[j] = qv[i][j] * er;
        kh[j] = kv[i][j] * ir;
        qb[j] = t1 ? qt[j] * e1[j] : qt[j];
        ke16[j][i] = (_Float16)(kh[j] * (t1 ? f1[j] : f0[j]));
        kb16[j][i] = (_Float16)(betar[i] * (t1 ? kt[j] * e1[j] : kt[j]));
      }
      bf16x4_t ktb, qhb, qlb;
      f16x4_t qbf;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ktb[j] = (__bf16)kt[j];
        qhb[j] = (__bf16)qt[j];
        qlb[j] = (__bf16)(qt[j] - (float)qhb[j]);
        qbf[j] = (_Float16)qb[j];
      }
      *reinterpret_cast<bf16x4_t*>(sKT + r * LB + 4 * cq) = ktb;
      *reinterpret_cast<bf16x4_t*>(sQH + r * LB + 4 * cq) = qhb;
      *reinterpret_cast<bf16x4_t*>(sQL + r * LB + 4 * cq) = qlb;
      *reinterpret_cast<f16x4_t*>(sQB + r * LB + 4 * cq) = qbf;
      bf16x4_t khh, khl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        khh[j] = (__bf16)kh[j];
        khl[j] = (__bf16)(kh[j] - (float)khh[j]);
      }
      *reinterpret_cast<bf16x4_t*>(sKHH + r * LB + 4 * cq) = khh;
      *reinterpret_cast<bf16x4_t*>(sKHL + r * LB + 4 * cq) = khl;
      if (!t1) {  // column operand of the off-diagonal tile: Kh exp(p_1) <= 1
        bf16x4_t k1h, k1l;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float y = kh[j] * e1[j];
          k1h[j] = (__bf16)y;
          k1l[j] = (__bf16)(y - (float)k1h[j]);
        }
        *reinterpret_cast<bf16x4_t*>(sK1H + r * LB + 4 * cq) = k1h;
        *reinterpret_cast<bf16x4_t*>(sK1L + r * LB + 4 * cq) = k1l;
      }
      if (cq == 0) sBeta[r] = betar[i];
    }
    // transposed [channel][row] operands: RPT consecutive rows per channel
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 4 * cq + j;
      if constexpr (RPT == 1) {
        sKE[c * LT + rg] = __builtin_bit_cast(uint16_t, ke16[j][0]);
        sKB[c * LT + rg] = __builtin_bit_cast(uint16_t, kb16[j][0]);
      } else {
        typedef __attribute__((ext_vector_type(RPT))) _Float16 f16xr_t;
        f16xr_t ve, vb;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          ve[i] = ke16[j][i];
          vb[i] = kb16[j][i];
        }
        *reinterpret_cast<f16xr_t*>(sKE + c * LT + RPT * rg) = ve;
        *reinterpret_cast<f16xr_t*>(sKB + c * LT + RPT * rg) = vb;
      }
    }
    if (c0 + kC < tok_end) load_qka(c0 + kC, cq, rg);  // next chunk, consumed in its S1
    lds_barrier();

    // ---- S3a: A tiles (waves 0-2) | P tiles --------------------------------------
    // tile job 0: (row tile 0, column tile 0); 1: (1, 0); 2: (1, 1)
    auto a_job = [&](int job) {
      const int tr = job == 0 ? 0 : 1, ti = job == 2 ? 1 : 0;
      const uint16_t* colh = job == 1 ? sK1H : sKHH;  // (1,0) uses Kh exp(p_1)
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int cb = 32 * kb + 8 * g;
        acc = mma_bf16(lds8<bf16x8_t>(sKT + (16 * tr + li) * LB + cb),
                       lds8<bf16x8_t>(colh + (16 * ti + li) * LB + cb), acc);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * tr + 4 * g + jj, i = 16 * ti + li;
        sA[r * LX + i] = i < r ? acc[jj] * sBeta[r] : 0.f;
      }
    };
    auto p_job = [&](int job) {
      const int tr = job == 0 ? 0 : 1, ti = job == 2 ? 1 : 0;
      const uint16_t* colh = job == 1 ? sK1H : sKHH;
      const uint16_t* coll = job == 1 ? sK1L : sKHL;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int cb = 32 * kb + 8 * g;
        acc = mma_x3(lds8<bf16x8_t>(sQH + (16 * tr + li) * LB + cb),
                     lds8<bf16x8_t>(sQL + (16 * tr + li) * LB + cb),
                     lds8<bf16x8_t>(colh + (16 * ti + li) * LB + cb),
                     lds8<bf16x8_t>(coll + (16 * ti + li) * LB + cb), acc);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * tr + 4 * g + jj, i = 16 * ti + li;
        const float pv = i <= r ? acc[jj] : 0.f;
        const __bf16 ph = (__bf16)pv;
        sPH[r * LT + i] = __builtin_bit_cast(uint16_t, ph);
        sPL[r * LT + i] = __builtin_bit_cast(uint16_t, (__bf16)(pv - (float)ph));
      }
      if (job == 0) {  // the upper tile (0, 1) of P is zero
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          sPH[(4 * g + jj) * LT + 16 + li] = 0;
          sPL[(4 * g + jj) * LT + 16 + li] = 0;
        }
      }
    };
    if (wave < 3) {
      a_job(wave);
    } else if (NW >= 6) {
      if (wave < 6) p_job(wave - 3);
    } else if (wave == 3) {
      p_job(0);
    }
    lds_barrier();

    // ---- S3b: X = (I + A)^-1 (wave 0) | remaining P tiles; then O = Qbar S ------
    if (wave == 0) {
      // Diagonal 16x16 blocks: lane group g < 2 owns block g, lane li column li;
      // right-looking forward substitution.
      if (g < 2) {
        const int o16 = 16 * g;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = r == li ? 1.f : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
          for (int i = r + 1; i < 16; ++i) x[i] -= sA[(o16 + i) * LX + o16 + r] * x[r];
          __builtin_amdgcn_sched_barrier(0);  // bound the load-hoisting window
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sX[(o16 + r) * LX + o16 + li] = x[r];
      }
      lds_wave_fence();
      // X10 = -X11 (A10 X00); lane holds rows 4g + jj, column li.
      float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const float xv = sX[kk * LX + li];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) y[jj] += sA[(16 + 4 * g + jj) * LX + kk] * xv;
        if (kk % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sX[(4 * g + jj) * LX + 16 + li] = y[jj];  // staged in X01
      lds_wave_fence();
      float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const float yv = sX[kk * LX + 16 + li];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) z[jj] += sX[(16 + 4 * g + jj) * LX + 16 + kk] * yv;
        if (kk % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
      lds_wave_fence();
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        sX[(16 + 4 * g + jj) * LX + li] = -z[jj];
        sX[(4 * g + jj) * LX + 16 + li] = 0.f;
      }
    } else if (NW < 6 && wave < 3) {
      p_job(wave);  // P tiles 1 and 2 on waves 1 and 2
    }
    // O = Qbar S for this wave's columns (fp16); S as fp16 B operand.
    auto s_f16 = [&](int kb) {
      f16x8_t r;
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = (_Float16)S[2 * kb + (j >> 2)][j & 3];
      return r;
    };
    f32x4_t O[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      O[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        O[rt] = mma_f16(lds4x2<f16x8_t>(sQB + (16 * rt + li) * LB + 32 * kb + 4 * g), s_f16(kb),
                        O[rt]);
    }
    lds_barrier();

    // ---- S4: W^T = (beta Kbar)^T X^T (fp16), U0 = X beta V (bf16 hi/lo) --------
    {
      f16x8_t xt[2];  // X^T as B operand: lane (li, g) holds X[16 rt + li][8 g + j]
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        float xx[8];
        lds_f32x8(sX + (16 * rt + li) * LX + 8 * g, xx);
        xt[rt] = pack_f16x8(xx);
      }
      constexpr int NWT = 2 * NCT;  // W^T tiles
#pragma unroll
      for (int tile = wave; tile < NWT; tile += NW) {
        const int ct = tile / 2, rt = tile % 2;
        const f32x4_t acc = mma_f16(lds8<f16x8_t>(sKB + (16 * ct + li) * LT + 8 * g), xt[rt],
                                    f32x4_t{0.f, 0.f, 0.f, 0.f});
        // acc[jj] = W[16 rt + li][16 ct + 4 g + jj]; store -W
        const f16x4_t wv = {(_Float16)(-acc[0]), (_Float16)(-acc[1]), (_Float16)(-acc[2]),
                            (_Float16)(-acc[3])};
        *reinterpret_cast<f16x4_t*>(sW + (16 * rt + li) * LB + 16 * ct + 4 * g) = wv;
      }
    }
    f32x4_t U[2];
    {
      float rr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) rr[j] = sBeta[16 * (j >> 2) + 4 * g + (j & 3)] * bf16lo(rv_[j]);
      bf16x8_t rh, rl;
      split_bf16x8(rr, rh, rl);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        float xx[8];
        lds_f32x4x2(sX + (16 * rt + li) * LX + 4 * g, xx);
        bf16x8_t xh, xl;
        split_bf16x8(xx, xh, xl);
        U[rt] = mma_x3(xh, xl, rh, rl, f32x4_t{0.f, 0.f, 0.f, 0.f});
      }
    }
    lds_barrier();

    // ---- S5: the state chain ----------------------------------------------------
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const f16x8_t sbk = s_f16(kb);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        U[rt] = mma_f16(lds4x2<f16x8_t>(sW + (16 * rt + li) * LB + 32 * kb + 4 * g), sbk, U[rt]);
    }
    f16x8_t uf;
    bf16x8_t uh, ul;
    {
      float uu[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) uu[j] = U[j >> 2][j & 3];
      uf = pack_f16x8(uu);
      split_bf16x8(uu, uh, ul);
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int off = (16 * rt + li) * LT + 4 * g;
      O[rt] = mma_x3(lds4x2<bf16x8_t>(sPH + off), lds4x2<bf16x8_t>(sPL + off), uh, ul, O[rt]);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4_t acc;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[jj] = sGE[16 * ct + 4 * g + jj] * S[ct][jj];
      S[ct] = mma_f16(lds4x2<f16x8_t>(sKE + (16 * ct + li) * LT + 4 * g), uf, acc);
    }
    // Epilogue: output gate and store.
    {
      const auto ob_ = sbase(o + (c0 * H + h) * DV);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 16 * (j >> 2) + 4 * g + (j & 3);
        if (r < nrows) {
          float y = O[j >> 2][j & 3];
          if (gate) y *= rcpf_fast(1.f + exp2f_fast(-kLog2e * bf16lo(rgt_[j])));
          ob_[vo_lane + (uint32_t)((16 * (j >> 2) + (j & 3)) * H * DV)] = y;
        }
      }
    }
    if (c0 + kC < tok_end) load_vg(c0 + kC, g, jcol);
    lds_barrier();
  }

  if (s_final) {
    const auto sp = sbase(s_final + st_off);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sp[st_lane + (16 * ct + jj) * DV] = S[ct][jj];
  }
}

template <int DK, int NW>
hipError_t launch_cfg(const FwdArgs& p, hipStream_t stream) {
  auto kern = chunk_fwd_bf16_kernel<DK, NW>;  // LDS is static (Cfg<DK, NW>::bytes)
  const int64_t grid = (int64_t)p.num_seqs * p.num_heads;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * NW), 0, stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v,
                     (const uint16_t*)p.a, (const uint16_t*)p.b, (const uint16_t*)p.gate,
                     p.cu_seqlens, p.initial_state, (float*)p.o, p.final_state, p.num_heads);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_chunked_bf16(const FwdArgs& p, hipStream_t stream) {
  if ((int64_t)p.num_seqs * p.num_heads == 0) return hipSuccess;
  if (p.dk == 128)
    return p.dv == 128 ? launch_cfg<128, 8>(p, stream) : launch_cfg<128, 4>(p, stream);
  return p.dv == 128 ? launch_cfg<64, 8>(p, stream) : launch_cfg<64, 4>(p, stream);
}

}  // namespace kda
