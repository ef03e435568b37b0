// kda_split_bf16.hip - the bf16 chunked KDA forward in two passes (gfx950).
//
// The recurrence of page "[Paper Review] Kimi K3...", section "Kimi Delta
// Attention (KDA)", in the same chunkwise form, chunk length, operand
// precisions and LDS layouts as the fused kernel (kda_chunk_bf16.hip), cut
// where that kernel hands chunk operands from its prep waves to its state
// waves:
//
//   pass 1  chunk_prep_bf16_kernel   for every (sequence, head, 32-token
//           chunk), independently: the decay-scaled operands, A, P, the
//           inverse X = (I + A)^-1 and W, written as one "chunk record"
//           (X fp32, P bf16 hi/lo, Gamma_end, beta, 1/|q|, 1/|k|, Qbar fp16,
//           -W fp16, Kend^T fp16: 33,664 bytes at d_k = 128);
//   pass 2  chunk_state_bf16_kernel  per (sequence, head, d_v slice), the
//           sequential chain over the records: U0 = X diag(beta) V,
//           U = U0 - W S, O = diag(nq) Qbar S + P U, S <- diag(Gamma_end) S
//           + Kend^T diag(nk) U, y = sigmoid(gate) O.
//
// Why two passes: the fused kernel runs the key-side work once per d_v slice
// and ties it to the state chain's pace; here it runs once per head with no
// dependence between chunks, so pass 1 fills every compute unit, and pass 2
// is a light streaming loop.  The price is the records' round trip through
// HBM (about 1 KB per token-head at d_k = 128).  A long input is processed
// in blocks of chunks: for each block, a plan kernel places the block's
// records densely in the workspace, pass 1 fills them and pass 2 consumes
// them, carrying the state from block to block through the workspace.
#include <algorithm>
#include <type_traits>

#include "kda_chunk_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

// Chunk record: LDS layout (padded rows, as the fused kernel's hand-over
// buffer) and the compact global layout (same regions in the same order,
// rows unpadded), moved in 16-byte segments.
template <int DK>
struct Rec {
  static constexpr int NP = DK / 16;  // pass-1 waves (16 key channels each)
  static constexpr int LB = DK + 8;   // 16-bit [32][DK] rows
  static constexpr int LT = kC + 8;   // 16-bit [DK][32] and [32][32] rows
  static constexpr int LX = kC + 4;   // fp32 [32][32] rows
  static constexpr int LA = 20;       // fp32 [16][16] scratch rows
  static constexpr int dX = 0;                       // X fp32 [32][LX]
  static constexpr int dPH = dX + kC * LX * 4;       // P hi bf16 [32][LT]
  static constexpr int dPL = dPH + kC * LT * 2;      // P lo bf16 [32][LT]
  static constexpr int dGE = dPL + kC * LT * 2;      // Gamma_end fp32 [DK]
  static constexpr int dBeta = dGE + DK * 4;         // beta fp32 [32]
  static constexpr int dNQ = dBeta + kC * 4;         // 1/|q| fp32 [32]
  static constexpr int dNK = dNQ + kC * 4;           // 1/|k| fp32 [32]
  static constexpr int dQB = dNK + kC * 4;           // Qbar fp16 [32][LB]
  static constexpr int dW = dQB + kC * LB * 2;       // -W fp16 [32][LB]
  static constexpr int dKE = dW + kC * LB * 2;       // Kend^T fp16 [DK][LT]
  static constexpr int dSize = dKE + DK * LT * 2;
  static constexpr int kSegs = (kC * 128 + 2 * kC * 64 + DK * 4 + 3 * kC * 4 +
                                2 * kC * DK * 2 + DK * 64) / 16;
  static constexpr int kBytes = 16 * kSegs;
  static_assert(dSize % 16 == 0, "alignment");
};

// LDS byte offset of compact segment s of a record (0 past the end).
template <int DK>
__device__ __forceinline__ int rec_lds_offset(int s) {
  using R = Rec<DK>;
  constexpr int rows[10] = {kC, kC, kC, 1, 1, 1, 1, kC, kC, DK};
  constexpr int rowb[10] = {kC * 4, kC * 2, kC * 2, DK * 4, kC * 4, kC * 4, kC * 4,
                            DK * 2, DK * 2, kC * 2};
  constexpr int off[10] = {R::dX, R::dPH, R::dPL, R::dGE, R::dBeta, R::dNQ, R::dNK,
                           R::dQB, R::dW, R::dKE};
  constexpr int stride[10] = {R::LX * 4, R::LT * 2, R::LT * 2, 0, 0, 0, 0,
                              R::LB * 2, R::LB * 2, R::LT * 2};
  int base = 0, out = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const int per = rowb[r] / 16, nseg = rows[r] * per;
    if (s >= base && s < base + nseg) {
      const int i = s - base;
      out = off[r] + (i / per) * stride[r] + (i % per) * 16;
    }
    base += nseg;
  }
  return out;
}

// Chunks of sequence n in the block [c_begin, c_begin + bc), and their dense
// placement: slot_base[n] = sum of those counts over the sequences before n
// (a sequence's records are then laid out head by head, chunk by chunk).
constexpr int kPlanThreads = 1024;

__global__ void __launch_bounds__(kPlanThreads)
    split_plan_kernel(const int32_t* __restrict__ cu_seqlens, int N, int c_begin, int bc,
                      int32_t* __restrict__ slot_base) {
  __shared__ int scan[kPlanThreads];
  const int t = threadIdx.x;
  const int per = (N + kPlanThreads - 1) / kPlanThreads;
  const int n0 = min(N, t * per), n1 = min(N, n0 + per);
  auto count = [&](int n) {
    const int nch = (int)(((int64_t)cu_seqlens[n + 1] - cu_seqlens[n] + kC - 1) / kC);
    return max(0, min(nch - c_begin, bc));
  };
  int mine = 0;
  for (int n = n0; n < n1; ++n) mine += count(n);
  scan[t] = mine;
  __syncthreads();
  for (int d = 1; d < kPlanThreads; d <<= 1) {  // inclusive Hillis-Steele scan
    const int x = t >= d ? scan[t - d] : 0;
    __syncthreads();
    scan[t] += x;
    __syncthreads();
  }
  int off = scan[t] - mine;
  for (int n = n0; n < n1; ++n) {
    slot_base[n] = off;
    off += count(n);
  }
  if (t == 0) slot_base[N] = scan[kPlanThreads - 1];
}

// ============================ pass 1 ==========================================
// One workgroup of DK/16 waves per (sequence, head, group of `cpw` chunks of
// the block).  Per chunk the stages of the fused kernel's prep waves:
//   E   elementwise decay scaling and operands; per-wave partial squared
//       norms of the q and k rows
//   N   (one wave) 1/|q|, 1/|k| of the 32 rows
//   AP  A diagonal blocks and their inverses (waves 0, 1), A10 (wave 2), P
//   W   X10 = -X11 A10 X00 and the W^T tiles
// then every thread copies its segments of the record to global memory.  The
// record buffer is double-buffered in LDS, so the copy of chunk c overlaps the
// E stage of chunk c + 1.
template <int DK>
__global__ void __launch_bounds__(64 * (DK / 16))
    chunk_prep_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                           const uint16_t* __restrict__ a, const uint16_t* __restrict__ bl,
                           const int32_t* __restrict__ cu_seqlens,
                           const int32_t* __restrict__ slot_base, int H, int num_items,
                           int c_begin, int bc, int cpw, unsigned char* __restrict__ rec) {
  using R = Rec<DK>;
  constexpr int NP = R::NP, NT = 64 * NP;
  constexpr int LB = R::LB, LT = R::LT, LX = R::LX, LA = R::LA;
  constexpr int NKB = DK / 32;
  constexpr int NSEG = (R::kSegs + NT - 1) / NT;
  constexpr int oAT = 0;                          // A diagonal blocks^T fp32 [2][16][LA]
  constexpr int oA10 = oAT + 2 * 16 * LA * 4;     // A10 fp32 [16][LA]
  constexpr int oPart = oA10 + 16 * LA * 4;       // squared-norm partials fp32 [NP][64]
  constexpr int oRec = oPart + NP * 64 * 4;       // two record buffers
  constexpr int oKT = oRec + 2 * R::dSize;        // Kt bf16 [32][LB]
  constexpr int oQH = oKT + kC * LB * 2;          // Qt hi
  constexpr int oQL = oQH + kC * LB * 2;          // Qt lo
  constexpr int oKHH = oQL + kC * LB * 2;         // Kh hi
  constexpr int oKHL = oKHH + kC * LB * 2;        // Kh lo
  constexpr int oK1H = oKHL + kC * LB * 2;        // Kh exp(p_1) hi, rows 0-15
  constexpr int oK1L = oK1H + 16 * LB * 2;        // Kh exp(p_1) lo
  constexpr int oKBT = oK1L + 16 * LB * 2;        // Kbar^T fp16 [DK][LT]
  constexpr int kLds = oKBT + DK * LT * 2;
  static_assert(oRec % 16 == 0 && kLds <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  float* sAT = reinterpret_cast<float*>(smem + oAT);
  float* sA10 = reinterpret_cast<float*>(smem + oA10);
  float* sPart = reinterpret_cast<float*>(smem + oPart);
  uint16_t* sKT = reinterpret_cast<uint16_t*>(smem + oKT);
  uint16_t* sQH = reinterpret_cast<uint16_t*>(smem + oQH);
  uint16_t* sQL = reinterpret_cast<uint16_t*>(smem + oQL);
  uint16_t* sKHH = reinterpret_cast<uint16_t*>(smem + oKHH);
  uint16_t* sKHL = reinterpret_cast<uint16_t*>(smem + oKHL);
  uint16_t* sK1H = reinterpret_cast<uint16_t*>(smem + oK1H);
  uint16_t* sK1L = reinterpret_cast<uint16_t*>(smem + oK1L);
  uint16_t* sKBT = reinterpret_cast<uint16_t*>(smem + oKBT);

  const int ngrp = (bc + cpw - 1) / cpw;
  const int item = blockIdx.x / ngrp, grp = blockIdx.x - item * ngrp;
  if (item >= num_items) return;
  const int n = item / H, h = item % H;
  const int64_t tok_beg = cu_seqlens[n], tok_end = cu_seqlens[n + 1];
  const int nch = (int)((tok_end - tok_beg + kC - 1) / kC);
  const int c_lo = c_begin + grp * cpw;
  const int c_hi = min(min(c_lo + cpw, c_begin + bc), nch);
  if (c_lo >= c_hi) return;  // whole workgroup, before any barrier
  const int cnt = min(nch - c_begin, bc);  // chunks of this sequence in the block
  unsigned char* rec_item = rec + ((int64_t)H * slot_base[n] + (int64_t)h * cnt) * R::kBytes;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);

  int segl[NSEG];  // LDS offsets of this thread's record segments
#pragma unroll
  for (int i = 0; i < NSEG; ++i) segl[i] = rec_lds_offset<DK>((int)threadIdx.x + NT * i);

  // Lane (li, g): rows li (tile 0) and 16 + li (tile 1), key channels
  // 16 * wave + 4g .. +3; the tokens of a tile run along a 16-lane DPP row.
  u32x2_t rq[2], rk[2], ra[2];
  uint16_t rb[2];
  auto load = [&](int64_t c0, int li, int g) {
    const int nr = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
    const int64_t tb = c0 * H + h;
    const auto qb_ = sbase(q + tb * DK);
    const auto kb_ = sbase(k + tb * DK);
    const auto ab_ = sbase(a + tb * DK);
    const auto bb_ = sbase(bl + tb);
    // Rows past the end of the sequence re-load its last row (in bounds,
    // finite); they get g = 0 and beta = 0, which removes every contribution
    // they could make.
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int r = 16 * tau + li;
      const int rr = r < nr ? r : nr - 1;
      const uint32_t off = (uint32_t)(rr * H * DK) + 16 * wave + 4 * g;
      rq[tau] = *reinterpret_cast<const gptr<const u32x2_t>>(qb_ + off);
      rk[tau] = *reinterpret_cast<const gptr<const u32x2_t>>(kb_ + off);
      ra[tau] = *reinterpret_cast<const gptr<const u32x2_t>>(ab_ + off);
      rb[tau] = bb_[(uint32_t)(rr * H)];
    }
  };
  {
    const int lane = threadIdx.x % 64;
    load(tok_beg + (int64_t)kC * c_lo, lane % 16, lane / 16);
  }

  for (int c = c_lo; c < c_hi; ++c) {
    const int64_t c0 = tok_beg + (int64_t)kC * c;
    unsigned char* rbuf = smem + oRec + ((c - c_lo) & 1) * R::dSize;
    float* rX = reinterpret_cast<float*>(rbuf + R::dX);
    uint16_t* rPH = reinterpret_cast<uint16_t*>(rbuf + R::dPH);
    uint16_t* rPL = reinterpret_cast<uint16_t*>(rbuf + R::dPL);
    float* rGE = reinterpret_cast<float*>(rbuf + R::dGE);
    float* rBeta = reinterpret_cast<float*>(rbuf + R::dBeta);
    float* rNQ = reinterpret_cast<float*>(rbuf + R::dNQ);
    float* rNK = reinterpret_cast<float*>(rbuf + R::dNK);
    uint16_t* rQB = reinterpret_cast<uint16_t*>(rbuf + R::dQB);
    uint16_t* rW = reinterpret_cast<uint16_t*>(rbuf + R::dW);
    uint16_t* rKE = reinterpret_cast<uint16_t*>(rbuf + R::dKE);
    int t_ = threadIdx.x;
    __asm__ volatile("" : "+v"(t_));
    const int lane = t_ % 64, li = lane % 16, g = lane / 16;

    // ---- E: elementwise ----------------------------------------------------
    {
      const int nrows = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
      float qf[2][4], kf[2][4], cum[2][4];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        qf[tau][0] = bf16lo(rq[tau][0]); qf[tau][1] = bf16hi(rq[tau][0]);
        qf[tau][2] = bf16lo(rq[tau][1]); qf[tau][3] = bf16hi(rq[tau][1]);
        kf[tau][0] = bf16lo(rk[tau][0]); kf[tau][1] = bf16hi(rk[tau][0]);
        kf[tau][2] = bf16lo(rk[tau][1]); kf[tau][3] = bf16hi(rk[tau][1]);
        const float av[4] = {bf16lo(ra[tau][0]), bf16hi(ra[tau][0]), bf16lo(ra[tau][1]),
                             bf16hi(ra[tau][1])};
#pragma unroll
        for (int j = 0; j < 4; ++j)  // g in log2 units: -5 log2(e) sigmoid(a)
          cum[tau][j] = (kGMin * kLog2e) * rcpf_fast(1.f + exp2f_fast(-kLog2e * av[j]));
      }
      float beta[2];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
        beta[tau] = rcpf_fast(1.f + exp2f_fast(-kLog2e * __uint_as_float((uint32_t)rb[tau] << 16)));
      // squared norms of rows li and 16 + li over this lane's four channels,
      // summed over the four lanes (g) that share the rows
      float pq[2], pk[2];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        pq[tau] = qf[tau][0] * qf[tau][0] + qf[tau][1] * qf[tau][1] +
                  qf[tau][2] * qf[tau][2] + qf[tau][3] * qf[tau][3];
        pk[tau] = kf[tau][0] * kf[tau][0] + kf[tau][1] * kf[tau][1] +
                  kf[tau][2] * kf[tau][2] + kf[tau][3] * kf[tau][3];
        pq[tau] += __shfl_xor(pq[tau], 16, 64);
        pk[tau] += __shfl_xor(pk[tau], 16, 64);
        pq[tau] += __shfl_xor(pq[tau], 32, 64);
        pk[tau] += __shfl_xor(pk[tau], 32, 64);
      }
      if (g == 0) {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          sPart[wave * 64 + 16 * tau + li] = pq[tau];
          sPart[wave * 64 + 32 + 16 * tau + li] = pk[tau];
        }
      }
      if (nrows < kC) {  // padding rows: g = 0, beta = 0
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          const bool valid = 16 * tau + li < nrows;
#pragma unroll
          for (int j = 0; j < 4; ++j) cum[tau][j] = valid ? cum[tau][j] : 0.f;
          beta[tau] = valid ? beta[tau] : 0.f;
        }
      }
      // decay accumulated within each tile (inclusive), and the tile totals
      scan16_x8(cum);
      float tot[2][4];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int j = 0; j < 4; ++j) tot[tau][j] = row_last16(cum[tau][j]);
      const int cb = 16 * wave + 4 * g;
      float e0[4], fend[2][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e0[j] = exp2f_fast(tot[0][j]);       // exp(p_1): decay over tile 0
        fend[1][j] = exp2f_fast(tot[1][j]);  // exp(b_end - p_1)
        fend[0][j] = e0[j] * fend[1][j];     // exp(b_end - p_0) = Gamma_end
      }
      if (li == 0)
        *reinterpret_cast<float4*>(rGE + cb) =
            make_float4(fend[0][0], fend[0][1], fend[0][2], fend[0][3]);
      if (wave == 0 && g == 0) {
        rBeta[li] = beta[0];
        rBeta[16 + li] = beta[1];
      }
      uint16_t* kbt = sKBT + cb * LT + li;  // [channel cb + j][token 16 tau + li]
      uint16_t* ket = rKE + cb * LT + li;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int r = 16 * tau + li;
        bf16x4_t ktb, qhb, qlb, khh, khl, k1h, k1l;
        f16x4_t qbf;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = cum[tau][j];  // log2(e) (b - p) <= 0
          const float er = exp2f_fast(x), ir = exp2f_fast(-x);
          const float kt = kf[tau][j] * er, kh = kf[tau][j] * ir;
          const float qt = qf[tau][j] * er;
          const float qbar = tau ? qt * e0[j] : qt;
          qhb[j] = (__bf16)qt;
          qlb[j] = (__bf16)(qt - (float)qhb[j]);
          qbf[j] = (_Float16)qbar;
          const float kbar = tau ? kt * e0[j] : kt;
          const float kend = kh * fend[tau][j];
          ktb[j] = (__bf16)kt;
          khh[j] = (__bf16)kh;
          khl[j] = (__bf16)(kh - (float)khh[j]);
          kbt[j * LT + 16 * tau] = f16_bits(kbar);
          ket[j * LT + 16 * tau] = f16_bits(kend);
          if (tau == 0) {  // column operand of the off-diagonal tile: Kh exp(p_1) <= 1
            const float y = kh * e0[j];
            k1h[j] = (__bf16)y;
            k1l[j] = (__bf16)(y - (float)k1h[j]);
          }
        }
        *reinterpret_cast<bf16x4_t*>(sKT + r * LB + cb) = ktb;
        *reinterpret_cast<bf16x4_t*>(sKHH + r * LB + cb) = khh;
        *reinterpret_cast<bf16x4_t*>(sKHL + r * LB + cb) = khl;
        *reinterpret_cast<bf16x4_t*>(sQH + r * LB + cb) = qhb;
        *reinterpret_cast<bf16x4_t*>(sQL + r * LB + cb) = qlb;
        *reinterpret_cast<f16x4_t*>(rQB + r * LB + cb) = qbf;
        if (tau == 0) {
          *reinterpret_cast<bf16x4_t*>(sK1H + li * LB + cb) = k1h;
          *reinterpret_cast<bf16x4_t*>(sK1L + li * LB + cb) = k1l;
        }
      }
      // next chunk's inputs (this chunk's again after the last), requested
      // when this chunk's raw registers are dead
      load(c + 1 < c_hi ? c0 + kC : c0, li, g);
    }
    lds_barrier();  // B0: operands and norm partials in LDS

    // ---- N: 1/|q| (lanes 0-31) and 1/|k| (lanes 32-63) of the 32 rows ------
    if (wave == NP - 1) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NP; ++w) s += sPart[w * 64 + lane];
      (lane < 32 ? rNQ : rNK)[lane & 31] = rsqrtf(s + kNormEps);
    }
    lds_barrier();  // B1

    // ---- AP: A and X (waves 0, 1) | A10 (wave 2) | P tiles --------------------
    {
      // Row scale beta_r nk_r and column scale nk_i of the A tiles.
      auto a_tile = [&](int tr, int ti, const uint16_t* col) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int cc = 32 * kb + 8 * g;
          acc = mma_bf16(lds8<bf16x8_t>(sKT + (16 * tr + li) * LB + cc), lds8<bf16x8_t>(col + cc),
                         acc);
        }
        const float nkc = rNK[16 * ti + li];
        const float4 nkr = *reinterpret_cast<const float4*>(rNK + 16 * tr + 4 * g);
        const float4 ber = *reinterpret_cast<const float4*>(rBeta + 16 * tr + 4 * g);
        acc[0] *= ber.x * nkr.x * nkc; acc[1] *= ber.y * nkr.y * nkc;
        acc[2] *= ber.z * nkr.z * nkc; acc[3] *= ber.w * nkr.w * nkc;
        return acc;
      };
      auto p_job = [&](int job) {  // 0 = (0,0), 1 = (1,0), 2 = (1,1)
        const int tr = job == 0 ? 0 : 1, ti = job == 2 ? 1 : 0;
        const uint16_t* colh = job == 1 ? sK1H + li * LB : sKHH + (16 * ti + li) * LB;
        const uint16_t* coll = job == 1 ? sK1L + li * LB : sKHL + (16 * ti + li) * LB;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int cc = 32 * kb + 8 * g;
          acc = mma_x3(lds8<bf16x8_t>(sQH + (16 * tr + li) * LB + cc),
                       lds8<bf16x8_t>(sQL + (16 * tr + li) * LB + cc),
                       lds8<bf16x8_t>(colh + cc), lds8<bf16x8_t>(coll + cc), acc);
        }
        const float nki = rNK[16 * ti + li];
        const float4 nqr = *reinterpret_cast<const float4*>(rNQ + 16 * tr + 4 * g);
        const float nqv[4] = {nqr.x, nqr.y, nqr.z, nqr.w};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 16 * tr + 4 * g + jj, i = 16 * ti + li;
          const float pv = i <= r ? acc[jj] * nqv[jj] * nki : 0.f;
          const __bf16 hv = (__bf16)pv;
          rPH[r * LT + i] = __builtin_bit_cast(uint16_t, hv);
          rPL[r * LT + i] = bf16_bits(pv - (float)hv);
        }
        if (job == 0) {  // the upper tile (0, 1) of P is zero
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            rPH[(4 * g + jj) * LT + 16 + li] = 0;
            rPL[(4 * g + jj) * LT + 16 + li] = 0;
          }
        }
      };
      if (wave < 2) {
        // Diagonal block tau = wave: A_tt, then X_tt = (I + A_tt)^-1.
        const int tau = wave;
        const f32x4_t acc = a_tile(tau, tau, sKHH + (16 * tau + li) * LB);
        float4 at;
        at.x = li < 4 * g + 0 ? acc[0] : 0.f;  // strictly lower: A[4g + jj][li], li < 4g + jj
        at.y = li < 4 * g + 1 ? acc[1] : 0.f;
        at.z = li < 4 * g + 2 ? acc[2] : 0.f;
        at.w = li < 4 * g + 3 ? acc[3] : 0.f;
        float* atb = sAT + 16 * tau * LA;
        *reinterpret_cast<float4*>(atb + li * LA + 4 * g) = at;  // row m of sAT = column m of A
        lds_wave_fence();
        // Forward substitution, four lanes per column: lane (j = lane/4,
        // qd = lane%4) holds rows 4qd..4qd+3 of column j; the pivot x[m] is
        // broadcast within each quad of lanes.
        const int jc = lane >> 2, qd = lane & 3;
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = 4 * qd + i == jc ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 15; ++m) {
          const float4 am = *reinterpret_cast<const float4*>(atb + m * LA + 4 * qd);
          const float xm = quad_bcast(x[m & 3], m >> 2);
          x[0] -= am.x * xm;
          x[1] -= am.y * xm;
          x[2] -= am.z * xm;
          x[3] -= am.w * xm;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) rX[(16 * tau + 4 * qd + i) * LX + 16 * tau + jc] = x[i];
      } else {
        if (wave == 2) {  // A10, kept row-major for the W stage
          const f32x4_t acc = a_tile(1, 0, sK1H + li * LB);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) sA10[(4 * g + jj) * LA + li] = acc[jj];
        }
        if constexpr (NP >= 6) {
          if (wave >= 3 && wave < 6) p_job(wave - 3);
        } else {
          if (wave == 2) {
            p_job(0);
          } else {
            p_job(1);
            p_job(2);
          }
        }
      }
    }
    lds_barrier();  // B2: X diagonal blocks, A10 and P in LDS

    // ---- W: X10 = -X11 A10 X00; W^T = Kbar^T diag(beta nk) X^T; store -W ----
    {
      // X10^T = -X00^T (A10^T X11^T) on the fp32 matrix cores (every wave forms
      // it for its own W tiles); lane (li, g) ends with X10[li][4g + jj].
      f32x4_t p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        p1 = mma_f32(sA10[(4 * s + g) * LA + li], rX[(16 + li) * LX + 16 + 4 * s + g], p1);
      f32x4_t x10 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) x10 = mma_f32(rX[(4 * g + s) * LX + li], p1[s], x10);
      x10 = -x10;
      float bs[8];  // beta nk at the tokens of slots j (k order 4g..4g+3, 16+4g..16+4g+3)
      {
        const float4 b0 = *reinterpret_cast<const float4*>(rBeta + 4 * g);
        const float4 b1 = *reinterpret_cast<const float4*>(rBeta + 16 + 4 * g);
        const float4 n0 = *reinterpret_cast<const float4*>(rNK + 4 * g);
        const float4 n1 = *reinterpret_cast<const float4*>(rNK + 16 + 4 * g);
        bs[0] = b0.x * n0.x; bs[1] = b0.y * n0.y; bs[2] = b0.z * n0.z; bs[3] = b0.w * n0.w;
        bs[4] = b1.x * n1.x; bs[5] = b1.y * n1.y; bs[6] = b1.z * n1.z; bs[7] = b1.w * n1.w;
      }
      const f16x8_t kbt = lds4x2<f16x8_t>(sKBT + (16 * wave + li) * LT + 4 * g);
      float xx[2][8];
      {
        const float4 x00 = *reinterpret_cast<const float4*>(rX + li * LX + 4 * g);
        const float4 x11 = *reinterpret_cast<const float4*>(rX + (16 + li) * LX + 16 + 4 * g);
        xx[0][0] = x00.x; xx[0][1] = x00.y; xx[0][2] = x00.z; xx[0][3] = x00.w;
        xx[0][4] = xx[0][5] = xx[0][6] = xx[0][7] = 0.f;
        xx[1][0] = x10[0]; xx[1][1] = x10[1]; xx[1][2] = x10[2]; xx[1][3] = x10[3];
        xx[1][4] = x11.x; xx[1][5] = x11.y; xx[1][6] = x11.z; xx[1][7] = x11.w;
      }
      if (wave == 0) {  // complete X for pass 2: X10, and X01 = 0 (blocks no wave reads here)
        *reinterpret_cast<float4*>(rX + (16 + li) * LX + 4 * g) =
            make_float4(x10[0], x10[1], x10[2], x10[3]);
        *reinterpret_cast<float4*>(rX + li * LX + 16 + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int j = 0; j < 8; ++j) xx[rt][j] *= bs[j];
        const f32x4_t acc = mma_f16(kbt, pack_f16x8(xx[rt]), f32x4_t{0.f, 0.f, 0.f, 0.f});
        // acc[jj] = W[16 rt + li][16 wave + 4 g + jj]
        const f16x4_t wv = {(_Float16)(-acc[0]), (_Float16)(-acc[1]), (_Float16)(-acc[2]),
                            (_Float16)(-acc[3])};
        *reinterpret_cast<f16x4_t*>(rW + (16 * rt + li) * LB + 16 * wave + 4 * g) = wv;
      }
    }
    lds_barrier();  // B3: the record is complete in LDS

    // ---- copy the record out (overlaps the next chunk's E stage) -------------
    {
      const auto dst = sbase(rec_item + (int64_t)(c - c_begin) * R::kBytes);
#pragma unroll
      for (int i = 0; i < NSEG; ++i) {
        const int s = (int)threadIdx.x + NT * i;
        if (s < R::kSegs)
          *reinterpret_cast<gptr<u32x4_t>>(dst + 16 * s) =
              *reinterpret_cast<const u32x4_t*>(rbuf + segl[i]);
      }
    }
  }
}

// ============================ pass 2 ==========================================
// One workgroup of DV/16 waves per (sequence, head, d_v slice of DV columns);
// wave s owns state columns [16 s, 16 s + 16) of the slice in MFMA
// accumulator registers for the block.  Records stream global -> registers ->
// LDS (two LDS buffers, two register sets): the record of chunk c + 2 is
// requested while chunk c is computed and written to LDS one chunk later, so
// one workgroup barrier per chunk orders everything.  Every global request
// and store issues on every iteration (indices clamped, store ranges emptied
// when inactive), so the in-order memory counter never needs a full drain.
template <int DK, int DV, bool CKPT>
__global__ void __launch_bounds__(64 * (DV / 16))
    chunk_state_bf16_kernel(const uint16_t* __restrict__ v, const uint16_t* __restrict__ gate,
                            const int32_t* __restrict__ cu_seqlens,
                            const int32_t* __restrict__ slot_base,
                            const unsigned char* __restrict__ rec,
                            const float* __restrict__ s_init, float* __restrict__ carry,
                            float* __restrict__ s_final, float* __restrict__ o, int H,
                            int num_items, int dvt, int nsl, int c_begin, int bc, int ckpt_iv,
                            float* __restrict__ ckpt, long long ckpt_cap) {
  using R = Rec<DK>;
  constexpr int NS = DV / 16, NT = 64 * NS, NCT = DK / 16, NKB = DK / 32;
  constexpr int LB = R::LB, LT = R::LT, LX = R::LX;
  constexpr int NSEG = (R::kSegs + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * R::dSize];

  // Block -> (item, slice): the nsl slices of an item sit 8 blocks apart, on
  // the same XCD, so the second slice's record reads hit that XCD's L2.
  const int blk = blockIdx.x;
  const int item = (blk / (8 * nsl)) * 8 + blk % 8;
  const int col0 = ((blk / 8) % nsl) * DV;
  if (item >= num_items) return;
  const int n = item / H, h = item % H;
  const int64_t tok_beg = cu_seqlens[n], tok_end = cu_seqlens[n + 1];
  const int nch = (int)((tok_end - tok_beg + kC - 1) / kC);
  if (c_begin > 0 && c_begin >= nch) return;  // finished in an earlier block
  const int c_end = min(c_begin + bc, nch);
  const int cnt = c_end - c_begin;
  const float* s_src = c_begin == 0 ? s_init : carry;
  float* s_dst = c_begin + bc >= nch ? s_final : carry;
  const int sw = __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
  const int64_t st_off = (int64_t)item * DK * dvt + col0;

  f32x4_t S[NCT];
  {
    const int lane = threadIdx.x % 64, g = lane / 16, li = lane % 16;
    const uint32_t st_lane = 4 * g * dvt + 16 * sw + li;
    if (s_src) {
      const auto sp = sbase(s_src + st_off);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) S[ct][jj] = sp[st_lane + (16 * ct + jj) * dvt];
    } else {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) S[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }

  if (cnt > 0) {
    int64_t ck_off = 0;  // first recorded-state slot of this sequence
    if (CKPT)
      for (int m = 0; m < n; ++m) ck_off += (int64_t)(cu_seqlens[m + 1] - cu_seqlens[m]) / ckpt_iv;
    const unsigned char* rec_item =
        rec + ((int64_t)H * slot_base[n] + (int64_t)h * cnt) * R::kBytes;
    const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(rec_item), 0, cnt * R::kBytes, kBufferRsrcFlags);
    int segl[NSEG];      // LDS offsets of this thread's record segments
    uint32_t segg[NSEG];  // their byte offsets in a record
#pragma unroll
    for (int i = 0; i < NSEG; ++i) {
      const int s = (int)threadIdx.x + NT * i;
      segl[i] = rec_lds_offset<DK>(s);
      segg[i] = 16u * (uint32_t)(s < R::kSegs ? s : R::kSegs - 1);
    }
    u32x4_t Rg[2][NSEG];
    auto rec_load = [&](int cc, u32x4_t(&dst)[NSEG]) __attribute__((always_inline)) {
      const int soff = (cc - c_begin) * R::kBytes;
#pragma unroll
      for (int i = 0; i < NSEG; ++i)
        dst[i] = __builtin_bit_cast(u32x4_t,
                                    __builtin_amdgcn_raw_buffer_load_b128(rrs, segg[i], soff, 0));
    };
    auto rec_to_lds = [&](int b, const u32x4_t(&src)[NSEG]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NSEG; ++i)
        if ((int)threadIdx.x + NT * i < R::kSegs)
          *reinterpret_cast<u32x4_t*>(smem + b * R::dSize + segl[i]) = src[i];
    };

    int t0_ = threadIdx.x;
    __asm__ volatile("" : "+v"(t0_));
    const int lane = t0_ % 64, g = lane / 16, li = lane % 16;
    const int jcol = 16 * sw + li;
    const uint32_t hsh = 16u * (li & 1);  // which half of a loaded word is this lane's
    // v and gate of a chunk: lane (li, g) reads rows 16 (i / 4) + 4 g + i % 4,
    // as the aligned 32-bit word holding its bf16 (the lane pair (jcol & ~1,
    // jcol | 1) shares it); rows past the sequence's end read as zero.
    // Every offset a range check must see is in the lane offset (the
    // wave-uniform offset is kept out of it).
    uint32_t vgo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      vgo[i] = 2u * (uint32_t)((16 * (i / 4) + 4 * g + (i % 4)) * H * dvt + (jcol & ~1));
    uint32_t rv[8], rgr[8];
    float rg[8];
    auto load_vg = [&](int cc) __attribute__((always_inline)) {
      const int64_t c0 = tok_beg + (int64_t)kC * cc;
      const int nr = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
      const uint32_t range = (uint32_t)nr * (uint32_t)(H * dvt) * 2u;
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(v + (c0 * H + h) * dvt + col0), 0, range, kBufferRsrcFlags);
      // Without a gate the same rows of v are read (and ignored), so the
      // number of requests never depends on the gate.
      const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>((gate ? gate : v) + (c0 * H + h) * dvt + col0), 0, range,
          kBufferRsrcFlags);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        rv[i] = __builtin_amdgcn_raw_buffer_load_b32(vr, vgo[i], 0, 0);
        rgr[i] = __builtin_amdgcn_raw_buffer_load_b32(gr, vgo[i], 0, 0);
      }
    };
    f32x4_t O[2], U[2];
    // Chunk cc from LDS buffer b: U0, U = U0 - W S, O = diag(nq) Qbar S + P U,
    // then (when act) S <- diag(Gamma_end) S + Kend^T diag(nk) U.
    auto compute = [&](int b, int cc, bool act) __attribute__((always_inline)) {
      const unsigned char* rb = smem + b * R::dSize;
      const float* xb = reinterpret_cast<const float*>(rb + R::dX);
      const float* be = reinterpret_cast<const float*>(rb + R::dBeta);
      const float* nq = reinterpret_cast<const float*>(rb + R::dNQ);
      const float* nk = reinterpret_cast<const float*>(rb + R::dNK);
      const float* ge = reinterpret_cast<const float*>(rb + R::dGE);
      const uint16_t* wp = reinterpret_cast<const uint16_t*>(rb + R::dW);
      const uint16_t* qbp = reinterpret_cast<const uint16_t*>(rb + R::dQB);
      const uint16_t* ph = reinterpret_cast<const uint16_t*>(rb + R::dPH);
      const uint16_t* pl = reinterpret_cast<const uint16_t*>(rb + R::dPL);
      const uint16_t* kep = reinterpret_cast<const uint16_t*>(rb + R::dKE);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        rg[j] = rcpf_fast(1.f + exp2f_fast(-kLog2e * __uint_as_float((rgr[j] >> hsh) << 16)));
      {
        float rr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          rr[j] = be[16 * (j >> 2) + 4 * g + (j & 3)] * __uint_as_float((rv[j] >> hsh) << 16);
        bf16x8_t rh, rl;
        split_bf16x8(rr, rh, rl);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          float xx[8];
          lds_f32x4x2(xb + (16 * rt + li) * LX + 4 * g, xx);
          bf16x8_t xh, xl;
          split_bf16x8(xx, xh, xl);
          U[rt] = mma_x3(xh, xl, rh, rl, f32x4_t{0.f, 0.f, 0.f, 0.f});
        }
      }
      O[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      O[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        f16x8_t sbk;
#pragma unroll
        for (int j = 0; j < 8; ++j) sbk[j] = (_Float16)S[2 * kb + (j >> 2)][j & 3];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          U[rt] = mma_f16(lds4x2<f16x8_t>(wp + (16 * rt + li) * LB + 32 * kb + 4 * g), sbk, U[rt]);
          O[rt] = mma_f16(lds4x2<f16x8_t>(qbp + (16 * rt + li) * LB + 32 * kb + 4 * g), sbk, O[rt]);
        }
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float4 nr = *reinterpret_cast<const float4*>(nq + 16 * rt + 4 * g);
        O[rt][0] *= nr.x; O[rt][1] *= nr.y; O[rt][2] *= nr.z; O[rt][3] *= nr.w;
      }
      f16x8_t uf;
      bf16x8_t uh, ul;
      {
        float uu[8], us[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) uu[j] = U[j >> 2][j & 3];
        const float4 n0 = *reinterpret_cast<const float4*>(nk + 4 * g);
        const float4 n1 = *reinterpret_cast<const float4*>(nk + 16 + 4 * g);
        us[0] = uu[0] * n0.x; us[1] = uu[1] * n0.y; us[2] = uu[2] * n0.z; us[3] = uu[3] * n0.w;
        us[4] = uu[4] * n1.x; us[5] = uu[5] * n1.y; us[6] = uu[6] * n1.z; us[7] = uu[7] * n1.w;
        uf = pack_f16x8(us);
        split_bf16x8(uu, uh, ul);
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int off = (16 * rt + li) * LT + 4 * g;
        O[rt] = mma_x3(lds4x2<bf16x8_t>(ph + off), lds4x2<bf16x8_t>(pl + off), uh, ul, O[rt]);
      }
      if (act) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const float4 gv = *reinterpret_cast<const float4*>(ge + 16 * ct + 4 * g);
          f32x4_t acc;
          acc[0] = gv.x * S[ct][0]; acc[1] = gv.y * S[ct][1];
          acc[2] = gv.z * S[ct][2]; acc[3] = gv.w * S[ct][3];
          S[ct] = mma_f16(lds4x2<f16x8_t>(kep + (16 * ct + li) * LT + 4 * g), uf, acc);
        }
      }
    };
    auto record = [&](int cc) __attribute__((always_inline)) {
      const int64_t done = (int64_t)kC * (cc + 1);
      if (done % ckpt_iv == 0 && done <= tok_end - tok_beg) {
        const int64_t slot = ck_off + done / ckpt_iv - 1;
        if (slot < ckpt_cap) {
          const uint32_t st_lane = 4 * g * dvt + 16 * sw + li;
          // lane address held in vector registers (no scalar base)
          uint64_t ad = reinterpret_cast<uint64_t>(ckpt + (slot * H + h) * DK * dvt + col0 + st_lane);
          __asm__ volatile("" : "+v"(ad));
          float* sp = reinterpret_cast<float*>(ad);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sp[(16 * ct + jj) * dvt] = S[ct][jj];
        }
      }
    };
    // Gated output of chunk cc through a buffer resource whose range ends
    // after the chunk's last valid row (0 when inactive): the eight stores
    // always issue and the hardware drops the rest.
    auto epilogue = [&](int cc, bool act) __attribute__((always_inline)) {
      const int64_t c0 = tok_beg + (int64_t)kC * (act ? cc : c_begin);
      const int nr = act ? (int)(tok_end - c0 < kC ? tok_end - c0 : kC) : 0;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          o + (c0 * H + h) * dvt + col0, 0, nr * H * dvt * 4, kBufferRsrcFlags);
      const uint32_t vo_lane = (4 * g) * H * dvt + jcol;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float y = O[j >> 2][j & 3];
        if (gate) y *= rg[j];
        __builtin_amdgcn_raw_buffer_store_b32(
            __float_as_uint(y), rs, 4 * (vo_lane + (uint32_t)((16 * (j >> 2) + (j & 3)) * H * dvt)),
            0, 0);
      }
    };
    // Iteration for chunk cc, LDS buffer and register set B = (cc - c_begin) & 1.
    auto step = [&](int cc, auto Bc) __attribute__((always_inline)) {
      constexpr int B = decltype(Bc)::value;
      const bool act = cc < c_end;
      rec_load(min(cc + 2, c_end - 1), Rg[B]);
      compute(B, cc, act);
      if constexpr (CKPT)
        if (act) record(cc);
      load_vg(min(cc + 1, c_end - 1));
      epilogue(cc, act);
      rec_to_lds(B ^ 1, Rg[B ^ 1]);
      lds_barrier();
    };

    rec_load(c_begin, Rg[0]);
    rec_load(min(c_begin + 1, c_end - 1), Rg[1]);
    load_vg(c_begin);
    // Let everything requested so far arrive before the loop: a request still
    // pending on entry would make the loop's waits count its own stores too.
    __builtin_amdgcn_s_waitcnt(0);
    rec_to_lds(0, Rg[0]);
    lds_barrier();
    for (int cc = c_begin; cc < c_end; cc += 2) {
      step(cc, std::integral_constant<int, 0>());
      step(cc + 1, std::integral_constant<int, 1>());
    }
  }

  if (s_dst) {
    const int lane = threadIdx.x % 64, g = lane / 16, li = lane % 16;
    const uint32_t st_lane = 4 * g * dvt + 16 * sw + li;
    const auto sp = sbase(s_dst + st_off);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sp[st_lane + (16 * ct + jj) * dvt] = S[ct][jj];
  }
}

template <int DK>
constexpr uint64_t rec_bytes() {
  return (uint64_t)Rec<DK>::kBytes;
}

}  // namespace

SplitLayout split_layout(int64_t num_seqs, int64_t total_tokens, int64_t num_heads, int dk,
                         int dv) {
  SplitLayout w{};
  const uint64_t rb = dk == 128 ? rec_bytes<128>() : rec_bytes<64>();
  const uint64_t N = (uint64_t)num_seqs, H = (uint64_t)num_heads;
  const uint64_t nch_max = std::max<uint64_t>(1, ((uint64_t)total_tokens + kC - 1) / kC);
  const uint64_t all = H * (nch_max + N);  // records of every chunk (upper bound)
  const uint64_t budget = kSplitRecordBudget / rb;
  uint64_t bc, recs;
  if (all <= budget) {
    bc = nch_max;
    recs = all;
  } else {
    bc = std::max<uint64_t>(8, budget / std::max<uint64_t>(1, H * N));
    recs = std::min(all, H * N * bc);
  }
  bc = std::min<uint64_t>(bc, 0x7fffffffull / rb);  // a sequence's block stays under 2 GiB
  bc = std::min(bc, nch_max);
  recs = std::min(recs, H * N * bc);
  auto up = [](uint64_t x) { return (x + 255) / 256 * 256; };
  w.bc = (int)bc;
  w.blocks = (int)((nch_max + bc - 1) / bc);
  w.rec = 0;
  w.slot = up(recs * rb);
  w.carry = w.slot + up((N + 1) * 4);
  w.total = w.carry + (w.blocks > 1 ? up(N * H * (uint64_t)dk * (uint64_t)dv * 4) : 0);
  return w;
}

hipError_t launch_fwd_split_bf16(const FwdArgs& p, void* workspace, hipStream_t stream) {
  const int64_t items = (int64_t)p.num_seqs * p.num_heads;
  if (items == 0) return hipSuccess;
  const SplitLayout w = split_layout(p.num_seqs, p.total_tokens, p.num_heads, p.dk, p.dv);
  unsigned char* base = static_cast<unsigned char*>(workspace);
  unsigned char* rec = base + w.rec;
  int32_t* slot = reinterpret_cast<int32_t*>(base + w.slot);
  float* carry = w.blocks > 1 ? reinterpret_cast<float*>(base + w.carry) : nullptr;
  const int H = p.num_heads, N = p.num_seqs;
  const int nsl = p.dv == 128 && 2 * items <= device_cus() ? 2 : 1;
  const int dvs = p.dv / nsl;  // columns per pass-2 workgroup
  const int64_t sgrid = (items + 7) / 8 * 8 * nsl;
  const bool ck = p.ckpt_interval > 0;
  // chunks per pass-1 workgroup: enough workgroups to fill the GPU several
  // times over, at most 16 chunks each
  const int64_t want = 8LL * device_cus();
  int cpw = 16;
  while (cpw > 1 && items * ((w.bc + cpw - 1) / cpw) < want) cpw /= 2;
  const int64_t pgrid = items * ((w.bc + cpw - 1) / cpw);
  for (int blk = 0; blk < w.blocks; ++blk) {
    const int c_begin = blk * w.bc;
    hipLaunchKernelGGL(split_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p.cu_seqlens,
                       N, c_begin, w.bc, slot);
    if (p.dk == 128)
      hipLaunchKernelGGL(chunk_prep_bf16_kernel<128>, dim3((unsigned)pgrid), dim3(64 * 8), 0,
                         stream, (const uint16_t*)p.q, (const uint16_t*)p.k,
                         (const uint16_t*)p.a, (const uint16_t*)p.b, p.cu_seqlens, slot, H,
                         (int)items, c_begin, w.bc, cpw, rec);
    else
      hipLaunchKernelGGL(chunk_prep_bf16_kernel<64>, dim3((unsigned)pgrid), dim3(64 * 4), 0,
                         stream, (const uint16_t*)p.q, (const uint16_t*)p.k,
                         (const uint16_t*)p.a, (const uint16_t*)p.b, p.cu_seqlens, slot, H,
                         (int)items, c_begin, w.bc, cpw, rec);
    auto launch_state = [&](auto kern, int threads) {
      hipLaunchKernelGGL(kern, dim3((unsigned)sgrid), dim3(threads), 0, stream,
                         (const uint16_t*)p.v, (const uint16_t*)p.gate, p.cu_seqlens, slot,
                         (const unsigned char*)rec, p.initial_state, carry, p.final_state,
                         (float*)p.o, H, (int)items, p.dv, nsl, c_begin, w.bc, p.ckpt_interval,
                         p.ckpt, (long long)p.ckpt_capacity);
    };
    if (p.dk == 128) {
      if (dvs == 128)
        ck ? launch_state(chunk_state_bf16_kernel<128, 128, true>, 512)
           : launch_state(chunk_state_bf16_kernel<128, 128, false>, 512);
      else
        ck ? launch_state(chunk_state_bf16_kernel<128, 64, true>, 256)
           : launch_state(chunk_state_bf16_kernel<128, 64, false>, 256);
    } else {
      if (dvs == 128)
        ck ? launch_state(chunk_state_bf16_kernel<64, 128, true>, 512)
           : launch_state(chunk_state_bf16_kernel<64, 128, false>, 512);
      else
        ck ? launch_state(chunk_state_bf16_kernel<64, 64, true>, 256)
           : launch_state(chunk_state_bf16_kernel<64, 64, false>, 256);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kda
