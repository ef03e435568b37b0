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
//           inverse X = (I + A)^-1 and W, written as one "chunk record" with
//           every row scale folded in: X diag(beta) (bf16 hi/lo), P (bf16
//           hi/lo, lower block-triangular parts only), Gamma_end, diag(nq)
//           Qbar, -W and Kend diag(nk) (fp16), 30,208 bytes at d_k = 128
//           (nq, nk: 1/|q|, 1/|k|);
//   pass 2  chunk_state_bf16_kernel  per (sequence, head) -- or per
//           (sequence, head, 64-column d_v slice) when there are few items --
//           the sequential chain over the records: U0 = X diag(beta) V,
//           U = U0 - W S, O = Qbar' S + P U, S <- diag(Gamma_end) S
//           + Kend'^T U, y = sigmoid(gate) O.
//
// Why two passes: the fused kernel runs the key-side work once per d_v slice
// and ties it to the state chain's pace; here it runs once per head with no
// dependence between chunks, so pass 1 fills every compute unit, and pass 2
// is a light streaming loop.  The price is the records' round trip through
// HBM (about 1 KB per token-head at d_k = 128).  A long input is processed
// in blocks of chunks: for each block, a plan kernel places the block's
// records densely in the workspace, pass 1 fills them and pass 2 consumes
// them, carrying the state from block to block through the workspace.
// Pass 2 of a block runs on a second stream beside pass 1 of the next; with
// whole-head state workgroups (87 KB of LDS, alone on their compute units)
// the two passes split the GPU between them.
#include <algorithm>
#include <mutex>
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
  // LDS rows of the record in pass 2, whose reads are 8-byte MFMA operand
  // pieces from 16 consecutive rows: a row stride of 2 (mod 32) dwords puts
  // the 16 rows' pieces on distinct banks.
  static constexpr int RB = DK + 4;   // 16-bit [32][DK] rows
  static constexpr int RT = kC + 4;   // 16-bit [DK][32] and [32][32] rows
  static constexpr int dXH = 0;                      // X diag(beta) hi bf16 [32][RT]
  static constexpr int dXL = dXH + kC * RT * 2;      // X diag(beta) lo bf16 [32][RT]
  static constexpr int dPH = dXL + kC * RT * 2;      // P hi bf16 [32][RT]
  static constexpr int dPL = dPH + kC * RT * 2;      // P lo bf16 [32][RT]
  static constexpr int dGE = dPL + kC * RT * 2;      // Gamma_end fp32 [DK]
  static constexpr int dQB = dGE + DK * 4;           // diag(nq) Qbar fp16 [32][RB]
  static constexpr int dW = dQB + kC * RB * 2;       // -W fp16 [32][RB]
  static constexpr int dKE = dW + kC * RB * 2;       // (Kend diag(nk))^T fp16 [DK][RT]
  // (globally Kend diag(nk) is stored token-major [32][DK], transposed into
  // LDS by pass 2)
  static constexpr int dSize = dKE + DK * RT * 2;
  // compact (global) byte offsets, same regions in the same order; the 32x32
  // matrices X diag(beta) and P are lower block-triangular with lower
  // triangular diagonal blocks, and keep rows 0-7: columns 0-7, rows 8-15:
  // 0-15, rows 16-23: 0-23, rows 24-31: 0-31 (see tri_off); kTri is the
  // bytes of one such matrix (80 segments of 16 bytes)
  static constexpr int kTri = (8 * 8 + 8 * 16 + 8 * 24 + 8 * 32) * 2;
  static constexpr int cXH = 0;
  static constexpr int cXL = cXH + kTri;
  static constexpr int cPH = cXL + kTri;
  static constexpr int cPL = cPH + kTri;
  static constexpr int cGE = cPL + kTri;
  static constexpr int cQB = cGE + DK * 4;
  static constexpr int cW = cQB + kC * DK * 2;
  static constexpr int cKE = cW + kC * DK * 2;
  static constexpr int kBytes = cKE + DK * kC * 2;
  static constexpr int kSegs = cKE / 16;  // segments copied as they are (all but Kend)
  static_assert(dSize % 16 == 0 && (RB * 2) % 8 == 0 && (RT * 2) % 8 == 0, "alignment");
};

// Element offset of (r, c) in the compact form of a 32x32 lower
// block-triangular matrix with lower triangular 16x16 diagonal blocks: row r
// keeps columns 0 .. 8 (r / 8) + 7 (c must be within them).
__device__ __forceinline__ int tri_off(int r, int c) {
  const int q = r / 8;  // row group: 8 (q + 1) columns kept
  return 8 * 8 * q * (q + 1) / 2 + (r % 8) * 8 * (q + 1) + c;
}
// Whether column c of row r is kept (the columns beyond are zero).
__device__ __forceinline__ bool tri_kept(int r, int c) { return c < 8 * (r / 8 + 1); }

// LDS byte offset of compact segment s of a record (0 past the end).
template <int DK>
__device__ __forceinline__ int rec_lds_offset(int s) {
  using R = Rec<DK>;
  int out = 0;
  // X diag(beta) hi, lo, P hi, lo: 80 segments each (row group q: 8 rows of
  // q + 1 segments)
  constexpr int tri[4] = {R::dXH, R::dXL, R::dPH, R::dPL};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int i = s - 80 * m;
    if (i >= 0 && i < 80) {
      const int q = i < 8 ? 0 : i < 24 ? 1 : i < 48 ? 2 : 3;
      const int j = i - 4 * q * (q + 1);  // segment within the row group
      const int row = 8 * q + j / (q + 1), sr = j % (q + 1);
      out = tri[m] + row * R::RT * 2 + sr * 16;
    }
  }
  constexpr int rows[3] = {1, kC, kC};
  constexpr int rowb[3] = {DK * 4, DK * 2, DK * 2};
  constexpr int off[3] = {R::dGE, R::dQB, R::dW};
  constexpr int stride[3] = {0, R::RB * 2, R::RB * 2};
  int base = 4 * 80;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
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

// b [T, H] -> bt [H, T] (16-bit), so that the record pass reads a head's
// write-strength logits as contiguous runs instead of one 2-byte value per
// H-element row.  64 tokens x 64 heads per workgroup through LDS.
constexpr int kBtTile = 64;
__global__ void __launch_bounds__(256)
    b_transpose_kernel(const uint16_t* __restrict__ b, uint16_t* __restrict__ bt, long long T,
                       int H) {
  __shared__ uint16_t tile[kBtTile][kBtTile + 2];
  const int64_t t0 = (int64_t)blockIdx.x * kBtTile;
  const int h0 = blockIdx.y * kBtTile;
  for (int i = threadIdx.x; i < kBtTile * kBtTile; i += 256) {
    const int r = i / kBtTile, c = i % kBtTile;  // token r, head c of the tile
    const int64_t t = t0 + r;
    const int hh = h0 + c;
    tile[r][c] = (t < T && hh < H) ? b[t * H + hh] : (uint16_t)0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBtTile * kBtTile; i += 256) {
    const int r = i / kBtTile, c = i % kBtTile;  // head r, token c of the tile
    const int64_t t = t0 + c;
    const int hh = h0 + r;
    if (t < T && hh < H) bt[(int64_t)hh * T + t] = tile[c][r];
  }
}

// ============================ pass 1 ==========================================
// One workgroup of DK/16 waves per (sequence, head, group of `cpw` chunks of
// the block).  Per chunk the stages of the fused kernel's prep waves:
//   E   elementwise decay scaling and operands; per-wave partial squared
//       norms of the q and k rows
//   N   (one wave) 1/|q|, 1/|k| of the 32 rows
//   AP  A diagonal blocks and their inverses (waves 0, 1), A10 (wave 2), P
//   W   X10 = -X11 A10 X00 and the W^T tiles
// Each lane writes its parts of the record straight to global memory (small
// stores that the L2 merges into whole lines), so the LDS holds only the
// stage operands (73 KB at d_k = 128: two workgroups per CU).
template <int DK>
__global__ void __launch_bounds__(64 * (DK / 16))
    chunk_prep_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                           const uint16_t* __restrict__ a, const uint16_t* __restrict__ bt,
                           long long T,
                           const int32_t* __restrict__ cu_seqlens,
                           const int32_t* __restrict__ slot_base, int H, int num_items,
                           int c_begin, int bc, int cpw, unsigned char* __restrict__ rec) {
  using R = Rec<DK>;
  constexpr int NP = R::NP, NT = 64 * NP;
  constexpr int LB = R::LB, LT = R::LT, LX = R::LX, LA = R::LA;
  constexpr int NKB = DK / 32;
  constexpr int oAT = 0;                          // A diagonal blocks^T fp32 [2][16][LA]
  constexpr int oA10 = oAT + 2 * 16 * LA * 4;     // A10 fp32 [16][LA]
  constexpr int oPart = oA10 + 16 * LA * 4;       // squared-norm partials fp32 [NP][64]
  constexpr int oX = oPart + NP * 64 * 4;         // X fp32 [32][LX]
  constexpr int oBeta = oX + kC * LX * 4;         // beta fp32 [32]
  constexpr int oNQ = oBeta + kC * 4;             // 1/|q| fp32 [32]
  constexpr int oNK = oNQ + kC * 4;               // 1/|k| fp32 [32]
  constexpr int oKT = oNK + kC * 4;               // Kt bf16 [32][LB]
  constexpr int oQH = oKT + kC * LB * 2;          // Qt hi
  constexpr int oQL = oQH + kC * LB * 2;          // Qt lo
  constexpr int oKHH = oQL + kC * LB * 2;         // Kh hi
  constexpr int oKHL = oKHH + kC * LB * 2;        // Kh lo
  constexpr int oK1H = oKHL + kC * LB * 2;        // Kh exp(p_1) hi, rows 0-15
  constexpr int oK1L = oK1H + 16 * LB * 2;        // Kh exp(p_1) lo
  constexpr int oKBT = oK1L + 16 * LB * 2;        // Kbar^T fp16 [DK][LT]
  constexpr int kLds = oKBT + DK * LT * 2;
  static_assert(oKT % 16 == 0 && kLds <= 80 * 1024, "LDS budget: two workgroups per CU");

  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  float* sAT = reinterpret_cast<float*>(smem + oAT);
  float* sA10 = reinterpret_cast<float*>(smem + oA10);
  float* sPart = reinterpret_cast<float*>(smem + oPart);
  float* rX = reinterpret_cast<float*>(smem + oX);
  float* rBeta = reinterpret_cast<float*>(smem + oBeta);
  float* rNQ = reinterpret_cast<float*>(smem + oNQ);
  float* rNK = reinterpret_cast<float*>(smem + oNK);
  uint16_t* sKT = reinterpret_cast<uint16_t*>(smem + oKT);
  uint16_t* sQH = reinterpret_cast<uint16_t*>(smem + oQH);
  uint16_t* sQL = reinterpret_cast<uint16_t*>(smem + oQL);
  uint16_t* sKHH = reinterpret_cast<uint16_t*>(smem + oKHH);
  uint16_t* sKHL = reinterpret_cast<uint16_t*>(smem + oKHL);
  uint16_t* sK1H = reinterpret_cast<uint16_t*>(smem + oK1H);
  uint16_t* sK1L = reinterpret_cast<uint16_t*>(smem + oK1L);
  uint16_t* sKBT = reinterpret_cast<uint16_t*>(smem + oKBT);

  const int ngrp = (bc + cpw - 1) / cpw;
  // Block -> (item, chunk group): head-major with one sequence (each head's
  // records written in one run); with several, group-major, so that the
  // groups past a shorter sequence's end (they exit at once) come after all
  // the busy ones.  Interleaved head-major with a short period, they left
  // most compute units without work: 3.4x the time per chunk on 4 x 4096
  // tokens x 32 heads.
  const bool gmaj = num_items > H;
  const int item = gmaj ? (int)(blockIdx.x % (unsigned)num_items) : (int)(blockIdx.x / ngrp);
  const int grp = gmaj ? (int)(blockIdx.x / (unsigned)num_items) : (int)(blockIdx.x % ngrp);
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


  // Lane (li, g): rows li (tile 0) and 16 + li (tile 1), key channels
  // 16 * wave + 4g .. +3; the tokens of a tile run along a 16-lane DPP row.
  u32x2_t rq[2], rk[2], ra[2];
  uint16_t rb[2];
  // Requests for the rows of the chunk starting at token c0 through buffer
  // resources whose range ends at the sequence's last row (rows past it read
  // as zero; they also get g = 0 and beta = 0, which removes every
  // contribution they could make); an empty range (`live` false) issues the
  // same requests without touching memory.
  auto load = [&](int64_t c0, bool live, int li, int g) {
    const int nr = live ? (int)(tok_end - c0 < kC ? tok_end - c0 : kC) : 0;
    const int64_t tb = c0 * H + h;
    const uint32_t rows = (uint32_t)nr * (uint32_t)H;
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(q + tb * DK), 0, rows * DK * 2u, kBufferRsrcFlags);
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(k + tb * DK), 0, rows * DK * 2u, kBufferRsrcFlags);
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a + tb * DK), 0, rows * DK * 2u, kBufferRsrcFlags);
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(bt + (int64_t)h * T + c0), 0, (uint32_t)nr * 2u, kBufferRsrcFlags);
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const uint32_t r = 16 * tau + li;
      const uint32_t off = 2u * (r * (uint32_t)(H * DK) + 16 * wave + 4 * g);
      rq[tau] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(qr, off, 0, 0));
      rk[tau] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(kr, off, 0, 0));
      ra[tau] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(ar, off, 0, 0));
      rb[tau] = __builtin_amdgcn_raw_buffer_load_b16(br, 2u * r, 0, 0);
    }
  };
  {
    const int lane = threadIdx.x % 64;
    load(tok_beg + (int64_t)kC * c_lo, true, lane % 16, lane / 16);
  }

  for (int c = c_lo; c < c_hi; ++c) {
    const int64_t c0 = tok_beg + (int64_t)kC * c;
    // this chunk's record (compact layout), written straight from registers
    const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc(
        rec_item + (int64_t)(c - c_begin) * R::kBytes, 0, R::kBytes, kBufferRsrcFlags);
    auto st64 = [&](int off, auto x) __attribute__((always_inline)) {  // 8 bytes
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, x), dst, off, 0, 0);
    };
    int t_ = threadIdx.x;
    __asm__ volatile("" : "+v"(t_));
    const int lane = t_ % 64, li = lane % 16, g = lane / 16;

    // Qbar and Kend of rows li, 16 + li at channels cb..cb+3, kept until the
    // norms are known and folded in (AP stage).
    float qbr[2][4], ker[2][4];
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
          cum[tau][j] = log2_decay(av[j]);
      }
      float beta[2] = {0.f, 0.f};  // only wave 0 publishes them
      if (wave == 0) {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
          beta[tau] = rcpf_fast(1.f + exp2f_fast(-kLog2e * __uint_as_float((uint32_t)rb[tau] << 16)));
      }
      // squared norms of rows li and 16 + li over this lane's four channels,
      // summed over the four lanes (g) that share the rows
      float pq[2], pk[2];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        pq[tau] = sq2_bf16(rq[tau][1], sq2_bf16(rq[tau][0], 0.f));
        pk[tau] = sq2_bf16(rk[tau][1], sq2_bf16(rk[tau][0], 0.f));
        pq[tau] = rows4_sum(pq[tau]);
        pk[tau] = rows4_sum(pk[tau]);
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
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4_t, f32x4_t{fend[0][0], fend[0][1], fend[0][2], fend[0][3]}),
            dst, R::cGE + 4 * cb, 0, 0);
      if (wave == 0 && g == 0) {
        rBeta[li] = beta[0];
        rBeta[16 + li] = beta[1];
      }
      uint16_t* kbt = sKBT + cb * LT + li;  // [channel cb + j][token 16 tau + li]
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int r = 16 * tau + li;
        bf16x4_t ktb, qhb, qlb, khh, khl, k1h, k1l;
        float qt4[4], kt4[4], kh4[4], y4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = cum[tau][j];  // log2(e) (b - p) <= 0
          const float er = exp2f_fast(x), ir = exp2f_fast(-x);
          const float kt = kf[tau][j] * er, kh = kf[tau][j] * ir;
          const float qt = qf[tau][j] * er;
          qt4[j] = qt;
          qbr[tau][j] = tau ? qt * e0[j] : qt;
          const float kbar = tau ? kt * e0[j] : kt;
          // tile 0's rows: (kh exp(p_1)) exp(b_end - p_1), both factors
          // normal wherever the product is not negligible
          ker[tau][j] = tau ? kh * fend[1][j] : (kh * e0[j]) * fend[1][j];
          kt4[j] = kt;
          kh4[j] = kh;
          kbt[j * LT + 16 * tau] = f16_bits(kbar);
          // column operand of the off-diagonal tile (tile 0): Kh exp(p_1) <= 1
          y4[j] = kh * e0[j];
        }
        split_bf16x4(qt4, qhb, qlb);
        ktb = pack_bf16x4(kt4);
        split_bf16x4(kh4, khh, khl);
        if (tau == 0) split_bf16x4(y4, k1h, k1l);
        *reinterpret_cast<bf16x4_t*>(sKT + r * LB + cb) = ktb;
        *reinterpret_cast<bf16x4_t*>(sKHH + r * LB + cb) = khh;
        *reinterpret_cast<bf16x4_t*>(sKHL + r * LB + cb) = khl;
        *reinterpret_cast<bf16x4_t*>(sQH + r * LB + cb) = qhb;
        *reinterpret_cast<bf16x4_t*>(sQL + r * LB + cb) = qlb;
        if (tau == 0) {
          *reinterpret_cast<bf16x4_t*>(sK1H + li * LB + cb) = k1h;
          *reinterpret_cast<bf16x4_t*>(sK1L + li * LB + cb) = k1l;
        }
      }
      // next chunk's inputs (an empty request after the last), requested
      // when this chunk's raw registers are dead
      load(c0 + kC, c + 1 < c_hi, li, g);
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
      {  // diag(nq) Qbar and Kend diag(nk) of this lane's rows into the record
        const int cb = 16 * wave + 4 * g;
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          const int r = 16 * tau + li;
          const float nqr = rNQ[r], nkr = rNK[r];
          f16x4_t qv, kv;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            qv[j] = (_Float16)(qbr[tau][j] * nqr);
            kv[j] = (_Float16)(ker[tau][j] * nkr);
          }
          st64(R::cQB + 2 * (r * DK + cb), qv);
          st64(R::cKE + 2 * (r * DK + cb), kv);
        }
      }
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
      // P tile (tr, ti) formed transposed (the key operand on the matrix
      // cores' A side), so that lane (li, g) ends with row 16 tr + li, columns
      // 16 ti + 4g .. +3: one 8-byte store each for the hi and lo parts.
      auto p_job = [&](int job) {  // 0 = (0,0), 1 = (1,0), 2 = (1,1)
        const int tr = job == 0 ? 0 : 1, ti = job == 2 ? 1 : 0;
        const uint16_t* colh = job == 1 ? sK1H + li * LB : sKHH + (16 * ti + li) * LB;
        const uint16_t* coll = job == 1 ? sK1L + li * LB : sKHL + (16 * ti + li) * LB;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int cc = 32 * kb + 8 * g;
          acc = mma_x3(lds8<bf16x8_t>(colh + cc), lds8<bf16x8_t>(coll + cc),
                       lds8<bf16x8_t>(sQH + (16 * tr + li) * LB + cc),
                       lds8<bf16x8_t>(sQL + (16 * tr + li) * LB + cc), acc);
        }
        const int r = 16 * tr + li;
        const float nqr = rNQ[r];
        const float4 nki = *reinterpret_cast<const float4*>(rNK + 16 * ti + 4 * g);
        const float nkv[4] = {nki.x, nki.y, nki.z, nki.w};
        bf16x4_t hv, lv;
        float pv4[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int i = 16 * ti + 4 * g + jj;
          pv4[jj] = i <= r ? acc[jj] * nqr * nkv[jj] : 0.f;
        }
        split_bf16x4(pv4, hv, lv);
        // (the upper tile (0, 1) of P and the upper parts of the diagonal
        // tiles beyond the kept columns are zero and not stored)
        if (tri_kept(r, 16 * ti + 4 * g)) {
          st64(R::cPH + 2 * tri_off(r, 16 * ti + 4 * g), hv);
          st64(R::cPL + 2 * tri_off(r, 16 * ti + 4 * g), lv);
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
      // X diag(beta) as bf16 hi + lo (blocks X00, X10, X11; X01 = 0 is not
      // stored): one block each on three waves that are idle in the AP stage
      // (with fewer than eight waves, all three on the last)
      auto xb_block = [&](int rt, int half) __attribute__((always_inline)) {
        const float4 b4 = *reinterpret_cast<const float4*>(rBeta + 16 * half + 4 * g);
        const float bt[4] = {b4.x, b4.y, b4.z, b4.w};
        bf16x4_t hv, lv;
        float xv4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xv4[j] = xx[rt][4 * half + j] * bt[j];
        split_bf16x4(xv4, hv, lv);
        if (tri_kept(16 * rt + li, 16 * half + 4 * g)) {
          const int off = 2 * tri_off(16 * rt + li, 16 * half + 4 * g);
          st64(R::cXH + off, hv);
          st64(R::cXL + off, lv);
        }
      };
      if constexpr (NP >= 8) {
        if (wave == 5) xb_block(0, 0);
        if (wave == 6) xb_block(1, 0);
        if (wave == 7) xb_block(1, 1);
      } else if (wave == NP - 1) {
        xb_block(0, 0);
        xb_block(1, 0);
        xb_block(1, 1);
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int j = 0; j < 8; ++j) xx[rt][j] *= bs[j];
        const f32x4_t acc = mma_f16(kbt, pack_f16x8(xx[rt]), f32x4_t{0.f, 0.f, 0.f, 0.f});
        // acc[jj] = W[16 rt + li][16 wave + 4 g + jj]
        const f16x4_t wv = {(_Float16)(-acc[0]), (_Float16)(-acc[1]), (_Float16)(-acc[2]),
                            (_Float16)(-acc[3])};
        st64(R::cW + 2 * ((16 * rt + li) * DK + 16 * wave + 4 * g), wv);
      }
    }
    lds_barrier();  // B3: scratch free for the next chunk
  }
}

// ============================ pass 2 ==========================================
// One workgroup per (sequence, head), or per (sequence, head, 64-column d_v
// slice) when there are few items, with two wave groups:
//   state waves (SW)  wave s owns state columns [16 CT s, 16 CT (s + 1)) as CT
//                     tiles of 16 in MFMA accumulator registers for the whole
//                     block and runs the chain of chunk c from LDS; its
//                     column tiles share each operand read (SW CT = d_v / 16);
//   stream waves (4)  move the record and the v tile of chunk c + 1 from
//                     global memory into the other LDS buffer, with the
//                     requests for the next kAhead chunks in flight in their
//                     own registers.
// One workgroup barrier per chunk orders the two LDS buffers.  The state
// waves read their gate values straight from global memory one chunk ahead
// and store the outputs; every step (idle tail steps included) issues the same
// loads and stores in the same order, so a wait for the gate values never has
// to cover the previous chunk's stores.  The stream waves' only global
// accesses are loads, consumed in request order.
// With many (sequence, head) items at d_v = 128 a workgroup covers a whole
// head: four state waves of two column tiles (one state and one stream wave
// per SIMD) and 87 KB of LDS, so it has its compute unit to itself (a
// workgroup above 80 KB of LDS shares it with no other large one): the state
// pass of a block takes one CU per head and the record pass of the next block
// runs at full rate on the others; two column tiles per state wave halve the
// LDS operand reads.  With few items, 64-column slices (one tile per state
// wave, 80 KB) halve the state chain's work per step instead.
constexpr int kStateWaves = 4;
constexpr int kStreamWaves = 4;
constexpr int kWideItems = 32;   // above this many items, one workgroup per item at d_v = 128
constexpr int kAhead = 2;        // chunks requested ahead of the one written to LDS
constexpr int kStepPeriod = 2;   // chunks per iteration of the stream waves' unrolled loop

// NORM (whole-head workgroups only): the output row of each (token, head)
// passes a head-wise RMSNorm with weight norm_w [d_v] and norm_eps before the
// gate (page "[Paper Review] Kimi K3...", section "Kimi Delta Attention
// (KDA)", "Full-rank gate" paragraph), applied by the stream waves, which hold
// whole rows in the output stage.
template <int DK, int SW, int CT, bool CKPT, bool GATE, bool NORM = false>
__global__ void __launch_bounds__(64 * (SW + kStreamWaves))
    chunk_state_bf16_kernel(const uint16_t* __restrict__ v, const uint16_t* __restrict__ gate,
                            const int32_t* __restrict__ cu_seqlens,
                            const int32_t* __restrict__ slot_base,
                            const unsigned char* __restrict__ rec,
                            const float* __restrict__ s_init, float* __restrict__ carry,
                            float* __restrict__ s_final, float* __restrict__ o, int H,
                            int num_items, int dvt, int nsl, int c_begin, int bc, int ckpt_iv,
                            float* __restrict__ ckpt, long long ckpt_cap,
                            const float* __restrict__ norm_w, float norm_eps) {
  using R = Rec<DK>;
  constexpr int DV = 16 * CT * SW;
  constexpr int NCT = DK / 16, NKB = DK / 32;
  constexpr int LB = R::RB, LT = R::RT;
  // LDS buffer: record, then the v tile [32][VS] (16-bit); the 8-byte row
  // padding puts the four rows a state-wave read touches on distinct banks.
  constexpr int VS = DV + 4;
  constexpr int dV = R::dSize, dBuf = dV + kC * VS * 2;
  constexpr int NTS = 64 * kStreamWaves;            // stream threads
  constexpr int NSEG = (R::kSegs + NTS - 1) / NTS;  // record segments per stream thread
  constexpr int VPR = DV * 2 / 16;                  // 16-byte segments per tile row
  constexpr int VSEG = kC * VPR / NTS;              // tile segments per stream thread
  static_assert(dBuf % 16 == 0 && (kC * VPR) % NTS == 0 && VSEG >= 1, "layout");
  // With the norm (whole-head workgroups), the stream waves also run the
  // output stage: the state waves leave each chunk's unscaled output rows in
  // one half of an fp32 buffer [2][32][OP]; in the next step the stream
  // waves, which hold whole rows there, apply the head-wise RMSNorm and
  // sigmoid(gate) and store them with 16-byte accesses.  (Without the norm
  // the state waves store their own outputs: handing that stage over as well
  // measured 1.5 ms slower on the 1M-token forward.)
  constexpr bool OS = CT == 2 && NORM;
  static_assert(!NORM || OS, "the norm needs whole-head workgroups");
  static_assert(!NORM || !CKPT, "no recorded states with the norm");
  constexpr int OP = DV + 4;  // fp32 row pitch of the output buffer
  constexpr int dO = 2 * dBuf;
  constexpr int kOutBytes = OS ? 2 * kC * OP * 4 : 0;
  static_assert(2 * dBuf + kOutBytes <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * dBuf + kOutBytes];

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
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
  const unsigned char* rec_item = rec + ((int64_t)H * slot_base[n] + (int64_t)h * max(cnt, 0)) * R::kBytes;

  if (wave >= SW) {
    // ======================= stream waves =====================================
    if (cnt == 0) return;  // the state waves then run no barrier either
    const int st = (int)threadIdx.x - 64 * SW;
    const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(rec_item), 0, cnt * R::kBytes, kBufferRsrcFlags);
    int segl[NSEG];       // LDS offsets of this thread's record segments
    uint32_t segg[NSEG];  // their byte offsets in a record
#pragma unroll
    for (int i = 0; i < NSEG; ++i) {
      const int sg = st + NTS * i;
      segl[i] = rec_lds_offset<DK>(sg);
      segg[i] = 16u * (uint32_t)(sg < R::kSegs ? sg : R::kSegs - 1);
    }
    int vl[VSEG];       // LDS offsets (within a tile) of this thread's v / gate segments
    uint32_t vgo[VSEG];  // their byte offsets from the chunk's first row
#pragma unroll
    for (int i = 0; i < VSEG; ++i) {
      const int sv = st + NTS * i, row = sv / VPR, c8 = sv % VPR;
      vl[i] = row * VS * 2 + c8 * 16;
      vgo[i] = 2u * (uint32_t)(row * H * dvt + 8 * c8);
    }
    // Kend' arrives token-major; thread st < KJOBS transposes tokens 2 kp and
    // 2 kp + 1 of channels 8 kg .. 8 kg + 7 (consecutive lanes: consecutive
    // token pairs, so the 32-bit LDS writes fall on distinct banks).
    constexpr int KJOBS = 16 * (DK / 8);
    const int kp = st % 16, kg = (st % KJOBS) / 16;
    const uint32_t kgo = 2u * (uint32_t)(R::cKE / 2 + 2 * kp * DK + 8 * kg);
    u32x4_t Rr[kAhead][NSEG], Rv[kAhead][VSEG], Rk[kAhead][2];
    // Requests for chunk c_begin + min(s, cnt - 1) into register set K; rows
    // past the sequence's end read as zero (their range is empty).
    auto fetch = [&](int s, auto Kc) __attribute__((always_inline)) {
      constexpr int K = decltype(Kc)::value;
      const int cs = min(s, cnt - 1);
      const int soff = cs * R::kBytes;
#pragma unroll
      for (int i = 0; i < NSEG; ++i)
        Rr[K][i] = __builtin_bit_cast(u32x4_t,
                                      __builtin_amdgcn_raw_buffer_load_b128(rrs, segg[i], soff, 0));
      // (every thread requests, so the count of requests in flight is the
      // same on every path; threads past KJOBS repeat a job)
      Rk[K][0] = __builtin_bit_cast(u32x4_t,
                                    __builtin_amdgcn_raw_buffer_load_b128(rrs, kgo, soff, 0));
      Rk[K][1] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rrs, kgo + 2 * DK, soff, 0));
      const int64_t c0 = tok_beg + (int64_t)kC * (c_begin + cs);
      const int nr = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
      const uint32_t range = (uint32_t)nr * (uint32_t)(H * dvt) * 2u;
      const int64_t eoff = (c0 * H + h) * dvt + col0;
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(v + eoff), 0, range, kBufferRsrcFlags);
#pragma unroll
      for (int i = 0; i < VSEG; ++i)
        Rv[K][i] = __builtin_bit_cast(u32x4_t,
                                      __builtin_amdgcn_raw_buffer_load_b128(vr, vgo[i], 0, 0));
    };
    // Register set K into LDS buffer b (8-byte writes: padded rows).
    auto put = [&](int b, auto Kc) __attribute__((always_inline)) {
      constexpr int K = decltype(Kc)::value;
      unsigned char* base = smem + b * dBuf;
#pragma unroll
      for (int i = 0; i < NSEG; ++i)
        if (st + NTS * i < R::kSegs) {
          u32x2_t* d = reinterpret_cast<u32x2_t*>(base + segl[i]);
          d[0] = u32x2_t{Rr[K][i][0], Rr[K][i][1]};
          d[1] = u32x2_t{Rr[K][i][2], Rr[K][i][3]};
        }
      if (st < KJOBS) {
        // channel 8 kg + e: (token 2 kp, token 2 kp + 1) as one 32-bit word
        uint32_t* d = reinterpret_cast<uint32_t*>(base + R::dKE) + ((8 * kg) * LT + 2 * kp) / 2;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          d[e * LT / 2] = __builtin_amdgcn_perm(Rk[K][1][e / 2], Rk[K][0][e / 2],
                                                (e & 1) ? 0x07060302u : 0x05040100u);
      }
#pragma unroll
      for (int i = 0; i < VSEG; ++i) {
        u32x2_t* d = reinterpret_cast<u32x2_t*>(base + dV + vl[i]);
        d[0] = u32x2_t{Rv[K][i][0], Rv[K][i][1]};
        d[1] = u32x2_t{Rv[K][i][2], Rv[K][i][3]};
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    static_assert(kAhead == 2, "the unrolled loop below rotates two register sets");
    fetch(0, I0());
    fetch(1, I1());
    // The zero parts of X diag(beta) and P beyond each row's kept columns are
    // not in the record: write them into both LDS buffers once (nothing
    // overwrites them).
#pragma unroll
    for (int rp = 0; rp < 8; ++rp) {
      const int idx = st + NTS * rp;  // 0 .. 2047: buffer, matrix, row, 4-column piece
      const int b = idx / 1024, m = (idx / 256) % 4, row = (idx / 8) % 32, q4 = idx % 8;
      const int mb = m == 0 ? R::dXH : m == 1 ? R::dXL : m == 2 ? R::dPH : R::dPL;
      if (!tri_kept(row, 4 * q4))
        *reinterpret_cast<u32x2_t*>(smem + b * dBuf + mb + row * LT * 2 + 8 * q4) =
            u32x2_t{0u, 0u};
    }
    static_assert(NTS * 8 == 2 * 4 * 32 * 8, "8-byte zero pieces: eight per thread");
    // Output stage (OS): thread st owns row ro, columns oc .. oc + 15 of a
    // chunk's output; gate words of chunk j arrive one step ahead in set j & 1.
    const int ro = st >> 3, oc = 16 * (st & 7);
    u32x4_t Rg[2][2] = {};
    float nwo[16];  // the norm's weight at those columns
#pragma unroll
    for (int i = 0; i < 16; ++i) nwo[i] = NORM && norm_w ? norm_w[oc + i] : 1.f;
    auto gate_fetch_o = [&](int j, auto Kc) __attribute__((always_inline)) {
      constexpr int K = decltype(Kc)::value;
      if constexpr (OS && GATE) {
        const int64_t c0 = tok_beg + (int64_t)kC * (c_begin + min(j, cnt - 1));
        const int nr = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
        const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(gate + (c0 * H + h) * dvt + col0), 0,
            (uint32_t)nr * (uint32_t)(H * dvt) * 2u, kBufferRsrcFlags);
        const uint32_t off = 2u * (uint32_t)(ro * H * dvt + oc);
        Rg[K][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(gr, off, 0, 0));
        Rg[K][1] =
            __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(gr, off + 16, 0, 0));
      }
    };
    // Chunk c_begin + j's rows from output half j & 1 (every step issues the
    // same stores; an empty range when there is no such chunk).
    auto out_stage = [&](int j, auto Kc) __attribute__((always_inline)) {
      constexpr int K = decltype(Kc)::value;
      if constexpr (OS) {
        const bool live = j >= 0 && j < cnt;
        const int64_t c0 = tok_beg + (int64_t)kC * (c_begin + max(min(j, cnt - 1), 0));
        const int nr = live ? (int)(tok_end - c0 < kC ? tok_end - c0 : kC) : 0;
        const float* ob = reinterpret_cast<const float*>(smem + dO) + K * kC * OP + ro * OP + oc;
        float y[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 x = *reinterpret_cast<const float4*>(ob + 4 * i);
          y[4 * i] = x.x; y[4 * i + 1] = x.y; y[4 * i + 2] = x.z; y[4 * i + 3] = x.w;
        }
        if constexpr (NORM) {  // the row's mean square over its 8 threads
          float ss = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) ss += y[i] * y[i];
          ss += __shfl_xor(ss, 1, 64);
          ss += __shfl_xor(ss, 2, 64);
          ss += __shfl_xor(ss, 4, 64);
          const float rsq = rsqrtf(ss * (1.f / DV) + norm_eps);
#pragma unroll
          for (int i = 0; i < 16; ++i) y[i] *= rsq * nwo[i];
        }
        if constexpr (GATE) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t w = Rg[K][i / 8][(i % 8) / 2];
            const float gv = (i & 1) ? bf16hi(w) : bf16lo(w);
            y[i] *= rcpf_fast(1.f + exp2f_fast(-kLog2e * gv));
          }
        }
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            o + (c0 * H + h) * dvt + col0, 0, nr * H * dvt * 4, kBufferRsrcFlags);
        const uint32_t off = 4u * (uint32_t)(ro * H * dvt + oc);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u32x4_t, f32x4_t{y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]}),
              rs, off + 16u * i, 0, 0);
      }
    };
    put(0, I0());
    fetch(2, I0());
    gate_fetch_o(0, I0());
    lds_barrier();
    // Step s: chunk s + 1 (register set (s + 1) % 2) into buffer (s + 1) & 1,
    // then chunk s + 3 requested into that set; with the output stage, chunk
    // s - 1's rows out and chunk s + 1's gate words requested.  Two steps per
    // iteration make both indices static; a step past the last chunk repeats
    // it (the state waves run the same number of barriers), so every request
    // is issued on every path and each wait covers exactly one set.
    for (int s0 = 0; s0 < cnt; s0 += kStepPeriod) {
      put(1, I1()); fetch(s0 + 3, I1());
      out_stage(s0 - 1, I1()); gate_fetch_o(s0 + 1, I1());
      lds_barrier();
      put(0, I0()); fetch(s0 + 4, I0());
      out_stage(s0, I0()); gate_fetch_o(s0 + 2, I0());
      lds_barrier();
    }
    // the last step's rows (an empty range when that step was idle)
    out_stage(((cnt + kStepPeriod - 1) / kStepPeriod) * kStepPeriod - 1, I1());
    return;
  }

  // ======================= state waves ========================================
  const float* s_src = c_begin == 0 ? s_init : carry;
  float* s_dst = c_begin + bc >= nch ? s_final : carry;
  const int sw = wave;
  const int64_t st_off = (int64_t)item * DK * dvt + col0;
  int t0_ = threadIdx.x;
  __asm__ volatile("" : "+v"(t0_));
  const int lane = t0_ % 64, g = lane / 16, li = lane % 16;
  // column tile t of this wave: columns 16 (CT sw + t) .. + 15 of the slice
  const uint32_t st_lane = 4 * g * dvt + 16 * CT * sw + li;
  f32x4_t S[CT][NCT];
  if (s_src) {
    const auto sp = sbase(s_src + st_off);
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) S[t][ct][jj] = sp[st_lane + 16 * t + (16 * ct + jj) * dvt];
  } else {
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) S[t][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // column tile t of the state is held as S 2^(esc[t] - 127) (fp16 range of
  // the state-chain operands)
  int esc[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) esc[t] = 127;

  if (cnt > 0) {
    int64_t ck_off = 0;  // first recorded-state slot of this sequence
    if (CKPT)
      for (int m = 0; m < n; ++m) ck_off += (int64_t)(cu_seqlens[m + 1] - cu_seqlens[m]) / ckpt_iv;
    const int jcol = 16 * CT * sw + li;  // the lane's column in tile 0 (tile t: + 16 t)
    // v / gate words of rows 16 (i / 4) + 4 g + i % 4 at the lane's column
    // (the aligned 32-bit word holding its bf16), and the perm selector of
    // the lane's half
    int vwo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) vwo[i] = ((16 * (i / 4) + 4 * g + (i % 4)) * VS + (jcol & ~1)) * 2;
    const uint32_t hsh = 16u * (li & 1);
    const uint32_t vsel = (li & 1) ? 0x07060302u : 0x05040100u;
    // gate words of those rows (byte offsets from the chunk's first row), in
    // two sets: set s & 1 holds chunk c_begin + s, requested one step ahead
    uint32_t gwo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      gwo[i] = 2u * (uint32_t)((16 * (i / 4) + 4 * g + (i % 4)) * H * dvt + (jcol & ~1));
    uint32_t gw[2][CT][8];
    // Requests for the gate words of chunk c_begin + min(s, cnt - 1) into set
    // K; rows past the sequence's end read as zero (their range is empty).
    auto gate_fetch = [&](int s, auto Kc) __attribute__((always_inline)) {
      constexpr int K = decltype(Kc)::value;
      if constexpr (GATE && !OS) {
        const int64_t c0 = tok_beg + (int64_t)kC * (c_begin + min(s, cnt - 1));
        const int nr = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
        const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(gate + (c0 * H + h) * dvt + col0), 0,
            (uint32_t)nr * (uint32_t)(H * dvt) * 2u, kBufferRsrcFlags);
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            gw[K][t][i] = __builtin_amdgcn_raw_buffer_load_b32(gr, gwo[i] + 32u * t, 0, 0);
      }
    };
    // The output stores of a step past the last chunk: empty range, so
    // nothing is written, but the count of memory operations per step stays
    // the same on every path.
    auto idle_stores = [&]() __attribute__((always_inline)) {
      if constexpr (GATE && !OS) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(o, 0, 0, kBufferRsrcFlags);
#pragma unroll
        for (int j = 0; j < 8 * CT; ++j) __builtin_amdgcn_raw_buffer_store_b32(0u, rs, 4 * j, 0, 0);
      }
    };
    f32x4_t O[CT][2], U[CT][2];
    // Chunk c_begin + s from LDS buffer B (gate words in set B).
    auto chunk_step = [&](int s, auto Bc) __attribute__((always_inline)) {
      constexpr int B = decltype(Bc)::value;
      const int cc = c_begin + s;
      gate_fetch(s + 1, std::integral_constant<int, B ^ 1>());
      // the state columns' range for this chunk's fp16 operands
#pragma unroll
      for (int t = 0; t < CT; ++t) rescale_state(S[t], esc[t]);
      const unsigned char* rb = smem + B * dBuf;
      const uint16_t* xh = reinterpret_cast<const uint16_t*>(rb + R::dXH);
      const uint16_t* xl = reinterpret_cast<const uint16_t*>(rb + R::dXL);
      const uint16_t* ph = reinterpret_cast<const uint16_t*>(rb + R::dPH);
      const uint16_t* pl = reinterpret_cast<const uint16_t*>(rb + R::dPL);
      const float* ge = reinterpret_cast<const float*>(rb + R::dGE);
      const uint16_t* qbp = reinterpret_cast<const uint16_t*>(rb + R::dQB);
      const uint16_t* wp = reinterpret_cast<const uint16_t*>(rb + R::dW);
      const uint16_t* kep = reinterpret_cast<const uint16_t*>(rb + R::dKE);
      // operands of the chunk (shared by the wave's column tiles), requested first
      bf16x8_t aXH[2], aXL[2], aPH[2], aPL[2];
      f16x8_t aW[2][NKB], aQ[2][NKB];
      uint32_t rv[CT][8];
#pragma unroll
      for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          rv[t][i] = *reinterpret_cast<const uint32_t*>(rb + dV + vwo[i] + 32 * t);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int off = (16 * rt + li) * LT + 4 * g;
        aXH[rt] = lds4x2<bf16x8_t>(xh + off);
        aXL[rt] = lds4x2<bf16x8_t>(xl + off);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          aW[rt][kb] = lds4x2<f16x8_t>(wp + (16 * rt + li) * LB + 32 * kb + 4 * g);
          aQ[rt][kb] = lds4x2<f16x8_t>(qbp + (16 * rt + li) * LB + 32 * kb + 4 * g);
        }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int off = (16 * rt + li) * LT + 4 * g;
        aPH[rt] = lds4x2<bf16x8_t>(ph + off);
        aPL[rt] = lds4x2<bf16x8_t>(pl + off);
      }
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        // U0 = (X diag(beta))_hi V + (X diag(beta))_lo V; v is exact in bf16
        bf16x8_t vb;
        {
          u32x4_t w;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] = __builtin_amdgcn_perm(rv[t][2 * i + 1], rv[t][2 * i], vsel);
          vb = __builtin_bit_cast(bf16x8_t, w);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          U[t][rt] = mma_bf16(aXH[rt], vb, mma_bf16(aXL[rt], vb, f32x4_t{0.f, 0.f, 0.f, 0.f}));
        O[t][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        O[t][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // U0 on the state column's scale
        const float sc = pow2f(esc[t]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) U[t][rt][jj] *= sc;
      }
      // U += (-W) S, O = Qbar' S
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int t = 0; t < CT; ++t) {
          f16x8_t sbk;
#pragma unroll
          for (int j = 0; j < 8; ++j) sbk[j] = (_Float16)S[t][2 * kb + (j >> 2)][j & 3];
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            U[t][rt] = mma_f16(aW[rt][kb], sbk, U[t][rt]);
            O[t][rt] = mma_f16(aQ[rt][kb], sbk, O[t][rt]);
          }
        }
      // O += P U (U as bf16 hi + lo); Kend'^T U takes U as fp16 hi + lo (the
      // state keeps the product to fp16's rounding of Kend' alone)
      f16x8_t uf[CT], ufl[CT];
      float uinv[CT];
      bool ub = false;
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        bf16x8_t uh, ul;
        float uu[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) uu[j] = U[t][j >> 2][j & 3];
        split_bf16x8(uu, uh, ul);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) O[t][rt] = mma_x3(aPH[rt], aPL[rt], uh, ul, O[t][rt]);
        bool big;
        uinv[t] = u_range(uu, big);
        ub |= big;
        split_f16x8(uu, uf[t], ufl[t]);
      }
      // a column of U beyond fp16's range (rare): S <- 1/f (f diag(Gamma_end) S
      // + Kend'^T (f U)), the state pre- and post-scaled by powers of two
      if (ub) {
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) S[t][ct][jj] *= pow2f(254 - bexp(uinv[t]));
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float4 gv = *reinterpret_cast<const float4*>(ge + 16 * ct + 4 * g);
        const f16x8_t ke = lds4x2<f16x8_t>(kep + (16 * ct + li) * LT + 4 * g);
#pragma unroll
        for (int t = 0; t < CT; ++t) {
          f32x4_t acc;
          acc[0] = gv.x * S[t][ct][0]; acc[1] = gv.y * S[t][ct][1];
          acc[2] = gv.z * S[t][ct][2]; acc[3] = gv.w * S[t][ct][3];
          S[t][ct] = mma_f16(ke, uf[t], mma_f16(ke, ufl[t], acc));
        }
      }
      if (ub) {
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) S[t][ct][jj] *= uinv[t];
      }
      if constexpr (CKPT) {
        // the state after the first `done` tokens, when that is a multiple of
        // the recording interval
        const int64_t done = (int64_t)kC * (cc + 1);
        if (done % ckpt_iv == 0 && done <= tok_end - tok_beg) {
          const int64_t slot = ck_off + done / ckpt_iv - 1;
          if (slot < ckpt_cap) {
            // lane address held in vector registers (no scalar base)
            uint64_t ad = reinterpret_cast<uint64_t>(ckpt + (slot * H + h) * DK * dvt + col0 + st_lane);
            __asm__ volatile("" : "+v"(ad));
            float* sp = reinterpret_cast<float*>(ad);
#pragma unroll
            for (int t = 0; t < CT; ++t) {
              const float isc = pow2f(254 - esc[t]);
#pragma unroll
              for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                  sp[16 * t + (16 * ct + jj) * dvt] = S[t][ct][jj] * isc;
            }
          }
        }
      }
      if constexpr (OS) {
        // the unscaled output rows into half s & 1 of the output buffer (the
        // stream waves gate and store them in the next step)
        float* ob = reinterpret_cast<float*>(smem + dO) + (s & 1) * kC * OP;
#pragma unroll
        for (int t = 0; t < CT; ++t) {
          const float isc = pow2f(254 - esc[t]);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            ob[(16 * (j >> 2) + 4 * g + (j & 3)) * OP + 16 * (CT * sw + t) + li] =
                O[t][j >> 2][j & 3] * isc;
        }
      } else {
        // gated output through a buffer resource whose range ends after the
        // chunk's last valid row
        const int64_t c0 = tok_beg + (int64_t)kC * cc;
        const int nr = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            o + (c0 * H + h) * dvt + col0, 0, nr * H * dvt * 4, kBufferRsrcFlags);
        const uint32_t vo_lane = (4 * g) * H * dvt + jcol;
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            float y = O[t][j >> 2][j & 3] * pow2f(254 - esc[t]);
            if constexpr (GATE)
              y *= rcpf_fast(1.f + exp2f_fast(-kLog2e * __uint_as_float((gw[B][t][j] >> hsh) << 16)));
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint(y), rs,
                4 * (vo_lane + 16 * t + (uint32_t)((16 * (j >> 2) + (j & 3)) * H * dvt)), 0, 0);
          }
      }
      lds_barrier();
    };
    // the first chunk's gate words, followed by the same stores as a step
    gate_fetch(0, std::integral_constant<int, 0>());
    idle_stores();
    lds_barrier();  // the first buffer is in LDS
    const int steps = (cnt + kStepPeriod - 1) / kStepPeriod * kStepPeriod;  // as many barriers as the stream waves
    static_assert(kStepPeriod == 2, "two LDS buffers and gate sets per iteration");
    for (int s = 0; s < steps; s += 2) {
      if (s < cnt) {
        chunk_step(s, std::integral_constant<int, 0>());
      } else {
        gate_fetch(s + 1, std::integral_constant<int, 1>());
        idle_stores();
        lds_barrier();
      }
      if (s + 1 < cnt) {
        chunk_step(s + 1, std::integral_constant<int, 1>());
      } else {
        gate_fetch(s + 2, std::integral_constant<int, 0>());
        idle_stores();
        lds_barrier();
      }
    }
  }

  if (s_dst) {
    const auto sp = sbase(s_dst + st_off);
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      const float isc = pow2f(254 - esc[t]);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          sp[st_lane + 16 * t + (16 * ct + jj) * dvt] = S[t][ct][jj] * isc;
    }
  }
}

template <int DK>
constexpr uint64_t rec_bytes() {
  return (uint64_t)Rec<DK>::kBytes;
}

}  // namespace

SplitLayout split_layout(int64_t num_seqs, int64_t total_tokens, int64_t num_heads, int dk,
                         int dv, uint64_t record_budget, int buffers) {
  SplitLayout w{};
  const uint64_t rb = dk == 128 ? rec_bytes<128>() : rec_bytes<64>();
  const uint64_t N = (uint64_t)num_seqs, H = (uint64_t)num_heads;
  const uint64_t nch_max = std::max<uint64_t>(1, ((uint64_t)total_tokens + kC - 1) / kC);
  const uint64_t all = H * (nch_max + N);  // records of every chunk (upper bound)
  const uint64_t budget = record_budget / rb;
  const uint64_t nb = buffers > 1 ? 2 : 1;
  uint64_t bc, recs;
  if (all <= budget) {  // one block
    bc = nch_max;
    recs = all;
  } else {  // blocks in (two) record buffers, so that a block's records are
            // built while the previous block's are consumed
    bc = std::max<uint64_t>(8, budget / nb / std::max<uint64_t>(1, H * N));
    recs = std::min(all, H * N * bc);
  }
  bc = std::min<uint64_t>(bc, 0x7fffffffull / rb);  // a sequence's block stays under 2 GiB
  bc = std::min(bc, nch_max);
  recs = std::min(recs, H * N * bc);
  auto up = [](uint64_t x) { return (x + 255) / 256 * 256; };
  w.bc = (int)bc;
  w.blocks = (int)((nch_max + bc - 1) / bc);
  w.nbuf = w.blocks > 1 ? (int)nb : 1;
  uint64_t off = 0;
  for (int i = 0; i < w.nbuf; ++i) {
    w.rec[i] = off;
    off += up(recs * rb);
  }
  for (int i = 0; i < w.nbuf; ++i) {
    w.slot[i] = off;
    off += up((N + 1) * 4);
  }
  w.carry = off;
  w.bt = w.carry + (w.blocks > 1 ? up(N * H * (uint64_t)dk * (uint64_t)dv * 4) : 0);
  w.total = w.bt + up(H * (uint64_t)std::max<int64_t>(total_tokens, 0) * 2);
  return w;
}

namespace {

// Per device: a second stream (default priority) for the state pass, and
// the events that order it against the chunk-record pass on the caller's
// stream.  Created on the first multi-block call on that device (on the
// device of the caller's stream) and kept for the process; one mutex
// serialises the enqueueing (not the GPU work) of concurrent calls, which on
// one device share this stream.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t start = nullptr, built[2] = {nullptr, nullptr}, used[2] = {nullptr, nullptr};
};
std::mutex g_side_mu;
SideStream g_side[64];

hipError_t side_stream(hipStream_t stream, SideStream** out) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    SideStream made;
    e = hipStreamCreateWithFlags(&made.s, hipStreamNonBlocking);
    hipEvent_t* evs[5] = {&made.start, &made.built[0], &made.built[1], &made.used[0],
                          &made.used[1]};
    for (hipEvent_t* ev : evs)
      if (e == hipSuccess) e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    ss = made;
  }
  *out = &ss;
  return hipSuccess;
}

}  // namespace

hipError_t device_side_stream(hipStream_t stream, hipStream_t* out) {
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream* side = nullptr;
  const hipError_t e = side_stream(stream, &side);
  if (e == hipSuccess) *out = side->s;
  return e;
}

bool split_whole_head(int64_t num_seqs, int64_t num_heads, int dv) {
  return dv == 128 && num_seqs * num_heads > kWideItems;
}

// Block b's plan and record pass run on the caller's stream into buffer
// b % 2; its state pass runs on the side stream once they are done, while
// block b + 1's records are built.  Block b + 2 reuses buffer b % 2 after
// block b's state pass; the caller's stream waits for the last state pass.
hipError_t launch_fwd_split_bf16(const FwdArgs& p, void* workspace, hipStream_t stream,
                                 const SplitLayout* layout) {
  const int64_t items = (int64_t)p.num_seqs * p.num_heads;
  if (items == 0) return hipSuccess;
  const SplitLayout w =
      layout ? *layout : split_layout(p.num_seqs, p.total_tokens, p.num_heads, p.dk, p.dv);
  unsigned char* base = static_cast<unsigned char*>(workspace);
  float* carry = w.blocks > 1 ? reinterpret_cast<float*>(base + w.carry) : nullptr;
  uint16_t* bt = reinterpret_cast<uint16_t*>(base + w.bt);
  const int H = p.num_heads, N = p.num_seqs;
  // Pass-2 workgroups: one per item with two 16-column tiles per state wave
  // (128 columns) when there are enough items to fill the GPU with both
  // passes running side by side (blocks overlapped on two streams), when the
  // norm is applied in the output stage, or when the slices would not fit
  // one round (a slice workgroup, VGPR-bound, has its CU to itself);
  // otherwise 64-column slices (one tile per state wave, two workgroups per
  // item), which shorten the chain where it runs alone (one block, or blocks
  // in sequence).
  const bool wide =
      p.norm || (split_whole_head(p.num_seqs, p.num_heads, p.dv) &&
                 ((!layout && w.blocks > 1) || 2 * items > device_cus()));
  const int nsl = wide ? 1 : p.dv / 64;
  const int64_t sgrid = (items + 7) / 8 * 8 * nsl;
  const bool ck = p.ckpt_interval > 0;
  // Block schedule: with several blocks the first is a quarter of the
  // others (its record pass runs alone, before any state pass) and the last
  // takes the remainder (its state pass runs alone); block b covers chunks
  // [b0, b0 + nb) of every sequence.
  const int64_t nch_max = std::max<int64_t>(1, (p.total_tokens + kC - 1) / kC);
  const int first = w.blocks > 1 ? std::max(8, w.bc / 4) : w.bc;
  const int nblocks = w.blocks > 1 ? 1 + (int)((nch_max - first + w.bc - 1) / w.bc) : 1;
  // chunks per pass-1 workgroup: enough workgroups to fill the GPU several
  // times over, at most 16 chunks each
  const int64_t want = 8LL * device_cus();

  std::unique_lock<std::mutex> lock(g_side_mu, std::defer_lock);
  if (!layout) lock.lock();  // the side stream is shared per device
  SideStream* side = nullptr;
  hipStream_t s2 = stream;  // one block: everything on the caller's stream
  hipError_t e;
  if (p.total_tokens > 0) {  // the record pass reads b as [H, T]
    const dim3 grid((unsigned)((p.total_tokens + kBtTile - 1) / kBtTile),
                    (unsigned)((H + kBtTile - 1) / kBtTile));
    hipLaunchKernelGGL(b_transpose_kernel, grid, dim3(256), 0, stream, (const uint16_t*)p.b, bt,
                       (long long)p.total_tokens, H);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (w.blocks > 1 && !layout) {
    if ((e = side_stream(stream, &side)) != hipSuccess) return e;
    s2 = side->s;
    if ((e = hipEventRecord(side->start, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(s2, side->start, 0)) != hipSuccess) return e;
  }
  for (int blk = 0; blk < nblocks; ++blk) {
    const int c_begin = blk == 0 ? 0 : first + (blk - 1) * w.bc;
    const int nb = blk == 0 ? first : w.bc;
    const int bi = blk % w.nbuf;
    int cpw = 16;
    while (cpw > 1 && items * ((nb + cpw - 1) / cpw) < want) cpw /= 2;
    const int64_t pgrid = items * ((nb + cpw - 1) / cpw);
    unsigned char* rec = base + w.rec[bi];
    int32_t* slot = reinterpret_cast<int32_t*>(base + w.slot[bi]);
    if (side && blk >= 2 && (e = hipStreamWaitEvent(stream, side->used[bi], 0)) != hipSuccess)
      return e;
    // The plan also orders the two passes on the GPU: block b's state pass
    // and block b + 1's record pass become ready together (both wait for
    // block b's record pass), and this plan puts a few microseconds between
    // them, so the state pass's 96 workgroups take their CUs first.  Planned
    // ahead for every block instead, the record pass won that race, filled
    // every CU, and each state pass took 3 ms instead of 1.75 (133 against
    // 80 ms per forward).
    hipLaunchKernelGGL(split_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p.cu_seqlens,
                       N, c_begin, nb, slot);
    if (p.dk == 128)
      hipLaunchKernelGGL(chunk_prep_bf16_kernel<128>, dim3((unsigned)pgrid), dim3(64 * 8), 0,
                         stream, (const uint16_t*)p.q, (const uint16_t*)p.k,
                         (const uint16_t*)p.a, bt, (long long)p.total_tokens, p.cu_seqlens,
                         slot, H, (int)items, c_begin, nb, cpw, rec);
    else
      hipLaunchKernelGGL(chunk_prep_bf16_kernel<64>, dim3((unsigned)pgrid), dim3(64 * 4), 0,
                         stream, (const uint16_t*)p.q, (const uint16_t*)p.k,
                         (const uint16_t*)p.a, bt, (long long)p.total_tokens, p.cu_seqlens,
                         slot, H, (int)items, c_begin, nb, cpw, rec);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (side) {
      if ((e = hipEventRecord(side->built[bi], stream)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(s2, side->built[bi], 0)) != hipSuccess) return e;
    }
    auto launch_state = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3((unsigned)sgrid), dim3(64 * (kStateWaves + kStreamWaves)), 0,
                         s2, (const uint16_t*)p.v, (const uint16_t*)p.gate, p.cu_seqlens, slot,
                         (const unsigned char*)rec, p.initial_state, carry, p.final_state,
                         (float*)p.o, H, (int)items, p.dv, nsl, c_begin, nb, p.ckpt_interval,
                         p.ckpt, (long long)p.ckpt_capacity, p.norm_weight, p.norm_eps);
    };
    const bool gt = p.gate != nullptr;
    auto pick = [&](auto dkc, auto ctc) {
      constexpr int K = decltype(dkc)::value, T = decltype(ctc)::value;
      if constexpr (T == 2) {
        if (p.norm) {  // whole-head workgroups only (the caller checks)
          gt ? launch_state(chunk_state_bf16_kernel<K, kStateWaves, T, false, true, true>)
             : launch_state(chunk_state_bf16_kernel<K, kStateWaves, T, false, false, true>);
          return;
        }
      }
      if (ck)
        gt ? launch_state(chunk_state_bf16_kernel<K, kStateWaves, T, true, true>)
           : launch_state(chunk_state_bf16_kernel<K, kStateWaves, T, true, false>);
      else
        gt ? launch_state(chunk_state_bf16_kernel<K, kStateWaves, T, false, true>)
           : launch_state(chunk_state_bf16_kernel<K, kStateWaves, T, false, false>);
    };
    using D128 = std::integral_constant<int, 128>;
    using D64 = std::integral_constant<int, 64>;
    using T2 = std::integral_constant<int, 2>;
    using T1 = std::integral_constant<int, 1>;
    if (p.dk == 128)
      wide ? pick(D128(), T2()) : pick(D128(), T1());
    else
      wide ? pick(D64(), T2()) : pick(D64(), T1());
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (side && (e = hipEventRecord(side->used[bi], s2)) != hipSuccess) return e;
  }
  if (side && (e = hipStreamWaitEvent(stream, side->used[(nblocks - 1) % w.nbuf], 0)) !=
                  hipSuccess)
    return e;
  return hipSuccess;
}

// ---- workspace of the forward that allocates nothing -------------------------
// A fixed device array, one per device the library runs on (each device's
// code object holds its own copy, at its own address); host code never
// passes the array's name to a kernel, only the address resolved below.
namespace {
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};
}  // namespace

bool noalloc_layout(int64_t num_seqs, int64_t total_tokens, int64_t num_heads, int dk, int dv,
                    SplitLayout* out) {
  auto up = [](uint64_t x) { return (x + 255) / 256 * 256; };
  const uint64_t N = (uint64_t)num_seqs, H = (uint64_t)num_heads;
  // the parts whose size does not depend on the block length: record
  // offsets, carried states, b transposed
  const uint64_t fixed = up((N + 1) * 4) + up(N * H * (uint64_t)dk * (uint64_t)dv * 4) +
                         up(H * (uint64_t)std::max<int64_t>(total_tokens, 0) * 2);
  if (fixed + 256 >= kNoAllocScratchBytes) return false;
  const SplitLayout w = split_layout(num_seqs, total_tokens, num_heads, dk, dv,
                                     kNoAllocScratchBytes - fixed - 256, 1);
  if (w.total > kNoAllocScratchBytes) return false;  // 8 chunks of every pair do not fit
  *out = w;
  return true;
}

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {  // once per device, with that device current
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace kda
