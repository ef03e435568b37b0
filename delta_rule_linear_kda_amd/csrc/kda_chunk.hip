// kda_chunk.hip - chunked KDA forward over packed variable-length sequences,
// gfx950 (MI355X): the fp32-input kernel (fp32 matrix-core products, for the
// 1e-4 accuracy of fp32 inputs).  bf16 inputs use kda_chunk_bf16.hip.
//
// Method: the KDA recurrence (page "[Paper Review] Kimi K3...", section "Kimi
// Delta Attention (KDA)") evaluated in its chunkwise-parallel form (same
// section: recurrent but parallelisable per chunk).  Each 64-token chunk is
// split into four 16-token tiles; because the log-decay is bounded below by
// g_min = -5 ("Lower-bounded decay" paragraph), the cumulative log-decay of a
// tile lies in [-80, 0] and every pairwise decay exp(b_r - b_i) can be
// factored into a row factor exp(b_r - p) <= 1 and a column factor
// exp(p - b_i) <= e^80 (p = cumulative decay before row r's tile), both
// finite in bf16, so every intra-chunk tile -- diagonal or not -- is a dense
// matrix product on the matrix cores.
//
// Per chunk (n <= 64 rows, start state S, b = chunk-local cumsum of g):
//   A   = diag(beta) strict_lower(Kt Kh^T)      P = lower(Qt Kh^T)
//   X   = (I + A)^-1                            (block forward substitution)
//   W   = X diag(beta) Kbar,   U0 = X diag(beta) V
//   U   = U0 - W S
//   O   = Qbar S + P U,        y = sigmoid(gate) * O
//   S  <- diag(Gamma_end) S + Kend^T U
// with Kt = kh*exp(b - p), Kh = kh*exp(p - b) (off-diagonal tiles rescaled by
// exp(p_row_tile - p_col_tile) <= 1), Qt = qh*exp(b - p), Qbar = qh*exp(b),
// Kbar = kh*exp(b), Kend = kh*exp(b_end - b), Gamma_end = exp(b_end); Kend's row
// factor is taken in two steps, to the tile's end and from there to the chunk's.
//
// Work decomposition: one workgroup of 4 wavefronts per (sequence, head,
// 64-column slice of d_v).  The fp32 state slice (dk x 64) stays in MFMA
// accumulator registers for the whole sequence: wave w owns columns
// [16w, 16w+16).  MFMA output tiles are consumed directly as the next
// product's B operand (a C tile's row index equals the B operand's k index up
// to a fixed permutation of k, applied identically to the A operand), so S and
// U never leave registers; the dk-side operands shared by the waves are staged
// through LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 64;      // chunk length (tokens)
constexpr int kTile = 16;   // tile length (tokens)
constexpr int kThreads = 256;
constexpr int kDvs = 64;    // d_v columns per workgroup

// ---------------------------------------------------------------------------
// Matrix-core precision policies.  For one 32-wide block of the contraction
// index, each lane supplies 8 fp32 values of the A operand (row m = lane%16)
// and 8 of the B operand (column n = lane%16); slot j of lane group g = lane/16
// stands for contraction index kmap(g, j), any bijection onto 0..31 in which
// the four lane groups hold four distinct indices in each slot.  The result
// accumulates sum_k A[m][k] B[k][n] into a 16x16 fp32 tile whose lane l holds
// rows 4*(l/16) + 0..3 of column l%16.
// ---------------------------------------------------------------------------

// fp32 inputs: v_mfma_f32_16x16x4_f32, one instruction per slot (the four lane
// groups are the instruction's four k values).
struct PolicyF32 {
  static __device__ __forceinline__ void mma(f32x4_t& acc, const float (&a)[8],
                                             const float (&b)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
  }
};

// Contraction index of slot j for lane group g when the B operand is formed
// from two stacked 16-row accumulator tiles (rows 0-15 then 16-31).
__device__ __forceinline__ int kperm(int g, int j) {
  return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

// Index of the ordered tile pair (t, u), u < t, among the six such pairs.
__device__ __forceinline__ int pair_idx(int t, int u) { return t * (t - 1) / 2 + u; }

// Lower-triangular tile pairs (row tile, column tile) of a 4x4 tiled chunk.
__constant__ int8_t kLowerPairs[10][2] = {{0, 0}, {1, 0}, {1, 1}, {2, 0}, {2, 1},
                                          {2, 2}, {3, 0}, {3, 1}, {3, 2}, {3, 3}};
__constant__ int8_t kUpperPairs[6][2] = {{0, 1}, {0, 2}, {0, 3}, {1, 2}, {1, 3}, {2, 3}};

// 16x16 block product on the vector ALU: lane l receives rows 4*(l/16)+jj,
// column l%16 of M N (M, N in LDS with leading dimensions ldm, ldn).
__device__ __forceinline__ void blk_mm(float (&out)[4], const float* M, int ldm, const float* N,
                                       int ldn, int g, int li) {
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) out[jj] = 0.f;
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    const float nv = N[kk * ldn + li];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) out[jj] += M[(4 * g + jj) * ldm + kk] * nv;
  }
}

template <int DK>
struct Layout {
  static constexpr int LDK = DK + 4;     // padded row stride of [64][DK] tiles
  static constexpr int L64 = kC + 4;     // padded row stride of [64][64] tiles
  static constexpr int LDV = kDvs + 4;
  static constexpr int oQt = 0;                  // Qt; X = (I+A)^-1 after the A/P stage
  static constexpr int oKt = oQt + kC * LDK;     // Kt; -W after the W stage
  static constexpr int oKh = oKt + kC * LDK;     // Kh
  static constexpr int oA = oKh + kC * LDK;      // A (+P: cumsum scratch during loads)
  static constexpr int oP = oA + kC * L64;       // P
  static constexpr int oV = oP + kC * L64;       // V slice
  static constexpr int oE = oV + kC * LDV;       // [4][DK] exp(p_tile)
  static constexpr int oF = oE + 4 * DK;         // [4][DK] exp(e_tile - p_tile)
  static constexpr int oD = oF + 4 * DK;         // [6][DK] exp(p_t - p_u), u < t
  static constexpr int oGe = oD + 6 * DK;        // [DK]    exp(b_end)
  static constexpr int oBeta = oGe + DK;         // [64]    beta
  static constexpr int oF2 = oBeta + kC;         // [4][DK] exp(b_end - e_tile)
  static constexpr int total = oF2 + 4 * DK;     // floats
  static_assert(total * 4 <= 160 * 1024, "LDS budget");
  static_assert(kC * LDK <= 2 * kC * L64, "cumsum scratch must fit in the A and P tiles");
};

template <typename TI, int DK, class Pol>
__global__ void __launch_bounds__(kThreads)
    chunk_fwd_kernel(const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v,
                     const TI* __restrict__ a, const TI* __restrict__ bl,
                     const TI* __restrict__ gate, const int32_t* __restrict__ cu_seqlens,
                     const float* __restrict__ s_init, float* __restrict__ o,
                     float* __restrict__ s_final, int H, int DV, int SDV, int ckpt_iv,
                     float* __restrict__ ckpt, long long ckpt_cap) {
  using L = Layout<DK>;
  constexpr int LDK = L::LDK, L64 = L::L64, LDV = L::LDV;
  constexpr int NSEG = DK / 8;                 // 8-channel segments per row
  constexpr int IT = kC * NSEG / kThreads;     // row segments per thread
  constexpr int NCT = DK / 16;                 // 16-row state tiles
  constexpr int NKB = DK / 32;                 // 32-wide k blocks over dk

  extern __shared__ float smem[];
  float* sQt = smem + L::oQt;
  float* sX = sQt;
  float* sKt = smem + L::oKt;
  float* sW = sKt;
  float* sKh = smem + L::oKh;
  float* sA = smem + L::oA;
  float* sG = sA;
  float* sP = smem + L::oP;
  float* sV = smem + L::oV;
  float* sE = smem + L::oE;
  float* sF = smem + L::oF;
  float* sF2 = smem + L::oF2;
  float* sD = smem + L::oD;
  float* sGe = smem + L::oGe;
  float* sBeta = smem + L::oBeta;

  // State rows hold SDV columns: d_v, or d_v + d_k for the transition form,
  // whose columns [d_v, d_v + d_k) carry the transition matrix (value rows
  // zero, start state the identity; no outputs are written).
  const int nslices = SDV / kDvs;
  const int slice = blockIdx.x % nslices;
  const int item = blockIdx.x / nslices;  // sequence * H + head
  const int n = item / H, h = item % H;
  const int j0 = slice * kDvs;
  const int t = threadIdx.x, wave = t / 64, lane = t % 64, g = lane / 16, li = lane % 16;
  const int64_t tok_beg = cu_seqlens[n], tok_end = cu_seqlens[n + 1];
  const int64_t st_off = (int64_t)item * DK * SDV;
  const int jcol = j0 + 16 * wave + li;  // this lane's state / output column
  const bool tslice = j0 >= DV;          // a slice of transition columns

  // State slice in accumulator layout: S[ct] holds rows 16ct + 4g + jj, column jcol.
  f32x4_t S[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 16 * ct + 4 * g + jj;
      S[ct][jj] = tslice ? (r == jcol - DV ? 1.f : 0.f)
                  : s_init ? s_init[st_off + (int64_t)r * SDV + jcol] : 0.f;
    }

  // First recorded-state slot of this sequence (the slots of the sequences
  // before it come first).
  int64_t ck_off = 0;
  if (ckpt_iv > 0)
    for (int m = 0; m < n; ++m) ck_off += (int64_t)(cu_seqlens[m + 1] - cu_seqlens[m]) / ckpt_iv;

  for (int64_t c0 = tok_beg; c0 < tok_end; c0 += kC) {
    const int nrows = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);

    // ---- stage 1: loads, L2 norms, log-decay g, beta, V slice ------------
    float qh[IT][8], kh[IT][8];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = t + kThreads * it, row = idx / NSEG, seg = idx % NSEG;
      float qx[8], kx[8], ax[8];
      const bool valid = row < nrows;
      if (valid) {
        const int64_t off = ((c0 + row) * H + h) * (int64_t)DK + seg * 8;
        if (q) {  // the transition form reads no queries
          ld8(q + off, qx);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) qx[j] = 0.f;
        }
        ld8(k + off, kx);
        ld8(a + off, ax);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) qx[j] = kx[j] = ax[j] = 0.f;
      }
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sq += qx[j] * qx[j];
        sk += kx[j] * kx[j];
      }
      sq = group_sum<NSEG>(sq);
      sk = group_sum<NSEG>(sk);
      const float rq = rsqrtf(sq + kNormEps), rk = rsqrtf(sk + kNormEps);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        qh[it][j] = qx[j] * rq;
        kh[it][j] = kx[j] * rk;
        sG[row * LDK + seg * 8 + j] = valid ? kGMin * sigmoidf(ax[j]) : 0.f;
      }
    }
    // V slice [64][64] and beta.
#pragma unroll
    for (int it = 0; it < kC * (kDvs / 8) / kThreads; ++it) {
      const int idx = t + kThreads * it, row = idx / (kDvs / 8), seg = idx % (kDvs / 8);
      float vx[8];
      if (row < nrows && !tslice)
        ld8(v + ((c0 + row) * H + h) * (int64_t)DV + j0 + seg * 8, vx);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) vx[j] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) sV[row * LDV + seg * 8 + j] = vx[j];
    }
    if (t < kC) sBeta[t] = t < nrows ? sigmoidf(ld_elem(bl, (c0 + t) * H + h)) : 0.f;
    lds_barrier();

    // ---- stage 2: chunk-local inclusive cumsum of g per key channel --------
    {
      constexpr int NPC = kThreads / DK;  // threads per channel
      constexpr int RPT = kC / NPC;       // rows per thread
      const int c = t % DK, part = t / DK;
      float tot = 0.f;
#pragma unroll 8
      for (int r = part * RPT; r < (part + 1) * RPT; ++r) tot += sG[r * LDK + c];
      sE[part * DK + c] = tot;  // scratch, overwritten in stage 3
      lds_barrier();
      float run = 0.f;
      for (int p = 0; p < part; ++p) run += sE[p * DK + c];
#pragma unroll 8
      for (int r = part * RPT; r < (part + 1) * RPT; ++r) {
        run += sG[r * LDK + c];
        sG[r * LDK + c] = run;
      }
    }
    lds_barrier();

    // ---- stage 3: per-tile reference factors and scaled operands ----------
    if (t < DK) {
      const int c = t;
      float p[4];
      p[0] = 0.f;
#pragma unroll
      for (int tt = 1; tt < 4; ++tt) p[tt] = sG[(kTile * tt - 1) * LDK + c];
      const float be = sG[(kC - 1) * LDK + c];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        // Kend of a row of tile tt is kh exp(p - b) exp(e - p) exp(b_end - e)
        // with e the cumulative decay at the tile's last row: both tile
        // factors stay normal wherever the product is not negligible (a
        // single exp(b_end - p) would fall below fp32's normal range while
        // exp(p - b) reaches e^80)
        const float e = tt < 3 ? p[tt + 1] : be;
        sE[tt * DK + c] = fast_exp(p[tt]);
        sF[tt * DK + c] = fast_exp(e - p[tt]);
        sF2[tt * DK + c] = fast_exp(be - e);
#pragma unroll
        for (int u = 0; u < tt; ++u) sD[pair_idx(tt, u) * DK + c] = fast_exp(p[tt] - p[u]);
      }
      sGe[c] = fast_exp(be);
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = t + kThreads * it, row = idx / NSEG, seg = idx % NSEG;
      const int tt = row / kTile;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = seg * 8 + j;
        const float p = tt == 0 ? 0.f : sG[(kTile * tt - 1) * LDK + c];
        const float x = sG[row * LDK + c] - p;  // in [-80, 0]
        const float er = fast_exp(x);
        sQt[row * LDK + c] = qh[it][j] * er;
        sKt[row * LDK + c] = kh[it][j] * er;
        sKh[row * LDK + c] = kh[it][j] * fast_exp(-x);
      }
    }
    lds_barrier();

    // ---- stage 4: A, P tiles (matrix cores) and O = Qbar S ---------------
    for (int idx = t; idx < 6 * 256; idx += kThreads) {  // zero the upper tiles of P
      const int pr = idx / 256, e = idx % 256;
      sP[(16 * kUpperPairs[pr][0] + e / 16) * L64 + 16 * kUpperPairs[pr][1] + e % 16] = 0.f;
    }
    for (int job = wave; job < 20; job += 4) {
      const bool isP = job >= 10;
      const int tr = kLowerPairs[job % 10][0], ti = kLowerPairs[job % 10][1];
      const float* rows = isP ? sQt : sKt;
      const float* dvec = ti < tr ? sD + pair_idx(tr, ti) * DK : nullptr;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float av[8], bv[8];
        const int cb = 32 * kb + 8 * g;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          av[j] = rows[(16 * tr + li) * LDK + cb + j];
          const float kx = sKh[(16 * ti + li) * LDK + cb + j];
          bv[j] = dvec ? kx * dvec[cb + j] : kx;
        }
        Pol::mma(acc, av, bv);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * tr + 4 * g + jj, i = 16 * ti + li;
        if (isP)
          sP[r * L64 + i] = i <= r ? acc[jj] : 0.f;
        else
          sA[r * L64 + i] = i < r ? acc[jj] * sBeta[r] : 0.f;
      }
    }
    f32x4_t O[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      O[tt] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float av[8], bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = 32 * kb + kperm(g, j);
          av[j] = sQt[(16 * tt + li) * LDK + c] * sE[tt * DK + c];
          bv[j] = S[2 * kb + (j >> 2)][j & 3];
        }
        Pol::mma(O[tt], av, bv);
      }
    }
    lds_barrier();

    // ---- stage 5: X = (I + A)^-1, unit lower triangular, into sX ----------
    // Diagonal 16x16 blocks: lane (block l/16, column l%16) runs the 16-step
    // forward substitution for its column.  Other waves zero the upper blocks.
    if (wave == 0) {
      const int tb = g, jc = li;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = r == jc ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) s -= sA[(16 * tb + r) * L64 + 16 * tb + i] * x[i];
        x[r] = s;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sX[(16 * tb + r) * L64 + 16 * tb + jc] = x[r];
    } else {
      for (int idx = t - 64; idx < 6 * 256; idx += kThreads - 64) {
        const int pr = idx / 256, e = idx % 256;
        sX[(16 * kUpperPairs[pr][0] + e / 16) * L64 + 16 * kUpperPairs[pr][1] + e % 16] = 0.f;
      }
      // Kh is not read again before the state update: turn it into Kend in
      // place, (Kh exp(e - p)) exp(b_end - e) per row of tile tt
      for (int idx = t - 64; idx < kC * DK; idx += kThreads - 64) {
        const int row = idx / DK, c = idx % DK, tt = row / kTile;
        sKh[row * LDK + c] = sKh[row * LDK + c] * sF[tt * DK + c] * sF2[tt * DK + c];
      }
    }
    lds_barrier();
    // Off-diagonal blocks: X_st = -X_ss sum_{t<=u<s} A_su X_ut, by levels s - t = 1, 2, 3.
    // Scratch for the inner sums: the (dead) diagonal blocks of A.
#pragma unroll 1
    for (int lev = 1; lev <= 3; ++lev) {
      const int nb = 4 - lev;  // blocks at this level
      float y[4];
      if (wave < nb) {
        const int tb = wave, sb = wave + lev;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int u = tb; u < sb; ++u) {
          blk_mm(y, sA + (16 * sb) * L64 + 16 * u, L64, sX + (16 * u) * L64 + 16 * tb, L64, g, li);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[jj] += y[jj];
        }
        float* tmp = sA + (16 * wave) * L64 + 16 * wave;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) tmp[(4 * g + jj) * L64 + li] = acc[jj];
      }
      lds_barrier();
      if (wave < nb) {
        const int tb = wave, sb = wave + lev;
        blk_mm(y, sX + (16 * sb) * L64 + 16 * sb, L64, sA + (16 * wave) * L64 + 16 * wave, L64, g,
               li);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sX[(16 * sb + 4 * g + jj) * L64 + 16 * tb + li] = -y[jj];
      }
      lds_barrier();
    }

    // ---- stage 6: W = X diag(beta) Kbar (all dk columns), U0 = X diag(beta) V
    constexpr int CTW = NCT / 4;  // W column tiles per wave
    f32x4_t Wt[4][CTW];
    f32x4_t U[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      U[tt] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cw = 0; cw < CTW; ++cw) Wt[tt][cw] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && tt < 2) continue;  // X is zero there
        float av[8], bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) av[j] = sX[(16 * tt + li) * L64 + 32 * kb + 8 * g + j];
#pragma unroll
        for (int cw = 0; cw < CTW; ++cw) {
          const int c = 16 * (wave + 4 * cw) + li;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 32 * kb + 8 * g + j;
            bv[j] = sBeta[i] * sKt[i * LDK + c] * sE[(i / kTile) * DK + c];
          }
          Pol::mma(Wt[tt][cw], av, bv);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 32 * kb + 8 * g + j;
          bv[j] = sBeta[i] * sV[i * LDV + 16 * wave + li];
        }
        Pol::mma(U[tt], av, bv);
      }
    }
    lds_barrier();  // every wave is done reading Kt
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int cw = 0; cw < CTW; ++cw)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          sW[(16 * tt + 4 * g + jj) * LDK + 16 * (wave + 4 * cw) + li] = -Wt[tt][cw][jj];
    lds_barrier();

    // ---- stage 7: the state chain (per wave, registers only) -------------
    // U = U0 - W S
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float av[8], bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          av[j] = sW[(16 * tt + li) * LDK + 32 * kb + kperm(g, j)];
          bv[j] = S[2 * kb + (j >> 2)][j & 3];
        }
        Pol::mma(U[tt], av, bv);
      }
    }
    // O += P U
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && tt < 2) continue;
        float av[8], bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          av[j] = sP[(16 * tt + li) * L64 + 32 * kb + kperm(g, j)];
          bv[j] = U[2 * kb + (j >> 2)][j & 3];
        }
        Pol::mma(O[tt], av, bv);
      }
    }
    // S <- diag(Gamma_end) S + Kend^T U
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4_t acc;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[jj] = sGe[16 * ct + 4 * g + jj] * S[ct][jj];
      const int c = 16 * ct + li;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float av[8], bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 32 * kb + kperm(g, j);
          av[j] = sKh[i * LDK + c];  // Kend (formed in place in stage 5)
          bv[j] = U[2 * kb + (j >> 2)][j & 3];
        }
        Pol::mma(acc, av, bv);
      }
      S[ct] = acc;
    }
    // Record the state after the first `done` tokens when that is a multiple
    // of the recording interval.
    const int64_t done = c0 + kC - tok_beg;
    if (ckpt_iv > 0 && done % ckpt_iv == 0 && done <= tok_end - tok_beg) {
      const int64_t slot = ck_off + done / ckpt_iv - 1;
      if (slot < ckpt_cap) {
        const int64_t cp = (slot * H + h) * (int64_t)DK * DV;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            ckpt[cp + (int64_t)(16 * ct + 4 * g + jj) * DV + jcol] = S[ct][jj];
      }
    }
    // Epilogue: output gate and store.
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * tt + 4 * g + jj;
        if (o && r < nrows) {
          const int64_t off = ((c0 + r) * H + h) * (int64_t)DV + jcol;
          float y = O[tt][jj];
          if (gate) y *= sigmoidf(ld_elem(gate, off));
          o[off] = y;
        }
      }
    }
    lds_barrier();  // LDS is rewritten by the next chunk
  }

  if (s_final) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        s_final[st_off + (int64_t)(16 * ct + 4 * g + jj) * SDV + jcol] = S[ct][jj];
  }
}

template <typename TI, int DK, class Pol>
hipError_t launch_t(const FwdArgs& p, hipStream_t stream) {
  const size_t lds = sizeof(float) * Layout<DK>::total;
  auto kern = chunk_fwd_kernel<TI, DK, Pol>;
  // Dynamic LDS above the default limit: set on every call (the attribute is
  // the device's, and a process may drive several devices or threads).
  {
    const hipError_t e = hipFuncSetAttribute((const void*)kern,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const bool tr = p.transition != nullptr;
  const int sdv = tr ? p.dv + p.dk : p.dv;
  const int64_t grid = (int64_t)p.num_seqs * p.num_heads * (sdv / kDvs);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, stream, (const TI*)p.q,
                     (const TI*)p.k, (const TI*)p.v, (const TI*)p.a, (const TI*)p.b,
                     tr ? nullptr : (const TI*)p.gate, p.cu_seqlens,
                     tr ? nullptr : p.initial_state, tr ? nullptr : (float*)p.o,
                     tr ? p.transition : p.final_state, p.num_heads, p.dv, sdv,
                     tr ? 0 : p.ckpt_interval, p.ckpt, (long long)p.ckpt_capacity);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_chunked(const FwdArgs& p, hipStream_t stream) {
  if ((int64_t)p.num_seqs * p.num_heads == 0) return hipSuccess;
  if (p.in_bf16) return launch_fwd_chunked_bf16(p, stream);
  return p.dk == 128 ? launch_t<float, 128, PolicyF32>(p, stream)
                     : launch_t<float, 64, PolicyF32>(p, stream);
}

}  // namespace kda
