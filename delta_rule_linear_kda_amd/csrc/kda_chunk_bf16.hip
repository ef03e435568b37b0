// kda_chunk_bf16.hip - chunked KDA forward for bf16 inputs on gfx950 (MI355X).
//
// The KDA recurrence (page "[Paper Review] Kimi K3...", section "Kimi Delta
// Attention (KDA)") in its chunkwise-parallel form, on 32-token chunks of two
// 16-token tiles.  The log-decay is bounded below by g_min = -5 (the
// "Lower-bounded decay" paragraph), so the cumulative log-decay over a
// 16-token tile lies in [-80, 0] and every pairwise decay exp(b_r - b_i)
// splits into a row factor exp(b_r - p) <= 1 and a column factor
// exp(p - b_i) <= e^80 (p = cumulative decay before the tile): both finite in
// bf16, so every intra-chunk tile, diagonal or not, is a dense matrix-core
// product.
//
// Per chunk (rows r < 32, start state S, b = chunk-local cumsum of g, and the
// raw q, k rows with their L2 norms nq, nk applied to the products' rows and
// columns rather than to the operands):
//   A      = diag(beta nk) strict_lower(Kt Kh^T) diag(nk)    bf16
//   P      = diag(nq) lower(Qt Kh^T) diag(nk)                bf16 hi/lo split
//   X      = (I + A)^-1                                      fp32
//   W      = X diag(beta nk) Kbar                            fp16 (formed as W^T)
//   U0     = X diag(beta) V                                  bf16 hi/lo
//   U      = U0 - W S                                        fp16
//   O      = diag(nq) Qbar S + P U,   y = sigmoid(gate) O    fp16 / bf16 hi/lo
//   S     <- diag(Gamma_end) S + Kend^T diag(nk) U           fp16
// Kt = k exp(b-p), Kh = k exp(p-b) (the off-diagonal tile's column operand is
// rescaled by exp(p_1) <= 1), Qt = q exp(b-p), Qbar = q exp(b), Kbar = k exp(b),
// Kend = k exp(b_end - b).  bf16 is used wherever the e^80 column factors
// appear; the hi/lo splits (Henry, Tang & Heinecke, ARITH 2019) are where the
// 2e-2 accuracy budget needs more than one 16-bit product.  Accumulation and
// the state are fp32 throughout.
//
// Work decomposition: one workgroup per (sequence, head), software-pipelined
// over chunks with two groups of wavefronts:
//   prep waves  (DK/16)  build chunk c's operands: elementwise decay scaling,
//                        A, P, X and W, into LDS;
//   state waves (DV/16)  run chunk c-1's state chain: wave s owns state
//                        columns [16s, 16s+16) for the whole sequence in MFMA
//                        accumulator registers, and also forms the L2 norms of
//                        chunk c's q and k rows.
// The operands that cross from prep to state are double-buffered in LDS, so
// each chunk needs three workgroup barriers:
//   E  prep: elementwise            | state: norms(c), U0, U, Qbar S  (c-1)
//   AP prep: A, X (wave 0); P tiles | state: P U, state update        (c-1)
//   W  prep: W^T tiles              | state: gated output store       (c-1)
// Every barrier orders LDS only (s_waitcnt lgkmcnt(0); s_barrier), so global
// prefetches and output stores stay in flight across it.  Both groups run
// loops of identical trip count with three barriers per iteration.
//
// TRANS = true is the segment-transition form of context parallelism (page
// "[Paper Review] Kimi K3...", section "Infrastructure: how to actually run
// trillion-scale", KDA co-design item): each sequence is a segment and the
// state has d_v + d_k columns, the first d_v from a zero start with the real
// values (the segment's local state S_loc), the last d_k from the identity
// with value rows zero (U0 = 0, so each chunk applies
// diag(Gamma_end) - Kend^T W: the product is the segment's transition M).
// No queries, gate or outputs: Qt, Qbar, P, Qbar S, P U and the stores drop
// out, and the final state [S_loc | M] is the result.
#include "kda_chunk_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <int DK, int DV>
struct Cfg {
  static constexpr int NP = DK / 16;         // prep waves (16 key channels each)
  static constexpr int NS = DV / 16;         // state waves (16 state columns each)
  static constexpr int NT = 64 * (NP + NS);  // threads
  static constexpr int CPL = DK / 16;        // channels per lane in the norm mapping
  static constexpr int RPW = kC / NS;        // norm rows per state wave
  static_assert(RPW % 4 == 0, "norm rows");
  // LDS strides (elements)
  // Row strides: 16-byte operand reads from 16 rows (the prep waves' [32][DK]
  // arrays) hit distinct banks with a stride of 4 (mod 32) dwords, 8-byte
  // reads (the hand-over arrays and Kbar^T) with 2 (mod 32) dwords.
  static constexpr int LB = DK + 8;          // 16-bit [32][DK], 16-byte reads
  static constexpr int RB = DK + 4;          // 16-bit [32][DK], 8-byte reads
  static constexpr int LT = kC + 4;          // 16-bit [DK][32] and [32][32], 8-byte reads
  static constexpr int LX = kC + 4;          // fp32 [32][32]
  static constexpr int LA = 20;              // fp32 [16][16] scratch
  // byte offsets.  Wave 0's scratch for the inverse first (many accesses).
  static constexpr int oAT = 0;                             // A diag blocks^T fp32 [2][16][LA]
  static constexpr int oA10 = oAT + 2 * 16 * LA * 4;        // A10 fp32 [16][LA]
  // double-buffered operands handed from prep (chunk c) to state (read at c+1)
  static constexpr int dX = 0;                              // X fp32 [32][LX]
  static constexpr int dPH = dX + kC * LX * 4;              // P hi bf16 [32][LT]
  static constexpr int dPL = dPH + kC * LT * 2;             // P lo bf16 [32][LT]
  static constexpr int dGE = dPL + kC * LT * 2;             // Gamma_end fp32 [DK]
  static constexpr int dBeta = dGE + DK * 4;                // beta fp32 [32]
  static constexpr int dNQ = dBeta + kC * 4;                // 1/|q| fp32 [32]
  static constexpr int dNK = dNQ + kC * 4;                  // 1/|k| fp32 [32]
  static constexpr int dQB = dNK + kC * 4;                  // Qbar fp16 [32][RB]
  static constexpr int dW = dQB + kC * RB * 2;              // -W fp16 [32][RB]
  static constexpr int dKE = dW + kC * RB * 2;              // Kend^T fp16 [DK][LT]
  static constexpr int dSize = dKE + DK * LT * 2;
  static constexpr int oBuf = oA10 + 16 * LA * 4;           // two copies
  // prep-only scratch (written and read within one chunk)
  static constexpr int oKT = oBuf + 2 * dSize;              // Kt bf16 [32][LB]
  static constexpr int oQH = oKT + kC * LB * 2;             // Qt hi
  static constexpr int oQL = oQH + kC * LB * 2;             // Qt lo
  static constexpr int oKHH = oQL + kC * LB * 2;            // Kh hi
  static constexpr int oKHL = oKHH + kC * LB * 2;           // Kh lo
  static constexpr int oK1H = oKHL + kC * LB * 2;           // Kh exp(p_1) hi, rows 0-15
  static constexpr int oK1L = oK1H + 16 * LB * 2;           // Kh exp(p_1) lo
  static constexpr int oKBT = oK1L + 16 * LB * 2;           // Kbar^T fp16 [DK][LT]
  static constexpr int bytes = oKBT + DK * LT * 2;
  static_assert(dSize % 16 == 0 && oBuf % 16 == 0, "alignment");
  static_assert(bytes <= 160 * 1024, "LDS budget");
};

template <int DK, int DV, bool TRANS>
__global__ void __launch_bounds__(64 * (DK / 16 + DV / 16))
    chunk_fwd_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                          const uint16_t* __restrict__ v, const uint16_t* __restrict__ a,
                          const uint16_t* __restrict__ bl, const uint16_t* __restrict__ gate,
                          const int32_t* __restrict__ cu_seqlens, const float* __restrict__ s_init,
                          float* __restrict__ o, float* __restrict__ s_final, int H,
                          int num_items, int dvt, int nsl, int ckpt_iv, float* __restrict__ ckpt,
                          long long ckpt_cap) {
  using L = Cfg<DK, DV>;
  constexpr int NP = L::NP, CPL = L::CPL, RPW = L::RPW;
  constexpr int LB = L::LB, RB = L::RB, LT = L::LT, LX = L::LX, LA = L::LA;
  constexpr int NCT = DK / 16, NKB = DK / 32;

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::bytes];
  float* sAT = reinterpret_cast<float*>(smem + L::oAT);
  float* sA10 = reinterpret_cast<float*>(smem + L::oA10);
  uint16_t* sKT = reinterpret_cast<uint16_t*>(smem + L::oKT);
  uint16_t* sQH = reinterpret_cast<uint16_t*>(smem + L::oQH);
  uint16_t* sQL = reinterpret_cast<uint16_t*>(smem + L::oQL);
  uint16_t* sKHH = reinterpret_cast<uint16_t*>(smem + L::oKHH);
  uint16_t* sKHL = reinterpret_cast<uint16_t*>(smem + L::oKHL);
  uint16_t* sK1H = reinterpret_cast<uint16_t*>(smem + L::oK1H);
  uint16_t* sK1L = reinterpret_cast<uint16_t*>(smem + L::oK1L);
  uint16_t* sKBT = reinterpret_cast<uint16_t*>(smem + L::oKBT);
  // double-buffered views; chunk c uses buffer c & 1
  auto buf = [&](int p, int off) { return smem + L::oBuf + p * L::dSize + off; };
  auto bX = [&](int p) { return reinterpret_cast<float*>(buf(p, L::dX)); };
  auto bPH = [&](int p) { return reinterpret_cast<uint16_t*>(buf(p, L::dPH)); };
  auto bPL = [&](int p) { return reinterpret_cast<uint16_t*>(buf(p, L::dPL)); };
  auto bGE = [&](int p) { return reinterpret_cast<float*>(buf(p, L::dGE)); };
  auto bBeta = [&](int p) { return reinterpret_cast<float*>(buf(p, L::dBeta)); };
  auto bNQ = [&](int p) { return reinterpret_cast<float*>(buf(p, L::dNQ)); };
  auto bNK = [&](int p) { return reinterpret_cast<float*>(buf(p, L::dNK)); };
  auto bQB = [&](int p) { return reinterpret_cast<uint16_t*>(buf(p, L::dQB)); };
  auto bW = [&](int p) { return reinterpret_cast<uint16_t*>(buf(p, L::dW)); };
  auto bKE = [&](int p) { return reinterpret_cast<uint16_t*>(buf(p, L::dKE)); };

  // Block -> (item = sequence * H + head, d_v slice): the nsl slices of an item
  // sit 8 blocks apart, on the same XCD (blocks go round-robin over the 8
  // XCDs), so the second slice's q, k, a reads hit that XCD's L2.
  const int blk = blockIdx.x;
  const int item = (blk / (8 * nsl)) * 8 + blk % 8;
  const int col0 = ((blk / 8) % nsl) * DV;  // first state / v column of this slice
  if (item >= num_items) return;            // whole workgroup; before any barrier
  const int h = item % H;
  // Sequences longest first: workgroups start in block order, so the item
  // ranks go to the sequences in decreasing length (ties by index), which
  // shortens the tail of a batch of unequal lengths (longest-processing-time
  // list scheduling).  With more than 256 sequences (a ranking loop of that
  // length per workgroup, and tails short against the batch), in index order.
  int n = item / H;
  {
    const int N = num_items / H;
    if (N > 1 && N <= 256) {  // uniform over the workgroup
      int* sl = reinterpret_cast<int*>(smem);  // lengths [N], then the answer
      const int t = threadIdx.x;
      if (t < N) sl[t] = cu_seqlens[t + 1] - cu_seqlens[t];
      __syncthreads();
      if (t < N) {
        const int lt = sl[t];
        int rank = 0;
        for (int m = 0; m < N; ++m) {
          const int lm = sl[m];
          rank += (lm > lt || (lm == lt && m < t)) ? 1 : 0;
        }
        if (rank == n) sl[L::NT] = t;
      }
      __syncthreads();
      n = sl[L::NT];
      __syncthreads();  // the LDS is the kernel's own from here on
    }
  }
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
  const int64_t tok_beg = cu_seqlens[n], tok_end = cu_seqlens[n + 1];
  const int nch = (int)((tok_end - tok_beg + kC - 1) / kC);

  if (wave < NP) {
    // ======================= prep waves =======================================
    // Lane (li, g): rows li (tile 0) and 16 + li (tile 1), key channels
    // 16 * wave + 4g .. +3.  The tokens of a tile run along the 16 lanes of a
    // DPP row.
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
      // finite); they get g = 0 and beta = 0 below, which removes every
      // contribution they could make, and their outputs are never stored.
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int r = 16 * tau + li;
        const int rr = r < nr ? r : nr - 1;
        const uint32_t off = (uint32_t)(rr * H * DK) + 16 * wave + 4 * g;
        if constexpr (!TRANS) rq[tau] = *gat<const u32x2_t>(qb_, off);
        rk[tau] = *gat<const u32x2_t>(kb_, off);
        ra[tau] = *gat<const u32x2_t>(ab_, off);
        rb[tau] = *gat<const uint16_t>(bb_, (uint32_t)(rr * H));
      }
    };
    if (nch > 0) {
      const int lane = threadIdx.x % 64;
      load(tok_beg, lane % 16, lane / 16);
    }

    // Both wave groups skip the loop together when the sequence is empty.
    for (int it = 0; nch > 0 && it <= nch; ++it) {
      const int64_t c0 = tok_beg + (int64_t)kC * it;
      const bool act = it < nch;
      const int p = it & 1;
      // Lane indices re-derived from an opaque copy each chunk (keeps the
      // optimiser from hoisting every lane-dependent address out of the loop).
      int t_ = threadIdx.x;
      __asm__ volatile("" : "+v"(t_));
      const int lane = t_ % 64, li = lane % 16, g = lane / 16;

      // ---- E: elementwise --------------------------------------------------
      if (act) {
        const int nrows = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
        float qf[2][4], kf[2][4], cum[2][4];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          if constexpr (!TRANS) {
            qf[tau][0] = bf16lo(rq[tau][0]); qf[tau][1] = bf16hi(rq[tau][0]);
            qf[tau][2] = bf16lo(rq[tau][1]); qf[tau][3] = bf16hi(rq[tau][1]);
          }
          kf[tau][0] = bf16lo(rk[tau][0]); kf[tau][1] = bf16hi(rk[tau][0]);
          kf[tau][2] = bf16lo(rk[tau][1]); kf[tau][3] = bf16hi(rk[tau][1]);
          const float av[4] = {bf16lo(ra[tau][0]), bf16hi(ra[tau][0]), bf16lo(ra[tau][1]),
                               bf16hi(ra[tau][1])};
#pragma unroll
          for (int j = 0; j < 4; ++j)  // g in log2 units: -5 log2(e) sigmoid(a)
            cum[tau][j] = log2_decay(av[j]);
        }
        float beta[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
          beta[tau] = rcpf_fast(1.f + exp2f_fast(-kLog2e * __uint_as_float((uint32_t)rb[tau] << 16)));
        if (nrows < kC) {  // padding rows: g = 0, beta = 0
#pragma unroll
          for (int tau = 0; tau < 2; ++tau) {
            const bool valid = 16 * tau + li < nrows;
#pragma unroll
            for (int j = 0; j < 4; ++j) cum[tau][j] = valid ? cum[tau][j] : 0.f;
            beta[tau] = valid ? beta[tau] : 0.f;
          }
        }
        // decay accumulated within each tile (inclusive; the eight scans are
        // interleaved step by step), and the tile totals
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
          e0[j] = exp2f_fast(tot[0][j]);    // exp(p_1): decay over tile 0
          fend[1][j] = exp2f_fast(tot[1][j]);  // exp(b_end - p_1)
          fend[0][j] = e0[j] * fend[1][j];     // exp(b_end - p_0) = Gamma_end
        }
        if (li == 0)
          *reinterpret_cast<float4*>(bGE(p) + cb) =
              make_float4(fend[0][0], fend[0][1], fend[0][2], fend[0][3]);
        if (wave == 0 && g == 0) {
          bBeta(p)[li] = beta[0];
          bBeta(p)[16 + li] = beta[1];
        }
        uint16_t* qbp = bQB(p);
        uint16_t* kbt = sKBT + cb * LT + li;  // [channel cb + j][token 16 tau + li]
        uint16_t* ket = bKE(p) + cb * LT + li;
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          const int r = 16 * tau + li;
          bf16x4_t ktb, qhb, qlb, khh, khl, k1h, k1l;
          f16x4_t qbf;
          float qt4[4], kt4[4], kh4[4], y4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = cum[tau][j];  // log2(e) (b - p) <= 0
            const float er = exp2f_fast(x), ir = exp2f_fast(-x);
            const float kt = kf[tau][j] * er, kh = kf[tau][j] * ir;
            if constexpr (!TRANS) {
              const float qt = qf[tau][j] * er;
              const float qbar = tau ? qt * e0[j] : qt;
              qt4[j] = qt;
              qbf[j] = (_Float16)qbar;
            }
            const float kbar = tau ? kt * e0[j] : kt;
            // tile 0's rows: (kh exp(p_1)) exp(b_end - p_1), both factors
            // normal wherever the product is not negligible
            const float kend = tau ? kh * fend[1][j] : (kh * e0[j]) * fend[1][j];
            kt4[j] = kt;
            kh4[j] = kh;
            kbt[j * LT + 16 * tau] = f16_bits(kbar);
            ket[j * LT + 16 * tau] = f16_bits(kend);
            // column operand of the off-diagonal tile (tile 0): Kh exp(p_1) <= 1
            y4[j] = kh * e0[j];
          }
          if constexpr (!TRANS) split_bf16x4(qt4, qhb, qlb);
          ktb = pack_bf16x4(kt4);
          split_bf16x4(kh4, khh, khl);
          if (tau == 0) split_bf16x4(y4, k1h, k1l);
          *reinterpret_cast<bf16x4_t*>(sKT + r * LB + cb) = ktb;
          *reinterpret_cast<bf16x4_t*>(sKHH + r * LB + cb) = khh;
          *reinterpret_cast<bf16x4_t*>(sKHL + r * LB + cb) = khl;
          if constexpr (!TRANS) {
            *reinterpret_cast<bf16x4_t*>(sQH + r * LB + cb) = qhb;
            *reinterpret_cast<bf16x4_t*>(sQL + r * LB + cb) = qlb;
            *reinterpret_cast<f16x4_t*>(qbp + r * RB + cb) = qbf;
          }
          if (tau == 0) {
            *reinterpret_cast<bf16x4_t*>(sK1H + li * LB + cb) = k1h;
            *reinterpret_cast<bf16x4_t*>(sK1L + li * LB + cb) = k1l;
          }
        }
        // Next chunk's inputs, consumed in its E stage.  Requested last, when
        // this chunk's raw registers are dead, and unconditionally (the last
        // chunk re-reads itself), so the loads land directly in the registers
        // carried to the next iteration and nothing here waits for them.
        load(it + 1 < nch ? c0 + kC : c0, li, g);
      }
      lds_barrier();  // B1: operands, beta (prep) and norms (state) in LDS

      // ---- AP: A and X (wave 0) | P tiles ------------------------------------
      if (act) {
        const float* nk = bNK(p);
        const float* nq = bNQ(p);
        const float* be = bBeta(p);
        // Row scale beta_r nk_r and column scale nk_i of the A tiles.
        auto a_tile = [&](int tr, int ti, const uint16_t* col) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            const int c = 32 * kb + 8 * g;
            acc = mma_bf16(lds8<bf16x8_t>(sKT + (16 * tr + li) * LB + c), lds8<bf16x8_t>(col + c),
                           acc);
          }
          const float nkc = nk[16 * ti + li];
          const float4 nkr = *reinterpret_cast<const float4*>(nk + 16 * tr + 4 * g);
          const float4 ber = *reinterpret_cast<const float4*>(be + 16 * tr + 4 * g);
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
            const int c = 32 * kb + 8 * g;
            acc = mma_x3(lds8<bf16x8_t>(sQH + (16 * tr + li) * LB + c),
                         lds8<bf16x8_t>(sQL + (16 * tr + li) * LB + c),
                         lds8<bf16x8_t>(colh + c), lds8<bf16x8_t>(coll + c), acc);
          }
          uint16_t* ph = bPH(p);
          uint16_t* pl = bPL(p);
          const float nki = nk[16 * ti + li];
          const float4 nqr = *reinterpret_cast<const float4*>(nq + 16 * tr + 4 * g);
          const float nqv[4] = {nqr.x, nqr.y, nqr.z, nqr.w};
          float pv[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * tr + 4 * g + jj, i = 16 * ti + li;
            pv[jj] = i <= r ? acc[jj] * nqv[jj] * nki : 0.f;
          }
          uint32_t hw[2], lw[2];
          split_pk_bf16(pv[0], pv[1], hw[0], lw[0]);
          split_pk_bf16(pv[2], pv[3], hw[1], lw[1]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * tr + 4 * g + jj, i = 16 * ti + li;
            ph[r * LT + i] = (uint16_t)(hw[jj / 2] >> (16 * (jj % 2)));
            pl[r * LT + i] = (uint16_t)(lw[jj / 2] >> (16 * (jj % 2)));
          }
          if (job == 0) {  // the upper tile (0, 1) of P is zero
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              ph[(4 * g + jj) * LT + 16 + li] = 0;
              pl[(4 * g + jj) * LT + 16 + li] = 0;
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
          // broadcast within each quad of lanes.  A[r][m] = 0 for r <= m, so
          // no row needs masking.
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
          float* xb = bX(p);
#pragma unroll
          for (int i = 0; i < 4; ++i) xb[(16 * tau + 4 * qd + i) * LX + 16 * tau + jc] = x[i];
        } else {
          if (wave == 2) {  // A10, kept row-major for the W stage
            const f32x4_t acc = a_tile(1, 0, sK1H + li * LB);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sA10[(4 * g + jj) * LA + li] = acc[jj];
          }
          if constexpr (TRANS) {
            // no outputs: P is not needed
          } else if constexpr (NP >= 6) {
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
      lds_barrier();  // B2: X and P in LDS

      // ---- W: X10 = -X11 A10 X00; W^T = Kbar^T diag(beta nk) X^T; store -W ----
      if (act) {
        float* xb = bX(p);
        const float* be = bBeta(p);
        const float* nk = bNK(p);
        // X10^T = -X00^T (A10^T X11^T) on the fp32 matrix cores (every prep
        // wave forms it for its own W tiles); lane (li, g) ends with
        // X10[li][4g + jj] in x10[jj].
        f32x4_t p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          p1 = mma_f32(sA10[(4 * s + g) * LA + li], xb[(16 + li) * LX + 16 + 4 * s + g], p1);
        f32x4_t x10 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) x10 = mma_f32(xb[(4 * g + s) * LX + li], p1[s], x10);
        x10 = -x10;
        if (wave == 0) {  // complete X for the state waves: X10, and X01 = 0
          *reinterpret_cast<float4*>(xb + (16 + li) * LX + 4 * g) =
              make_float4(x10[0], x10[1], x10[2], x10[3]);
          *reinterpret_cast<float4*>(xb + li * LX + 16 + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        // beta nk at the tokens of slots j (k order 4g..4g+3, 16+4g..16+4g+3)
        float bs[8];
        {
          const float4 b0 = *reinterpret_cast<const float4*>(be + 4 * g);
          const float4 b1 = *reinterpret_cast<const float4*>(be + 16 + 4 * g);
          const float4 n0 = *reinterpret_cast<const float4*>(nk + 4 * g);
          const float4 n1 = *reinterpret_cast<const float4*>(nk + 16 + 4 * g);
          bs[0] = b0.x * n0.x; bs[1] = b0.y * n0.y; bs[2] = b0.z * n0.z; bs[3] = b0.w * n0.w;
          bs[4] = b1.x * n1.x; bs[5] = b1.y * n1.y; bs[6] = b1.z * n1.z; bs[7] = b1.w * n1.w;
        }
        const f16x8_t kbt = lds4x2<f16x8_t>(sKBT + (16 * wave + li) * LT + 4 * g);
        uint16_t* wp = bW(p);
        float xx[2][8];
        {
          const float4 x00 = *reinterpret_cast<const float4*>(xb + li * LX + 4 * g);
          const float4 x11 = *reinterpret_cast<const float4*>(xb + (16 + li) * LX + 16 + 4 * g);
          xx[0][0] = x00.x; xx[0][1] = x00.y; xx[0][2] = x00.z; xx[0][3] = x00.w;
          xx[0][4] = xx[0][5] = xx[0][6] = xx[0][7] = 0.f;
          xx[1][0] = x10[0]; xx[1][1] = x10[1]; xx[1][2] = x10[2]; xx[1][3] = x10[3];
          xx[1][4] = x11.x; xx[1][5] = x11.y; xx[1][6] = x11.z; xx[1][7] = x11.w;
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
          for (int j = 0; j < 8; ++j) xx[rt][j] *= bs[j];
          const f32x4_t acc = mma_f16(kbt, pack_f16x8(xx[rt]), f32x4_t{0.f, 0.f, 0.f, 0.f});
          // acc[jj] = W[16 rt + li][16 wave + 4 g + jj]
          const f16x4_t wv = {(_Float16)(-acc[0]), (_Float16)(-acc[1]), (_Float16)(-acc[2]),
                              (_Float16)(-acc[3])};
          *reinterpret_cast<f16x4_t*>(wp + (16 * rt + li) * RB + 16 * wave + 4 * g) = wv;
        }
      }
      lds_barrier();  // B3: W in LDS; scratch free for the next chunk
    }
  } else {
    // ======================= state waves ======================================
    const int sw = wave - NP;  // owns state columns [16 sw, 16 sw + 16)
    // State row length: d_v, or d_v + d_k for the transition form, whose
    // columns [d_v, d_v + d_k) carry the transition matrix (value rows zero).
    const int sdv = TRANS ? dvt + DK : dvt;
    const bool tslice = TRANS && col0 >= dvt;  // a slice of transition columns
    const int64_t st_off = ((int64_t)n * H + h) * DK * sdv + col0;
    // First recorded-state slot of this sequence: the slots of the sequences
    // before it come first.
    int64_t ck_off = 0;
    if (ckpt_iv > 0)
      for (int m = 0; m < n; ++m) ck_off += (int64_t)(cu_seqlens[m + 1] - cu_seqlens[m]) / ckpt_iv;
    f32x4_t S[NCT];
    {
      const int lane = threadIdx.x % 64, g = lane / 16, li = lane % 16;
      const uint32_t st_lane = 4 * g * sdv + 16 * sw + li;  // state element (row 4g, column)
      if (tslice) {  // transition columns start from the identity
        const int mc = col0 - dvt + 16 * sw + li;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) S[ct][jj] = 16 * ct + 4 * g + jj == mc ? 1.f : 0.f;
      } else if (s_init && !TRANS) {
        const auto sp = sbase(s_init + st_off);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) S[ct][jj] = *gat<const float>(sp, st_lane + (16 * ct + jj) * dvt);
      } else {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) S[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    // this wave's state columns are held as S 2^(esc - 127) (fp16 range of the
    // state-chain operands)
    int esc = 127;
    typedef __attribute__((ext_vector_type(CPL / 2))) uint32_t uvec_t;
    constexpr int NPASS = RPW / 4;
    uvec_t nq_[NPASS], nk_[NPASS];  // q, k rows for the norms of the next chunk
    uint32_t rv[8];                 // v of the chunk the chain works on (word with the bf16)
    uint32_t rgr[8];                // gate of that chunk (word with the bf16)
    f32x4_t O[2], U[2];
    auto load_qk = [&](int64_t c0, int g, int li) {
      const int nr = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
      const int64_t tb = c0 * H + h;
      const auto qb_ = sbase(q + tb * DK);
      const auto kb_ = sbase(k + tb * DK);
#pragma unroll
      for (int ps = 0; ps < NPASS; ++ps) {
        const int r = RPW * sw + 4 * ps + g;
        const int rr = r < nr ? r : nr - 1;
        const uint32_t off = (uint32_t)(rr * H * DK) + CPL * li;
        if constexpr (!TRANS) nq_[ps] = *gat<const uvec_t>(qb_, off);
        nk_[ps] = *gat<const uvec_t>(kb_, off);
      }
    };
    // v and gate arrive as the aligned 32-bit word holding the lane's bf16
    // element (the lane pair (jcol & ~1, jcol | 1) shares it); the half is
    // picked at use.  Whole-register loads keep the loop-carried registers
    // free of zero-extension masks, which would have to wait for the loads.
    auto load_v = [&](int64_t c0, int g, int jcol) {
      const int nr = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
      const auto vb_ = sbase(reinterpret_cast<const uint32_t*>(v + (c0 * H + h) * dvt + col0));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 16 * (i / 4) + 4 * g + (i % 4);
        const int rr = r < nr ? r : nr - 1;
        rv[i] = *gat<const uint32_t>(vb_, (uint32_t)(rr * H * dvt + (jcol & ~1)) / 2);
      }
    };
    auto load_g = [&](int64_t c0, int g, int jcol) {
      const int nr = (int)(tok_end - c0 < kC ? tok_end - c0 : kC);
      // Without a gate the same rows of v are read (and ignored), so the
      // number of requests in flight never depends on the gate.
      const auto gb_ = sbase(
          reinterpret_cast<const uint32_t*>((gate ? gate : v) + (c0 * H + h) * dvt + col0));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 16 * (i / 4) + 4 * g + (i % 4);
        const int rr = r < nr ? r : nr - 1;
        rgr[i] = *gat<const uint32_t>(gb_, (uint32_t)(rr * H * dvt + (jcol & ~1)) / 2);
      }
    };
    // Gated output of chunk c (its O accumulators), stored fp32 through a
    // buffer resource whose range ends after the chunk's last valid row: all
    // eight stores always issue, on every iteration (so the in-order count of
    // outstanding memory operations is the same on every path and the waits
    // that follow never have to cover them), and the hardware drops the
    // padding rows of a partial chunk, or every row when there is no chunk to
    // store yet (nrows = 0, first iteration).
    auto epilogue = [&](int64_t c0, int nrows, int g, int jcol) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          o + (c0 * H + h) * dvt + col0, 0, nrows * H * dvt * 4, kBufferRsrcFlags);
      const uint32_t vo_lane = (4 * g) * H * dvt + jcol;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float y = O[j >> 2][j & 3] * pow2f(254 - esc);
        if (gate)  // sigmoid(gate) of the chunk, from its loaded words
          y *= rcpf_fast(
              1.f + exp2f_fast(-kLog2e * __uint_as_float((rgr[j] >> (16u * (jcol & 1))) << 16)));
        __builtin_amdgcn_raw_buffer_store_b32(
            __float_as_uint(y), rs, 4 * (vo_lane + (uint32_t)((16 * (j >> 2) + (j & 3)) * H * dvt)),
            0, 0);
      }
    };
    if (nch > 0) {  // q, k rows of chunk 0 for its norms
      const int lane = threadIdx.x % 64;
      load_qk(tok_beg, lane / 16, lane % 16);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) rv[j] = rgr[j] = 0u;  // first read before their first load
    // Let the initial state and chunk 0's rows arrive before the loop: the
    // memory counter completes in order, so a load still pending on entry
    // would make the compiler's loop-invariant waits count the loop's own
    // output stores as well (every iteration would wait for them).
    __builtin_amdgcn_s_waitcnt(0);
    // Iteration it: the chain works on chunk c = it - 1.
    for (int it = 0; nch > 0 && it <= nch; ++it) {
      const bool act = it >= 1;
      const int p = (it - 1) & 1;
      int t_ = threadIdx.x;
      __asm__ volatile("" : "+v"(t_));
      const int lane = t_ % 64, g = lane / 16, li = lane % 16;
      const int jcol = 16 * sw + li;
      const uint32_t hsh = 16u * (li & 1);  // which half of a loaded word is this lane's

      auto s_f16 = [&](int kb) {
        f16x8_t r;
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = (_Float16)S[2 * kb + (j >> 2)][j & 3];
        return r;
      };

      // ---- E: norms of chunk it; U0, U = U0 - W S, O = Qbar S
      // The consumers of the registers loaded in the previous W stage run on
      // every iteration (at it = 0 the gate words are unused, at it = nch the
      // norms of the clamped chunk go to the LDS buffer no one reads then), so
      // every path waits for those loads at the same place and no later
      // reuse of their registers needs a drain of the memory counter, which
      // would also wait for the output stores.
      {
        float* nqo = bNQ(it & 1);
        float* nko = bNK(it & 1);
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
          float sq = 0.f, sk = 0.f;
#pragma unroll
          for (int e = 0; e < CPL / 2; ++e) {
            if constexpr (!TRANS) sq = sq2_bf16(nq_[ps][e], sq);
            sk = sq2_bf16(nk_[ps][e], sk);
          }
          if constexpr (!TRANS) sq = row_sum16(sq);
          sk = row_sum16(sk);
          if (li == 0) {
            const int r = RPW * sw + 4 * ps + g;
            if constexpr (!TRANS) nqo[r] = rsqrtf(sq + kNormEps);
            nko[r] = rsqrtf(sk + kNormEps);
          }
        }
      }
      if (act) {
        // the state columns' range for this chunk's fp16 operands
        rescale_state(S, esc);
        const float* xb = bX(p);
        const float* be = bBeta(p);
        if (tslice) {  // no value rows: U0 = 0
          U[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          U[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        } else {
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
          const float sc = pow2f(esc);  // U0 on the state columns' scale
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) U[rt][jj] *= sc;
        }
        const uint16_t* wp = bW(p);
        const uint16_t* qbp = bQB(p);
        O[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        O[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const f16x8_t sbk = s_f16(kb);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            U[rt] = mma_f16(lds4x2<f16x8_t>(wp + (16 * rt + li) * RB + 32 * kb + 4 * g), sbk, U[rt]);
            if constexpr (!TRANS)
              O[rt] = mma_f16(lds4x2<f16x8_t>(qbp + (16 * rt + li) * RB + 32 * kb + 4 * g), sbk,
                              O[rt]);
          }
        }
        if constexpr (!TRANS) {
          const float* nq = bNQ(p);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            const float4 nr = *reinterpret_cast<const float4*>(nq + 16 * rt + 4 * g);
            O[rt][0] *= nr.x; O[rt][1] *= nr.y; O[rt][2] *= nr.z; O[rt][3] *= nr.w;
          }
        }
      }
      lds_barrier();  // B1

      // ---- AP: O += P U; S <- diag(Gamma_end) S + Kend^T diag(nk) U -------------
      if (act) {
        const float* nk = bNK(p);
        f16x8_t uf, ufl;  // diag(nk) U as fp16 hi + lo for Kend^T U
        float uinv;
        bool ubig;
        {
          float uu[8], us[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) uu[j] = U[j >> 2][j & 3];
          if constexpr (!TRANS) {  // O += P U first (U as bf16 hi + lo)
            bf16x8_t uh, ul;
            split_bf16x8(uu, uh, ul);
            const uint16_t* ph = bPH(p);
            const uint16_t* pl = bPL(p);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
              const int off = (16 * rt + li) * LT + 4 * g;
              O[rt] = mma_x3(lds4x2<bf16x8_t>(ph + off), lds4x2<bf16x8_t>(pl + off), uh, ul, O[rt]);
            }
          }
          const float4 n0 = *reinterpret_cast<const float4*>(nk + 4 * g);
          const float4 n1 = *reinterpret_cast<const float4*>(nk + 16 + 4 * g);
          us[0] = uu[0] * n0.x; us[1] = uu[1] * n0.y; us[2] = uu[2] * n0.z; us[3] = uu[3] * n0.w;
          us[4] = uu[4] * n1.x; us[5] = uu[5] * n1.y; us[6] = uu[6] * n1.z; us[7] = uu[7] * n1.w;
          // the fp16 copy of diag(nk) U: its column's range (rare: a factor f)
          uinv = u_range(us, ubig);
          split_f16x8(us, uf, ufl);
        }
        const float* ge = bGE(p);
        const uint16_t* kep = bKE(p);
        // S <- 1/f (f diag(Gamma_end) S + Kend^T (f diag(nk) U)); f = 1 but on
        // the rare path
        const bool ub = ubig;
        if (ub) {
          const float f = pow2f(254 - bexp(uinv));
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) S[ct][jj] *= f;
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const float4 gv = *reinterpret_cast<const float4*>(ge + 16 * ct + 4 * g);
          f32x4_t acc;
          acc[0] = gv.x * S[ct][0]; acc[1] = gv.y * S[ct][1];
          acc[2] = gv.z * S[ct][2]; acc[3] = gv.w * S[ct][3];
          const f16x8_t ke = lds4x2<f16x8_t>(kep + (16 * ct + li) * LT + 4 * g);
          S[ct] = mma_f16(ke, uf, mma_f16(ke, ufl, acc));
        }
        if (ub) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) S[ct][jj] *= uinv;
        }
        // Record the state after the first `done` tokens when that is a
        // multiple of the recording interval.
        const int64_t done = (int64_t)kC * it;
        if (!TRANS && ckpt_iv > 0 && done % ckpt_iv == 0 && done <= tok_end - tok_beg) {
          const int64_t slot = ck_off + done / ckpt_iv - 1;
          if (slot < ckpt_cap) {
            const uint32_t st_lane = 4 * g * dvt + 16 * sw + li;
            const auto sp = sbase(ckpt + (slot * H + h) * DK * dvt + col0);
            const float isc = pow2f(254 - esc);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) *gat<float>(sp, st_lane + (16 * ct + jj) * dvt) = S[ct][jj] * isc;
          }
        }
      }
      lds_barrier();  // B2

      // ---- W: chunk c's gated output, then the requests for the next iteration
      // The stores issue first and the loads last, so no instruction after a
      // load can touch its destination registers (which would make it wait
      // for the load, and, the memory counter being in order, for everything
      // before it).  The requests are unconditional (chunk index clamped to
      // the last chunk), so they land directly in the carried registers; the
      // next stage's waits for them also cover these stores, issued just
      // before and no slower to complete.
      if constexpr (!TRANS) {
        const int64_t c_out = tok_beg + (int64_t)kC * (act ? it - 1 : 0);
        const int n_out = act ? (int)(tok_end - c_out < kC ? tok_end - c_out : kC) : 0;
        epilogue(c_out, n_out, g, jcol);
      }
      {
        const int64_t c_this = tok_beg + (int64_t)kC * (it < nch ? it : nch - 1);
        const int64_t c_next = tok_beg + (int64_t)kC * (it + 1 < nch ? it + 1 : nch - 1);
        if constexpr (!TRANS) load_g(c_this, g, jcol);  // chunk it's gate and v, for it+1
        if (!tslice) load_v(c_this, g, jcol);
        load_qk(c_next, g, li);  // norms at it+1
      }
      lds_barrier();  // B3
    }

    if (s_final) {
      const int lane = threadIdx.x % 64, g = lane / 16, li = lane % 16;
      const uint32_t st_lane = 4 * g * sdv + 16 * sw + li;
      const auto sp = sbase(s_final + st_off);
      const float isc = pow2f(254 - esc);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) *gat<float>(sp, st_lane + (16 * ct + jj) * sdv) = S[ct][jj] * isc;
    }
  }
}

template <int DK, int DV, bool TRANS>
hipError_t launch_cfg(const FwdArgs& p, int nsl, hipStream_t stream) {
  auto kern = chunk_fwd_bf16_kernel<DK, DV, TRANS>;  // LDS is static (Cfg<DK, DV>::bytes)
  const int64_t items = (int64_t)p.num_seqs * p.num_heads;
  const int64_t grid = (items + 7) / 8 * 8 * nsl;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg<DK, DV>::NT), 0, stream,
                     (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.v,
                     (const uint16_t*)p.a, (const uint16_t*)p.b,
                     TRANS ? nullptr : (const uint16_t*)p.gate, p.cu_seqlens,
                     TRANS ? nullptr : p.initial_state, TRANS ? nullptr : (float*)p.o,
                     TRANS ? p.transition : p.final_state, p.num_heads, (int)items, p.dv, nsl,
                     TRANS ? 0 : p.ckpt_interval, p.ckpt, (long long)p.ckpt_capacity);
  return hipGetLastError();
}

}  // namespace

// One workgroup per (sequence, head) when that fills the GPU; with fewer
// items than half the compute units, d_v = 128 is split into two 64-column
// slices per item (the key-side work is repeated, the state work halves),
// unless the caller asks for whole items.
//
// The transition form has state rows of d_v + d_k columns: 64-column slices
// while they fit the GPU in one round, otherwise (d_k = d_v = 128) two
// 128-column slices per item.
hipError_t launch_fwd_chunked_bf16(const FwdArgs& p, hipStream_t stream) {
  const int64_t items = (int64_t)p.num_seqs * p.num_heads;
  if (items == 0) return hipSuccess;
  if (p.transition) {
    const int nsl64 = (p.dv + p.dk) / 64;
    if (p.dk == 128) {
      if (p.dv == 128 && nsl64 * items > device_cus()) return launch_cfg<128, 128, true>(p, 2, stream);
      return launch_cfg<128, 64, true>(p, nsl64, stream);
    }
    return launch_cfg<64, 64, true>(p, nsl64, stream);
  }
  const bool split = !p.whole_items && p.dv == 128 && 2 * items <= device_cus();
  if (p.dk == 128) {
    if (p.dv == 128 && !split) return launch_cfg<128, 128, false>(p, 1, stream);
    return launch_cfg<128, 64, false>(p, p.dv / 64, stream);
  }
  if (p.dv == 128 && !split) return launch_cfg<64, 128, false>(p, 1, stream);
  return launch_cfg<64, 64, false>(p, p.dv / 64, stream);
}

}  // namespace kda
