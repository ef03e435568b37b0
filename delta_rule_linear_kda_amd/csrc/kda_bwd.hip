// kda_bwd.hip - backward of the KDA recurrence on gfx950: gradients of
// L = sum_t <dy_t, y_t> + <dS_final, S_final> with respect to q, k, v, a, b,
// gate and the initial state.
//
// The recurrence is the one of page "[Paper Review] Kimi K3...", section
// "Kimi Delta Attention (KDA)" (the pages describe no backward; training at
// scale implies one).  Reverse mode through one token, with S' = Diag(alpha)
// S_{t-1}, w = S'^T kh, u = beta (v - w), S_t = S' + kh u^T, o = S_t^T qh and
// dS the adjoint of S_t:
//   do = dy sigmoid(gate),  dgate = dy o sigmoid'(gate),  dS += qh do^T
//   dqh = S_t do,  du = dS^T kh,  dv = beta du,  dbeta = du . (v - w)
//   dkh = dS u - beta S' du,  dS' = dS - beta kh du^T
//   dalpha = rowsum(dS' * S_{t-1}),  dS_{t-1} = Diag(alpha) dS'
// and through the input maps (L2 normalisation, alpha = exp(-5 sigmoid(a)),
// beta = sigmoid(b)) in the reduction kernel.
//
// Work decomposition.  The state columns are independent given the keys, so
// one wavefront owns (sequence, head, 8 state columns): lane l holds rows
// RPT l .. RPT l + RPT - 1 (RPT = dk / 64) of the state slice and of its
// adjoint in registers.  The sequence is walked backwards in 64-token chunks;
// each chunk's start state is the forward's recorded state (states every 64
// tokens), the chunk is replayed once to record the starts of its 4-token
// sub-chunks, and each sub-chunk, last first, is replayed again to record
// the state before each of its tokens, then the adjoint runs through it
// token by token.  The sub-chunk starts live in a per-wavefront global
// scratch and the per-token states in LDS (16 KB at d_k = 128), so about
// nine single-wave workgroups share a CU: the per-token chains are short
// dependent reductions, and other waves on the SIMD hide their latency.
// The per-row partial sums over the wavefront's columns
// (dqh, dkh, dalpha, and the scalar dbeta) go to per-slice buffers, which the
// reduction kernel adds in a fixed order (no atomics: bitwise repeatable).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kSC = 8;        // state columns per wavefront
constexpr int kChunk = 64;    // tokens between recorded forward states
constexpr int kSub = 4;       // tokens per replayed sub-chunk
constexpr int kNSub = kChunk / kSub;
static_assert(kNSub == kBwdSubStarts && kSub * kSC <= 64, "sub-chunk layout");

__device__ __forceinline__ float sigm(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum of x over the 64 lanes for each of 8 values, returned uniform: a
// transposing butterfly (each step halves the values a lane carries), then a
// read of the lane that ended with each total.
__device__ __forceinline__ void reduce8(const float (&x)[8], float (&out)[8], int lane) {
  float k4[4], k2[2];
  const bool hi32 = lane & 32, hi16 = lane & 16, hi8 = lane & 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float send = hi32 ? x[i] : x[4 + i];
    k4[i] = (hi32 ? x[4 + i] : x[i]) + __shfl_xor(send, 32, 64);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float send = hi16 ? k4[i] : k4[2 + i];
    k2[i] = (hi16 ? k4[2 + i] : k4[i]) + __shfl_xor(send, 16, 64);
  }
  // within a 16-lane row: exchange with lane ^ 8 (row_ror:8), then sums over
  // aligned groups of 8 (xor 1, xor 2 by quad permutes, the other quad of the
  // group by row_half_mirror) -- DPP, no LDS round trip
  float k1;
  {
    const float send = hi8 ? k2[0] : k2[1];
    k1 = (hi8 ? k2[1] : k2[0]) + dpp_mov<0x128>(send);
  }
  k1 += dpp_mov<0xB1>(k1);   // quad_perm [1,0,3,2]
  k1 += dpp_mov<0x4E>(k1);   // quad_perm [2,3,0,1]
  k1 += dpp_mov<0x141>(k1);  // row_half_mirror
  // lane L holds the total of value 4 (L>>5 & 1) + 2 (L>>4 & 1) + (L>>3 & 1)
#pragma unroll
  for (int v = 0; v < 8; ++v)
    out[v] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                           __builtin_bit_cast(int, k1),
                                           32 * (v >> 2) + 16 * ((v >> 1) & 1) + 8 * (v & 1)));
}

template <typename TI, int RPT>
__device__ __forceinline__ void load_rows(const TI* p, float (&x)[RPT]) {
#pragma unroll
  for (int r = 0; r < RPT; ++r) x[r] = ld_elem(p, r);
}

// State slice in LDS: element (row RPT l + r, column j) of a DK x 8 slice at
// ((r * 2 + j / 4) * 64 + l) * 4 + j % 4, so that each lane's four columns are
// one 16-byte access and a wave's access is one contiguous 1 KB.
template <int RPT>
struct SliceLds {
  static __device__ __forceinline__ void store(float* base, int lane, const float (&S)[RPT][kSC]) {
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<float4*>(base + ((r * 2 + h) * 64 + lane) * 4) =
            make_float4(S[r][4 * h], S[r][4 * h + 1], S[r][4 * h + 2], S[r][4 * h + 3]);
  }
  static __device__ __forceinline__ void load(const float* base, int lane, float (&S)[RPT][kSC]) {
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 v = *reinterpret_cast<const float4*>(base + ((r * 2 + h) * 64 + lane) * 4);
        S[r][4 * h] = v.x; S[r][4 * h + 1] = v.y; S[r][4 * h + 2] = v.z; S[r][4 * h + 3] = v.w;
      }
  }
};

template <typename TI, int DK>
__global__ void __launch_bounds__(64)
    bwd_token_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                     const TI* __restrict__ v, const TI* __restrict__ a,
                     const TI* __restrict__ bl, const TI* __restrict__ gate,
                     const float* __restrict__ dy, const float* __restrict__ o_raw,
                     const int32_t* __restrict__ cu_seqlens, const float* __restrict__ s_init,
                     const float* __restrict__ ckpt, const float* __restrict__ d_sfinal,
                     float* __restrict__ dv_out, float* __restrict__ dgate_out,
                     float* __restrict__ d_s0, float* __restrict__ p_dqh,
                     float* __restrict__ p_dkh, float* __restrict__ p_dal,
                     float* __restrict__ p_dbeta, float* __restrict__ sub_ws, int H, int DV,
                     long long T_tot) {
  constexpr int RPT = DK / 64;
  constexpr int SL = DK * kSC;  // floats per state slice
  using LS = SliceLds<RPT>;
  __shared__ __attribute__((aligned(16))) float sTok[kSub * SL];   // state before each token
  __shared__ float sV[kSub][kSC], sDO[kSub][kSC], sVW[kSub][kSC];  // per token, slice columns
  __shared__ float sBeta[kSub];

  const int nsl = DV / kSC;
  const int slice = blockIdx.x % nsl;
  const int item = blockIdx.x / nsl;
  const int n = item / H, h = item % H;
  const int col0 = slice * kSC;
  const int lane = threadIdx.x;
  // this wavefront's sub-chunk start states (global scratch, same layout as LDS)
  float* sSub = sub_ws + (int64_t)blockIdx.x * kNSub * SL;
  const int64_t tok_beg = cu_seqlens[n], tok_end = cu_seqlens[n + 1];
  const int64_t L = tok_end - tok_beg;
  const int64_t st_off = (int64_t)item * DK * DV;
  int64_t ck_off = 0;  // first recorded state of this sequence
  for (int m = 0; m < n; ++m) ck_off += (int64_t)(cu_seqlens[m + 1] - cu_seqlens[m]) / kChunk;

  float S[RPT][kSC], dS[RPT][kSC];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
#pragma unroll
    for (int j = 0; j < kSC; ++j)
      dS[r][j] = d_sfinal ? d_sfinal[st_off + (int64_t)(RPT * lane + r) * DV + col0 + j] : 0.f;

  // Inputs of one sub-chunk (tokens t0 .. t0 + ls - 1; rows past the end
  // repeat the last token and are never used), requested together: the rows
  // this lane owns of kh = k / |k|, alpha and (with the adjoint) qh = q / |q|
  // in registers; v, beta and do = dy sigmoid(gate) of the slice columns in
  // LDS (lane l requests token l / 8, column l % 8); dgate, elementwise, is
  // written here.
  float KH[kSub][RPT], AL[kSub][RPT], QH[kSub][RPT];
  auto stage = [&](int64_t t0, int ls, bool adj) {
    float kr[kSub][RPT], qr[kSub][RPT];
#pragma unroll
    for (int i = 0; i < kSub; ++i) {
      const int64_t th = (t0 + (i < ls ? i : ls - 1)) * H + h;
      load_rows<TI, RPT>(k + th * DK + RPT * lane, kr[i]);
      load_rows<TI, RPT>(a + th * DK + RPT * lane, AL[i]);
      if (adj) load_rows<TI, RPT>(q + th * DK + RPT * lane, qr[i]);
    }
    if (lane < kSub * kSC) {
      const int ti = lane / kSC, j = lane % kSC;
      const int64_t th = (t0 + (ti < ls ? ti : ls - 1)) * H + h;
      const int64_t e = th * DV + col0 + j;
      sV[ti][j] = ld_elem(v, e);
      if (j == 0) sBeta[ti] = sigm(ld_elem(bl, th));
      if (adj) {
        const float dyj = dy[e];
        float sg = 1.f;
        if (gate) {
          sg = sigm(ld_elem(gate, e));
          if (ti < ls) dgate_out[e] = dyj * o_raw[e] * sg * (1.f - sg);
        }
        sDO[ti][j] = dyj * sg;
      }
    }
    float part[8], tot[8];  // (reduce8 sums eight values; the rest are zero)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      part[i] = 0.f;
      if (i < kSub)
#pragma unroll
        for (int r = 0; r < RPT; ++r) part[i] += kr[i < kSub ? i : 0][r] * kr[i < kSub ? i : 0][r];
    }
    reduce8(part, tot, lane);
#pragma unroll
    for (int i = 0; i < kSub; ++i) {
      const float rk = rsqrtf(tot[i] + kNormEps);
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        KH[i][r] = kr[i][r] * rk;
        AL[i][r] = __expf(kGMin * sigm(AL[i][r]));
      }
    }
    if (adj) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        part[i] = 0.f;
        if (i < kSub)
#pragma unroll
          for (int r = 0; r < RPT; ++r) part[i] += qr[i < kSub ? i : 0][r] * qr[i < kSub ? i : 0][r];
      }
      reduce8(part, tot, lane);
#pragma unroll
      for (int i = 0; i < kSub; ++i) {
        const float rq = rsqrtf(tot[i] + kNormEps);
#pragma unroll
        for (int r = 0; r < RPT; ++r) QH[i][r] = qr[i][r] * rq;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the LDS table is visible to every lane
  };

  // One forward step of sub-chunk token i on the state slice; records v - w.
  auto fwd_step = [&](int i) {
    float part[kSC], w[kSC];
#pragma unroll
    for (int j = 0; j < kSC; ++j) {
      part[j] = 0.f;
#pragma unroll
      for (int r = 0; r < RPT; ++r) part[j] += AL[i][r] * KH[i][r] * S[r][j];
    }
    reduce8(part, w, lane);
    const float beta = sBeta[i];
    float u[kSC];
#pragma unroll
    for (int j = 0; j < kSC; ++j) {
      const float vw = sV[i][j] - w[j];
      u[j] = beta * vw;
      if (lane == 0) sVW[i][j] = vw;
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
      for (int j = 0; j < kSC; ++j) S[r][j] = AL[i][r] * S[r][j] + KH[i][r] * u[j];
  };

  const int nchunks = (int)((L + kChunk - 1) / kChunk);
  for (int m = nchunks - 1; m >= 0; --m) {
    const int64_t c0 = tok_beg + (int64_t)kChunk * m;
    const int lc = (int)(tok_end - c0 < kChunk ? tok_end - c0 : kChunk);
    const int nsub = (lc + kSub - 1) / kSub;
    // chunk start state: the initial state, or the forward's record after 64 m tokens
    {
      const float* src = m == 0 ? s_init : ckpt + ((ck_off + m - 1) * H + h) * (int64_t)DK * DV;
#pragma unroll
      for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int j = 0; j < kSC; ++j)
          S[r][j] = src ? src[(m == 0 ? st_off : 0) + (int64_t)(RPT * lane + r) * DV + col0 + j]
                        : 0.f;
    }
    // replay 1: the starts of the sub-chunks (each lane writes and later reads
    // back only its own part of the scratch)
    for (int s = 0; s < nsub; ++s) {
      const int ls = lc - kSub * s < kSub ? lc - kSub * s : kSub;
      LS::store(sSub + s * SL, lane, S);
      stage(c0 + kSub * s, ls, false);
#pragma unroll
      for (int i = 0; i < kSub; ++i)
        if (i < ls) fwd_step(i);
    }
    // sub-chunks, last first: replay 2 records the state before each token,
    // then the adjoint runs back through them
    for (int s = nsub - 1; s >= 0; --s) {
      const int ls = lc - kSub * s < kSub ? lc - kSub * s : kSub;
      stage(c0 + kSub * s, ls, true);
      LS::load(sSub + s * SL, lane, S);
#pragma unroll
      for (int i = 0; i < kSub; ++i)
        if (i < ls) {
          LS::store(sTok + i * SL, lane, S);
          fwd_step(i);
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      // S now holds the state after the sub-chunk's last token
#pragma unroll
      for (int i = kSub - 1; i >= 0; --i) {
        if (i >= ls) continue;
        const int64_t t = c0 + kSub * s + i;
        float Sp[RPT][kSC];  // state before token t; S holds the state after it
        LS::load(sTok + i * SL, lane, Sp);
        const float beta = sBeta[i];
        float doj[kSC], vw[kSC];
#pragma unroll
        for (int j = 0; j < kSC; ++j) {
          doj[j] = sDO[i][j];
          vw[j] = sVW[i][j];
        }
        float dqh[RPT], part[kSC];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          dqh[r] = 0.f;
#pragma unroll
          for (int j = 0; j < kSC; ++j) {
            dS[r][j] += QH[i][r] * doj[j];
            dqh[r] += S[r][j] * doj[j];
          }
        }
#pragma unroll
        for (int j = 0; j < kSC; ++j) {
          part[j] = 0.f;
#pragma unroll
          for (int r = 0; r < RPT; ++r) part[j] += dS[r][j] * KH[i][r];
        }
        float du[kSC];
        reduce8(part, du, lane);
        float dbeta = 0.f;
#pragma unroll
        for (int j = 0; j < kSC; ++j) dbeta += du[j] * vw[j];
        const int64_t th = t * H + h;
        if (lane < kSC) {
          float dvj = 0.f;
#pragma unroll
          for (int j = 0; j < kSC; ++j) dvj = lane == j ? beta * du[j] : dvj;
          dv_out[th * DV + col0 + lane] = dvj;
        }
        float dkh[RPT], dal[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          dkh[r] = 0.f;
          dal[r] = 0.f;
#pragma unroll
          for (int j = 0; j < kSC; ++j) {
            const float sp = AL[i][r] * Sp[r][j];
            dkh[r] += dS[r][j] * beta * vw[j] - beta * sp * du[j];
            const float dsp = dS[r][j] - beta * KH[i][r] * du[j];
            dal[r] += dsp * Sp[r][j];
            dS[r][j] = AL[i][r] * dsp;
          }
        }
        const int64_t po = ((int64_t)slice * T_tot + t) * H + h;  // partial-sum row
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          p_dqh[po * DK + RPT * lane + r] = dqh[r];
          p_dkh[po * DK + RPT * lane + r] = dkh[r];
          p_dal[po * DK + RPT * lane + r] = dal[r];
        }
        if (lane == 0) p_dbeta[po] = dbeta;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
          for (int j = 0; j < kSC; ++j) S[r][j] = Sp[r][j];
      }
    }
  }
  if (d_s0) {
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
      for (int j = 0; j < kSC; ++j) d_s0[st_off + (int64_t)(RPT * lane + r) * DV + col0 + j] = dS[r][j];
  }
}

// Per (token, head) row: add the slices' partial sums in slice order, then the
// input maps: dq = r dqh - r^3 (q . dqh) q (r = (|q|^2 + eps)^-1/2, same for
// k), da = dalpha alpha (-5) sigmoid(a) (1 - sigmoid(a)),
// db = dbeta beta (1 - beta).  One 16-lane DPP row per (token, head) row.
template <int CTRL>
__device__ __forceinline__ float dpp_sum_step(float x) {
  return x + __builtin_bit_cast(
                 float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf,
                                                    0xf, true));
}
__device__ __forceinline__ float row16_total(float x) {
  x = dpp_sum_step<0x128>(x);
  x = dpp_sum_step<0x124>(x);
  x = dpp_sum_step<0x122>(x);
  return dpp_sum_step<0x121>(x);
}

template <typename TI, int DK>
__global__ void __launch_bounds__(256)
    bwd_reduce_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                      const TI* __restrict__ a, const TI* __restrict__ bl,
                      const float* __restrict__ p_dqh, const float* __restrict__ p_dkh,
                      const float* __restrict__ p_dal, const float* __restrict__ p_dbeta,
                      float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ da,
                      float* __restrict__ db, int nsl, long long rows) {
  constexpr int CPL = DK / 16;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int li = lane % 16, rsub = lane / 16;
  const int64_t row = (int64_t)blockIdx.x * 16 + 4 * wave + rsub;
  if (row >= rows) return;  // uniform within each 16-lane row
  const int c0 = CPL * li;
  float dqh[CPL], dkh[CPL], dal[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) dqh[c] = dkh[c] = dal[c] = 0.f;
  float dbeta = 0.f;
  for (int s = 0; s < nsl; ++s) {
    const int64_t po = (int64_t)s * rows + row;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      dqh[c] += p_dqh[po * DK + c0 + c];
      dkh[c] += p_dkh[po * DK + c0 + c];
      dal[c] += p_dal[po * DK + c0 + c];
    }
    dbeta += p_dbeta[po];
  }
  float qv[CPL], kv[CPL], sq = 0.f, sk = 0.f, qd = 0.f, kd = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    qv[c] = ld_elem(q, row * DK + c0 + c);
    kv[c] = ld_elem(k, row * DK + c0 + c);
    sq += qv[c] * qv[c];
    sk += kv[c] * kv[c];
    qd += qv[c] * dqh[c];
    kd += kv[c] * dkh[c];
  }
  sq = row16_total(sq);
  sk = row16_total(sk);
  qd = row16_total(qd);
  kd = row16_total(kd);
  const float rq = rsqrtf(sq + kNormEps), rk = rsqrtf(sk + kNormEps);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    dq[row * DK + c0 + c] = rq * dqh[c] - rq * rq * rq * qd * qv[c];
    dk[row * DK + c0 + c] = rk * dkh[c] - rk * rk * rk * kd * kv[c];
    const float av = ld_elem(a, row * DK + c0 + c);
    const float sa = sigm(av);
    const float al = __expf(kGMin * sa);
    // sigmoid'(a) = sigmoid(a) sigmoid(-a): no cancellation as sigmoid(a) -> 1
    da[row * DK + c0 + c] = dal[c] * al * kGMin * sa * sigm(-av);
  }
  if (li == 0) {
    const float beta = sigm(ld_elem(bl, row));
    db[row] = dbeta * beta * (1.f - beta);
  }
}

template <typename TI>
hipError_t launch_bwd_t(const BwdArgs& p, hipStream_t stream) {
  const int nsl = p.dv / kSC;
  const int64_t items = (int64_t)p.num_seqs * p.num_heads;
  const int64_t rows = p.total_tokens * p.num_heads;
  if (items > 0) {
    auto kern = p.dk == 128 ? bwd_token_kernel<TI, 128> : bwd_token_kernel<TI, 64>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(items * nsl)), dim3(64), 0, stream,
                       (const TI*)p.q, (const TI*)p.k, (const TI*)p.v, (const TI*)p.a,
                       (const TI*)p.b, (const TI*)p.gate, p.dy, p.o_raw, p.cu_seqlens,
                       p.initial_state, p.ckpt, p.d_final_state, p.dv_out, p.dgate_out, p.d_s0,
                       p.p_dqh, p.p_dkh, p.p_dal, p.p_dbeta, p.sub_ws, p.num_heads, p.dv,
                       (long long)p.total_tokens);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (rows > 0) {
    auto kern = p.dk == 128 ? bwd_reduce_kernel<TI, 128> : bwd_reduce_kernel<TI, 64>;
    hipLaunchKernelGGL(kern, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream,
                       (const TI*)p.q, (const TI*)p.k, (const TI*)p.a, (const TI*)p.b, p.p_dqh,
                       p.p_dkh, p.p_dal, p.p_dbeta, p.dq_out, p.dk_out, p.da_out, p.db_out,
                       nsl, (long long)rows);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& p, hipStream_t stream) {
  return p.in_bf16 ? launch_bwd_t<uint16_t>(p, stream) : launch_bwd_t<float>(p, stream);
}

}  // namespace kda
