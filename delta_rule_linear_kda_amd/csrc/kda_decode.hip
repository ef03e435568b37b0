// kda_decode.hip - one-token KDA recurrent update (decode), gfx950.
//
// Per (sequence, head) the fp32 state S (DK x DV, row = key channel) is read
// once from HBM, updated, and written back in place:
//     s1 = S^T (alpha * kh),  s2 = S^T (alpha * qh)
//     u  = beta (v - s1)                         (delta-rule correction)
//     o  = s2 + (kh . qh) u                      (= S_new^T qh)
//     S  = Diag(alpha) S + kh u^T                (= (I - beta kh kh^T) Diag(alpha) S + beta kh v^T)
//     y  = sigmoid(gate) * o
// This is the recurrence of page "[Paper Review] Kimi K3...", section "Kimi
// Delta Attention (KDA)", rearranged so the state is streamed once: the two
// reductions over key channels are taken before the state is modified.
//
// The kernel is HBM-bound (128 KiB of state traffic per (sequence, head) at
// DK = DV = 128 against ~1.3 KiB of token inputs).  A workgroup of 512
// threads (8 waves) updates one (sequence, head) item, and two workgroups
// share a compute unit (it holds 16 waves), so one workgroup's reductions
// and stores overlap the other's state loads: measured 5.8-5.9 TB/s against
// 5.6-5.8 TB/s for two items per 1024-thread workgroup (one per CU) and
// ~5.4 TB/s for one item per 256-thread workgroup.  Each thread holds
// DK*DV/512 floats of its item's state in registers as float4 columns, so
// every byte of S is read and written exactly once with 16-byte nontemporal
// accesses, consecutive lanes covering consecutive addresses.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kTPI = 512;    // threads per (sequence, head) item
constexpr int kItems = 1;    // items per workgroup

template <typename TI, int DK, int DV>
__global__ void __launch_bounds__(kTPI * kItems)
    decode_kernel(const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v,
                  const TI* __restrict__ a, const TI* __restrict__ b, const TI* __restrict__ gate,
                  float* __restrict__ state, float* __restrict__ o, int64_t num_items) {
  constexpr int CG = DV / 4;      // column groups of 4 floats
  constexpr int RG = kTPI / CG;   // row groups
  constexpr int RPT = DK / RG;    // rows per thread
  constexpr int NWI = kTPI / 64;  // waves per item
  static_assert(RPT * RG == DK && RPT >= 1, "row split");

  const int part = threadIdx.x / kTPI;  // which item of the workgroup
  const int t = threadIdx.x % kTPI;
  const int64_t item_raw = (int64_t)blockIdx.x * kItems + part;  // sequence * H + head
  const bool valid = item_raw < num_items;  // an odd item count leaves one half idle
  const int64_t item = valid ? item_raw : num_items - 1;
  const int cg = t % CG, rg = t / CG;
  float* S = state + item * (int64_t)(DK * DV);

  // 1. The token's inputs first, then the state: the memory counter
  //    completes in order, so the small loads the norms and the correction
  //    wait for must not sit behind the state's 64 KB.  Every thread issues
  //    the same loads (channel t % DK; the gate's place taken by v when there
  //    is no gate), so the waits do not depend on the path.  The state: rows
  //    rg, rg+RG, ... ; the lanes of a wave cover 64 / CG consecutive rows.
  const int tc = t % DK;
  const float qc0 = ld_elem(q, item * DK + tc);
  const float kc0 = ld_elem(k, item * DK + tc);
  const float ac0 = ld_elem(a, item * DK + tc);
  const float braw = ld_elem(b, item);
  float vj[4], gj[4];
  ld4(v + item * DV + 4 * cg, vj);
  ld4((gate ? gate : v) + item * DV + 4 * cg, gj);
  f32x4_t s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(S + (rg + RG * i) * DV) + cg);

  __shared__ float sh_red[kItems][3][NWI];
  __shared__ float sh_kh[kItems][DK], sh_akh[kItems][DK], sh_aqh[kItems][DK], sh_alpha[kItems][DK];
  __shared__ float4 sh_part[kItems][2][RG][CG];

  // 2. Norms and k.q: threads t < DK of each item own key channel c = t.
  const int wave = t / 64;
  const float qc = t < DK ? qc0 : 0.f, kc = t < DK ? kc0 : 0.f, ac = ac0;
  float r0 = wave_sum(qc * qc), r1 = wave_sum(kc * kc), r2 = wave_sum(qc * kc);
  if ((t & 63) == 0 && wave < DK / 64) {
    sh_red[part][0][wave] = r0;
    sh_red[part][1][wave] = r1;
    sh_red[part][2][wave] = r2;
  }
  __syncthreads();
  float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
  for (int w = 0; w < DK / 64; ++w) {
    sq += sh_red[part][0][w];
    sk += sh_red[part][1][w];
    sqk += sh_red[part][2][w];
  }
  const float rq = rsqrtf(sq + kNormEps), rk = rsqrtf(sk + kNormEps);
  const float kq = sqk * rq * rk;  // kh . qh
  if (t < DK) {
    const float al = fast_exp(kGMin * sigmoidf(ac));
    const float kh = kc * rk;
    sh_kh[part][t] = kh;
    sh_alpha[part][t] = al;
    sh_akh[part][t] = al * kh;
    sh_aqh[part][t] = al * qc * rq;
  }
  __syncthreads();

  // 3. Partial reductions over this thread's rows for its 4 columns.
  float4 p1 = {0.f, 0.f, 0.f, 0.f}, p2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    const float x1 = sh_akh[part][r], x2 = sh_aqh[part][r];
    p1.x += x1 * s[i][0]; p1.y += x1 * s[i][1]; p1.z += x1 * s[i][2]; p1.w += x1 * s[i][3];
    p2.x += x2 * s[i][0]; p2.y += x2 * s[i][1]; p2.z += x2 * s[i][2]; p2.w += x2 * s[i][3];
  }
  sh_part[part][0][rg][cg] = p1;
  sh_part[part][1][rg][cg] = p2;
  __syncthreads();
  float4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int gi = 0; gi < RG; ++gi) {
    const float4 x1 = sh_part[part][0][gi][cg], x2 = sh_part[part][1][gi][cg];
    s1.x += x1.x; s1.y += x1.y; s1.z += x1.z; s1.w += x1.w;
    s2.x += x2.x; s2.y += x2.y; s2.z += x2.z; s2.w += x2.w;
  }

  // 4. Correction u and the output for columns 4cg..4cg+3.
  const float beta = sigmoidf(braw);
  const float4 u = {beta * (vj[0] - s1.x), beta * (vj[1] - s1.y), beta * (vj[2] - s1.z),
                    beta * (vj[3] - s1.w)};
  if (!valid) return;  // after the last barrier: the idle half stores nothing
  if (rg == 0) {
    float4 y = {s2.x + kq * u.x, s2.y + kq * u.y, s2.z + kq * u.z, s2.w + kq * u.w};
    if (gate) {
      y.x *= sigmoidf(gj[0]); y.y *= sigmoidf(gj[1]); y.z *= sigmoidf(gj[2]); y.w *= sigmoidf(gj[3]);
    }
    reinterpret_cast<float4*>(o + item * DV)[cg] = y;
  }

  // 5. S = Diag(alpha) S + kh u^T, written back in place.
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    const float al = sh_alpha[part][r], kh = sh_kh[part][r];
    f32x4_t x = s[i];
    x[0] = al * x[0] + kh * u.x;
    x[1] = al * x[1] + kh * u.y;
    x[2] = al * x[2] + kh * u.z;
    x[3] = al * x[3] + kh * u.w;
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4_t*>(S + r * DV) + cg);
  }
}

template <typename TI, int DK, int DV>
hipError_t launch_t(const DecodeArgs& p, hipStream_t stream) {
  const int64_t items = (int64_t)p.num_seqs * p.num_heads;
  const int64_t blocks = (items + kItems - 1) / kItems;
  hipLaunchKernelGGL((decode_kernel<TI, DK, DV>), dim3((unsigned)blocks), dim3(kTPI * kItems), 0,
                     stream, (const TI*)p.q, (const TI*)p.k, (const TI*)p.v, (const TI*)p.a,
                     (const TI*)p.b, (const TI*)p.gate, p.state, (float*)p.o, items);
  return hipGetLastError();
}

template <typename TI>
hipError_t launch_d(const DecodeArgs& p, hipStream_t stream) {
  if (p.dk == 128 && p.dv == 128) return launch_t<TI, 128, 128>(p, stream);
  if (p.dk == 128 && p.dv == 64) return launch_t<TI, 128, 64>(p, stream);
  if (p.dk == 64 && p.dv == 128) return launch_t<TI, 64, 128>(p, stream);
  return launch_t<TI, 64, 64>(p, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& p, hipStream_t stream) {
  if ((int64_t)p.num_seqs * p.num_heads == 0) return hipSuccess;
  return p.in_bf16 ? launch_d<uint16_t>(p, stream) : launch_d<float>(p, stream);
}

}  // namespace kda
