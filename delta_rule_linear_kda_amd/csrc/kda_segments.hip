// kda_segments.hip - the segment-transition form of the KDA forward on one
// GPU (gfx950): the segment table and the composition of segment transitions.
//
// Context parallelism for KDA (page "[Paper Review] Kimi K3...", section
// "Infrastructure: how to actually run trillion-scale", the KDA co-design
// item, and the "Parallelism" row of the summary table) splits a sequence into segments,
// computes each segment's state transition on its own and combines the
// transitions associatively, so only fixed-size states cross segment
// boundaries.  For one segment, the recurrence is affine in the start state:
//   S_end = M S_start + S_loc
// with M (dk x dk) the product of the per-token factors
// (I - beta kh kh^T) Diag(alpha), latest on the left, and S_loc the state the
// segment reaches from a zero start.  The chunked kernels produce [S_loc | M]
// as one recurrence over d_v + d_k state columns (value rows zero and an
// identity start for the M columns).  This file turns a packed-sequence
// layout into segments and chains the transitions in order:
//   S_start(first segment) = initial state,  S_start(next) = M S_start + S_loc.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kTableThreads = 1024;

// Segment table for segments of `seg_len` tokens (the last segment of a
// sequence may be shorter; an empty sequence has none):
//   seg_off[n]  first segment of sequence n (seg_off[N] = segment count)
//   seg_cu[j]   first token of segment j, seg_cu[count] = T; entries up to
//               seg_cu[cap] repeat T (empty trailing segments).
// One workgroup: thread t takes a contiguous run of sequences, and an
// exclusive scan over the threads' segment counts places the runs.
__global__ void __launch_bounds__(kTableThreads)
    segment_table_kernel(const int32_t* __restrict__ cu_seqlens, int N, int seg_len,
                         int cap, int32_t* __restrict__ seg_cu, int32_t* __restrict__ seg_off) {
  __shared__ int scan[kTableThreads];
  const int t = threadIdx.x;
  const int per = (N + kTableThreads - 1) / kTableThreads;
  const int n0 = min(N, t * per), n1 = min(N, n0 + per);
  int mine = 0;
  for (int n = n0; n < n1; ++n)
    mine += (int)(((int64_t)cu_seqlens[n + 1] - cu_seqlens[n] + seg_len - 1) / seg_len);
  scan[t] = mine;
  __syncthreads();
  // Hillis-Steele inclusive scan over the counts.
  for (int d = 1; d < kTableThreads; d <<= 1) {
    const int x = t >= d ? scan[t - d] : 0;
    __syncthreads();
    scan[t] += x;
    __syncthreads();
  }
  int off = scan[t] - mine;  // exclusive prefix
  for (int n = n0; n < n1; ++n) {
    const int beg = cu_seqlens[n], len = cu_seqlens[n + 1] - beg;
    const int cnt = (int)(((int64_t)len + seg_len - 1) / seg_len);
    seg_off[n] = off;
    for (int j = 0; j < cnt; ++j) seg_cu[off + j] = beg + j * seg_len;
    off += cnt;
  }
  const int total = scan[kTableThreads - 1];
  const int T = cu_seqlens[N];
  if (t == 0) seg_off[N] = total;
  for (int j = total + t; j <= cap; j += kTableThreads) seg_cu[j] = T;
}

// Composition, one workgroup per (sequence, head, 16 state columns); thread
// (r0 = t / 16, c = t % 16) owns rows r0 + 16 i of column c.  Per segment the
// transition M is staged in LDS and S <- M S + S_loc is formed in fp32.
constexpr int kComposeThreads = 256;

template <int DK>
__global__ void __launch_bounds__(kComposeThreads)
    compose_kernel(const int32_t* __restrict__ seg_off, const float* __restrict__ trans,
                   const float* __restrict__ s_init, float* __restrict__ seg_start,
                   float* __restrict__ s_final, int H, int dv) {
  constexpr int LM = DK + 4;         // padded LDS row of M
  constexpr int RPT = DK / 16;       // rows per thread
  __shared__ __attribute__((aligned(16))) float sM[DK * LM];
  __shared__ float sS[DK * 16];
  const int ncb = dv / 16;
  const int cb = blockIdx.x % ncb;
  const int item = blockIdx.x / ncb;  // sequence * H + head
  const int n = item / H, h = item % H;
  const int t = threadIdx.x, c = t % 16, r0 = t / 16;
  const int col = 16 * cb + c;
  const int sdv = dv + DK;

  float s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = r0 + 16 * i;
    s[i] = s_init ? s_init[((int64_t)item * DK + r) * dv + col] : 0.f;
  }
  const int j0 = seg_off[n], j1 = seg_off[n + 1];
  for (int j = j0; j < j1; ++j) {
    const int64_t tb = ((int64_t)j * H + h) * DK * sdv;  // [S_loc | M] rows of segment j
    if (seg_start) {
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        seg_start[(((int64_t)j * H + h) * DK + r0 + 16 * i) * dv + col] = s[i];
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) sS[(r0 + 16 * i) * 16 + c] = s[i];
    for (int e = t; e < DK * DK / 4; e += kComposeThreads) {
      const int r = e / (DK / 4), k4 = 4 * (e % (DK / 4));
      *reinterpret_cast<float4*>(sM + r * LM + k4) =
          *reinterpret_cast<const float4*>(trans + tb + (int64_t)r * sdv + dv + k4);
    }
    float acc[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) acc[i] = trans[tb + (int64_t)(r0 + 16 * i) * sdv + col];
    __syncthreads();
    for (int k4 = 0; k4 < DK; k4 += 4) {
      const float x0 = sS[(k4 + 0) * 16 + c], x1 = sS[(k4 + 1) * 16 + c];
      const float x2 = sS[(k4 + 2) * 16 + c], x3 = sS[(k4 + 3) * 16 + c];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float4 m = *reinterpret_cast<const float4*>(sM + (r0 + 16 * i) * LM + k4);
        acc[i] += m.x * x0 + m.y * x1 + m.z * x2 + m.w * x3;
      }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = acc[i];
    __syncthreads();  // sM and sS are rewritten for the next segment
  }
  if (s_final) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) s_final[((int64_t)item * DK + r0 + 16 * i) * dv + col] = s[i];
  }
}

}  // namespace

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

hipError_t launch_segment_table(const int32_t* cu_seqlens, int32_t num_seqs, int32_t seg_len,
                                int32_t cap, int32_t* seg_cu, int32_t* seg_off,
                                hipStream_t stream) {
  hipLaunchKernelGGL(segment_table_kernel, dim3(1), dim3(kTableThreads), 0, stream, cu_seqlens,
                     num_seqs, seg_len, cap, seg_cu, seg_off);
  return hipGetLastError();
}

hipError_t launch_compose(const ComposeArgs& p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.num_seqs * p.num_heads * (p.dv / 16);
  if (grid == 0) return hipSuccess;
  auto kern = p.dk == 128 ? compose_kernel<128> : compose_kernel<64>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kComposeThreads), 0, stream, p.seg_offsets,
                     p.trans, p.initial_state, p.seg_start, p.final_state, p.num_heads, p.dv);
  return hipGetLastError();
}

}  // namespace kda
