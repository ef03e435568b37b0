// kda_layer.hip - the KDA layer operations around the core recurrence, gfx950.
//
// Page "[Paper Review] Kimi K3...", section "Kimi Delta Attention (KDA)":
//   * projections paragraph: query and key pass through a short convolution,
//     then Swish, and are L2-normalised -> conv_swish_l2_kernel, one pass;
//   * "Full-rank gate" paragraph: the sigmoid output gate follows a head-wise
//     RMSNorm of the head's output -> rmsnorm_gate_kernel, one pass.
// Both are HBM-bound elementwise/row-reduction passes.  A 16-lane row of a
// wavefront owns one (token, head) row of the tensor (d channels, d / 16 per
// lane, one 16- or 32-byte access per lane), so the row reductions are
// four DPP steps inside the row, and a wave covers four rows at a time.
//
// Readings (the pages print neither the convolution nor the norm's details):
// causal depthwise convolution over a sequence's tokens, width W <= 4,
// weight [H, d, W] fp32 with w[.., W-1] on the current token, no bias;
// positions before a sequence's first token come from a carried state
// [N, H, d, W-1] (oldest first) or are zero; Swish(c) = c sigmoid(c); L2
// normalisation with eps = 1e-6 under the root; RMSNorm over the head's d_v
// channels with a weight [d_v] shared by the heads and a caller-given eps.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kLayerThreads = 256;  // 4 waves x 4 rows of 16 lanes
constexpr int kConvTokens = 256;    // tokens per wave in the convolution pass
constexpr int kGroup = 8;           // rows requested together
constexpr float kLog2eL = 1.4426950408889634f;

// Sum over the 16 lanes of each DPP row, in every lane of the row.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(
                 float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf,
                                                    0xf, true));
}
__device__ __forceinline__ float row16_sum(float x) {
  x = dpp_add<0x128>(x);  // row_ror:8
  x = dpp_add<0x124>(x);  // row_ror:4
  x = dpp_add<0x122>(x);  // row_ror:2
  return dpp_add<0x121>(x);  // row_ror:1
}

__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2eL * x));
}

// CPL consecutive elements of a row <-> floats.
template <typename T, int CPL>
struct RowIO;
template <int CPL>
struct RowIO<float, CPL> {
  static constexpr int RW = CPL;  // 32-bit words per lane and row
  static __device__ __forceinline__ void load_raw(const float* p, uint32_t (&w)[RW]) {
#pragma unroll
    for (int i = 0; i < CPL; i += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + i);
      w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
    }
  }
  static __device__ __forceinline__ float elem(const uint32_t (&w)[RW], int c) {
    return __uint_as_float(w[c]);
  }
  static __device__ __forceinline__ void load(const float* p, float (&x)[CPL]) {
#pragma unroll
    for (int i = 0; i < CPL; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(p + i);
      x[i] = v.x; x[i + 1] = v.y; x[i + 2] = v.z; x[i + 3] = v.w;
    }
  }
  static __device__ __forceinline__ void store(float* p, const float (&x)[CPL]) {
#pragma unroll
    for (int i = 0; i < CPL; i += 4)
      *reinterpret_cast<float4*>(p + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
  }
};
template <int CPL>
struct RowIO<uint16_t, CPL> {  // bf16
  static constexpr int RW = CPL / 2;
  static __device__ __forceinline__ void load_raw(const uint16_t* p, uint32_t (&w)[RW]) {
    if constexpr (CPL == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x; w[1] = v.y;
    }
  }
  static __device__ __forceinline__ float elem(const uint32_t (&w)[RW], int c) {
    return c % 2 ? __uint_as_float(w[c / 2] & 0xFFFF0000u) : __uint_as_float(w[c / 2] << 16);
  }
  static __device__ __forceinline__ void load(const uint16_t* p, float (&x)[CPL]) {
    static_assert(CPL == 8 || CPL == 4, "row split");
    uint32_t w[CPL / 2];
    if constexpr (CPL == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x; w[1] = v.y;
    }
#pragma unroll
    for (int j = 0; j < CPL / 2; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float (&x)[CPL]) {
    uint32_t w[CPL / 2];
#pragma unroll
    for (int j = 0; j < CPL / 2; ++j)
      w[j] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x[2 * j]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x[2 * j + 1]) << 16);
    if constexpr (CPL == 8) {
      *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    }
  }
};

// Short convolution -> Swish -> L2.  Grid: x = blocks of kConvTokens packed
// tokens, y = groups of 16 heads; wave w, row r of the block handles head
// 16 y + 4 w + r over the block's tokens in order, carrying the W - 1
// previous inputs of its row in registers.
template <typename T, int DIM>
__global__ void __launch_bounds__(kLayerThreads)
    conv_swish_l2_kernel(const T* __restrict__ x, const float* __restrict__ w,
                         const int32_t* __restrict__ cu_seqlens, const T* __restrict__ st_in,
                         T* __restrict__ y, int N, long long T_tot, int H, int W) {
  constexpr int CPL = DIM / 16;  // channels per lane
  using IO = RowIO<T, CPL>;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int li = lane % 16, r = lane / 16;
  const int h = 16 * blockIdx.y + 4 * wave + r;
  const bool hv = h < H;  // rows past the last head do nothing (no memory access)
  const int hh = hv ? h : 0;
  const int c0 = CPL * li;
  const int64_t t0 = (int64_t)blockIdx.x * kConvTokens;
  const int64_t t1 = t0 + kConvTokens < T_tot ? t0 + kConvTokens : T_tot;

  float wr[CPL][4];  // wr[c][i]: tap for the token i steps back
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wr[c][i] = (hv && i < W) ? w[((int64_t)hh * DIM + c0 + c) * W + (W - 1 - i)] : 0.f;

  // Sequence holding t0: the largest n with cu[n] <= t0 (then cu[n+1] > t0).
  int lo = 0, hi = N;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if ((int64_t)cu_seqlens[mid] <= t0) lo = mid; else hi = mid - 1;
  }
  int n = lo;
  int64_t s_beg = cu_seqlens[n], s_end = cu_seqlens[n + 1];

  float hist[3][CPL];  // inputs 1, 2, 3 tokens back
  auto fill_history = [&](int64_t t) {  // history of token t in sequence n
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      float v[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) v[c] = 0.f;
      const int64_t p = t - i;
      if (hv && i < W) {
        if (p >= s_beg) {
          IO::load(x + (p * H + hh) * DIM + c0, v);
        } else if (st_in) {  // carried state: index p - s_beg + W - 1 (>= 0)
          const int j = (int)(p - s_beg) + W - 1;
#pragma unroll
          for (int c = 0; c < CPL; ++c)
            v[c] = ld_elem(st_in, (((int64_t)n * H + hh) * DIM + c0 + c) * (W - 1) + j);
        }
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) hist[i - 1][c] = v[c];
    }
  };
  if (t0 < t1) fill_history(t0);

  for (int64_t tg = t0; tg < t1; tg += kGroup) {
    uint32_t xr[kGroup][IO::RW];  // the group's rows as loaded (unpacked at use)
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {  // rows of the group (clamped to the block)
      const int64_t t = tg + u < t1 ? tg + u : t1 - 1;
      if (hv) {
        IO::load_raw(x + (t * H + hh) * DIM + c0, xr[u]);
      } else {
#pragma unroll
        for (int j = 0; j < IO::RW; ++j) xr[u][j] = 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int64_t t = tg + u;
      if (t >= t1) break;
      if (t >= s_end) {  // next non-empty sequence starts here
        while ((int64_t)cu_seqlens[n + 1] <= t) ++n;
        s_beg = cu_seqlens[n];
        s_end = cu_seqlens[n + 1];
        fill_history(t);
      }
      float s[CPL], xc[CPL], ss = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        xc[c] = IO::elem(xr[u], c);
        float cv = wr[c][0] * xc[c];
#pragma unroll
        for (int i = 1; i < 4; ++i) cv += wr[c][i] * hist[i - 1][c];
        s[c] = cv * sigmoid_fast(cv);
        ss += s[c] * s[c];
      }
      const float rn = rsqrtf(row16_sum(ss) + kNormEps);
#pragma unroll
      for (int c = 0; c < CPL; ++c) s[c] *= rn;
      if (hv) IO::store(y + (t * H + hh) * DIM + c0, s);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        hist[2][c] = hist[1][c];
        hist[1][c] = hist[0][c];
        hist[0][c] = xc[c];
      }
    }
  }
}

// Carried state after each sequence: the last W - 1 inputs of
// [state_in, sequence].  One thread per (sequence, head, channel); runs after
// conv_swish_l2_kernel (which reads state_in), so state_out may be state_in.
template <typename T>
__global__ void __launch_bounds__(256)
    conv_state_kernel(const T* __restrict__ x, const int32_t* __restrict__ cu_seqlens,
                      const T* st_in, T* st_out, int N, int H, int DIM, int W) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)N * H * DIM) return;
  const int c = (int)(idx % DIM);
  const int h = (int)((idx / DIM) % H);
  const int n = (int)(idx / ((int64_t)DIM * H));
  const int64_t s_beg = cu_seqlens[n], s_end = cu_seqlens[n + 1];
  for (int j = 0; j < W - 1; ++j) {  // increasing j: reads stay at or after the write
    const int64_t p = s_end - (W - 1) + j;
    T v;
    if (p >= s_beg) {
      v = x[(p * H + h) * DIM + c];
    } else if (st_in) {
      v = st_in[idx * (W - 1) + (p - s_beg) + W - 1];
    } else {
      v = T(0);
    }
    st_out[idx * (W - 1) + j] = v;
  }
}

// y = sigmoid(gate) * weight * o / sqrt(mean(o^2) + eps) per (token, head)
// row.  Each 16-lane row of a wave owns one row; lane li holds the channels
// 64 k + 4 li .. + 3 (k < DV / 64), so every load instruction of the wave
// reads whole contiguous segments of the rows.  A workgroup walks 64 rows;
// each thread issues the loads of all four of its rows before the first
// store (y may be o: every element is read and then written by the same
// thread, so the order is safe, and four rows' loads are in flight at once).
template <typename TG, int DV>
__global__ void __launch_bounds__(kLayerThreads)
    rmsnorm_gate_kernel(const float* o, const TG* __restrict__ gate,
                        const float* __restrict__ weight, float eps, float* y,
                        long long rows) {
  constexpr int NCH = DV / 64;  // 4-channel pieces per lane
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int li = lane % 16, r = lane / 16;
  float wt[NCH][4];
#pragma unroll
  for (int k = 0; k < NCH; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) wt[k][j] = weight ? weight[64 * k + 4 * li + j] : 1.f;
  constexpr int GW = sizeof(TG);  // 32-bit gate words per lane and 4 channels
  float v[4][NCH][4];
  uint32_t gr[4][NCH][GW];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int64_t row = (int64_t)blockIdx.x * 64 + it * 16 + 4 * wave + r;
    if (row >= rows) break;  // uniform within each 16-lane row
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const f32x4_t q =
          __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(o + row * DV + 64 * k + 4 * li));
      v[it][k][0] = q[0]; v[it][k][1] = q[1]; v[it][k][2] = q[2]; v[it][k][3] = q[3];
      if (gate) {
        if constexpr (GW == 2) {
          typedef __attribute__((ext_vector_type(2))) float f32x2_t;
          const f32x2_t u = __builtin_nontemporal_load(
              reinterpret_cast<const f32x2_t*>(gate + row * DV + 64 * k + 4 * li));
          gr[it][k][0] = __float_as_uint(u[0]); gr[it][k][1] = __float_as_uint(u[1]);
        } else {
          const uint4 u = *reinterpret_cast<const uint4*>(gate + row * DV + 64 * k + 4 * li);
          gr[it][k][0] = u.x; gr[it][k][1] = u.y; gr[it][k][2] = u.z; gr[it][k][3] = u.w;
        }
      }
    }
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int64_t row = (int64_t)blockIdx.x * 64 + it * 16 + 4 * wave + r;
    if (row >= rows) break;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) ss += v[it][k][j] * v[it][k][j];
    const float rn = rsqrtf(row16_sum(ss) * (1.f / DV) + eps);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      float gv[4] = {0.f, 0.f, 0.f, 0.f};
      if (gate) {
        if constexpr (GW == 2) {
          gv[0] = __uint_as_float(gr[it][k][0] << 16);
          gv[1] = __uint_as_float(gr[it][k][0] & 0xFFFF0000u);
          gv[2] = __uint_as_float(gr[it][k][1] << 16);
          gv[3] = __uint_as_float(gr[it][k][1] & 0xFFFF0000u);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) gv[j] = __uint_as_float(gr[it][k][j]);
        }
      }
      float* vv = v[it][k];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vv[j] *= rn * wt[k][j];
        if (gate) vv[j] *= sigmoid_fast(gv[j]);
      }
      __builtin_nontemporal_store(f32x4_t{vv[0], vv[1], vv[2], vv[3]},
                                  reinterpret_cast<f32x4_t*>(y + row * DV + 64 * k + 4 * li));
    }
  }
}

template <typename T>
hipError_t launch_conv_t(const ConvArgs& p, hipStream_t stream) {
  const T* x = static_cast<const T*>(p.x);
  if (p.total_tokens > 0) {
    const dim3 grid((unsigned)((p.total_tokens + kConvTokens - 1) / kConvTokens),
                    (unsigned)((p.num_heads + 15) / 16));
    auto kern = p.dim == 128 ? conv_swish_l2_kernel<T, 128> : conv_swish_l2_kernel<T, 64>;
    hipLaunchKernelGGL(kern, grid, dim3(kLayerThreads), 0, stream, x, p.weight, p.cu_seqlens,
                       static_cast<const T*>(p.state_in), static_cast<T*>(p.y), p.num_seqs,
                       (long long)p.total_tokens, p.num_heads, p.width);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.state_out && p.width > 1) {
    const int64_t n = (int64_t)p.num_seqs * p.num_heads * p.dim;
    hipLaunchKernelGGL(conv_state_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, x, p.cu_seqlens, static_cast<const T*>(p.state_in),
                       static_cast<T*>(p.state_out), p.num_seqs, p.num_heads, p.dim, p.width);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename TG>
hipError_t launch_rms_t(const RmsGateArgs& p, hipStream_t stream) {
  const int64_t rows = p.total_tokens * p.num_heads;
  if (rows == 0) return hipSuccess;
  auto kern = p.dv == 128 ? rmsnorm_gate_kernel<TG, 128> : rmsnorm_gate_kernel<TG, 64>;
  hipLaunchKernelGGL(kern, dim3((unsigned)((rows + 63) / 64)), dim3(kLayerThreads), 0, stream,
                     p.o, static_cast<const TG*>(p.gate), p.weight, p.eps, p.y,
                     (long long)rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_swish_l2(const ConvArgs& p, hipStream_t stream) {
  return p.in_bf16 ? launch_conv_t<uint16_t>(p, stream) : launch_conv_t<float>(p, stream);
}

hipError_t launch_rmsnorm_gate(const RmsGateArgs& p, hipStream_t stream) {
  return p.in_bf16 ? launch_rms_t<uint16_t>(p, stream) : launch_rms_t<float>(p, stream);
}

}  // namespace kda
