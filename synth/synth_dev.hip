// synth_dev.hip - device (gfx950) filler for the seeded synthetic inputs.
// Produces the same values as synth_host.c (same synth_core.h definition);
// used where a tensor is too large to generate on the host and upload
// (a 1M-token, 96-head tensor is 1.3e10 elements).
#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)
#define SYNTH_FN __host__ __device__ static inline
#include "synth_core.h"

namespace {

template <int DTYPE>
__global__ void __launch_bounds__(256) fill_kernel(void* __restrict__ out, uint64_t key, double mean,
                                                   double stdv, int64_t n_rows, int64_t row_len,
                                                   int64_t row_stride, int64_t base) {
  const int64_t total = n_rows * row_len;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += step) {
    const int64_t r = i / row_len;
    const int64_t c = i - r * row_len;
    const double x = synth_normal(key, (uint64_t)(base + r * row_stride + c), mean, stdv);
    const float f = (float)x;
    if (DTYPE == 0)
      ((float*)out)[i] = f;
    else
      ((uint16_t*)out)[i] = synth_f32_to_bf16(f);
  }
}

}  // namespace

extern "C" {

// out (device, dense n_rows x row_len) [r][c] = element base + r*row_stride + c.
// dtype 0 = fp32, 1 = bf16.  Enqueued on `stream` (a hipStream_t, NULL = default).
// Returns 0, -1 on a bad argument, -2 on a HIP launch error.
int synth_fill_normal_dev(void* out, int dtype, uint64_t key, double mean, double stdv,
                          int64_t n_rows, int64_t row_len, int64_t row_stride, int64_t base,
                          void* stream) {
  if (!out || n_rows < 0 || row_len < 0 || base < 0 || (dtype != 0 && dtype != 1)) return -1;
  const int64_t total = n_rows * row_len;
  if (total == 0) return 0;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == 0)
    hipLaunchKernelGGL(fill_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, out, key, mean, stdv,
                       n_rows, row_len, row_stride, base);
  else
    hipLaunchKernelGGL(fill_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, out, key, mean, stdv,
                       n_rows, row_len, row_stride, base);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

uint64_t synth_key_dev(uint64_t seed, uint32_t tensor, uint32_t step) {
  return synth_stream_key(seed, tensor, step);
}

}  // extern "C"
