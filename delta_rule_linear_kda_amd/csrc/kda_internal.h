// kda_internal.h - host-side launch interface between the C ABI layer
// (kda_api.cpp) and the kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
  int32_t num_seqs, num_heads, dk, dv;
  bool in_bf16;
  const void *q, *k, *v, *a, *b, *gate;  // gate may be null
  float* state;
  void* o;
};

struct FwdArgs {
  int32_t num_seqs, num_heads, dk, dv;
  int64_t total_tokens;
  bool in_bf16;
  const void *q, *k, *v, *a, *b, *gate;  // gate may be null
  const int32_t* cu_seqlens;
  const float* initial_state;  // may be null (zero state)
  void* o;
  float* final_state;  // may be null
  // Recorded states (kda_fwd_chunked_ckpt): every ckpt_interval tokens of a
  // sequence; 0 = none.  Slot layout as final_state, ckpt_capacity slots.
  int32_t ckpt_interval = 0;
  float* ckpt = nullptr;
  int64_t ckpt_capacity = 0;
};

hipError_t launch_decode(const DecodeArgs& p, hipStream_t stream);
hipError_t launch_fwd_chunked(const FwdArgs& p, hipStream_t stream);
// bf16-input kernel (kda_chunk_bf16.hip); launch_fwd_chunked dispatches to it.
hipError_t launch_fwd_chunked_bf16(const FwdArgs& p, hipStream_t stream);

}  // namespace kda
