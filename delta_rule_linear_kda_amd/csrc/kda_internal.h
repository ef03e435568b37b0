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
  // Transition form (kda_segment_transition): when set, each sequence is a
  // segment and [S_loc | M] rows of d_v + d_k columns are written here,
  // [N, H, dk, dv + dk]; gate, initial_state, o, final_state and the
  // recorded states are not used.
  float* transition = nullptr;
  // Head-wise RMSNorm before the gate (kda_fwd_chunked_rmsnorm_gate): only
  // on the two-pass form's whole-head state pass (split_norm_fused says
  // when); weight [dv] or null (ones).
  bool norm = false;
  const float* norm_weight = nullptr;
  float norm_eps = 0.f;
  // Fused bf16 form: one workgroup per (sequence, head) even when d_v slices
  // would fill more compute units (the backward's recomputation, which then
  // leaves the other half of the units to its adjoint chain).
  bool whole_items = false;
};

// Two-pass bf16 forward (kda_split_bf16.hip): workspace layout.  Chunks are
// processed in `blocks` blocks of `bc` chunks per sequence, alternating over
// `nbuf` (1 or 2) buffers of chunk records at rec[i] and per-sequence record
// offsets at slot[i]; with more than one block the carried states sit at
// [carry, total).
struct SplitLayout {
  int bc, blocks, nbuf;
  uint64_t rec[2], slot[2], carry, bt, total;  // bt: b transposed to [H, T] bf16
};
constexpr uint64_t kSplitRecordBudget = 4ull << 30;  // bytes of chunk records per block
// Layout for a record budget of `record_budget` bytes over `buffers` (1 or 2)
// record buffers.
SplitLayout split_layout(int64_t num_seqs, int64_t total_tokens, int64_t num_heads, int dk,
                         int dv, uint64_t record_budget = kSplitRecordBudget, int buffers = 2);
// With `layout` given, the blocks run one after another on `stream` alone
// (no second stream); otherwise the default layout and the overlapped
// schedule.
hipError_t launch_fwd_split_bf16(const FwdArgs& p, void* workspace, hipStream_t stream,
                                 const SplitLayout* layout = nullptr);
// Whether the two-pass form can run whole-head state workgroups for this
// shape: with the head-wise RMSNorm (applied in their output stage), and
// without it where a block's state pass runs beside the next block's record
// pass.
bool split_whole_head(int64_t num_seqs, int64_t num_heads, int dv);

// The forward entry point that allocates nothing (kda_fwd_chunked_noalloc)
// takes its workspace from a fixed device array of this many bytes, one per
// device, which the library holds until the process ends.
constexpr uint64_t kNoAllocScratchBytes = 256ull << 20;
// Layout of the two-pass form inside that array (one record buffer, blocks
// sized to what is left after the fixed parts); false when the shape does
// not fit.
bool noalloc_layout(int64_t num_seqs, int64_t total_tokens, int64_t num_heads, int dk, int dv,
                    SplitLayout* out);
// Device address of the array on the device of `stream` (resolved once per
// device).
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

// Backward: sub-chunks per 64-token chunk whose start states each
// wavefront keeps in global scratch (kda_bwd.hip).
constexpr int kBwdSubStarts = 16;

struct ComposeArgs {
  int32_t num_seqs, num_heads, dk, dv;
  const int32_t* seg_offsets;   // [N + 1], device
  const float* trans;           // [segments, H, dk, dv + dk]
  const float* initial_state;   // [N, H, dk, dv] or null (zero)
  float* seg_start;             // [segments, H, dk, dv] or null
  float* final_state;           // [N, H, dk, dv] or null
};

// Short convolution -> Swish -> L2 over [T, H, dim] rows (kda_layer.hip).
struct ConvArgs {
  int32_t num_seqs, num_heads, dim, width;
  int64_t total_tokens;
  bool in_bf16;
  const void* x;
  const float* weight;          // [H, dim, width]
  const int32_t* cu_seqlens;
  const void* state_in;         // [N, H, dim, width - 1] or null (zero)
  void* state_out;              // same layout or null; may equal state_in
  void* y;
};

// Head-wise RMSNorm then sigmoid gate over [T, H, dv] rows (kda_layer.hip).
struct RmsGateArgs {
  int32_t num_heads, dv;
  int64_t total_tokens;
  bool in_bf16;                 // dtype of gate
  const float* o;
  const void* gate;             // or null
  const float* weight;          // [dv] or null (ones)
  float eps;
  float* y;                     // may equal o
};

// Backward (kda_bwd.hip).  The forward's recorded states and ungated output
// are computed by the caller (kda_api.cpp) into the workspace first.
struct BwdArgs {
  int32_t num_seqs, num_heads, dk, dv;
  int64_t total_tokens;
  bool in_bf16;
  const void *q, *k, *v, *a, *b, *gate;  // gate may be null
  const int32_t* cu_seqlens;
  const float* initial_state;   // may be null
  const float* dy;              // [T, H, dv]
  const float* d_final_state;   // may be null
  const float* o_raw;           // [T, H, dv] ungated forward output
  const float* ckpt;            // states after every 64 tokens of each sequence
  float *dq_out, *dk_out, *dv_out, *da_out, *db_out, *dgate_out, *d_s0;  // dgate, d_s0 may be null
  float *p_dqh, *p_dkh, *p_dal, *p_dbeta;  // per-slice partial sums
  float* sub_ws;  // per-wavefront sub-chunk start states [N H dv/8][kBwdSubStarts][dk x 8]
};
hipError_t launch_bwd(const BwdArgs& p, hipStream_t stream);

// Chunked backward (kda_bwd_chunk.hip): the forward's states recorded every
// bwd_chunk_len() tokens (slot layout of kda_fwd_chunked_ckpt) and its
// ungated output are computed by the caller into the workspace first.
struct BwdChunkArgs {
  int32_t num_seqs, num_heads, dk, dv;
  int64_t total_tokens;
  bool in_bf16;
  const void *q, *k, *v, *a, *b, *gate;  // gate may be null
  const int32_t* cu_seqlens;
  const float* initial_state;   // may be null
  const float* dy;              // [T, H, dv]
  const float* d_final_state;   // may be null
  const float* o_raw;           // [T, H, dv] ungated forward output
  const float* ckpt;            // states after every bwd_chunk_len() tokens of each sequence
  float* dse;                   // [T / len + N, H, dk x dv]: adjoint state at each chunk's end (tile layout, kda_bwd_chunk.hip)
  float* crec;                  // [T / len + N, H, bwd_chain_record_floats(dk)]: chain operands
  int32_t *cbase, *kbase;       // [N + 1] each: chunk and recorded-state offsets
  float *dq_out, *dk_out, *dv_out, *da_out, *db_out, *dgate_out, *d_s0;  // dgate, d_s0 may be null
};
int bwd_chunk_len();
// fp32 values per (chunk, head) of the adjoint chain's operand record.
int bwd_chain_record_floats(int dk);
// Enqueues the whole chunked backward on `stream`: the chunk plan, the
// adjoint chain on the device's second stream beside the forward `f` (which
// records the states and the ungated output the gradients read), then the
// per-chunk gradients once both are done.
hipError_t launch_bwd_chunked(const BwdChunkArgs& p, const FwdArgs& f, hipStream_t stream);

// The per-device second stream (default priority, created on first use on the
// device of `stream` and kept for the process) that the forward's state
// passes and the backward's adjoint chain run on beside the caller's stream.
hipError_t device_side_stream(hipStream_t stream, hipStream_t* out);

// Compute units of the current device (cached per device).
int device_cus();

hipError_t launch_decode(const DecodeArgs& p, hipStream_t stream);
// kda_segments.hip
hipError_t launch_segment_table(const int32_t* cu_seqlens, int32_t num_seqs, int32_t seg_len,
                                int32_t cap, int32_t* seg_cu, int32_t* seg_off,
                                hipStream_t stream);
hipError_t launch_compose(const ComposeArgs& p, hipStream_t stream);
// kda_layer.hip
hipError_t launch_conv_swish_l2(const ConvArgs& p, hipStream_t stream);
hipError_t launch_rmsnorm_gate(const RmsGateArgs& p, hipStream_t stream);
hipError_t launch_fwd_chunked(const FwdArgs& p, hipStream_t stream);
// bf16-input kernel (kda_chunk_bf16.hip); launch_fwd_chunked dispatches to it.
hipError_t launch_fwd_chunked_bf16(const FwdArgs& p, hipStream_t stream);

}  // namespace kda
