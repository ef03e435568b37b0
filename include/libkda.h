/*
 * libkda.h - C ABI of libkda, a gfx950 (MI355X) implementation of Kimi Delta
 * Attention (KDA), the per-head delta-rule linear-attention token mixer with a
 * channel-wise forget gate described on the page "[Paper Review] Kimi K3: Open
 * Frontier Intelligence", section "Method / Architecture" -> "Kimi Delta
 * Attention (KDA)", and on the page "atlas.lewiswon.me/arch/moonshot-kimi-k3"
 * (overview paragraph).
 *
 * The operation, per sequence n and head h, with state S (dk x dv, row = key
 * channel) carried token by token:
 *     qh = q_t / sqrt(|q_t|^2 + 1e-6),  kh = k_t / sqrt(|k_t|^2 + 1e-6)
 *     g  = -5 * sigmoid(a_t)     per key channel (the lower-bounded
 *                                scaled-sigmoid log-decay, g_min = -5,
 *                                per-head log-scale A_h at its initial 0;
 *                                a caller with a trained A_h folds it into a)
 *     alpha = exp(g),  beta = sigmoid(b_t)
 *     S  = (I - beta kh kh^T) Diag(alpha) S + beta kh v_t^T
 *     o_t = sigmoid(gate_t) * (S^T qh)        (full-rank output gate)
 * The pages' displayed equations were lost in extraction; this is the form
 * their prose describes (retention Diag(alpha) decays the prior state, the
 * delta rule erases the key direction, then k v^T is written with strength
 * beta; the output is read from the updated state).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major, owned by the
 *     caller, 16-byte aligned -- except b, which needs only the alignment of
 *     its element type, and cu_seqlens (4 bytes).  The library never
 *     allocates or frees device memory, retains a pointer past the call, or
 *     synchronises; work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) and ordered by it.
 *   - One exception to statelessness: when the two-pass bf16 forward needs
 *     more than one block of chunk records (very long inputs, e.g. 1M tokens
 *     x 96 heads), it runs each block's state pass on a second stream beside
 *     the next block's record pass.  That stream and five events are created
 *     per device, on the device of the caller's stream, at the first such
 *     call and kept until the process ends; the enqueueing of such calls is
 *     serialised by a mutex, and concurrent calls on one device share the
 *     stream (their state passes run in call order).  The caller's stream
 *     waits for all of it, so the call is still ordered by `stream` alone.
 *     The bf16 backward (kda_bwd_chunked) uses the same per-device stream
 *     for its adjoint chain beside its forward recomputation, with two more
 *     events per device and a mutex of its own, under the same rules.
 *   - Host-checkable problems are reported by the return code BEFORE anything
 *     is enqueued.  Preconditions that live in device memory (cu_seqlens
 *     starting at 0, nondecreasing, ending at total_tokens) are the caller's
 *     responsibility; violating them is undefined behaviour.
 *   - A launch failure is reported as KDA_ERR_HIP.  No C++ exception crosses
 *     the ABI.  Functions may be called from any thread.
 *   - Results are deterministic: repeated calls on the same inputs give
 *     bitwise-identical outputs (no atomics in any reduction).
 */
#ifndef LIBKDA_H
#define LIBKDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 6u

#if defined(__GNUC__)
#define KDA_API __attribute__((visibility("default")))
#else
#define KDA_API
#endif

typedef enum kda_dtype {
  KDA_F32 = 0,  /* IEEE binary32 */
  KDA_BF16 = 1  /* bfloat16 */
} kda_dtype;

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL_POINTER = 1, /* a required pointer (or the shape) is NULL      */
  KDA_ERR_BAD_SHAPE = 2,    /* sizes out of range or inconsistent            */
  KDA_ERR_BAD_DTYPE = 3,    /* unsupported in_dtype / out_dtype              */
  KDA_ERR_MISALIGNED = 4,   /* a tensor pointer is not aligned as required   */
  KDA_ERR_WORKSPACE = 5,    /* workspace missing or smaller than required    */
  KDA_ERR_ALIAS = 6,        /* an output overlaps an input it must not       */
  KDA_ERR_HIP = 7,          /* the HIP runtime rejected a launch             */
  KDA_ERR_SCRATCH = 8       /* kda_fwd_chunked_noalloc: the problem needs    */
                            /* more than its fixed scratch                   */
} kda_status;

/* Problem description shared by both operations. */
typedef struct kda_shape {
  int32_t num_seqs;     /* N >= 0 sequences                                     */
  int64_t total_tokens; /* fwd: packed token count T = cu_seqlens[N];           */
                        /* decode: must equal num_seqs (one token each)         */
  int32_t num_heads;    /* H >= 1                                               */
  int32_t dk;           /* key/query head dim: 64 or 128                        */
  int32_t dv;           /* value head dim: 64 or 128                            */
  kda_dtype in_dtype;   /* dtype of q, k, v, a, b, gate: KDA_F32 or KDA_BF16    */
  kda_dtype out_dtype;  /* dtype of o: KDA_F32 (fp32 output only)               */
} kda_shape;

/* Bytes of device workspace kda_fwd_chunked (and kda_fwd_chunked_ckpt) need
 * for `shape` on the current device.  fp32 inputs: 0.  bf16 inputs run in
 * two passes over 32-token chunks (the chunk operands of every chunk first,
 * in parallel; then the state chain over them) with fewer (sequence, head)
 * pairs than the device has compute units, and at d_k = d_v = 128 also with
 * up to three pairs per four compute units when the records of every chunk
 * fit one block and sequences average at least 1024 tokens; the workspace
 * then holds one block of those chunk records: at most about 4 GiB (more
 * only when 8 chunks of every pair need more), the per-sequence record offsets,
 * the state carried between blocks and b transposed to [H, T] (2 H T
 * bytes).  Otherwise the single fused kernel runs and the size is 0.  The
 * size depends on the shape and the current device's compute-unit count.
 * Errors: KDA_ERR_NULL_POINTER, KDA_ERR_BAD_SHAPE, KDA_ERR_BAD_DTYPE. */
KDA_API kda_status kda_fwd_workspace_bytes(const kda_shape* shape, size_t* bytes);

/* Chunked forward over packed variable-length sequences.
 *
 * Computes the recurrence above for every (sequence, head) with the
 * chunkwise-parallel form the pages name (page "[Paper Review] Kimi K3...",
 * section "Kimi Delta Attention (KDA)": recurrent but parallelisable per
 * chunk; chunks of 16-token tiles whose pairwise decay factors stay inside
 * the bf16 range because g >= -5, "Lower-bounded decay" paragraph; 32-token
 * chunks for bf16 inputs, 64-token chunks for fp32 inputs).  The state is
 * carried across chunks in fp32.
 *
 *   q, k, a      [T, H, dk]   in_dtype
 *   v, gate      [T, H, dv]   in_dtype; gate may be NULL (no output gate)
 *   b            [T, H]       in_dtype (write-strength logit)
 *   cu_seqlens   [N + 1]      int32, device; cu[0] = 0, nondecreasing,
 *                             cu[N] = T; sequence n is tokens [cu[n], cu[n+1])
 *   initial_state [N, H, dk, dv] fp32, or NULL (= zero state)
 *   o            [T, H, dv]   out_dtype (fp32)
 *   final_state  [N, H, dk, dv] fp32, or NULL (= not written); it may be the
 *                same pointer as initial_state (in-place update), but may not
 *                overlap it partially.
 *   workspace    at least kda_fwd_workspace_bytes(shape) bytes, 16-byte
 *                aligned, overlapping no argument (may be NULL when 0 are
 *                required); its contents are scratch
 * A zero-length sequence produces no rows and final_state = initial_state
 * (or zeros).  o must not overlap any input.
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_DTYPE, MISALIGNED, WORKSPACE, ALIAS, HIP. */
KDA_API kda_status kda_fwd_chunked(const kda_shape* shape, const void* q, const void* k, const void* v,
                           const void* a, const void* b, const void* gate,
                           const int32_t* cu_seqlens, const float* initial_state, void* o,
                           float* final_state, void* workspace, size_t workspace_bytes,
                           void* stream);

/* kda_fwd_chunked that also records the state at regular positions of every
 * sequence: the hybrid cache of the serving stack keeps KDA states at fixed
 * token intervals (every 512 tokens on page "atlas.lewiswon.me/...", cache
 * paragraph), so a later request that shares a prefix resumes from the
 * nearest recorded state instead of recomputing it.
 *
 *   ckpt_interval  tokens between recorded states: a positive multiple of 64
 *   ckpt_states    [ckpt_capacity, H, dk, dv] fp32, device.  For sequence n of
 *                  length L_n, slot ckpt_offset(n) + j, j = 0 ..
 *                  floor(L_n / ckpt_interval) - 1, receives the state after the
 *                  first (j + 1) * ckpt_interval tokens of the sequence, where
 *                  ckpt_offset(n) = sum over m < n of floor(L_m / ckpt_interval)
 *                  (kda_fwd_ckpt_count gives the total).  Slots at or beyond
 *                  ckpt_capacity are not written.  May be NULL only when
 *                  ckpt_capacity is 0.  Must not overlap any other argument.
 * Everything else is as for kda_fwd_chunked (same results, bitwise).
 * Errors: as kda_fwd_chunked; BAD_SHAPE also for a bad ckpt_interval or a
 * negative ckpt_capacity. */
KDA_API kda_status kda_fwd_chunked_ckpt(const kda_shape* shape, const void* q, const void* k,
                                const void* v, const void* a, const void* b, const void* gate,
                                const int32_t* cu_seqlens, const float* initial_state, void* o,
                                float* final_state, int32_t ckpt_interval, float* ckpt_states,
                                int64_t ckpt_capacity, void* workspace, size_t workspace_bytes,
                                void* stream);

/* kda_fwd_chunked with the head-wise RMSNorm before the output gate (page
 * "[Paper Review] Kimi K3...", section "Kimi Delta Attention (KDA)",
 * "Full-rank gate" paragraph; weight and epsilon are not printed there):
 *     o_t  = S_t^T qh_t                      (the recurrence above)
 *     y_t  = sigmoid(gate_t) * norm_weight * o_t / sqrt(mean_c(o_t^2) + norm_eps)
 * the mean over the head's dv channels, for every (token, head) row.
 *   norm_weight  [dv] fp32 shared by the heads, or NULL (ones); 16-byte
 *                aligned; not overlapping o, final_state or the workspace
 *   norm_eps     in [0, 1]
 *   o            [T, H, dv] fp32 receives y
 * Everything else (workspace included) as for kda_fwd_chunked.  With bf16
 * inputs and enough (sequence, head) pairs for the two-pass form's
 * whole-head state pass (more than 32 pairs at dv = 128 and fewer pairs
 * than compute units, e.g. 1 x 1M tokens x 96 heads) the norm is applied in
 * the forward's output stage (no extra pass over o); otherwise the forward
 * writes the ungated output and one more pass applies norm and gate in
 * place.  Same results either way up to rounding.
 * Errors: as kda_fwd_chunked; BAD_SHAPE also for norm_eps outside [0, 1]. */
KDA_API kda_status kda_fwd_chunked_rmsnorm_gate(const kda_shape* shape, const void* q,
                                                const void* k, const void* v, const void* a,
                                                const void* b, const void* gate,
                                                const int32_t* cu_seqlens,
                                                const float* initial_state,
                                                const float* norm_weight, float norm_eps,
                                                void* o, float* final_state, void* workspace,
                                                size_t workspace_bytes, void* stream);

/* kda_fwd_chunked for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation and arguments without a workspace.  The scratch the
 * two-pass bf16 form needs (chunk records, carried states, b transposed) is
 * a fixed device array of 256 MiB held by the library on every device it
 * runs on until the process ends; nothing is allocated or freed per call,
 * and no second stream is used (all work on `stream`, blocks of chunks one
 * after another, sized to fit the array).  Limit: 2 H T + 4 N H dk dv bytes
 * (b transposed, carried states) plus 8 chunk records of every (sequence,
 * head) pair (8 x 30,208 bytes at dk = 128) must fit in 256 MiB, else
 * KDA_ERR_SCRATCH and nothing is enqueued -- e.g. 1 x 1,048,576 tokens x 96
 * heads fits, 2 x 1,048,576 x 96 does not.  Shapes that take the fused
 * kernel or fp32 inputs use no scratch at all.  Every call on a device
 * shares that device's array: calls that overlap in time on one device
 * (concurrent streams) race and give undefined results; calls ordered on
 * one stream are safe (each rewrites what it reads).
 * Errors: as kda_fwd_chunked (no WORKSPACE), plus SCRATCH. */
KDA_API kda_status kda_fwd_chunked_noalloc(const kda_shape* shape, const void* q, const void* k,
                                           const void* v, const void* a, const void* b,
                                           const void* gate, const int32_t* cu_seqlens,
                                           const float* initial_state, void* o,
                                           float* final_state, void* stream);

/* Number of state slots kda_fwd_chunked_ckpt fills for HOST-resident
 * cu_seqlens [num_seqs + 1] (same validity rules as the device array).
 * Errors: NULL_POINTER, BAD_SHAPE (num_seqs < 0, bad interval, decreasing
 * offsets). */
KDA_API kda_status kda_fwd_ckpt_count(int32_t num_seqs, const int32_t* cu_seqlens_host,
                              int32_t ckpt_interval, int64_t* count);

/* ---- Segment-transition form (context parallelism) -----------------------
 * KDA context parallelism (page "[Paper Review] Kimi K3...", section
 * "Infrastructure: how to actually run trillion-scale", KDA co-design item)
 * computes the state transition of every segment of a sequence on its own and
 * composes the transitions associatively, so segments proceed in parallel and
 * only fixed-size states cross segment boundaries.  For one segment and head,
 * the recurrence is affine in its start state S0:
 *     S_end = M S0 + S_loc
 * with M (dk x dk) the product of the per-token factors
 * (I - beta kh kh^T) Diag(alpha) over the segment, latest on the left, and
 * S_loc (dk x dv) the state the segment reaches from S0 = 0.
 */

/* Transitions of segments given as packed sequences (each sequence of
 * cu_seqlens is one segment; shape as for kda_fwd_chunked; gate, q and the
 * initial state play no part).
 *   k, a [T, H, dk]; v [T, H, dv]; b [T, H]   in_dtype
 *   trans [N, H, dk, dv + dk] fp32 out: row r of (n, h) holds S_loc[r, 0..dv)
 *         followed by M[r, 0..dk).  An empty segment gives S_loc = 0, M = I.
 * trans must not overlap any input.
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_DTYPE, MISALIGNED, ALIAS, HIP. */
KDA_API kda_status kda_segment_transition(const kda_shape* shape, const void* k, const void* v,
                                          const void* a, const void* b,
                                          const int32_t* cu_seqlens, float* trans, void* stream);

/* Composition of segment transitions, in token order, for every sequence n
 * and head h.  Sequence n owns segments seg_offsets[n] .. seg_offsets[n+1]-1:
 *     S = initial_state[n, h] (or 0);  for each segment j:  S <- M_j S + S_loc_j
 *   seg_offsets [num_seqs + 1] int32, device; 0 = seg_offsets[0] <=
 *               ... <= seg_offsets[num_seqs] <= num_segments (caller's duty)
 *   trans       [num_segments, H, dk, dv + dk] fp32 (kda_segment_transition)
 *   initial_state [num_seqs, H, dk, dv] fp32 or NULL (zero)
 *   seg_start   [num_segments, H, dk, dv] fp32 out or NULL: S before segment j
 *   final_state [num_seqs, H, dk, dv] fp32 out or NULL: S after the last
 *               segment; may be exactly initial_state (in place).
 * Outputs must not overlap inputs or each other otherwise.
 * Errors: NULL_POINTER, BAD_SHAPE, MISALIGNED, ALIAS, HIP. */
KDA_API kda_status kda_segment_compose(int32_t num_seqs, int32_t num_segments, int32_t num_heads,
                                       int32_t dk, int32_t dv, const int32_t* seg_offsets,
                                       const float* trans, const float* initial_state,
                                       float* seg_start, float* final_state, void* stream);

/* Bytes of workspace kda_fwd_chunked_kcp needs for `shape` and segment_len
 * (0 when the automatic choice is the direct form).
 * Errors: NULL_POINTER, BAD_SHAPE (bad segment_len, too many segments),
 * BAD_DTYPE. */
KDA_API kda_status kda_fwd_kcp_workspace_bytes(const kda_shape* shape, int32_t segment_len,
                                               size_t* bytes);

/* kda_fwd_chunked evaluated in segment-transition form on one GPU: every
 * sequence is cut into segments of segment_len tokens (the last may be
 * shorter); the transitions of all segments are formed in parallel, composed
 * in order, and every segment is then run through the chunked forward from its
 * true start state.  For few (sequence, head) pairs and long sequences this
 * keeps many more compute units busy than the direct form.  Results equal
 * kda_fwd_chunked up to rounding (not bitwise).
 *   segment_len  a positive multiple of 64, or 0: chosen from the shape and
 *                the current device (the direct form when segmenting would
 *                not pay; then no workspace is used)
 *   workspace    kda_fwd_kcp_workspace_bytes(shape, segment_len) bytes,
 *                16-byte aligned, disjoint from every other argument
 * Everything else as for kda_fwd_chunked.
 * Errors: as kda_fwd_chunked; BAD_SHAPE also for a bad segment_len. */
KDA_API kda_status kda_fwd_chunked_kcp(const kda_shape* shape, const void* q, const void* k,
                                       const void* v, const void* a, const void* b,
                                       const void* gate, const int32_t* cu_seqlens,
                                       const float* initial_state, void* o, float* final_state,
                                       int32_t segment_len, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* ---- Layer operations around the core ------------------------------------
 * Page "[Paper Review] Kimi K3...", section "Kimi Delta Attention (KDA)": the
 * query and key pass through a short convolution, then Swish, and are
 * L2-normalised (projections paragraph); the sigmoid output gate follows a
 * head-wise RMSNorm of the head's output ("Full-rank gate" paragraph).  The
 * pages print neither operation's details; the readings are stated below.
 */

/* Short convolution -> Swish -> L2 normalisation of one projection (q or k),
 * over packed sequences.  For sequence n, head h, channel c and token t:
 *     c_t = sum_{i < width} weight[h, c, width-1-i] * x_{t-i}
 *     s_t = c_t * sigmoid(c_t),   y_t = s_t / sqrt(|s_t|^2 + 1e-6)
 * (|.| over the head's dk channels) -- a causal depthwise convolution within
 * each sequence, no bias; positions before the sequence's first token are
 * taken from state_in, else zero.
 *   shape        num_seqs, total_tokens, num_heads, dk (= the channel count),
 *                in_dtype (of x, y and the states); dv and out_dtype unused
 *   width        1..4
 *   x, y         [T, H, dk] in_dtype; y must not overlap x
 *   weight       [H, dk, width] fp32
 *   cu_seqlens   [N + 1] int32, device, as for kda_fwd_chunked
 *   state_in     [N, H, dk, width-1] in_dtype (oldest position first), or NULL
 *   state_out    same layout, or NULL: the last width-1 inputs of
 *                [state_in, sequence] (the state a following call continues
 *                from; for decode, one token per sequence); may be state_in
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_DTYPE, MISALIGNED, ALIAS, HIP. */
KDA_API kda_status kda_shortconv_swish_l2(const kda_shape* shape, int32_t width, const void* x,
                                          const float* weight, const int32_t* cu_seqlens,
                                          const void* state_in, void* state_out, void* y,
                                          void* stream);

/* Head-wise RMSNorm, then the sigmoid output gate, per (token, head) row:
 *     y = sigmoid(gate) * weight * o / sqrt(mean(o^2) + eps)
 * (mean over the head's dv channels).  o is the core's output computed
 * without a gate (kda_fwd_chunked with gate = NULL).
 *   shape   total_tokens, num_heads, dv, in_dtype (of gate); others unused
 *   o, y    [T, H, dv] fp32; y may be o (in place), no other overlap
 *   gate    [T, H, dv] in_dtype, or NULL (no gate)
 *   weight  [dv] fp32 shared by the heads, or NULL (ones)
 *   eps     0 <= eps <= 1
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_DTYPE, MISALIGNED, ALIAS, HIP. */
KDA_API kda_status kda_rmsnorm_gate(const kda_shape* shape, const float* o, const void* gate,
                                    const float* weight, float eps, float* y, void* stream);

/* ---- Backward -------------------------------------------------------------
 * Training through the KDA mixer (the method page trains it at scale and
 * splits it over devices for training -- section "Infrastructure: how to
 * actually run trillion-scale", KDA co-design item -- but describes no
 * backward).  kda_bwd_chunked computes the gradients of
 *     L = sum_t <dy_t, y_t> + <d_final_state, S_final>
 * (y, S_final the outputs of kda_fwd_chunked on the same inputs) with respect
 * to q, k, v, a, b, gate and initial_state, by the chain rule through the
 * recurrence stated at the top of this header, in reverse token order.
 *   q, k, v, a, b, gate, cu_seqlens, initial_state: as for kda_fwd_chunked
 *   dy             [T, H, dv] fp32
 *   d_final_state  [N, H, dk, dv] fp32, or NULL (zero)
 *   dq, dk, da     [T, H, dk] fp32 out;  dv [T, H, dv] fp32 out;  db [T, H] fp32 out
 *   dgate          [T, H, dv] fp32 out (required when gate is given; unused otherwise)
 *   d_initial_state [N, H, dk, dv] fp32 out, or NULL
 *   workspace      kda_bwd_workspace_bytes(shape) bytes, 16-byte aligned
 * Outputs and workspace must not overlap any input or each other.  The
 * forward is recomputed inside.  bf16 inputs run the chunked form: the states
 * recorded every 32 tokens, the adjoint state carried back across 32-token
 * chunks on the device's second stream (beside the recomputation), then every
 * chunk's gradients in parallel on matrix-core products (bf16 hi + lo
 * operands, fp32 accumulation).  fp32 inputs run the token form in fp32
 * (states every 64 tokens, the adjoint carried token by token).  Results are
 * deterministic (no atomics).
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_DTYPE, MISALIGNED, WORKSPACE, ALIAS, HIP. */
KDA_API kda_status kda_bwd_workspace_bytes(const kda_shape* shape, size_t* bytes);
KDA_API kda_status kda_bwd_chunked(const kda_shape* shape, const void* q, const void* k,
                                   const void* v, const void* a, const void* b,
                                   const void* gate, const int32_t* cu_seqlens,
                                   const float* initial_state, const float* dy,
                                   const float* d_final_state, float* dq, float* dk, float* dv,
                                   float* da, float* db, float* dgate, float* d_initial_state,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* One decode step: one new token for each of N independent sequences, the
 * recurrent update the pages' serving section runs with dedicated decode
 * kernels on the fixed-size d_k x d_v per-head state (page "[Paper Review]
 * Kimi K3...", section "Infrastructure", "Inference serving"; page
 * "atlas.lewiswon.me/...", hybrid-cache paragraph).
 *
 *   q, k, a  [N, H, dk]  in_dtype     v, gate [N, H, dv] in_dtype (gate may be NULL)
 *   b        [N, H]      in_dtype
 *   state    [N, H, dk, dv] fp32, read and updated IN PLACE
 *   o        [N, H, dv]  out_dtype (fp32)
 * shape->total_tokens must equal shape->num_seqs.  o must not overlap state
 * or any input.  The same state layout is read and written by
 * kda_fwd_chunked, so fwd over T tokens followed by one decode step equals fwd
 * over T + 1 tokens (up to rounding).
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_DTYPE, MISALIGNED, ALIAS, HIP. */
KDA_API kda_status kda_decode_step(const kda_shape* shape, const void* q, const void* k, const void* v,
                           const void* a, const void* b, const void* gate, float* state,
                           void* o, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
KDA_API const char* kda_status_str(kda_status status);

/* KDA_ABI_VERSION of the built library. */
KDA_API uint32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBKDA_H */
