// kda_api.cpp - the libkda C ABI (include/libkda.h): argument validation and
// dispatch.  Every host-checkable problem is rejected here before any HIP
// call, so an invalid call enqueues nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/libkda.h"
#include "kda_internal.h"

namespace {

bool valid_dim(int32_t d) { return d == 64 || d == 128; }

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// b is read one element at a time: natural alignment of its dtype suffices.
bool aligned_elem(const void* p, kda_dtype dt) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) & (dt == KDA_BF16 ? 1u : 3u)) == 0;
}

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
  Span() = default;
  Span(const void* p, uint64_t bytes)
      : lo(reinterpret_cast<uintptr_t>(p)), hi(reinterpret_cast<uintptr_t>(p) + bytes) {
    if (!p || bytes == 0) lo = hi = 0;
  }
  bool empty() const { return lo == hi; }
};

bool overlap(const Span& x, const Span& y) {
  return !x.empty() && !y.empty() && x.lo < y.hi && y.lo < x.hi;
}

// Element counts must stay far from overflow of byte offsets.
constexpr int64_t kMaxElems = int64_t(1) << 56;

kda_status check_shape(const kda_shape* s) {
  if (!s) return KDA_ERR_NULL_POINTER;
  if (s->in_dtype != KDA_F32 && s->in_dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (s->out_dtype != KDA_F32) return KDA_ERR_BAD_DTYPE;
  if (s->num_seqs < 0 || s->total_tokens < 0 || s->num_heads < 1) return KDA_ERR_BAD_SHAPE;
  if (!valid_dim(s->dk) || !valid_dim(s->dv)) return KDA_ERR_BAD_SHAPE;
  if (s->total_tokens > kMaxElems / (int64_t(s->num_heads) * 128)) return KDA_ERR_BAD_SHAPE;
  if (int64_t(s->num_seqs) * s->num_heads > (int64_t(1) << 31) / 4) return KDA_ERR_BAD_SHAPE;
  return KDA_OK;
}

struct Sizes {
  uint64_t qk, v, b, o, st;
};

Sizes byte_sizes(const kda_shape* s, int64_t tokens) {
  const uint64_t es = s->in_dtype == KDA_BF16 ? 2 : 4;
  const uint64_t th = uint64_t(tokens) * uint64_t(s->num_heads);
  Sizes z;
  z.qk = th * uint64_t(s->dk) * es;
  z.v = th * uint64_t(s->dv) * es;
  z.b = th * es;
  z.o = th * uint64_t(s->dv) * 4;
  z.st = uint64_t(s->num_seqs) * uint64_t(s->num_heads) * uint64_t(s->dk) * uint64_t(s->dv) * 4;
  return z;
}

}  // namespace

extern "C" {

uint32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_str(kda_status st) {
  switch (st) {
    case KDA_OK: return "KDA_OK: success";
    case KDA_ERR_NULL_POINTER: return "KDA_ERR_NULL_POINTER: a required pointer is NULL";
    case KDA_ERR_BAD_SHAPE: return "KDA_ERR_BAD_SHAPE: sizes out of range or inconsistent";
    case KDA_ERR_BAD_DTYPE: return "KDA_ERR_BAD_DTYPE: unsupported dtype";
    case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED: a tensor pointer is not aligned as required";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
    case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: an output overlaps an input";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime rejected a launch";
    case KDA_ERR_SCRATCH:
      return "KDA_ERR_SCRATCH: the problem needs more scratch than the no-allocation forward holds";
  }
  return "unknown kda_status";
}

}  // extern "C"

namespace {

// bf16 inputs take the two-pass form when the fused kernel's workgroups
// ((sequence, head) pairs, times two d_v slices when that still fits in one
// round) would leave compute units of the current device idle.  With up to
// three pairs per four compute units at d_k = d_v = 128 they also take it
// when every chunk record fits one block and sequences average at least 1024
// tokens: the record pass then runs on the whole GPU and the state chain
// alone, at a quarter (64-column slices) to under half (whole heads) of the
// fused kernel's time per chunk (4 x 4096 tokens x 32 heads: 0.53-0.56
// against 0.66 ms; 6 x 4096 x 32: 0.75 against 0.83 ms; at 8 x 4096 x 32
// the record pass's share tips it: 0.95 against 0.74 ms).  Otherwise the
// fused kernel, which has no record round trip.
bool fwd_uses_split(const kda_shape& s) {
  if (s.in_dtype != KDA_BF16 || s.num_seqs <= 0) return false;
  const int64_t items = int64_t(s.num_seqs) * s.num_heads, cus = kda::device_cus();
  const int64_t fused_wgs = s.dv == 128 && 2 * items <= cus ? 2 * items : items;
  if (fused_wgs < cus) return true;
  return s.dk == 128 && s.dv == 128 && 4 * items <= 3 * cus &&
         s.total_tokens >= 1024 * int64_t(s.num_seqs) &&
         kda::split_layout(s.num_seqs, s.total_tokens, s.num_heads, s.dk, s.dv).blocks == 1;
}

}  // namespace

extern "C" {

kda_status kda_fwd_workspace_bytes(const kda_shape* shape, size_t* bytes) {
  if (!bytes) return KDA_ERR_NULL_POINTER;
  const kda_status st = check_shape(shape);
  if (st != KDA_OK) return st;
  const kda_shape& s = *shape;
  // the two-pass form's chunk records live here
  *bytes = fwd_uses_split(s)
               ? size_t(kda::split_layout(s.num_seqs, s.total_tokens, s.num_heads, s.dk, s.dv)
                            .total)
               : 0;
  return KDA_OK;
}

}  // extern "C"

namespace {

bool valid_interval(int32_t iv) { return iv > 0 && iv % 64 == 0; }

// Checks shared by the forward entry points, after check_shape.  Sets *empty
// when there is nothing to do (no sequences).
kda_status check_fwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                     const void* a, const void* b, const void* gate, const int32_t* cu_seqlens,
                     const float* initial_state, void* o, float* final_state,
                     int32_t ckpt_interval, float* ckpt, int64_t ckpt_capacity, bool* empty) {
  const kda_shape& s = *shape;
  *empty = s.num_seqs == 0;
  if (s.num_seqs == 0) return s.total_tokens == 0 ? KDA_OK : KDA_ERR_BAD_SHAPE;
  if (!cu_seqlens) return KDA_ERR_NULL_POINTER;
  if (s.total_tokens > 0 && (!q || !k || !v || !a || !b || !o)) return KDA_ERR_NULL_POINTER;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return KDA_ERR_MISALIGNED;
  for (const void* p : {q, k, v, a, gate, (const void*)initial_state, (const void*)o,
                        (const void*)final_state})
    if (!aligned16(p)) return KDA_ERR_MISALIGNED;
  if (!aligned_elem(b, s.in_dtype)) return KDA_ERR_MISALIGNED;

  const Sizes z = byte_sizes(shape, s.total_tokens);
  const Span in[] = {Span(q, z.qk), Span(k, z.qk), Span(v, z.v), Span(a, z.qk), Span(b, z.b),
                     Span(gate, z.v), Span(cu_seqlens, uint64_t(s.num_seqs + 1) * 4),
                     Span(initial_state, z.st)};
  const Span so(o, z.o), sf(final_state, z.st);
  for (const Span& x : in)
    if (overlap(so, x)) return KDA_ERR_ALIAS;
  if (overlap(so, sf)) return KDA_ERR_ALIAS;
  for (int i = 0; i < 7; ++i)
    if (overlap(sf, in[i])) return KDA_ERR_ALIAS;
  // final_state may be exactly initial_state (in place), never a partial overlap.
  if (overlap(sf, in[7]) && (const void*)final_state != (const void*)initial_state)
    return KDA_ERR_ALIAS;
  if (ckpt_interval != 0) {  // recorded states: disjoint from everything else
    const uint64_t slot = uint64_t(s.num_heads) * uint64_t(s.dk) * uint64_t(s.dv) * 4;
    if (uint64_t(ckpt_capacity) > uint64_t(kMaxElems) / slot) return KDA_ERR_BAD_SHAPE;
    const Span sc(ckpt, uint64_t(ckpt_capacity) * slot);
    for (const Span& x : in)
      if (overlap(sc, x)) return KDA_ERR_ALIAS;
    if (overlap(sc, so) || overlap(sc, sf)) return KDA_ERR_ALIAS;
  }
  return KDA_OK;
}

kda::FwdArgs fwd_args(const kda_shape& s, const void* q, const void* k, const void* v,
                      const void* a, const void* b, const void* gate, const int32_t* cu_seqlens,
                      const float* initial_state, void* o, float* final_state) {
  kda::FwdArgs p;
  p.num_seqs = s.num_seqs;
  p.num_heads = s.num_heads;
  p.dk = s.dk;
  p.dv = s.dv;
  p.total_tokens = s.total_tokens;
  p.in_bf16 = s.in_dtype == KDA_BF16;
  p.q = q; p.k = k; p.v = v; p.a = a; p.b = b; p.gate = gate;
  p.cu_seqlens = cu_seqlens;
  p.initial_state = initial_state;
  p.o = o;
  p.final_state = final_state;
  return p;
}

kda_status fwd_impl(const kda_shape* shape, const void* q, const void* k, const void* v,
                    const void* a, const void* b, const void* gate, const int32_t* cu_seqlens,
                    const float* initial_state, void* o, float* final_state,
                    int32_t ckpt_interval, float* ckpt, int64_t ckpt_capacity, void* workspace,
                    size_t workspace_bytes, void* stream, bool norm = false,
                    const float* norm_weight = nullptr, float norm_eps = 0.f) {
  kda_status st = check_shape(shape);
  if (st != KDA_OK) return st;
  const kda_shape& s = *shape;
  size_t need = 0;
  kda_fwd_workspace_bytes(shape, &need);
  if (workspace_bytes < need || (need > 0 && !workspace)) return KDA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return KDA_ERR_MISALIGNED;
  bool empty = false;
  st = check_fwd(shape, q, k, v, a, b, gate, cu_seqlens, initial_state, o, final_state,
                 ckpt_interval, ckpt, ckpt_capacity, &empty);
  if (st != KDA_OK || empty) return st;
  if (need > 0) {  // the workspace is disjoint from every argument
    const Sizes z = byte_sizes(shape, s.total_tokens);
    const Span ws(workspace, need);
    for (const Span& x : {Span(q, z.qk), Span(k, z.qk), Span(v, z.v), Span(a, z.qk),
                          Span(b, z.b), Span(gate, z.v),
                          Span(cu_seqlens, uint64_t(s.num_seqs + 1) * 4),
                          Span(initial_state, z.st), Span(o, z.o), Span(final_state, z.st)})
      if (overlap(ws, x)) return KDA_ERR_ALIAS;
    if (ckpt_interval != 0 &&
        overlap(ws, Span(ckpt, uint64_t(ckpt_capacity) * uint64_t(s.num_heads) *
                                   uint64_t(s.dk) * uint64_t(s.dv) * 4)))
      return KDA_ERR_ALIAS;
  }

  if (norm) {  // the norm's weight: read-only, disjoint from the output
    if (!(norm_eps >= 0.f) || norm_eps > 1.f) return KDA_ERR_BAD_SHAPE;
    if (!aligned16(norm_weight)) return KDA_ERR_MISALIGNED;
    const Sizes z = byte_sizes(shape, s.total_tokens);
    const Span sw(norm_weight, uint64_t(s.dv) * 4);
    if (overlap(sw, Span(o, z.o)) || overlap(sw, Span(final_state, z.st)) ||
        overlap(sw, Span(workspace, need)))
      return KDA_ERR_ALIAS;
  }

  kda::FwdArgs p = fwd_args(s, q, k, v, a, b, gate, cu_seqlens, initial_state, o, final_state);
  p.ckpt_interval = ckpt_capacity > 0 ? ckpt_interval : 0;
  p.ckpt = ckpt;
  p.ckpt_capacity = ckpt_capacity;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool split = fwd_uses_split(s);
  // The head-wise RMSNorm runs in the output stage of the two-pass form's
  // whole-head state pass; elsewhere the forward writes the ungated output
  // and one more pass applies norm and gate in place.
  const bool norm_fused = norm && split && kda::split_whole_head(s.num_seqs, s.num_heads, s.dv);
  if (norm_fused) {
    p.norm = true;
    p.norm_weight = norm_weight;
    p.norm_eps = norm_eps;
  } else if (norm) {
    p.gate = nullptr;
  }
  hipError_t e = split ? kda::launch_fwd_split_bf16(p, workspace, hs)
                       : kda::launch_fwd_chunked(p, hs);
  if (e != hipSuccess) return KDA_ERR_HIP;
  if (norm && !norm_fused && s.total_tokens > 0) {
    kda::RmsGateArgs r;
    r.num_heads = s.num_heads;
    r.dv = s.dv;
    r.total_tokens = s.total_tokens;
    r.in_bf16 = s.in_dtype == KDA_BF16;
    r.o = static_cast<const float*>(o);
    r.gate = gate;
    r.weight = norm_weight;
    r.eps = norm_eps;
    r.y = static_cast<float*>(o);
    if ((e = kda::launch_rmsnorm_gate(r, hs)) != hipSuccess) return KDA_ERR_HIP;
  }
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_fwd_chunked(const kda_shape* shape, const void* q, const void* k, const void* v,
                           const void* a, const void* b, const void* gate,
                           const int32_t* cu_seqlens, const float* initial_state, void* o,
                           float* final_state, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return fwd_impl(shape, q, k, v, a, b, gate, cu_seqlens, initial_state, o, final_state, 0,
                  nullptr, 0, workspace, workspace_bytes, stream);
}

kda_status kda_fwd_chunked_ckpt(const kda_shape* shape, const void* q, const void* k,
                                const void* v, const void* a, const void* b, const void* gate,
                                const int32_t* cu_seqlens, const float* initial_state, void* o,
                                float* final_state, int32_t ckpt_interval, float* ckpt_states,
                                int64_t ckpt_capacity, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (!valid_interval(ckpt_interval) || ckpt_capacity < 0) {
    const kda_status st = check_shape(shape);
    return st != KDA_OK ? st : KDA_ERR_BAD_SHAPE;
  }
  if (ckpt_capacity > 0 && !ckpt_states) return KDA_ERR_NULL_POINTER;
  if (!aligned16(ckpt_states)) return KDA_ERR_MISALIGNED;
  return fwd_impl(shape, q, k, v, a, b, gate, cu_seqlens, initial_state, o, final_state,
                  ckpt_interval, ckpt_states, ckpt_capacity, workspace, workspace_bytes, stream);
}

kda_status kda_fwd_chunked_rmsnorm_gate(const kda_shape* shape, const void* q, const void* k,
                                        const void* v, const void* a, const void* b,
                                        const void* gate, const int32_t* cu_seqlens,
                                        const float* initial_state, const float* norm_weight,
                                        float norm_eps, void* o, float* final_state,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(shape, q, k, v, a, b, gate, cu_seqlens, initial_state, o, final_state, 0,
                  nullptr, 0, workspace, workspace_bytes, stream, true, norm_weight, norm_eps);
}

kda_status kda_fwd_chunked_noalloc(const kda_shape* shape, const void* q, const void* k,
                                   const void* v, const void* a, const void* b, const void* gate,
                                   const int32_t* cu_seqlens, const float* initial_state, void* o,
                                   float* final_state, void* stream) {
  kda_status st = check_shape(shape);
  if (st != KDA_OK) return st;
  const kda_shape& s = *shape;
  bool empty = false;
  st = check_fwd(shape, q, k, v, a, b, gate, cu_seqlens, initial_state, o, final_state, 0,
                 nullptr, 0, &empty);
  if (st != KDA_OK || empty) return st;
  kda::FwdArgs p = fwd_args(s, q, k, v, a, b, gate, cu_seqlens, initial_state, o, final_state);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (!fwd_uses_split(s))  // the kernels of these shapes use no workspace
    return kda::launch_fwd_chunked(p, hs) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  kda::SplitLayout w;
  if (!kda::noalloc_layout(s.num_seqs, s.total_tokens, s.num_heads, s.dk, s.dv, &w))
    return KDA_ERR_SCRATCH;
  void* ws = nullptr;
  if (kda::noalloc_scratch(hs, &ws) != hipSuccess) return KDA_ERR_HIP;
  return kda::launch_fwd_split_bf16(p, ws, hs, &w) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_fwd_ckpt_count(int32_t num_seqs, const int32_t* cu_seqlens_host,
                              int32_t ckpt_interval, int64_t* count) {
  if (!count || (num_seqs > 0 && !cu_seqlens_host)) return KDA_ERR_NULL_POINTER;
  if (num_seqs < 0 || !valid_interval(ckpt_interval)) return KDA_ERR_BAD_SHAPE;
  int64_t total = 0;
  for (int32_t n = 0; n < num_seqs; ++n) {
    const int64_t len = int64_t(cu_seqlens_host[n + 1]) - int64_t(cu_seqlens_host[n]);
    if (len < 0 || (n == 0 && cu_seqlens_host[0] != 0)) return KDA_ERR_BAD_SHAPE;
    total += len / ckpt_interval;
  }
  *count = total;
  return KDA_OK;
}

kda_status kda_decode_step(const kda_shape* shape, const void* q, const void* k, const void* v,
                           const void* a, const void* b, const void* gate, float* state,
                           void* o, void* stream) {
  kda_status st = check_shape(shape);
  if (st != KDA_OK) return st;
  const kda_shape& s = *shape;
  if (s.total_tokens != s.num_seqs) return KDA_ERR_BAD_SHAPE;
  if (s.num_seqs == 0) return KDA_OK;
  if (!q || !k || !v || !a || !b || !state || !o) return KDA_ERR_NULL_POINTER;
  for (const void* p : {q, k, v, a, gate, (const void*)state, (const void*)o})
    if (!aligned16(p)) return KDA_ERR_MISALIGNED;
  if (!aligned_elem(b, s.in_dtype)) return KDA_ERR_MISALIGNED;
  const Sizes z = byte_sizes(shape, s.num_seqs);
  const Span in[] = {Span(q, z.qk), Span(k, z.qk), Span(v, z.v), Span(a, z.qk), Span(b, z.b),
                     Span(gate, z.v)};
  const Span so(o, z.o), ss(state, z.st);
  for (const Span& x : in)
    if (overlap(so, x) || overlap(ss, x)) return KDA_ERR_ALIAS;
  if (overlap(so, ss)) return KDA_ERR_ALIAS;

  kda::DecodeArgs p;
  p.num_seqs = s.num_seqs;
  p.num_heads = s.num_heads;
  p.dk = s.dk;
  p.dv = s.dv;
  p.in_bf16 = s.in_dtype == KDA_BF16;
  p.q = q; p.k = k; p.v = v; p.a = a; p.b = b; p.gate = gate;
  p.state = state;
  p.o = o;
  if (kda::launch_decode(p, static_cast<hipStream_t>(stream)) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Segment-transition form (context parallelism on one GPU).
// ---------------------------------------------------------------------------
namespace {

constexpr int32_t kSegQuantum = 64;        // segment lengths: multiples of both chunk sizes
constexpr int64_t kMinAutoSegment = 4096;  // shorter automatic segments do not pay

uint64_t round_up(uint64_t x, uint64_t m) { return (x + m - 1) / m * m; }

// Workspace of kda_fwd_chunked_kcp for segment length L: segment table,
// per-sequence segment offsets, [S_loc | M] per (segment, head) and the start
// state of every segment.  `cap` bounds the segment count:
// sum_n ceil(L_n / L) <= floor(T / L) + N.
struct KcpLayout {
  int64_t cap;
  uint64_t seg_cu, seg_off, trans, start, total;
};

KcpLayout kcp_layout(const kda_shape& s, int64_t L) {
  KcpLayout w;
  w.cap = s.total_tokens / L + s.num_seqs;
  const uint64_t hk = uint64_t(s.num_heads) * uint64_t(s.dk);
  w.seg_cu = 0;
  w.seg_off = round_up(uint64_t(w.cap + 1) * 4, 256);
  w.trans = w.seg_off + round_up(uint64_t(s.num_seqs + 1) * 4, 256);
  w.start = w.trans + round_up(uint64_t(w.cap) * hk * uint64_t(s.dv + s.dk) * 4, 256);
  w.total = w.start + round_up(uint64_t(w.cap) * hk * uint64_t(s.dv) * 4, 256);
  return w;
}

// Segment length for `segment_len` (0 = automatic); *L = 0 selects the direct
// form.  The segment form costs about three chunk passes per segment and head
// (the transition over d_v + d_k columns, then the forward), spread over the
// whole GPU, against one pass per (sequence, head) for the direct form, which
// runs at most 2 workgroups per pair.  The automatic choice therefore
// segments when there are at most cus / 4 (sequence, head) pairs, and aims at
// about one segment per compute unit and head.
kda_status kcp_resolve(const kda_shape& s, int32_t segment_len, int64_t* L) {
  if (segment_len < 0 || segment_len % kSegQuantum != 0) return KDA_ERR_BAD_SHAPE;
  *L = segment_len;
  if (segment_len == 0) {
    const int64_t items = int64_t(s.num_seqs) * s.num_heads;
    const int cus = kda::device_cus();
    if (items == 0 || 4 * items > cus) return KDA_OK;
    const int64_t target = std::max<int64_t>(2, cus / s.num_heads);
    const int64_t len = (int64_t)round_up((s.total_tokens + target - 1) / target, kSegQuantum);
    if (len >= kMinAutoSegment && s.total_tokens >= 2 * len * s.num_seqs) *L = len;
  }
  if (*L == 0) return KDA_OK;
  // The segment count must stay within the kernels' limits.
  const KcpLayout w = kcp_layout(s, *L);
  if (w.cap + 1 > INT32_MAX || w.cap * s.num_heads > (int64_t(1) << 31) / 4 ||
      w.total > uint64_t(kMaxElems))
    return KDA_ERR_BAD_SHAPE;
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_segment_transition(const kda_shape* shape, const void* k, const void* v,
                                  const void* a, const void* b, const int32_t* cu_seqlens,
                                  float* trans, void* stream) {
  kda_status st = check_shape(shape);
  if (st != KDA_OK) return st;
  const kda_shape& s = *shape;
  if (s.num_seqs == 0) return s.total_tokens == 0 ? KDA_OK : KDA_ERR_BAD_SHAPE;
  if (!cu_seqlens || !trans) return KDA_ERR_NULL_POINTER;
  if (s.total_tokens > 0 && (!k || !v || !a || !b)) return KDA_ERR_NULL_POINTER;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return KDA_ERR_MISALIGNED;
  for (const void* p : {k, v, a, (const void*)trans})
    if (!aligned16(p)) return KDA_ERR_MISALIGNED;
  if (!aligned_elem(b, s.in_dtype)) return KDA_ERR_MISALIGNED;
  const Sizes z = byte_sizes(shape, s.total_tokens);
  const uint64_t tb = uint64_t(s.num_seqs) * uint64_t(s.num_heads) * uint64_t(s.dk) *
                      uint64_t(s.dv + s.dk) * 4;
  const Span st_(trans, tb);
  for (const Span& x : {Span(k, z.qk), Span(v, z.v), Span(a, z.qk), Span(b, z.b),
                        Span(cu_seqlens, uint64_t(s.num_seqs + 1) * 4)})
    if (overlap(st_, x)) return KDA_ERR_ALIAS;
  kda::FwdArgs p = fwd_args(s, nullptr, k, v, a, b, nullptr, cu_seqlens, nullptr, nullptr, nullptr);
  p.transition = trans;
  if (kda::launch_fwd_chunked(p, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_HIP;
  return KDA_OK;
}

kda_status kda_segment_compose(int32_t num_seqs, int32_t num_segments, int32_t num_heads,
                               int32_t dk, int32_t dv, const int32_t* seg_offsets,
                               const float* trans, const float* initial_state, float* seg_start,
                               float* final_state, void* stream) {
  if (num_seqs < 0 || num_segments < 0 || num_heads < 1 || !valid_dim(dk) || !valid_dim(dv))
    return KDA_ERR_BAD_SHAPE;
  if (int64_t(num_seqs) * num_heads > (int64_t(1) << 31) / 4 ||
      int64_t(num_segments) * num_heads > (int64_t(1) << 31) / 4)
    return KDA_ERR_BAD_SHAPE;
  if (num_seqs == 0) return KDA_OK;
  if (!seg_offsets || (num_segments > 0 && !trans)) return KDA_ERR_NULL_POINTER;
  if ((reinterpret_cast<uintptr_t>(seg_offsets) & 3u) != 0) return KDA_ERR_MISALIGNED;
  for (const void* p : {(const void*)trans, (const void*)initial_state, (const void*)seg_start,
                        (const void*)final_state})
    if (!aligned16(p)) return KDA_ERR_MISALIGNED;
  const uint64_t hk = uint64_t(num_heads) * uint64_t(dk);
  const Span so(seg_offsets, uint64_t(num_seqs + 1) * 4);
  const Span stt(trans, uint64_t(num_segments) * hk * uint64_t(dv + dk) * 4);
  const Span si(initial_state, uint64_t(num_seqs) * hk * uint64_t(dv) * 4);
  const Span ss(seg_start, uint64_t(num_segments) * hk * uint64_t(dv) * 4);
  const Span sf(final_state, uint64_t(num_seqs) * hk * uint64_t(dv) * 4);
  for (const Span& x : {so, stt, si, sf})
    if (overlap(ss, x)) return KDA_ERR_ALIAS;
  if (overlap(sf, so) || overlap(sf, stt)) return KDA_ERR_ALIAS;
  if (overlap(sf, si) && (const void*)final_state != (const void*)initial_state)
    return KDA_ERR_ALIAS;
  kda::ComposeArgs p;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.dk = dk;
  p.dv = dv;
  p.seg_offsets = seg_offsets;
  p.trans = trans;
  p.initial_state = initial_state;
  p.seg_start = seg_start;
  p.final_state = final_state;
  if (kda::launch_compose(p, static_cast<hipStream_t>(stream)) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

kda_status kda_fwd_kcp_workspace_bytes(const kda_shape* shape, int32_t segment_len,
                                       size_t* bytes) {
  if (!bytes) return KDA_ERR_NULL_POINTER;
  kda_status st = check_shape(shape);
  if (st != KDA_OK) return st;
  int64_t L = 0;
  st = kcp_resolve(*shape, segment_len, &L);
  if (st != KDA_OK) return st;
  if (L == 0) return kda_fwd_workspace_bytes(shape, bytes);  // direct form
  *bytes = size_t(kcp_layout(*shape, L).total);
  return KDA_OK;
}

kda_status kda_fwd_chunked_kcp(const kda_shape* shape, const void* q, const void* k,
                               const void* v, const void* a, const void* b, const void* gate,
                               const int32_t* cu_seqlens, const float* initial_state, void* o,
                               float* final_state, int32_t segment_len, void* workspace,
                               size_t workspace_bytes, void* stream) {
  kda_status st = check_shape(shape);
  if (st != KDA_OK) return st;
  const kda_shape& s = *shape;
  int64_t L = 0;
  st = kcp_resolve(s, segment_len, &L);
  if (st != KDA_OK) return st;
  if (L == 0)  // direct form
    return fwd_impl(shape, q, k, v, a, b, gate, cu_seqlens, initial_state, o, final_state, 0,
                    nullptr, 0, workspace, workspace_bytes, stream);
  const KcpLayout w = kcp_layout(s, L);
  if (workspace_bytes < w.total || !workspace) return KDA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KDA_ERR_MISALIGNED;
  bool empty = false;
  st = check_fwd(shape, q, k, v, a, b, gate, cu_seqlens, initial_state, o, final_state, 0,
                 nullptr, 0, &empty);
  if (st != KDA_OK || empty) return st;
  {  // the workspace is disjoint from every argument
    const Sizes z = byte_sizes(shape, s.total_tokens);
    const Span ws(workspace, w.total);
    for (const Span& x : {Span(q, z.qk), Span(k, z.qk), Span(v, z.v), Span(a, z.qk),
                          Span(b, z.b), Span(gate, z.v),
                          Span(cu_seqlens, uint64_t(s.num_seqs + 1) * 4),
                          Span(initial_state, z.st), Span(o, z.o), Span(final_state, z.st)})
      if (overlap(ws, x)) return KDA_ERR_ALIAS;
  }
  unsigned char* base = static_cast<unsigned char*>(workspace);
  int32_t* seg_cu = reinterpret_cast<int32_t*>(base + w.seg_cu);
  int32_t* seg_off = reinterpret_cast<int32_t*>(base + w.seg_off);
  float* trans = reinterpret_cast<float*>(base + w.trans);
  float* start = reinterpret_cast<float*>(base + w.start);
  hipStream_t hs = static_cast<hipStream_t>(stream);

  // 1. segments  2. their transitions  3. composition (start states and the
  // final state)  4. the chunked forward of every segment from its start state.
  if (kda::launch_segment_table(cu_seqlens, s.num_seqs, (int32_t)L, (int32_t)w.cap, seg_cu,
                                seg_off, hs) != hipSuccess)
    return KDA_ERR_HIP;
  kda::FwdArgs pa = fwd_args(s, nullptr, k, v, a, b, nullptr, seg_cu, nullptr, nullptr, nullptr);
  pa.num_seqs = (int32_t)w.cap;
  pa.transition = trans;
  if (kda::launch_fwd_chunked(pa, hs) != hipSuccess) return KDA_ERR_HIP;
  kda::ComposeArgs pc;
  pc.num_seqs = s.num_seqs;
  pc.num_heads = s.num_heads;
  pc.dk = s.dk;
  pc.dv = s.dv;
  pc.seg_offsets = seg_off;
  pc.trans = trans;
  pc.initial_state = initial_state;
  pc.seg_start = start;
  pc.final_state = final_state;
  if (kda::launch_compose(pc, hs) != hipSuccess) return KDA_ERR_HIP;
  kda::FwdArgs pb = fwd_args(s, q, k, v, a, b, gate, seg_cu, start, o, nullptr);
  pb.num_seqs = (int32_t)w.cap;
  if (kda::launch_fwd_chunked(pb, hs) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Layer operations around the core: short convolution -> Swish -> L2 front,
// head-wise RMSNorm -> sigmoid gate back.
// ---------------------------------------------------------------------------
extern "C" {

kda_status kda_shortconv_swish_l2(const kda_shape* shape, int32_t width, const void* x,
                                  const float* weight, const int32_t* cu_seqlens,
                                  const void* state_in, void* state_out, void* y,
                                  void* stream) {
  kda_status st = check_shape(shape);
  if (st != KDA_OK) return st;
  const kda_shape& s = *shape;
  if (width < 1 || width > 4) return KDA_ERR_BAD_SHAPE;
  if (s.num_seqs == 0) return s.total_tokens == 0 ? KDA_OK : KDA_ERR_BAD_SHAPE;
  if (!cu_seqlens || !weight) return KDA_ERR_NULL_POINTER;
  if (s.total_tokens > 0 && (!x || !y)) return KDA_ERR_NULL_POINTER;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return KDA_ERR_MISALIGNED;
  for (const void* p : {x, (const void*)weight, (const void*)y})
    if (!aligned16(p)) return KDA_ERR_MISALIGNED;
  for (const void* p : {state_in, (const void*)state_out})
    if (!aligned_elem(p, s.in_dtype)) return KDA_ERR_MISALIGNED;
  const uint64_t es = s.in_dtype == KDA_BF16 ? 2 : 4;
  const uint64_t hk = uint64_t(s.num_heads) * uint64_t(s.dk);
  const Span sx(x, uint64_t(s.total_tokens) * hk * es), sy(y, uint64_t(s.total_tokens) * hk * es);
  const Span sw(weight, hk * uint64_t(width) * 4);
  const Span sc(cu_seqlens, uint64_t(s.num_seqs + 1) * 4);
  const uint64_t stb = uint64_t(s.num_seqs) * hk * uint64_t(width - 1) * es;
  const Span si(state_in, stb), so(state_out, stb);
  for (const Span& in : {sx, sw, sc, si})
    if (overlap(sy, in)) return KDA_ERR_ALIAS;
  if (overlap(sy, so)) return KDA_ERR_ALIAS;
  for (const Span& in : {sx, sw, sc})
    if (overlap(so, in)) return KDA_ERR_ALIAS;
  if (overlap(so, si) && state_out != state_in) return KDA_ERR_ALIAS;
  kda::ConvArgs p;
  p.num_seqs = s.num_seqs;
  p.num_heads = s.num_heads;
  p.dim = s.dk;
  p.width = width;
  p.total_tokens = s.total_tokens;
  p.in_bf16 = s.in_dtype == KDA_BF16;
  p.x = x;
  p.weight = weight;
  p.cu_seqlens = cu_seqlens;
  p.state_in = state_in;
  p.state_out = state_out;
  p.y = y;
  if (kda::launch_conv_swish_l2(p, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_HIP;
  return KDA_OK;
}

kda_status kda_rmsnorm_gate(const kda_shape* shape, const float* o, const void* gate,
                            const float* weight, float eps, float* y, void* stream) {
  kda_status st = check_shape(shape);
  if (st != KDA_OK) return st;
  const kda_shape& s = *shape;
  if (!(eps >= 0.f) || eps > 1.f) return KDA_ERR_BAD_SHAPE;
  if (s.total_tokens == 0) return KDA_OK;
  if (!o || !y) return KDA_ERR_NULL_POINTER;
  for (const void* p : {(const void*)o, gate, (const void*)weight, (const void*)y})
    if (!aligned16(p)) return KDA_ERR_MISALIGNED;
  const uint64_t rowsb = uint64_t(s.total_tokens) * uint64_t(s.num_heads) * uint64_t(s.dv);
  const Span so(o, rowsb * 4), sy(y, rowsb * 4);
  const Span sg(gate, rowsb * (s.in_dtype == KDA_BF16 ? 2 : 4)), sw(weight, uint64_t(s.dv) * 4);
  if (overlap(sy, sg) || overlap(sy, sw)) return KDA_ERR_ALIAS;
  if (overlap(sy, so) && (const void*)y != (const void*)o) return KDA_ERR_ALIAS;
  kda::RmsGateArgs p;
  p.num_heads = s.num_heads;
  p.dv = s.dv;
  p.total_tokens = s.total_tokens;
  p.in_bf16 = s.in_dtype == KDA_BF16;
  p.o = o;
  p.gate = gate;
  p.weight = weight;
  p.eps = eps;
  p.y = y;
  if (kda::launch_rmsnorm_gate(p, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KDA_ERR_HIP;
  return KDA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward.
// ---------------------------------------------------------------------------
namespace {

constexpr int32_t kBwdCkpt = 64;  // tokens between the forward states the token form restarts from
constexpr int32_t kBwdSlice = 8;  // state columns per token-form wavefront

// bf16 inputs run the chunked form (kda_bwd_chunk.hip): the forward's states
// every kda::bwd_chunk_len() tokens, its ungated output, the adjoint state at
// each chunk's end and the chunk offsets.  fp32 inputs run the token form
// (kda_bwd.hip): states every 64 tokens, the ungated output, per-slice
// partial sums and sub-chunk start states.
struct BwdLayout {
  bool chunked;
  uint64_t ckpt, o_raw, p_dqh, p_dkh, p_dal, p_dbeta, sub, dse, crec, cbase, kbase, total;
  int64_t slots;
};

BwdLayout bwd_layout(const kda_shape& s) {
  BwdLayout w{};
  const uint64_t th = uint64_t(s.total_tokens) * uint64_t(s.num_heads);
  const uint64_t st = uint64_t(s.num_heads) * s.dk * s.dv * 4;  // one state per head
  w.chunked = s.in_dtype == KDA_BF16;
  w.ckpt = 0;
  if (w.chunked) {
    const int64_t cl = kda::bwd_chunk_len();
    w.slots = s.total_tokens / cl;  // >= sum over sequences of floor(L_n / cl)
    w.o_raw = round_up(uint64_t(w.slots) * st, 256);
    w.dse = w.o_raw + round_up(th * s.dv * 4, 256);
    const uint64_t chunks = uint64_t(s.total_tokens / cl + s.num_seqs);  // >= sum of ceil(L_n / cl)
    w.crec = w.dse + round_up(chunks * st, 256);
    w.cbase = w.crec + round_up(chunks * uint64_t(s.num_heads) *
                                    uint64_t(kda::bwd_chain_record_floats(s.dk)) * 4,
                                256);
    w.kbase = w.cbase + round_up(uint64_t(s.num_seqs + 1) * 4, 256);
    w.total = w.kbase + round_up(uint64_t(s.num_seqs + 1) * 4, 256);
    return w;
  }
  const uint64_t nsl = uint64_t(s.dv / kBwdSlice);
  w.slots = s.total_tokens / kBwdCkpt;  // >= sum over sequences of floor(L_n / 64)
  w.o_raw = round_up(uint64_t(w.slots) * st, 256);
  w.p_dqh = w.o_raw + round_up(th * s.dv * 4, 256);
  w.p_dkh = w.p_dqh + round_up(nsl * th * s.dk * 4, 256);
  w.p_dal = w.p_dkh + round_up(nsl * th * s.dk * 4, 256);
  w.p_dbeta = w.p_dal + round_up(nsl * th * s.dk * 4, 256);
  w.sub = w.p_dbeta + round_up(nsl * th * 4, 256);
  // per (sequence, head, 8-column slice): the sub-chunk start states of a
  // 64-token chunk, dk x 8 fp32 each
  w.total = w.sub + round_up(uint64_t(s.num_seqs) * uint64_t(s.num_heads) * nsl *
                                 kda::kBwdSubStarts * s.dk * 8 * 4,
                             256);
  return w;
}

}  // namespace

extern "C" {

kda_status kda_bwd_workspace_bytes(const kda_shape* shape, size_t* bytes) {
  if (!bytes) return KDA_ERR_NULL_POINTER;
  const kda_status st = check_shape(shape);
  if (st != KDA_OK) return st;
  const BwdLayout w = bwd_layout(*shape);
  if (w.total > uint64_t(kMaxElems)) return KDA_ERR_BAD_SHAPE;
  *bytes = size_t(w.total);
  return KDA_OK;
}

kda_status kda_bwd_chunked(const kda_shape* shape, const void* q, const void* k, const void* v,
                           const void* a, const void* b, const void* gate,
                           const int32_t* cu_seqlens, const float* initial_state,
                           const float* dy, const float* d_final_state, float* dq, float* dk,
                           float* dv, float* da, float* db, float* dgate, float* d_initial_state,
                           void* workspace, size_t workspace_bytes, void* stream) {
  kda_status st = check_shape(shape);
  if (st != KDA_OK) return st;
  const kda_shape& s = *shape;
  if (s.num_seqs == 0) return s.total_tokens == 0 ? KDA_OK : KDA_ERR_BAD_SHAPE;
  const BwdLayout w = bwd_layout(s);
  if (w.total > uint64_t(kMaxElems)) return KDA_ERR_BAD_SHAPE;
  // the chunked form launches one workgroup per (chunk, head)
  if (w.chunked && (s.total_tokens / kda::bwd_chunk_len() + s.num_seqs) * int64_t(s.num_heads) >
                       int64_t(0x7fffffff))
    return KDA_ERR_BAD_SHAPE;
  if (!cu_seqlens) return KDA_ERR_NULL_POINTER;
  if (s.total_tokens > 0 &&
      (!q || !k || !v || !a || !b || !dy || !dq || !dk || !dv || !da || !db))
    return KDA_ERR_NULL_POINTER;
  if (gate && s.total_tokens > 0 && !dgate) return KDA_ERR_NULL_POINTER;
  if (workspace_bytes < w.total || !workspace) return KDA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return KDA_ERR_MISALIGNED;
  for (const void* p : {q, k, v, a, gate, (const void*)initial_state, (const void*)dy,
                        (const void*)d_final_state, (const void*)dq, (const void*)dk,
                        (const void*)dv, (const void*)da, (const void*)db, (const void*)dgate,
                        (const void*)d_initial_state, (const void*)workspace})
    if (!aligned16(p)) return KDA_ERR_MISALIGNED;
  if (!aligned_elem(b, s.in_dtype)) return KDA_ERR_MISALIGNED;
  {  // outputs and workspace: disjoint from every input and from each other
    const Sizes z = byte_sizes(shape, s.total_tokens);
    const uint64_t th = uint64_t(s.total_tokens) * uint64_t(s.num_heads);
    const Span in[] = {Span(q, z.qk), Span(k, z.qk), Span(v, z.v), Span(a, z.qk), Span(b, z.b),
                       Span(gate, z.v), Span(cu_seqlens, uint64_t(s.num_seqs + 1) * 4),
                       Span(initial_state, z.st), Span(dy, z.o), Span(d_final_state, z.st)};
    const Span out[] = {Span(dq, th * s.dk * 4), Span(dk, th * s.dk * 4), Span(dv, z.o),
                        Span(da, th * s.dk * 4), Span(db, th * 4), Span(dgate, z.o),
                        Span(d_initial_state, z.st), Span(workspace, w.total)};
    for (const Span& o : out)
      for (const Span& i : in)
        if (overlap(o, i)) return KDA_ERR_ALIAS;
    for (size_t i = 0; i < sizeof(out) / sizeof(out[0]); ++i)
      for (size_t j = i + 1; j < sizeof(out) / sizeof(out[0]); ++j)
        if (overlap(out[i], out[j])) return KDA_ERR_ALIAS;
  }
  unsigned char* base = static_cast<unsigned char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // 1. the forward with its states recorded and the ungated output
  kda::FwdArgs f = fwd_args(s, q, k, v, a, b, nullptr, cu_seqlens, initial_state,
                            base + w.o_raw, nullptr);
  f.ckpt_interval = w.chunked ? kda::bwd_chunk_len() : kBwdCkpt;
  f.ckpt = reinterpret_cast<float*>(base + w.ckpt);
  f.ckpt_capacity = w.slots;
  if (w.chunked) {
    // 2. the adjoint chain over chunks (beside the forward), then every
    // chunk's gradients
    kda::BwdChunkArgs c;
    c.num_seqs = s.num_seqs;
    c.num_heads = s.num_heads;
    c.dk = s.dk;
    c.dv = s.dv;
    c.total_tokens = s.total_tokens;
    c.in_bf16 = true;
    c.q = q; c.k = k; c.v = v; c.a = a; c.b = b; c.gate = gate;
    c.cu_seqlens = cu_seqlens;
    c.initial_state = initial_state;
    c.dy = dy;
    c.d_final_state = d_final_state;
    c.o_raw = reinterpret_cast<const float*>(base + w.o_raw);
    c.ckpt = reinterpret_cast<const float*>(base + w.ckpt);
    c.dse = reinterpret_cast<float*>(base + w.dse);
    c.crec = reinterpret_cast<float*>(base + w.crec);
    c.cbase = reinterpret_cast<int32_t*>(base + w.cbase);
    c.kbase = reinterpret_cast<int32_t*>(base + w.kbase);
    c.dq_out = dq; c.dk_out = dk; c.dv_out = dv; c.da_out = da; c.db_out = db;
    c.dgate_out = gate ? dgate : nullptr;
    c.d_s0 = d_initial_state;
    if (kda::launch_bwd_chunked(c, f, hs) != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
  }
  if (kda::launch_fwd_chunked(f, hs) != hipSuccess) return KDA_ERR_HIP;
  // 2. the adjoint recurrence token by token and the reduction over column slices
  kda::BwdArgs p;
  p.num_seqs = s.num_seqs;
  p.num_heads = s.num_heads;
  p.dk = s.dk;
  p.dv = s.dv;
  p.total_tokens = s.total_tokens;
  p.in_bf16 = s.in_dtype == KDA_BF16;
  p.q = q; p.k = k; p.v = v; p.a = a; p.b = b; p.gate = gate;
  p.cu_seqlens = cu_seqlens;
  p.initial_state = initial_state;
  p.dy = dy;
  p.d_final_state = d_final_state;
  p.o_raw = reinterpret_cast<const float*>(base + w.o_raw);
  p.ckpt = reinterpret_cast<const float*>(base + w.ckpt);
  p.dq_out = dq; p.dk_out = dk; p.dv_out = dv; p.da_out = da; p.db_out = db;
  p.dgate_out = gate ? dgate : nullptr;
  p.d_s0 = d_initial_state;
  p.p_dqh = reinterpret_cast<float*>(base + w.p_dqh);
  p.p_dkh = reinterpret_cast<float*>(base + w.p_dkh);
  p.p_dal = reinterpret_cast<float*>(base + w.p_dal);
  p.p_dbeta = reinterpret_cast<float*>(base + w.p_dbeta);
  p.sub_ws = reinterpret_cast<float*>(base + w.sub);
  if (kda::launch_bwd(p, hs) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

}  // extern "C"
