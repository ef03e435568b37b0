/*
 * kda_ref.h - fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this.  The product path
 * (libkda) never does; it shares no code with this file.
 *
 * What it computes (page "[Paper Review] Kimi K3: Open Frontier
 * Intelligence", section "Kimi Delta Attention (KDA)", and the lower-bounded
 * decay paragraph after it): for each sequence n and head h, with state
 * S (dk x dv) starting at s0[n,h] (or zero), token by token in order:
 *     qh = q_t / sqrt(|q_t|^2 + eps),  kh = k_t / sqrt(|k_t|^2 + eps),  eps = 1e-6
 *     g  = -5 * sigmoid(a_t)           (per key channel; g_min = -5)
 *     alpha = exp(g),  beta = sigmoid(b_t)
 *     S  = (I - beta kh kh^T) Diag(alpha) S + beta kh v_t^T
 *     o_t = S^T qh,   y_t = sigmoid(gate_t) * o_t   (gate NULL: y_t = o_t)
 * and s_final[n,h] = S after the last token.
 *
 * Layouts (row-major, T = cu_seqlens[num_seqs] packed tokens):
 *   q, k, a : [T, H, dk]      v, gate, o : [T, H, dv]      b : [T, H]
 *   s0, s_final, state : [num_seqs, H, dk, dv]   (row = key channel)
 * All buffers are host fp64, owned by the caller.
 */
#ifndef KDA_REF_H
#define KDA_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_REF_EPS 1e-6
#define KDA_REF_GMIN (-5.0)

/* Chunk-free token recurrence over packed variable-length sequences.
 * cu_seqlens: host int64 [num_seqs + 1], cu[0] = 0, nondecreasing.
 * gate, s0 may be NULL; s_final may be NULL (not written).
 * nthreads <= 0 means one thread.  Returns 0, or -1 on a bad argument. */
int kda_ref_fwd(int32_t num_seqs, const int64_t* cu_seqlens, int32_t H, int32_t dk, int32_t dv,
                const double* q, const double* k, const double* v, const double* a,
                const double* b, const double* gate, const double* s0, double* o,
                double* s_final, int nthreads);

/* One token per sequence: q, k, a [N, H, dk]; v, gate [N, H, dv]; b [N, H];
 * state [N, H, dk, dv] updated in place; o [N, H, dv].  Same recurrence. */
int kda_ref_decode_step(int32_t num_seqs, int32_t H, int32_t dk, int32_t dv, const double* q,
                        const double* k, const double* v, const double* a, const double* b,
                        const double* gate, double* state, double* o, int nthreads);

/* Segment transitions: every sequence of cu_seqlens is one segment.  For
 * segment n and head h, the recurrence maps a start state S0 to M S0 + S_loc;
 * trans [num_seqs, H, dk, dv + dk] receives, per row r, S_loc[r, :] then
 * M[r, :], with M = F_last ... F_first, F_t = (I - beta kh kh^T) Diag(alpha)
 * formed densely, and S_loc the state from S0 = 0.  Returns 0 or -1. */
int kda_ref_segment_transition(int32_t num_seqs, const int64_t* cu_seqlens, int32_t H,
                               int32_t dk, int32_t dv, const double* k, const double* v,
                               const double* a, const double* b, double* trans, int nthreads);

/* Backward: gradients of L = sum_t <dy_t, y_t> + <d_sfinal, S_final> with
 * respect to q, k, v, a, b, gate and s0, by the chain rule through the same
 * token recurrence in reverse.  dy [T, H, dv]; d_sfinal [N, H, dk, dv] or
 * NULL; outputs dq, dk, da [T, H, dk], dv [T, H, dv], db [T, H], dgate
 * [T, H, dv] (may be NULL; zero where gate is NULL), ds0 [N, H, dk, dv] or
 * NULL.  Returns 0 or -1. */
int kda_ref_bwd(int32_t num_seqs, const int64_t* cu_seqlens, int32_t H, int32_t dk, int32_t dv,
                const double* q, const double* k, const double* v, const double* a,
                const double* b, const double* gate, const double* s0, const double* dy,
                const double* d_sfinal, double* dq, double* dk_out, double* dv_out, double* da,
                double* db, double* dgate, double* ds0, int nthreads);

#ifdef __cplusplus
}
#endif

#endif /* KDA_REF_H */
