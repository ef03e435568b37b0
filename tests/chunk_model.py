"""Test-only fp64 model of the chunkwise-parallel (UT/WY) form of KDA.

It is an independent second formulation of the recurrence, used to pin the
token-by-token oracle: the two agree only if both are right.  It is also the
algebra the GPU chunk kernel implements, so a mistake in the derivation shows
up here on the CPU first.

Chunkwise parallel form: the pages say KDA is recurrent but parallelisable per
chunk (page "[Paper Review] Kimi K3...", section "Kimi Delta Attention (KDA)",
the paragraph after the projections), and that each chunk is split into
16-token tiles whose cumulative log-decay stays in (-80, 0) once the decay is
bounded below by g_min = -5 ("Lower-bounded decay" paragraph).  The displayed
equations are lost, so the form below is derived from the recurrence:

Within a chunk of n <= C tokens with start state S0, b_r = sum_{i<=r} g_i
(per key channel, chunk-local), Gamma_r = exp(b_r):
    A[r,i] = beta_r * sum_c kh[r,c] kh[i,c] exp(b[r,c] - b[i,c])      (i < r)
    P[r,i] =          sum_c qh[r,c] kh[i,c] exp(b[r,c] - b[i,c])      (i <= r)
    T      = I + A
    W      = T^-1 diag(beta) Kbar,   Kbar[i,c] = kh[i,c] Gamma_i[c]
    U0     = T^-1 diag(beta) V
    U      = U0 - W S0
    O      = Qbar S0 + P U,          Qbar[r,c] = qh[r,c] Gamma_r[c]
    S_n    = diag(Gamma_{n-1}) S0 + Kend^T U,  Kend[i,c] = kh[i,c] exp(b[n-1,c] - b[i,c])
The pairwise decay exp(b_r - b_i) is formed as the product of a row factor
exp(b_r - p) <= 1 and a column factor exp(p - b_i), with p the cumulative decay
at the start of row r's 16-token tile; ``tile_factors`` checks the bounds the
pages state for these factors.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6
G_MIN = -5.0
TILE = 16


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def pairwise_decay_tiled(bcum: np.ndarray, check: bool = True) -> np.ndarray:
    """E[r, i, c] = exp(b[r,c] - b[i,c]) for i <= r, built from per-tile
    reference factors; asserts the pages' range statements."""
    n, dk = bcum.shape
    E = np.zeros((n, n, dk))
    for r in range(n):
        t0 = (r // TILE) * TILE
        p = bcum[t0 - 1] if t0 > 0 else np.zeros(dk)     # decay accumulated before the tile
        row = np.exp(bcum[r] - p)                        # in [e^-80, 1]
        for i in range(r + 1):
            col = np.exp(p - bcum[i])                    # <= 1 off the tile, <= e^80 on it
            if check:
                assert np.all(row <= 1.0) and np.all(bcum[r] - p >= -80.0)
                if i < t0:
                    assert np.all(col <= 1.0)
                else:
                    assert np.all(p - bcum[i] <= 80.0)
            E[r, i] = row * col
    return E


def chunk_fwd(q, k, v, a, b, gate, cu_seqlens, s0=None, chunk: int = 64):
    """Same contract as oracle.fwd: returns (o [T,H,dv], s_final [N,H,dk,dv])."""
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu_seqlens) - 1
    o = np.zeros((T, H, dv))
    sf = np.zeros((N, H, dk, dv))
    for n in range(N):
        t_beg, t_end = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        for h in range(H):
            S = np.zeros((dk, dv)) if s0 is None else s0[n, h].astype(np.float64).copy()
            for c0 in range(t_beg, t_end, chunk):
                c1 = min(c0 + chunk, t_end)
                qc, kc, vc = q[c0:c1, h], k[c0:c1, h], v[c0:c1, h]
                qh = qc / np.sqrt((qc * qc).sum(-1, keepdims=True) + EPS)
                kh = kc / np.sqrt((kc * kc).sum(-1, keepdims=True) + EPS)
                g = G_MIN * _sigmoid(a[c0:c1, h])
                beta = _sigmoid(b[c0:c1, h])
                bc = np.cumsum(g, axis=0)
                E = pairwise_decay_tiled(bc)
                nr = c1 - c0
                A = np.zeros((nr, nr))
                P = np.zeros((nr, nr))
                for r in range(nr):
                    for i in range(r + 1):
                        P[r, i] = (qh[r] * kh[i] * E[r, i]).sum()
                        if i < r:
                            A[r, i] = beta[r] * (kh[r] * kh[i] * E[r, i]).sum()
                Tinv = np.linalg.inv(np.eye(nr) + A)
                Gam = np.exp(bc)
                Kbar = kh * Gam
                Qbar = qh * Gam
                Kend = kh * np.exp(bc[-1][None, :] - bc)
                W = Tinv @ (beta[:, None] * Kbar)
                U0 = Tinv @ (beta[:, None] * vc)
                U = U0 - W @ S
                O = Qbar @ S + P @ U
                S = Gam[-1][:, None] * S + Kend.T @ U
                if gate is not None:
                    O = _sigmoid(gate[c0:c1, h]) * O
                o[c0:c1, h] = O
            sf[n, h] = S
    return o, sf
