"""fp64 oracle for the KDA layer operations around the core recurrence.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the product
library shares no code with it.

Page "[Paper Review] Kimi K3: Open Frontier Intelligence", section "Kimi
Delta Attention (KDA)":
  * the per-head projections paragraph: query and key pass through a short
    convolution, then Swish, then L2 normalisation;
  * the "Full-rank gate" paragraph: the sigmoid output gate follows a
    head-wise RMSNorm of the head's output.
The pages print neither the convolution's width and weight layout nor the
RMSNorm's weight and epsilon; the readings used here are:
  * short convolution: causal and depthwise over tokens, within a sequence,
    width W; weight [H, d, W] with w[..., W - 1] on the current token and
    w[..., W - 1 - i] on the token i steps back; positions before a
    sequence's first token come from an optional carried state
    [N, H, d, W - 1] (oldest first), else zero; no bias;
  * Swish: s = c * sigmoid(c);
  * L2 normalisation over the head's d channels with eps = 1e-6 under the
    root, as the core's own normalisation;
  * head-wise RMSNorm over the head's d_v channels: o / sqrt(mean(o^2) + eps),
    times a weight [d_v] shared by the heads, then times sigmoid(gate).
Every function here is written out from those definitions, token by token.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

EPS_L2 = 1e-6


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def shortconv_swish_l2(x, w, cu_seqlens, state_in=None) -> Tuple[np.ndarray, np.ndarray]:
    """x [T, H, d]; w [H, d, W]; cu_seqlens [N+1]; state_in [N, H, d, W-1] or
    None.  Returns (y [T, H, d], state_out [N, H, d, W-1]) in fp64, where
    state_out holds the last W-1 inputs of each sequence (the carried state
    continued through the sequence)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, d = x.shape
    W = w.shape[2]
    N = len(cu) - 1
    y = np.zeros((T, H, d))
    state_out = np.zeros((N, H, d, W - 1))
    for n in range(N):
        for h in range(H):
            # inputs of this sequence and head, preceded by its carried history
            hist = (np.zeros((W - 1, d)) if state_in is None
                    else np.asarray(state_in[n, h], dtype=np.float64).T)   # [W-1, d]
            seq = np.concatenate([hist, x[cu[n]:cu[n + 1], h]], axis=0)    # [W-1+L, d]
            for t in range(cu[n + 1] - cu[n]):
                c = np.zeros(d)
                for i in range(W):             # i steps back from the current token
                    c += w[h, :, W - 1 - i] * seq[W - 1 + t - i]
                s = c * _sigmoid(c)
                y[cu[n] + t, h] = s / np.sqrt(np.dot(s, s) + EPS_L2)
            if W > 1:
                state_out[n, h] = seq[len(seq) - (W - 1):].T
    return y, state_out


def rmsnorm_gate(o, gate, weight, eps: float) -> np.ndarray:
    """o [T, H, dv]; gate [T, H, dv] or None; weight [dv] or None (ones).
    Returns y = sigmoid(gate) * weight * o / sqrt(mean(o^2) + eps), the mean
    over each (token, head) row, fp64."""
    o = np.asarray(o, dtype=np.float64)
    T, H, dv = o.shape
    wt = np.ones(dv) if weight is None else np.asarray(weight, dtype=np.float64)
    y = np.zeros_like(o)
    for t in range(T):
        for h in range(H):
            row = o[t, h]
            r = row / np.sqrt(np.mean(row * row) + eps) * wt
            if gate is not None:
                r = r * _sigmoid(np.asarray(gate[t, h], dtype=np.float64))
            y[t, h] = r
    return y
