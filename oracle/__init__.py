"""fp64 CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``delta_rule_linear_kda_amd``) never imports it and shares no code
with it.

The computation is the plain token-by-token recurrence written in
``kda_ref.c`` (plain C, fp64).  Its steps follow the page "[Paper Review] Kimi
K3: Open Frontier Intelligence", section "Kimi Delta Attention (KDA)": the
channel-wise forget gate Diag(alpha_t) on the prior state, the delta-rule
erase (I - beta_t k_t k_t^T) and write beta_t k_t v_t^T, L2-normalised q and
k, the lower-bounded scaled-sigmoid log-decay g = g_min * sigmoid(a) with
g_min = -5, beta = sigmoid(b), and the full-rank sigmoid output gate.

Every function here is pinned by tests in ``tests/test_oracle_pins.py``
against closed forms, brute-force matrix products, a chunked-algebra model
and the pages' bounds; nothing here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "libkda_ref.so")

EPS = 1e-6
G_MIN = -5.0


def build(verbose: bool = False) -> None:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           os.path.join(_HERE, "kda_ref.c"), "-o", LIB, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + r.stderr)
    if verbose:
        print(" ".join(cmd))


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run oracle.build()")
        lib = ctypes.CDLL(LIB)
        dp = ctypes.c_void_p
        lib.kda_ref_fwd.restype = ctypes.c_int
        lib.kda_ref_fwd.argtypes = [ctypes.c_int32, dp, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                    ctypes.c_int]
        lib.kda_ref_segment_transition.restype = ctypes.c_int
        lib.kda_ref_segment_transition.argtypes = [ctypes.c_int32, dp, ctypes.c_int32,
                                                   ctypes.c_int32, ctypes.c_int32, dp, dp, dp,
                                                   dp, dp, ctypes.c_int]
        lib.kda_ref_bwd.restype = ctypes.c_int
        lib.kda_ref_bwd.argtypes = [ctypes.c_int32, dp, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32] + [dp] * 16 + [ctypes.c_int]
        lib.kda_ref_decode_step.restype = ctypes.c_int
        lib.kda_ref_decode_step.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, dp, dp, dp, dp, dp, dp, dp, dp,
                                            ctypes.c_int]
        _lib = lib
    return _lib


def _f64(x: Optional[np.ndarray]) -> Optional[np.ndarray]:
    if x is None:
        return None
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(x: Optional[np.ndarray]):
    return None if x is None else x.ctypes.data


def threads() -> int:
    """Worker threads for the oracle: the cores this process may run on,
    capped at 16 (the host share that goes with one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fwd(q, k, v, a, b, gate, cu_seqlens, s0=None, *, nthreads: Optional[int] = None):
    """Token recurrence over packed sequences.

    q, k, a: [T, H, dk]; v, gate: [T, H, dv] (gate may be None); b: [T, H];
    cu_seqlens: [N+1]; s0: [N, H, dk, dv] or None.
    Returns (o [T, H, dv], s_final [N, H, dk, dv]) in fp64."""
    q, k, v, a, b, gate, s0 = map(_f64, (q, k, v, a, b, gate, s0))
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu) - 1
    assert cu[-1] == T and k.shape == q.shape and a.shape == q.shape and b.shape == (T, H)
    o = np.zeros((T, H, dv))
    sf = np.zeros((N, H, dk, dv))
    rc = _L().kda_ref_fwd(N, cu.ctypes.data, H, dk, dv, _p(q), _p(k), _p(v), _p(a), _p(b),
                          _p(gate), _p(s0), o.ctypes.data, sf.ctypes.data,
                          nthreads or threads())
    if rc != 0:
        raise ValueError("kda_ref_fwd: bad argument")
    return o, sf


def decode_step(q, k, v, a, b, gate, state, *, nthreads: Optional[int] = None):
    """One token per sequence.  q, k, a: [N, H, dk]; v, gate: [N, H, dv];
    b: [N, H]; state: [N, H, dk, dv] fp64, updated IN PLACE.  Returns o."""
    q, k, v, a, b, gate = map(_f64, (q, k, v, a, b, gate))
    assert state.dtype == np.float64 and state.flags.c_contiguous
    N, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((N, H, dv))
    rc = _L().kda_ref_decode_step(N, H, dk, dv, _p(q), _p(k), _p(v), _p(a), _p(b), _p(gate),
                                  state.ctypes.data, o.ctypes.data, nthreads or threads())
    if rc != 0:
        raise ValueError("kda_ref_decode_step: bad argument")
    return o


def segment_transition(k, v, a, b, cu_seqlens, *, nthreads: Optional[int] = None):
    """Transition of every segment (one segment per sequence of cu_seqlens):
    the recurrence maps a start state S0 to M S0 + S_loc.  Page "[Paper
    Review] Kimi K3...", section "Infrastructure: how to actually run
    trillion-scale", KDA co-design item (a cumulative transition plus a
    locally generated state).  Returns fp64 [N, H, dk, dv + dk]: per row
    S_loc then M."""
    k, v, a, b = map(_f64, (k, v, a, b))
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    T, H, dk = k.shape
    dv = v.shape[2]
    N = len(cu) - 1
    assert cu[-1] == T and a.shape == k.shape and b.shape == (T, H)
    tr = np.zeros((N, H, dk, dv + dk))
    rc = _L().kda_ref_segment_transition(N, cu.ctypes.data, H, dk, dv, _p(k), _p(v), _p(a),
                                         _p(b), tr.ctypes.data, nthreads or threads())
    if rc != 0:
        raise ValueError("kda_ref_segment_transition: bad argument")
    return tr


def segment_compose(seg_offsets, trans, dv: int, s0=None):
    """Chains segment transitions in token order, per sequence n and head h:
    S = s0[n, h] (or 0), then S <- M_j S + S_loc_j for the segments
    j = seg_offsets[n] .. seg_offsets[n+1]-1 (associative composition of the
    same KDA co-design item).  Returns (seg_start [S, H, dk, dv]: the state
    before each segment, final [N, H, dk, dv])."""
    trans = np.asarray(trans, dtype=np.float64)
    off = np.asarray(seg_offsets, dtype=np.int64)
    S_, H, dk, w = trans.shape
    assert w == dv + dk
    N = len(off) - 1
    starts = np.zeros((S_, H, dk, dv))
    final = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if s0 is None else np.array(s0[n, h], dtype=np.float64)
            for j in range(off[n], off[n + 1]):
                starts[j, h] = S
                S_loc, M = trans[j, h, :, :dv], trans[j, h, :, dv:]
                S = M @ S + S_loc
            final[n, h] = S
    return starts, final


def bwd(q, k, v, a, b, gate, cu_seqlens, s0, dy, d_sfinal=None, *,
        nthreads: Optional[int] = None):
    """Gradients of sum_t <dy_t, y_t> + <d_sfinal, S_final> (the outputs of
    ``fwd``) with respect to q, k, v, a, b, gate, s0, by reverse-mode chain
    rule through the token recurrence (``kda_ref_bwd``).  Returns a dict of
    fp64 arrays: dq, dk, dv, da, db, dgate (None without gate), ds0."""
    q, k, v, a, b, gate, s0, dy, d_sfinal = map(_f64, (q, k, v, a, b, gate, s0, dy, d_sfinal))
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(cu) - 1
    out = {"dq": np.zeros((T, H, dk)), "dk": np.zeros((T, H, dk)), "dv": np.zeros((T, H, dv)),
           "da": np.zeros((T, H, dk)), "db": np.zeros((T, H)),
           "dgate": np.zeros((T, H, dv)) if gate is not None else None,
           "ds0": np.zeros((N, H, dk, dv))}
    rc = _L().kda_ref_bwd(N, cu.ctypes.data, H, dk, dv, _p(q), _p(k), _p(v), _p(a), _p(b),
                          _p(gate), _p(s0), _p(dy), _p(d_sfinal), _p(out["dq"]), _p(out["dk"]),
                          _p(out["dv"]), _p(out["da"]), _p(out["db"]), _p(out["dgate"]),
                          _p(out["ds0"]), nthreads or threads())
    if rc != 0:
        raise ValueError("kda_ref_bwd: bad argument")
    return out
