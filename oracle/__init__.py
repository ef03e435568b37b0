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
