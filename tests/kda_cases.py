"""Helpers shared by the tests: seeded inputs of the five workloads, on the
host (for the oracle) or on the device (for the kernels), and the error
metric.  Inputs only ever flow host -> oracle and host/device-generator ->
kernel; nothing the kernels produce is fed to the oracle."""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

import synth

TOL_F32 = 1e-4   # max |gpu - ref| / RMS(ref), fp32-input path
TOL_BF16 = 2e-2  # same, bf16-input path


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |got_i - ref_i| / RMS(ref) over the whole array."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref))) / rms


# The seeded generators' whole-tensor helpers live in synth/; re-exported
# here for the tests.
host_tokens = synth.host_tokens
host_head_slice = synth.host_head_slice
host_state = synth.host_state
host_state_item = synth.host_state_item
host_inputs = synth.host_inputs
to_torch = synth.to_torch
torch_dtype = synth.torch_dtype
device_tokens = synth.device_tokens
device_state = synth.device_state
custom_workload = synth.custom_workload


def f64(x: Optional[np.ndarray]) -> Optional[np.ndarray]:
    return None if x is None else synth.to_f64(x)



class ErrAcc:
    """max |got - ref| and sum ref^2 accumulated over pieces of a tensor, so
    that rel_err of a tensor too large to hold can be formed slice by slice."""

    def __init__(self):
        self.mx, self.ss, self.n = 0.0, 0.0, 0

    def add(self, got: np.ndarray, ref: np.ndarray) -> None:
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        if ref.size:
            self.mx = max(self.mx, float(np.max(np.abs(got - ref))))
            self.ss += float(np.sum(ref * ref))
            self.n += ref.size

    def err(self) -> float:
        rms = (self.ss / self.n) ** 0.5 if self.n else 0.0
        return self.mx / rms if rms > 0 else self.mx


def oracle_stream(fetch, n_tokens: int, s0, gate: bool = True, slice_tokens: int = 65536,
                  on_slice=None):
    """The oracle over tokens [0, n_tokens) of some heads of one sequence, in
    slices with the state carried (the same recurrence as one run; bounded
    host memory).  fetch(t0, t1) -> dict of f64 arrays q, k, v, a, gate
    [n, Hs, L] and b [n, Hs]; on_slice(t0, t1, o_ref) receives each slice's
    outputs.  Returns the final state [1, Hs, dk, dv]."""
    import oracle

    state = s0
    for t0 in range(0, n_tokens, slice_tokens):
        t1 = min(n_tokens, t0 + slice_tokens)
        x = fetch(t0, t1)
        o_ref, state = oracle.fwd(x["q"], x["k"], x["v"], x["a"], x["b"],
                                  x["gate"] if gate else None, [0, t1 - t0], state)
        if on_slice is not None:
            on_slice(t0, t1, o_ref)
    return state


def device_rows_f64(t, t0: int, t1: int, heads) -> np.ndarray:
    """Rows [t0, t1) of heads `heads` of a device token tensor, widened exactly
    to fp64 on the host."""
    import torch

    x = t[t0:t1, heads].contiguous()
    if x.dtype == torch.bfloat16:
        return synth.to_f64(x.view(torch.int16).cpu().numpy().view(np.uint16))
    return x.cpu().numpy().astype(np.float64)


def rel_err_device(got, ref, rows: int = 65536) -> float:
    """max |got - ref| / RMS(ref) over whole device tensors, accumulated on
    the device in row slices (no full-size temporaries or host copies)."""
    mx, ss, n = 0.0, 0.0, 0
    for r0 in range(0, ref.shape[0], rows):
        g = got[r0:r0 + rows].double()
        f = ref[r0:r0 + rows].double()
        mx = max(mx, float((g - f).abs().max()))
        ss += float((f * f).sum())
        n += f.numel()
    return mx / (ss / n) ** 0.5
