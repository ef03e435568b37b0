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


def host_tokens(w: synth.Workload, name: str, T: int, step: int = 0) -> np.ndarray:
    """Whole token tensor [T, H, L] (b: [T, H]) as generator output (fp32 or
    bf16 bit patterns)."""
    L = synth.token_row_len(w, name)
    arr = synth.host_normal(synth.key(w.seed, name, step), T * w.heads, L, dtype=w.dtype,
                            std=w.std_of(name))
    return arr.reshape(T, w.heads) if name == "b" else arr.reshape(T, w.heads, L)


def host_head_slice(w: synth.Workload, name: str, t0: int, t1: int, h: int,
                    step: int = 0) -> np.ndarray:
    """Tokens [t0, t1) of head h only: [t1 - t0, L] (b: [t1 - t0])."""
    L = synth.token_row_len(w, name)
    arr = synth.host_normal(synth.key(w.seed, name, step), t1 - t0, L, dtype=w.dtype,
                            std=w.std_of(name), row_stride=w.heads * L, base=(t0 * w.heads + h) * L)
    return arr[:, 0] if name == "b" else arr


def host_state(w: synth.Workload, num_seqs: int) -> Optional[np.ndarray]:
    if w.s0_std is None:
        return None
    n = num_seqs * w.heads * w.dk
    return synth.host_normal(synth.key(w.seed, "s0"), n, w.dv, dtype=synth.F32,
                             std=w.s0_std).reshape(num_seqs, w.heads, w.dk, w.dv)


def host_state_item(w: synth.Workload, n: int, h: int) -> np.ndarray:
    base = (n * w.heads + h) * w.dk * w.dv
    return synth.host_normal(synth.key(w.seed, "s0"), w.dk, w.dv, dtype=synth.F32,
                             std=w.s0_std, base=base)


def to_torch(arr: np.ndarray, device="cuda"):
    import torch

    if arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr)
    return t.to(device)


def torch_dtype(w: synth.Workload):
    import torch

    return torch.float32 if w.dtype == synth.F32 else torch.bfloat16


def device_tokens(w: synth.Workload, name: str, T: int, step: int = 0, device="cuda"):
    """Token tensor generated directly on the device (same values as host_tokens)."""
    import torch

    L = synth.token_row_len(w, name)
    shape = (T, w.heads) if name == "b" else (T, w.heads, L)
    t = torch.empty(shape, dtype=torch_dtype(w), device=device)
    if t.numel():
        synth.device_normal(t.view(-1, L), synth.key(w.seed, name, step), std=w.std_of(name))
    return t


def device_state(w: synth.Workload, num_seqs: int, device="cuda"):
    import torch

    if w.s0_std is None:
        return None
    t = torch.empty((num_seqs, w.heads, w.dk, w.dv), dtype=torch.float32, device=device)
    synth.device_normal(t.view(-1, w.dv), synth.key(w.seed, "s0"), std=w.s0_std)
    return t


def host_inputs(w: synth.Workload, T: int, step: int = 0) -> Dict[str, np.ndarray]:
    return {name: host_tokens(w, name, T, step) for name in synth.TOKEN_TENSORS}


def f64(x: Optional[np.ndarray]) -> Optional[np.ndarray]:
    return None if x is None else synth.to_f64(x)


def custom_workload(base: synth.Workload, **kw) -> synth.Workload:
    import dataclasses

    return dataclasses.replace(base, **kw)
