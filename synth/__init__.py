"""Seeded synthetic inputs for the KDA kernels and their oracle.

This module is the only code shared by the GPU path's tests/benchmark and the
oracle's tests.  It holds no part of the KDA method: it turns
(seed, tensor id, step, element index) into numbers (see ``synth_core.h`` for
the exact definition: SplitMix64 streams, Box-Muller normals, fp64 -> fp32 ->
bf16 round-to-nearest-even) and it states the five workload recipes.

Two fillers produce identical values:
  * ``host_normal``   -- C on the CPU (``libsynth_host.so``, gcc),
  * ``device_normal`` -- a HIP kernel on the GPU (``libsynth_dev.so``, hipcc),
    for tensors too large to generate on the host and upload.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

# Tensor ids in the stream key.
TENSOR = {"q": 1, "k": 2, "v": 3, "a": 4, "b": 5, "gate": 6, "s0": 7, "lengths": 8,
          "conv_w": 9, "conv_state": 10, "norm_w": 11, "o": 12}

F32, BF16 = 0, 1


def build(verbose: bool = False) -> None:
    """Compile both fillers in-tree (gcc for the host, hipcc for gfx950)."""
    cmds = [
        ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-ffp-contract=off", "-std=c11",
         os.path.join(_HERE, "synth_host.c"), "-o", HOST_LIB, "-lm"],
        ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
         "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         os.path.join(_HERE, "synth_dev.hip"), "-o", DEV_LIB],
    ]
    for cmd in cmds:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("synth build failed:\n" + " ".join(cmd) + "\n" + r.stderr)
        if verbose:
            print(" ".join(cmd))


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run synth.build()")
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32]
        lib.synth_fill_normal.restype = ctypes.c_int
        lib.synth_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                          ctypes.c_double, ctypes.c_double, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int]
        lib.synth_uniform_ints.restype = ctypes.c_int
        lib.synth_uniform_ints.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64,
                                           ctypes.c_int32, ctypes.c_int32]
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run synth.build()")
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_fill_normal_dev.restype = ctypes.c_int
        lib.synth_fill_normal_dev.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                              ctypes.c_double, ctypes.c_double, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_void_p]
        lib.synth_key_dev.restype = ctypes.c_uint64
        lib.synth_key_dev.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32]
        _dev = lib
    return _dev


def key(seed: int, tensor: str, step: int = 0) -> int:
    return int(_host_lib().synth_key(seed, TENSOR[tensor], step))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def host_normal(k: int, n_rows: int, row_len: int, *, dtype: int = BF16, mean: float = 0.0,
                std: float = 1.0, row_stride: Optional[int] = None, base: int = 0,
                nthreads: Optional[int] = None) -> np.ndarray:
    """Dense [n_rows, row_len] array; element [r, c] is stream element
    ``base + r * row_stride + c``.  bf16 values come back as uint16 bit patterns."""
    if row_stride is None:
        row_stride = row_len
    out = np.empty((n_rows, row_len), dtype=np.float32 if dtype == F32 else np.uint16)
    rc = _host_lib().synth_fill_normal(out.ctypes.data, dtype, k, mean, std, n_rows, row_len,
                                       row_stride, base, nthreads or _threads())
    if rc != 0:
        raise ValueError("synth_fill_normal: bad argument")
    return out


def uniform_ints(k: int, n: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    if _host_lib().synth_uniform_ints(out.ctypes.data, n, k, lo, hi) != 0:
        raise ValueError("synth_uniform_ints: bad argument")
    return out


def device_normal(out, k: int, *, mean: float = 0.0, std: float = 1.0,
                  row_stride: Optional[int] = None, base: int = 0, stream=None) -> None:
    """Fill a contiguous 2-D (or flattened to [rows, last_dim]) torch GPU tensor
    of dtype float32 or bfloat16 with the same values ``host_normal`` gives."""
    import torch

    assert out.is_cuda and out.is_contiguous()
    dtype = {torch.float32: F32, torch.bfloat16: BF16}[out.dtype]
    row_len = out.shape[-1] if out.dim() > 0 else 1
    n_rows = out.numel() // max(row_len, 1)
    if row_stride is None:
        row_stride = row_len
    if stream is None:
        stream = torch.cuda.current_stream(out.device).cuda_stream
    rc = _dev_lib().synth_fill_normal_dev(out.data_ptr(), dtype, k, mean, std, n_rows, row_len,
                                          row_stride, base, stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal_dev failed ({rc})")


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_f64(arr: np.ndarray) -> np.ndarray:
    """Widen generator output (fp32, or bf16 bit patterns) exactly to fp64."""
    if arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return arr.astype(np.float64)


# ---------------------------------------------------------------------------
# Workload recipes (the five measured/tested configurations).
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    heads: int
    dk: int
    dv: int
    dtype: int                     # F32 or BF16 for q, k, v, a, b, gate
    a_std: float                   # std of the decay logits a
    s0_std: Optional[float]        # None: zero initial state
    fixed_len: Optional[int]       # every sequence this long, or None (drawn)
    len_range: Optional[tuple] = None   # (lo, hi) inclusive when drawn
    decode_steps: int = 0          # >0: decode workload (one token per sequence per step)
    seed: int = 0

    def seq_lens(self) -> List[int]:
        if self.fixed_len is not None:
            return [self.fixed_len] * self.num_seqs
        lo, hi = self.len_range
        return [int(x) for x in uniform_ints(key(self.seed, "lengths"), self.num_seqs, lo, hi)]

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seq_lens())]).astype(np.int64)

    def std_of(self, name: str) -> float:
        return self.a_std if name == "a" else 1.0


SQRT3 = float(np.sqrt(3.0))

WORKLOADS = {
    # fp32 everywhere, 1 x 256 tokens, H=2, d=64; all of q,k,v,a,b,gate ~ N(0,1); S0 = 0.
    0: Workload("kda_fwd_fp32_T256_H2_d64", 1, 2, 64, 64, F32, 1.0, None, 256),
    # bf16 prefill, 4 x 4096 tokens, H=32, d=128; a ~ N(0,3) (variance 3); S0 = 0.
    1: Workload("kda_fwd_bf16_4x4096_H32_d128", 4, 32, 128, 128, BF16, SQRT3, None, 4096),
    # bf16 packed varlen, 16 sequences with lengths uniform on [256, 16384],
    # H=96, d=128; per-sequence S0 ~ N(0, 0.02^2).
    2: Workload("kda_fwd_bf16_varlen16_H96_d128", 16, 96, 128, 128, BF16, SQRT3, 0.02, None,
                (256, 16384)),
    # bf16 long context, 1 x 1,048,576 tokens, H=96, d=128; S0 = 0.
    3: Workload("kda_fwd_bf16_T1M_H96_d128", 1, 96, 128, 128, BF16, SQRT3, None, 1 << 20),
    # decode: 256 sequences x 1 token per step, 64 steps, H=96, d=128;
    # state ~ N(0, 0.02^2) fp32, fresh bf16 tokens per step (step index in the key).
    4: Workload("kda_decode_bf16_N256_H96_d128", 256, 96, 128, 128, BF16, SQRT3, 0.02, 1,
                decode_steps=64),
}

TOKEN_TENSORS = ("q", "k", "v", "a", "b", "gate")


def token_row_len(w: Workload, name: str) -> int:
    """Per-token, per-head element count of a token tensor."""
    return {"q": w.dk, "k": w.dk, "a": w.dk, "v": w.dv, "gate": w.dv, "b": 1}[name]


# ---------------------------------------------------------------------------
# Whole tensors of a workload, on the host (generator output: fp32 arrays or
# bf16 bit patterns as uint16) or on the device (torch tensors, same values).
# ---------------------------------------------------------------------------

def custom_workload(base: Workload, **kw) -> Workload:
    """A copy of a workload recipe with some fields changed."""
    return dataclasses.replace(base, **kw)


def host_tokens(w: Workload, name: str, T: int, step: int = 0) -> np.ndarray:
    """Token tensor [T, H, L] (b: [T, H]) of workload w."""
    L = token_row_len(w, name)
    arr = host_normal(key(w.seed, name, step), T * w.heads, L, dtype=w.dtype, std=w.std_of(name))
    return arr.reshape(T, w.heads) if name == "b" else arr.reshape(T, w.heads, L)


def host_head_slice(w: Workload, name: str, t0: int, t1: int, h: int,
                    step: int = 0) -> np.ndarray:
    """Tokens [t0, t1) of head h only: [t1 - t0, L] (b: [t1 - t0])."""
    L = token_row_len(w, name)
    arr = host_normal(key(w.seed, name, step), t1 - t0, L, dtype=w.dtype, std=w.std_of(name),
                      row_stride=w.heads * L, base=(t0 * w.heads + h) * L)
    return arr[:, 0] if name == "b" else arr


def host_state(w: Workload, num_seqs: int) -> Optional[np.ndarray]:
    """Initial states [N, H, dk, dv] fp32, or None for a zero start."""
    if w.s0_std is None:
        return None
    n = num_seqs * w.heads * w.dk
    return host_normal(key(w.seed, "s0"), n, w.dv, dtype=F32,
                       std=w.s0_std).reshape(num_seqs, w.heads, w.dk, w.dv)


def host_state_item(w: Workload, n: int, h: int) -> np.ndarray:
    """Initial state [dk, dv] of sequence n, head h."""
    base = (n * w.heads + h) * w.dk * w.dv
    return host_normal(key(w.seed, "s0"), w.dk, w.dv, dtype=F32, std=w.s0_std, base=base)


def host_inputs(w: Workload, T: int, step: int = 0):
    return {name: host_tokens(w, name, T, step) for name in TOKEN_TENSORS}


def to_torch(arr: np.ndarray, device="cuda"):
    """Host generator output as a torch tensor (bf16 bit patterns -> bfloat16)."""
    import torch

    if arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr)
    return t.to(device)


def torch_dtype(w: Workload):
    import torch

    return torch.float32 if w.dtype == F32 else torch.bfloat16


def device_tokens(w: Workload, name: str, T: int, step: int = 0, device="cuda"):
    """Token tensor generated directly on the device (same values as host_tokens)."""
    import torch

    L = token_row_len(w, name)
    shape = (T, w.heads) if name == "b" else (T, w.heads, L)
    t = torch.empty(shape, dtype=torch_dtype(w), device=device)
    if t.numel():
        device_normal(t.view(-1, L), key(w.seed, name, step), std=w.std_of(name))
    return t


def device_state(w: Workload, num_seqs: int, device="cuda"):
    """Initial states generated on the device (same values as host_state)."""
    import torch

    if w.s0_std is None:
        return None
    t = torch.empty((num_seqs, w.heads, w.dk, w.dv), dtype=torch.float32, device=device)
    device_normal(t.view(-1, w.dv), key(w.seed, "s0"), std=w.s0_std)
    return t
