"""delta_rule_linear_kda_amd: Python binding of libkda (Kimi Delta Attention on gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libkda.so`` through its C ABI (``include/libkda.h``); PyTorch
supplies device memory and the current stream.  If the library is missing the
import of any entry point raises -- there is no fallback path.

Entry points (same names as the C ABI):
  * ``fwd_chunked(q, k, v, a, b, gate, cu_seqlens, initial_state=None, ...)``
  * ``decode_step(q, k, v, a, b, gate, state, ...)``
  * ``fwd_workspace_bytes(...)``, ``ckpt_count(...)``, ``status_str(code)``,
    ``abi_version()``
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
STATUS = {
    0: "KDA_OK", 1: "KDA_ERR_NULL_POINTER", 2: "KDA_ERR_BAD_SHAPE", 3: "KDA_ERR_BAD_DTYPE",
    4: "KDA_ERR_MISALIGNED", 5: "KDA_ERR_WORKSPACE", 6: "KDA_ERR_ALIAS", 7: "KDA_ERR_HIP",
}
EXPORTS = ("kda_fwd_workspace_bytes", "kda_fwd_chunked", "kda_fwd_chunked_ckpt",
           "kda_fwd_ckpt_count", "kda_decode_step", "kda_status_str", "kda_abi_version")


class KdaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_str(code)}")


class Shape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int64),
                ("num_heads", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkda.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run delta_rule_linear_kda_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, sp = ctypes.c_void_p, ctypes.POINTER(Shape)
        L.kda_fwd_workspace_bytes.restype = ctypes.c_int
        L.kda_fwd_workspace_bytes.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
        L.kda_fwd_chunked.restype = ctypes.c_int
        L.kda_fwd_chunked.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.c_size_t, vp]
        L.kda_fwd_chunked_ckpt.restype = ctypes.c_int
        L.kda_fwd_chunked_ckpt.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           ctypes.c_int32, vp, ctypes.c_int64, vp,
                                           ctypes.c_size_t, vp]
        L.kda_fwd_ckpt_count.restype = ctypes.c_int
        L.kda_fwd_ckpt_count.argtypes = [ctypes.c_int32, vp, ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_int64)]
        L.kda_decode_step.restype = ctypes.c_int
        L.kda_decode_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.kda_status_str.restype = ctypes.c_char_p
        L.kda_status_str.argtypes = [ctypes.c_int]
        L.kda_abi_version.restype = ctypes.c_uint32
        L.kda_abi_version.argtypes = []
        _lib = L
    return _lib


def status_str(code: int) -> str:
    return lib().kda_status_str(code).decode()


def abi_version() -> int:
    return int(lib().kda_abi_version())


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return KDA_F32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(device, stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def fwd_workspace_bytes(num_seqs: int, total_tokens: int, num_heads: int, dk: int, dv: int,
                        in_dtype: int = KDA_BF16) -> int:
    shape = Shape(num_seqs, total_tokens, num_heads, dk, dv, in_dtype, KDA_F32)
    out = ctypes.c_size_t(0)
    rc = lib().kda_fwd_workspace_bytes(ctypes.byref(shape), ctypes.byref(out))
    if rc != 0:
        raise KdaError(rc, "kda_fwd_workspace_bytes")
    return int(out.value)


def ckpt_count(cu_seqlens_host, interval: int) -> int:
    """Recorded-state slots kda_fwd_chunked_ckpt fills (C ABI
    ``kda_fwd_ckpt_count``) for host offsets ``cu_seqlens_host`` (int32 [N+1])."""
    import numpy as np

    cu = np.ascontiguousarray(cu_seqlens_host, dtype=np.int32)
    out = ctypes.c_int64(0)
    rc = lib().kda_fwd_ckpt_count(int(cu.size) - 1, cu.ctypes.data, int(interval), ctypes.byref(out))
    if rc != 0:
        raise KdaError(rc, "kda_fwd_ckpt_count")
    return int(out.value)


def fwd_chunked(q, k, v, a, b, gate, cu_seqlens, initial_state=None, *,
                output_final_state: bool = True, out=None, final_state=None,
                checkpoint_interval: Optional[int] = None, checkpoints=None,
                stream=None):
    """Chunked KDA forward over packed sequences (C ABI ``kda_fwd_chunked``, or
    ``kda_fwd_chunked_ckpt`` when ``checkpoint_interval`` is given).

    q, k, a: [T, H, dk]; v, gate: [T, H, dv] (gate may be None); b: [T, H]
    (all float32 or all bfloat16); cu_seqlens: int32 [N+1] on the device;
    initial_state: fp32 [N, H, dk, dv] or None.  Returns (o fp32 [T, H, dv],
    final_state fp32 [N, H, dk, dv] or None), plus the recorded states fp32
    [n_ckpt, H, dk, dv] as a third element when ``checkpoint_interval`` is
    given (slot layout: see ``kda_fwd_chunked_ckpt``).  ``final_state`` may be
    passed as the same tensor as ``initial_state`` for an in-place update."""
    import torch

    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.float32, device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    ws_bytes = fwd_workspace_bytes(N, T, H, dk, dv, dt)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    shape = Shape(N, T, H, dk, dv, dt, KDA_F32)
    if checkpoint_interval is None:
        rc = lib().kda_fwd_chunked(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                   _ptr(b), _ptr(gate), _ptr(cu_seqlens), _ptr(initial_state),
                                   _ptr(out), _ptr(final_state), _ptr(ws), ws_bytes,
                                   _stream(q.device, stream))
        if rc != 0:
            raise KdaError(rc, "kda_fwd_chunked")
        return out, final_state
    if checkpoints is None:
        n_ckpt = ckpt_count(cu_seqlens.cpu().numpy(), checkpoint_interval)
        checkpoints = torch.empty((n_ckpt, H, dk, dv), dtype=torch.float32, device=q.device)
    rc = lib().kda_fwd_chunked_ckpt(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                    _ptr(b), _ptr(gate), _ptr(cu_seqlens), _ptr(initial_state),
                                    _ptr(out), _ptr(final_state), int(checkpoint_interval),
                                    _ptr(checkpoints), int(checkpoints.shape[0]), _ptr(ws),
                                    ws_bytes, _stream(q.device, stream))
    if rc != 0:
        raise KdaError(rc, "kda_fwd_chunked_ckpt")
    return out, final_state, checkpoints


def decode_step(q, k, v, a, b, gate, state, *, out=None, stream=None):
    """One decode step (C ABI ``kda_decode_step``): q, k, a [N, H, dk];
    v, gate [N, H, dv]; b [N, H]; state fp32 [N, H, dk, dv] updated in place.
    Returns o fp32 [N, H, dv]."""
    import torch

    N, H, dk = q.shape
    dv = v.shape[2]
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=q.device)
    shape = Shape(N, N, H, dk, dv, _dtype_code(q), KDA_F32)
    rc = lib().kda_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                               _ptr(gate), _ptr(state), _ptr(out), _stream(q.device, stream))
    if rc != 0:
        raise KdaError(rc, "kda_decode_step")
    return out
