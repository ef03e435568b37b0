"""delta_rule_linear_kda_amd: Python binding of libkda (Kimi Delta Attention on gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libkda.so`` through its C ABI (``include/libkda.h``); PyTorch
supplies device memory and the current stream.  If the library is missing the
import of any entry point raises -- there is no fallback path.

Entry points (same names as the C ABI):
  * ``fwd_chunked(q, k, v, a, b, gate, cu_seqlens, initial_state=None, ...)``,
    ``fwd_chunked_noalloc(...)`` (same, without a workspace),
    ``fwd_chunked_rmsnorm_gate(...)`` (with the head-wise RMSNorm before the gate)
  * ``decode_step(q, k, v, a, b, gate, state, ...)``
  * ``segment_transition(k, v, a, b, cu_seqlens, ...)``,
    ``segment_compose(seg_offsets, trans, ...)``,
    ``fwd_chunked_kcp(q, k, v, a, b, gate, cu_seqlens, ...)``
  * ``shortconv_swish_l2(x, weight, cu_seqlens, ...)``,
    ``rmsnorm_gate(o, gate, weight, eps, ...)``
  * ``bwd_chunked(q, k, v, a, b, gate, cu_seqlens, initial_state, dy, ...)``
  * ``fwd_workspace_bytes(...)``, ``kcp_workspace_bytes(...)``, ``bwd_workspace_bytes(...)``,
    ``ckpt_count(...)``, ``status_str(code)``, ``abi_version()``
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
    8: "KDA_ERR_SCRATCH",
}
EXPORTS = ("kda_fwd_workspace_bytes", "kda_fwd_chunked", "kda_fwd_chunked_ckpt",
           "kda_fwd_ckpt_count", "kda_segment_transition", "kda_segment_compose",
           "kda_fwd_kcp_workspace_bytes", "kda_fwd_chunked_kcp", "kda_shortconv_swish_l2",
           "kda_rmsnorm_gate", "kda_bwd_workspace_bytes", "kda_bwd_chunked", "kda_decode_step",
           "kda_status_str", "kda_abi_version", "kda_fwd_chunked_noalloc",
           "kda_fwd_chunked_rmsnorm_gate")


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
        L.kda_fwd_chunked_rmsnorm_gate.restype = ctypes.c_int
        L.kda_fwd_chunked_rmsnorm_gate.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                   ctypes.c_float, vp, vp, vp, ctypes.c_size_t,
                                                   vp]
        L.kda_fwd_chunked_noalloc.restype = ctypes.c_int
        L.kda_fwd_chunked_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.kda_fwd_chunked_ckpt.restype = ctypes.c_int
        L.kda_fwd_chunked_ckpt.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           ctypes.c_int32, vp, ctypes.c_int64, vp,
                                           ctypes.c_size_t, vp]
        L.kda_fwd_ckpt_count.restype = ctypes.c_int
        L.kda_fwd_ckpt_count.argtypes = [ctypes.c_int32, vp, ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_int64)]
        L.kda_segment_transition.restype = ctypes.c_int
        L.kda_segment_transition.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp]
        i32 = ctypes.c_int32
        L.kda_segment_compose.restype = ctypes.c_int
        L.kda_segment_compose.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.kda_fwd_kcp_workspace_bytes.restype = ctypes.c_int
        L.kda_fwd_kcp_workspace_bytes.argtypes = [sp, i32, ctypes.POINTER(ctypes.c_size_t)]
        L.kda_fwd_chunked_kcp.restype = ctypes.c_int
        L.kda_fwd_chunked_kcp.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                          ctypes.c_size_t, vp]
        L.kda_shortconv_swish_l2.restype = ctypes.c_int
        L.kda_shortconv_swish_l2.argtypes = [sp, i32, vp, vp, vp, vp, vp, vp, vp]
        L.kda_rmsnorm_gate.restype = ctypes.c_int
        L.kda_rmsnorm_gate.argtypes = [sp, vp, vp, vp, ctypes.c_float, vp, vp]
        L.kda_bwd_workspace_bytes.restype = ctypes.c_int
        L.kda_bwd_workspace_bytes.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
        L.kda_bwd_chunked.restype = ctypes.c_int
        L.kda_bwd_chunked.argtypes = [sp] + [vp] * 18 + [ctypes.c_size_t, vp]
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
                workspace=None, stream=None):
    """Chunked KDA forward over packed sequences (C ABI ``kda_fwd_chunked``, or
    ``kda_fwd_chunked_ckpt`` when ``checkpoint_interval`` is given).

    q, k, a: [T, H, dk]; v, gate: [T, H, dv] (gate may be None); b: [T, H]
    (all float32 or all bfloat16); cu_seqlens: int32 [N+1] on the device;
    initial_state: fp32 [N, H, dk, dv] or None.  Returns (o fp32 [T, H, dv],
    final_state fp32 [N, H, dk, dv] or None), plus the recorded states fp32
    [n_ckpt, H, dk, dv] as a third element when ``checkpoint_interval`` is
    given (slot layout: see ``kda_fwd_chunked_ckpt``).  ``final_state`` may be
    passed as the same tensor as ``initial_state`` for an in-place update.
    ``workspace``: a uint8 device tensor of at least ``fwd_workspace_bytes``
    bytes to use instead of a fresh one."""
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
    if workspace is not None and ws_bytes:
        ws = workspace
        ws_bytes = workspace.numel()
    else:
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


def fwd_chunked_rmsnorm_gate(q, k, v, a, b, gate, cu_seqlens, initial_state=None,
                             norm_weight=None, norm_eps: float = 1e-6, *, out=None,
                             final_state=None, workspace=None, stream=None):
    """``kda_fwd_chunked_rmsnorm_gate``: y = sigmoid(gate) * norm_weight *
    o / sqrt(mean(o^2) + norm_eps) per (token, head) row of the forward's
    output o.  Returns (y fp32 [T, H, dv], final_state)."""
    import torch

    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.float32, device=q.device)
    if final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    ws_bytes = fwd_workspace_bytes(N, T, H, dk, dv, dt)
    if workspace is not None and ws_bytes:
        ws, ws_bytes = workspace, workspace.numel()
    else:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    shape = Shape(N, T, H, dk, dv, dt, KDA_F32)
    rc = lib().kda_fwd_chunked_rmsnorm_gate(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(a), _ptr(b), _ptr(gate), _ptr(cu_seqlens),
                                            _ptr(initial_state), _ptr(norm_weight),
                                            float(norm_eps), _ptr(out), _ptr(final_state),
                                            _ptr(ws), ws_bytes, _stream(q.device, stream))
    if rc != 0:
        raise KdaError(rc, "kda_fwd_chunked_rmsnorm_gate")
    return out, final_state


def fwd_chunked_noalloc(q, k, v, a, b, gate, cu_seqlens, initial_state=None, *, out=None,
                        final_state=None, stream=None):
    """``kda_fwd_chunked_noalloc``: the forward with its scratch in the
    library's fixed device array (no workspace; raises KdaError with
    KDA_ERR_SCRATCH when the shape needs more).  Arguments and results as
    ``fwd_chunked`` (out and final_state are allocated here when not given;
    pass them for a call that allocates nothing)."""
    import torch

    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.float32, device=q.device)
    if final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    shape = Shape(N, T, H, dk, dv, dt, KDA_F32)
    rc = lib().kda_fwd_chunked_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                       _ptr(b), _ptr(gate), _ptr(cu_seqlens),
                                       _ptr(initial_state), _ptr(out), _ptr(final_state),
                                       _stream(q.device, stream))
    if rc != 0:
        raise KdaError(rc, "kda_fwd_chunked_noalloc")
    return out, final_state


def segment_transition(k, v, a, b, cu_seqlens, *, out=None, stream=None):
    """Transitions of the segments given as packed sequences (C ABI
    ``kda_segment_transition``): k, a [T, H, dk]; v [T, H, dv]; b [T, H];
    cu_seqlens int32 [S+1] on the device (one segment per entry).  Returns
    fp32 [S, H, dk, dv + dk]: per row, the segment's zero-start state S_loc
    followed by its transition M."""
    import torch

    T, H, dk = k.shape
    dv = v.shape[2]
    S = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if out is None:
        out = torch.empty((S, H, dk, dv + dk), dtype=torch.float32, device=k.device)
    shape = Shape(S, T, H, dk, dv, _dtype_code(k), KDA_F32)
    rc = lib().kda_segment_transition(ctypes.byref(shape), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                      _ptr(cu_seqlens), _ptr(out), _stream(k.device, stream))
    if rc != 0:
        raise KdaError(rc, "kda_segment_transition")
    return out


def segment_compose(seg_offsets, trans, dv: int, initial_state=None, *, seg_start=None,
                    final_state=None, want_seg_start: bool = True, want_final: bool = True,
                    stream=None):
    """Composition of segment transitions in token order (C ABI
    ``kda_segment_compose``): seg_offsets int32 [N+1] on the device; trans
    fp32 [S, H, dk, dv + dk]; initial_state fp32 [N, H, dk, dv] or None.
    Returns (seg_start [S, H, dk, dv] or None, final_state [N, H, dk, dv] or
    None)."""
    import torch

    S, H, dk, w = trans.shape
    if w != dv + dk:
        raise ValueError("trans must be [S, H, dk, dv + dk]")
    N = seg_offsets.numel() - 1
    if seg_offsets.dtype != torch.int32:
        raise TypeError("seg_offsets must be int32")
    dev = trans.device
    if seg_start is None and want_seg_start:
        seg_start = torch.empty((S, H, dk, dv), dtype=torch.float32, device=dev)
    if final_state is None and want_final:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    rc = lib().kda_segment_compose(N, S, H, dk, dv, _ptr(seg_offsets), _ptr(trans),
                                   _ptr(initial_state), _ptr(seg_start), _ptr(final_state),
                                   _stream(dev, stream))
    if rc != 0:
        raise KdaError(rc, "kda_segment_compose")
    return seg_start, final_state


def kcp_workspace_bytes(num_seqs: int, total_tokens: int, num_heads: int, dk: int, dv: int,
                        segment_len: int = 0, in_dtype: int = KDA_BF16) -> int:
    shape = Shape(num_seqs, total_tokens, num_heads, dk, dv, in_dtype, KDA_F32)
    out = ctypes.c_size_t(0)
    rc = lib().kda_fwd_kcp_workspace_bytes(ctypes.byref(shape), int(segment_len),
                                           ctypes.byref(out))
    if rc != 0:
        raise KdaError(rc, "kda_fwd_kcp_workspace_bytes")
    return int(out.value)


def fwd_chunked_kcp(q, k, v, a, b, gate, cu_seqlens, initial_state=None, *,
                    segment_len: int = 0, output_final_state: bool = True, out=None,
                    final_state=None, workspace=None, stream=None):
    """Chunked forward in segment-transition form (C ABI
    ``kda_fwd_chunked_kcp``); arguments and results as ``fwd_chunked``.
    ``segment_len``: tokens per segment (a multiple of 64), 0 = automatic.
    ``workspace``: a uint8 device tensor of at least ``kcp_workspace_bytes``
    bytes, or None to allocate one."""
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
    ws_bytes = kcp_workspace_bytes(N, T, H, dk, dv, segment_len, dt)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    shape = Shape(N, T, H, dk, dv, dt, KDA_F32)
    rc = lib().kda_fwd_chunked_kcp(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                   _ptr(b), _ptr(gate), _ptr(cu_seqlens), _ptr(initial_state),
                                   _ptr(out), _ptr(final_state), int(segment_len),
                                   _ptr(workspace),
                                   int(workspace.numel()) if workspace is not None else 0,
                                   _stream(q.device, stream))
    if rc != 0:
        raise KdaError(rc, "kda_fwd_chunked_kcp")
    return out, final_state


def shortconv_swish_l2(x, weight, cu_seqlens, state_in=None, *, out=None, state_out=None,
                       want_state: bool = False, stream=None):
    """Short convolution -> Swish -> L2 of one projection (C ABI
    ``kda_shortconv_swish_l2``): x [T, H, d] (float32 or bfloat16); weight fp32
    [H, d, W]; cu_seqlens int32 [N+1] on the device; state_in [N, H, d, W-1]
    (x's dtype) or None.  Returns y (x's dtype), plus the carried state when
    ``want_state`` or ``state_out`` is given."""
    import torch

    T, H, d = x.shape
    W = weight.shape[2]
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if out is None:
        out = torch.empty_like(x)
    if state_out is None and want_state:
        state_out = torch.empty((N, H, d, W - 1), dtype=x.dtype, device=x.device)
    shape = Shape(N, T, H, d, d, _dtype_code(x), KDA_F32)
    rc = lib().kda_shortconv_swish_l2(ctypes.byref(shape), int(W), _ptr(x), _ptr(weight),
                                      _ptr(cu_seqlens), _ptr(state_in), _ptr(state_out),
                                      _ptr(out), _stream(x.device, stream))
    if rc != 0:
        raise KdaError(rc, "kda_shortconv_swish_l2")
    return (out, state_out) if (want_state or state_out is not None) else out


def rmsnorm_gate(o, gate, weight=None, eps: float = 1e-6, *, out=None, stream=None):
    """Head-wise RMSNorm then sigmoid gate (C ABI ``kda_rmsnorm_gate``):
    o fp32 [T, H, dv]; gate [T, H, dv] (float32 or bfloat16) or None; weight
    fp32 [dv] or None.  ``out`` may be ``o`` (in place).  Returns y fp32."""
    import torch

    T, H, dv = o.shape
    if out is None:
        out = torch.empty_like(o)
    shape = Shape(1, T, H, dv, dv, _dtype_code(gate) if gate is not None else KDA_BF16,
                  KDA_F32)
    rc = lib().kda_rmsnorm_gate(ctypes.byref(shape), _ptr(o), _ptr(gate), _ptr(weight),
                                float(eps), _ptr(out), _stream(o.device, stream))
    if rc != 0:
        raise KdaError(rc, "kda_rmsnorm_gate")
    return out


def bwd_workspace_bytes(num_seqs: int, total_tokens: int, num_heads: int, dk: int, dv: int,
                        in_dtype: int = KDA_BF16) -> int:
    shape = Shape(num_seqs, total_tokens, num_heads, dk, dv, in_dtype, KDA_F32)
    out = ctypes.c_size_t(0)
    rc = lib().kda_bwd_workspace_bytes(ctypes.byref(shape), ctypes.byref(out))
    if rc != 0:
        raise KdaError(rc, "kda_bwd_workspace_bytes")
    return int(out.value)


def bwd_chunked(q, k, v, a, b, gate, cu_seqlens, initial_state, dy, d_final_state=None, *,
                want_d_initial_state: bool = True, workspace=None, stream=None):
    """Gradients of sum <dy, y> + <d_final_state, S_final> for the forward of
    ``fwd_chunked`` on the same inputs (C ABI ``kda_bwd_chunked``).  dy fp32
    [T, H, dv]; d_final_state fp32 [N, H, dk, dv] or None.  Returns a dict of
    fp32 tensors: dq, dk, dv, da, db, dgate (None without gate), ds0 (None
    unless wanted)."""
    import torch

    T, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    dt = _dtype_code(q)
    f32 = dict(dtype=torch.float32, device=q.device)
    g = {"dq": torch.empty((T, H, dk), **f32), "dk": torch.empty((T, H, dk), **f32),
         "dv": torch.empty((T, H, dv), **f32), "da": torch.empty((T, H, dk), **f32),
         "db": torch.empty((T, H), **f32),
         "dgate": torch.empty((T, H, dv), **f32) if gate is not None else None,
         "ds0": torch.empty((N, H, dk, dv), **f32) if want_d_initial_state else None}
    ws_bytes = bwd_workspace_bytes(N, T, H, dk, dv, dt)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    shape = Shape(N, T, H, dk, dv, dt, KDA_F32)
    rc = lib().kda_bwd_chunked(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                               _ptr(gate), _ptr(cu_seqlens), _ptr(initial_state), _ptr(dy),
                               _ptr(d_final_state), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
                               _ptr(g["da"]), _ptr(g["db"]), _ptr(g["dgate"]), _ptr(g["ds0"]),
                               _ptr(workspace), int(workspace.numel()),
                               _stream(q.device, stream))
    if rc != 0:
        raise KdaError(rc, "kda_bwd_chunked")
    return g


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
