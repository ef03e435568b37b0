"""The C-ABI library on the host: it loads, exports every symbol the header
declares, and rejects every host-checkable invalid call with its status code
before touching the GPU.  No call here launches anything: every call is
constructed to fail validation (fake pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

import delta_rule_linear_kda_amd as kda
from delta_rule_linear_kda_amd import Shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULLP, SHAPE, DTYPE, MISAL, WS, ALIAS, SCRATCH = 0, 1, 2, 3, 4, 5, 6, 8


def header_symbols():
    syms = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            syms |= set(re.findall(r"KDA_API\s+[\w\s\*]+?\b(kda_\w+)\s*\(", text))
    return syms


def test_exports_every_declared_symbol():
    syms = header_symbols()
    assert syms == set(kda.EXPORTS)
    L = kda.lib()
    for s in syms:
        assert hasattr(L, s), s


def test_version_and_status_strings():
    assert kda.abi_version() == 6
    for code in range(9):
        assert kda.status_str(code).startswith(kda.STATUS[code])
    assert kda.status_str(99) == "unknown kda_status"


def _split_layout(N, T, H, dk, dv):
    """Host mirror of the two-pass forward's workspace: one block of chunk
    records (per 32-token chunk: X diag(beta) and P as bf16 hi/lo, each 32 x
    32 lower block-triangular with lower triangular diagonal blocks, stored
    as rows 8q .. 8q + 7 up to column 8q + 7 for q = 0 .. 3; Gamma_end fp32
    [dk]; Qbar', -W and Kend' fp16 32 x dk each; 30,208 / 17,664 bytes at
    d_k = 128 / 64), at most 4 GiB unless 8 chunks per
    sequence need more (two half-size buffers when the input needs more than
    one block), the per-sequence record offsets, the carried states when
    there is more than one block, and b transposed to [H, T] (bf16)."""
    rb = 4 * (8 * 8 + 8 * 16 + 8 * 24 + 8 * 32) * 2 + dk * 4 + 3 * 32 * dk * 2
    assert rb == {128: 30208, 64: 17664}[dk]
    nch_max = max(1, -(-T // 32))
    every = H * (nch_max + N)
    budget = (4 << 30) // rb
    if every <= budget:
        bc, recs = nch_max, every
    else:  # two record buffers (one block built while the previous is consumed)
        bc = max(8, budget // 2 // max(1, H * N))
        recs = min(every, H * N * bc)
    bc = min(bc, 0x7FFFFFFF // rb, nch_max)
    recs = min(recs, H * N * bc)
    blocks = -(-nch_max // bc)
    nbuf = 2 if blocks > 1 else 1
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    total = (nbuf * (up(recs * rb) + up((N + 1) * 4)) +
             (up(N * H * dk * dv * 4) if blocks > 1 else 0) + up(H * T * 2))
    return total, blocks


def _split_bytes(*args):
    return _split_layout(*args)[0]


def _uses_split(N, T, H, dk, dv, cus=256):
    """The two-pass form runs when the fused kernel's workgroups ((sequence,
    head) pairs, two d_v slices each when that fits one round) would leave
    compute units idle, and with up to three pairs per four compute units
    at d_k = d_v = 128 when all records fit one block and sequences average
    at least 1024 tokens (no GPU here: the library assumes 256 units)."""
    items = N * H
    fused = 2 * items if dv == 128 and 2 * items <= cus else items
    if fused < cus:
        return True
    return (dk == 128 and dv == 128 and 4 * items <= 3 * cus and T >= 1024 * N and
            _split_layout(N, T, H, dk, dv)[1] == 1)


def test_workspace_query():
    for args in [(4, 16384, 32, 128, 128), (1, 1 << 20, 96, 128, 128), (16, 131072, 96, 128, 128),
                 (3, 1000, 2, 64, 128), (1, 0, 4, 128, 64), (5000, 5000, 8, 128, 128),
                 (2, 4096, 12, 64, 64), (1, 1 << 20, 12, 128, 128), (4, 2048, 32, 128, 128),
                 (4, 16384, 32, 64, 128), (2, 1 << 20, 64, 128, 128), (6, 24576, 32, 128, 128),
                 (8, 32768, 32, 128, 128)]:
        N, T, H, dk, dv = args
        exp = _split_bytes(*args) if _uses_split(*args) else 0
        assert kda.fwd_workspace_bytes(*args) == exp, args
    # 4 x 4096 tokens x 32 heads: one block of records, then the chain alone
    assert kda.fwd_workspace_bytes(4, 16384, 32, 128, 128) == _split_bytes(4, 16384, 32, 128, 128)
    assert kda.fwd_workspace_bytes(4, 2048, 32, 128, 128) == 0      # short sequences: fused
    assert kda.fwd_workspace_bytes(8, 32768, 32, 128, 128) == 0     # 256 pairs: fused
    assert kda.fwd_workspace_bytes(16, 131072, 96, 128, 128) == 0   # 1536 pairs: fused
    # the 1M-token, 96-head workload runs in blocks of records within about
    # 4 GiB, plus b transposed (2 H T bytes: 192 MiB)
    assert kda.fwd_workspace_bytes(1, 1 << 20, 96, 128, 128) < (4 << 30) + (256 << 20)
    assert kda.fwd_workspace_bytes(4, 16384, 32, 128, 128, in_dtype=0) == 0   # fp32: none
    L = kda.lib()
    out = ctypes.c_size_t(0)
    assert L.kda_fwd_workspace_bytes(None, ctypes.byref(out)) == NULLP
    s = Shape(1, 10, 2, 96, 128, 1, 0)
    assert L.kda_fwd_workspace_bytes(ctypes.byref(s), ctypes.byref(out)) == SHAPE
    s = Shape(1, 10, 2, 128, 128, 1, 0)
    assert L.kda_fwd_workspace_bytes(ctypes.byref(s), None) == NULLP


# Fake, distinct, 16-byte aligned addresses, far apart (never dereferenced).
BASE = 1 << 40
P = {name: BASE + i * (1 << 36) for i, name in enumerate(
    ["q", "k", "v", "a", "b", "gate", "cu", "s0", "o", "sf", "ws"])}
P["ws_bytes"] = 1 << 34


def fwd(shape, **over):
    args = dict(P)
    args.update(over)
    return kda.lib().kda_fwd_chunked(
        ctypes.byref(shape) if shape is not None else None, args["q"], args["k"], args["v"],
        args["a"], args["b"], args["gate"], args["cu"], args["s0"], args["o"], args["sf"],
        args["ws"], args["ws_bytes"], None)


def dec(shape, **over):
    args = dict(P)
    args.update(over)
    return kda.lib().kda_decode_step(
        ctypes.byref(shape) if shape is not None else None, args["q"], args["k"], args["v"],
        args["a"], args["b"], args["gate"], args["s0"], args["o"], None)


def good_shape(**kw):
    d = dict(num_seqs=2, total_tokens=300, num_heads=4, dk=128, dv=128, in_dtype=1, out_dtype=0)
    d.update(kw)
    return Shape(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(dk=96), SHAPE), (dict(dv=32), SHAPE), (dict(num_heads=0), SHAPE),
    (dict(num_seqs=-1), SHAPE), (dict(total_tokens=-5), SHAPE),
    (dict(in_dtype=7), DTYPE), (dict(out_dtype=1), DTYPE),
    (dict(total_tokens=1 << 60), SHAPE),
    (dict(num_seqs=0, total_tokens=10), SHAPE),
])
def test_fwd_rejects_bad_shape(kw, code):
    assert fwd(good_shape(**kw)) == code


def test_fwd_rejects_null_and_misaligned():
    assert fwd(None) == NULLP
    for name in ["q", "k", "v", "a", "b", "o", "cu"]:
        assert fwd(good_shape(), **{name: None}) == NULLP, name
    for name in ["q", "k", "v", "a", "gate", "s0", "o", "sf"]:
        assert fwd(good_shape(), **{name: P[name] + 8}) == MISAL, name
    assert fwd(good_shape(), cu=P["cu"] + 2) == MISAL
    assert fwd(good_shape(), b=P["b"] + 1) == MISAL                # bf16 b: 2-byte alignment
    assert fwd(good_shape(in_dtype=0), b=P["b"] + 2) == MISAL      # fp32 b: 4-byte alignment


def test_fwd_rejects_aliasing():
    assert fwd(good_shape(), o=P["q"]) == ALIAS
    assert fwd(good_shape(), o=P["k"] + 64) == ALIAS
    assert fwd(good_shape(), sf=P["v"]) == ALIAS
    assert fwd(good_shape(), o=P["sf"]) == ALIAS
    assert fwd(good_shape(), sf=P["s0"] + 16) == ALIAS          # partial overlap with the state
    assert fwd(good_shape(), o=P["cu"] - 16) == ALIAS            # o runs into cu_seqlens


def test_fwd_rejects_bad_workspace():
    need = kda.fwd_workspace_bytes(2, 300, 4, 128, 128)
    assert need > 0
    assert fwd(good_shape(), ws_bytes=need - 1) == WS
    assert fwd(good_shape(), ws=None) == WS
    assert fwd(good_shape(), ws=P["ws"] + 8) == MISAL
    assert fwd(good_shape(), ws=P["q"]) == ALIAS                  # workspace over an input
    assert fwd(good_shape(), ws=P["o"] - 64) == ALIAS             # workspace runs into o


def test_decode_rejects():
    s = good_shape(num_seqs=8, total_tokens=8)
    assert dec(None) == NULLP
    assert dec(good_shape(num_seqs=8, total_tokens=9)) == SHAPE
    assert dec(good_shape(num_seqs=8, total_tokens=8, dk=100)) == SHAPE
    assert dec(good_shape(num_seqs=8, total_tokens=8, in_dtype=5)) == DTYPE
    for name in ["q", "k", "v", "a", "b", "s0", "o"]:
        assert dec(s, **{name: None}) == NULLP, name
    for name in ["q", "gate", "s0", "o"]:
        assert dec(s, **{name: P[name] + 4}) == MISAL, name
    assert dec(s, o=P["s0"]) == ALIAS
    assert dec(s, s0=P["q"]) == ALIAS
    assert dec(s, o=P["v"] + 32) == ALIAS


def test_zero_sequences_is_a_no_op():
    # N = 0, T = 0: nothing to do, nothing launched.
    assert fwd(good_shape(num_seqs=0, total_tokens=0)) == OK
    assert dec(good_shape(num_seqs=0, total_tokens=0)) == OK


def fwd_ckpt(shape, interval=512, ckpt=None, capacity=4, **over):
    args = dict(P)
    args.update(over)
    return kda.lib().kda_fwd_chunked_ckpt(
        ctypes.byref(shape), args["q"], args["k"], args["v"], args["a"], args["b"], args["gate"],
        args["cu"], args["s0"], args["o"], args["sf"], interval,
        BASE + 11 * (1 << 36) if ckpt is None else ckpt, capacity, args["ws"], args["ws_bytes"],
        None)


@pytest.mark.parametrize("interval,capacity,code", [(0, 4, SHAPE), (100, 4, SHAPE), (32, 4, SHAPE),
                                                    (-512, 4, SHAPE), (512, -1, SHAPE)])
def test_ckpt_rejects_bad_interval_or_capacity(interval, capacity, code):
    assert fwd_ckpt(good_shape(), interval=interval, capacity=capacity) == code


def test_ckpt_rejects_null_misaligned_and_aliasing():
    s = good_shape()
    assert fwd_ckpt(s, ckpt=0, capacity=4) == NULLP
    assert fwd_ckpt(s, ckpt=BASE + 11 * (1 << 36) + 8) == MISAL
    assert fwd_ckpt(s, ckpt=P["o"]) == ALIAS          # overlaps the output
    assert fwd_ckpt(s, ckpt=P["k"]) == ALIAS          # overlaps an input
    assert fwd_ckpt(s, ckpt=P["sf"]) == ALIAS         # overlaps the final state
    assert fwd_ckpt(s, ckpt=P["ws"] + 256) == ALIAS   # overlaps the workspace
    assert fwd_ckpt(good_shape(dk=96)) == SHAPE       # the shape is still checked


def test_ckpt_count():
    cu = [0, 1100, 1612, 1912, 1912, 3448]
    assert kda.ckpt_count(cu, 512) == 2 + 1 + 0 + 0 + 3
    assert kda.ckpt_count(cu, 64) == sum((cu[i + 1] - cu[i]) // 64 for i in range(5))
    assert kda.ckpt_count([0], 512) == 0
    for bad_cu, iv in [(cu, 100), ([0, 10, 5], 512), ([3, 600], 512)]:
        with pytest.raises(kda.KdaError) as e:
            kda.ckpt_count(bad_cu, iv)
        assert e.value.code == SHAPE
    out = ctypes.c_int64(0)
    assert kda.lib().kda_fwd_ckpt_count(2, None, 512, ctypes.byref(out)) == NULLP


# --- segment-transition form -------------------------------------------------
def _kcp_layout_bytes(N, T, H, dk, dv, L):
    up = lambda x: (x + 255) // 256 * 256
    cap = T // L + N
    return (up((cap + 1) * 4) + up((N + 1) * 4) + up(cap * H * dk * (dv + dk) * 4)
            + up(cap * H * dk * dv * 4))


def test_kcp_workspace_query():
    # explicit segment length: table, offsets, [S_loc | M] and start states
    assert kda.kcp_workspace_bytes(1, 1 << 20, 12, 128, 128, 4096) == \
        _kcp_layout_bytes(1, 1 << 20, 12, 128, 128, 4096)
    assert kda.kcp_workspace_bytes(3, 1000, 2, 64, 128, 128) == \
        _kcp_layout_bytes(3, 1000, 2, 64, 128, 128)
    # automatic: many (sequence, head) pairs keep the direct form (its workspace)
    assert kda.kcp_workspace_bytes(1, 1 << 20, 96, 128, 128, 0) == \
        kda.fwd_workspace_bytes(1, 1 << 20, 96, 128, 128)
    assert kda.kcp_workspace_bytes(4, 4096, 2, 128, 128, 0) == \
        kda.fwd_workspace_bytes(4, 4096, 2, 128, 128)                  # too short to segment
    for bad in (-64, 100, 32):
        with pytest.raises(kda.KdaError) as e:
            kda.kcp_workspace_bytes(1, 1 << 20, 12, 128, 128, bad)
        assert e.value.code == SHAPE
    with pytest.raises(kda.KdaError) as e:  # more segments than the kernels index
        kda.kcp_workspace_bytes(1, 1 << 30, 64, 128, 128, 64)
    assert e.value.code == SHAPE
    out = ctypes.c_size_t(0)
    assert kda.lib().kda_fwd_kcp_workspace_bytes(None, 0, ctypes.byref(out)) == NULLP
    s = good_shape()
    assert kda.lib().kda_fwd_kcp_workspace_bytes(ctypes.byref(s), 0, None) == NULLP


WSP = BASE + 12 * (1 << 36)


def fwd_kcp(shape, seg=128, ws=WSP, ws_bytes=1 << 34, **over):
    args = dict(P)
    args.update(over)
    return kda.lib().kda_fwd_chunked_kcp(
        ctypes.byref(shape), args["q"], args["k"], args["v"], args["a"], args["b"], args["gate"],
        args["cu"], args["s0"], args["o"], args["sf"], seg, ws, ws_bytes, None)


def test_kcp_rejects():
    s = good_shape()
    need = _kcp_layout_bytes(2, 300, 4, 128, 128, 128)
    assert fwd_kcp(good_shape(dk=96)) == SHAPE
    assert fwd_kcp(s, seg=96) == SHAPE
    assert fwd_kcp(s, seg=-128) == SHAPE
    assert fwd_kcp(s, ws=None) == WS
    assert fwd_kcp(s, ws_bytes=need - 1) == WS
    assert fwd_kcp(s, ws=WSP + 8) == MISAL
    assert fwd_kcp(s, ws=P["q"]) == ALIAS             # workspace over an input
    assert fwd_kcp(s, ws=P["o"] - 64) == ALIAS        # workspace runs into the output
    assert fwd_kcp(s, q=None) == NULLP                # the forward's own checks apply
    assert fwd_kcp(s, o=P["k"]) == ALIAS
    assert fwd_kcp(good_shape(num_seqs=0, total_tokens=0)) == OK


TRP = BASE + 13 * (1 << 36)


def seg_trans(shape, trans=TRP, **over):
    args = dict(P)
    args.update(over)
    return kda.lib().kda_segment_transition(ctypes.byref(shape), args["k"], args["v"], args["a"],
                                            args["b"], args["cu"], trans, None)


def test_segment_transition_rejects():
    s = good_shape()
    assert seg_trans(good_shape(dv=48)) == SHAPE
    assert seg_trans(good_shape(in_dtype=3)) == DTYPE
    assert seg_trans(s, trans=None) == NULLP
    for name in ["k", "v", "a", "b", "cu"]:
        assert seg_trans(s, **{name: None}) == NULLP, name
    assert seg_trans(s, trans=TRP + 4) == MISAL
    assert seg_trans(s, k=P["k"] + 8) == MISAL
    assert seg_trans(s, trans=P["v"]) == ALIAS
    assert seg_trans(s, trans=P["cu"] - 64) == ALIAS
    assert seg_trans(good_shape(num_seqs=0, total_tokens=0)) == OK


def compose(N=2, S=5, H=4, dk=128, dv=128, off=P["cu"], trans=TRP, s0=P["s0"],
            start=BASE + 14 * (1 << 36), sf=P["sf"]):
    return kda.lib().kda_segment_compose(N, S, H, dk, dv, off, trans, s0, start, sf, None)


def test_segment_compose_rejects():
    assert compose(dk=32) == SHAPE
    assert compose(N=-1) == SHAPE
    assert compose(S=-1) == SHAPE
    assert compose(H=0) == SHAPE
    assert compose(off=None) == NULLP
    assert compose(trans=None) == NULLP
    assert compose(off=P["cu"] + 2) == MISAL
    assert compose(trans=TRP + 8) == MISAL
    assert compose(start=TRP) == ALIAS                 # start states over the transitions
    assert compose(start=P["sf"]) == ALIAS             # over the final states
    assert compose(sf=TRP + 1024) == ALIAS
    assert compose(sf=P["s0"] + 16) == ALIAS           # partial overlap with the start
    assert compose(N=0) == OK


# --- layer operations: short convolution front, RMSNorm gate back ------------
XP, WP, YP, SIP, SOP = (BASE + (20 + i) * (1 << 36) for i in range(5))


def conv(shape, width=4, x=XP, w=WP, cu=P["cu"], si=SIP, so=SOP, y=YP):
    return kda.lib().kda_shortconv_swish_l2(ctypes.byref(shape), width, x, w, cu, si, so, y, None)


def test_shortconv_rejects():
    s = good_shape()
    assert conv(good_shape(dk=48)) == SHAPE
    assert conv(good_shape(in_dtype=9)) == DTYPE
    for wd in (0, 5, -1):
        assert conv(s, width=wd) == SHAPE
    assert conv(s, x=None) == NULLP
    assert conv(s, y=None) == NULLP
    assert conv(s, w=None) == NULLP
    assert conv(s, cu=None) == NULLP
    assert conv(s, x=XP + 8) == MISAL
    assert conv(s, w=WP + 4) == MISAL
    assert conv(s, si=SIP + 1) == MISAL            # bf16 state: 2-byte alignment
    assert conv(s, y=XP) == ALIAS                  # output over the input
    assert conv(s, so=WP) == ALIAS                 # state over the weights
    assert conv(s, so=YP) == ALIAS                 # state over the output
    assert conv(s, so=SIP + 2) == ALIAS            # partial overlap with the state in
    assert conv(good_shape(num_seqs=0, total_tokens=0)) == OK


def rms(shape, o=XP, gate=WP, w=SIP, eps=1e-6, y=YP):
    return kda.lib().kda_rmsnorm_gate(ctypes.byref(shape), o, gate, w, eps, y, None)


def test_rmsnorm_gate_rejects():
    s = good_shape()
    assert rms(good_shape(dv=100)) == SHAPE
    assert rms(s, eps=-1.0) == SHAPE
    assert rms(s, eps=float("nan")) == SHAPE
    assert rms(s, o=None) == NULLP
    assert rms(s, y=None) == NULLP
    assert rms(s, o=XP + 4) == MISAL
    assert rms(s, gate=WP + 2) == MISAL
    assert rms(s, y=WP) == ALIAS                   # output over the gate
    assert rms(s, y=XP + 16) == ALIAS              # partial overlap with o
    assert rms(good_shape(num_seqs=0, total_tokens=0)) == OK


# --- backward ----------------------------------------------------------------
GP = {name: BASE + (30 + i) * (1 << 36) for i, name in enumerate(
    ["dy", "dsf", "dq", "dk", "dv", "da", "db", "dgate", "ds0", "ws"])}


def bwd(shape, ws_bytes=1 << 40, **over):
    args = dict(P)
    args.update(GP)
    args.update(over)
    return kda.lib().kda_bwd_chunked(
        ctypes.byref(shape), args["q"], args["k"], args["v"], args["a"], args["b"], args["gate"],
        args["cu"], args["s0"], args["dy"], args["dsf"], args["dq"], args["dk"], args["dv"],
        args["da"], args["db"], args["dgate"], args["ds0"], args["ws"], ws_bytes, None)


def test_bwd_workspace_query():
    up = lambda x: (x + 255) // 256 * 256
    N, T, H, dk, dv = 2, 300, 4, 128, 128
    th, nsl = T * H, dv // 8
    st = H * dk * dv * 4
    # bf16 inputs (chunked form, 32-token chunks): states every 32 tokens, the
    # ungated output, the adjoint state at each chunk's end, the adjoint
    # chain's operand record per (chunk, head) (Qbar^T, (beta Kbar)^T, Kend:
    # 32 x dk each; P^T, X^T: 32 x 32; Gamma_end: dk; then Mkk: 32 x 32), two
    # offset tables
    chunks = T // 32 + N
    rec = 3 * 32 * dk + 3 * 32 * 32 + dk
    exp = (up((T // 32) * st) + up(th * dv * 4) + up(chunks * st) + up(chunks * H * rec * 4)
           + 2 * up((N + 1) * 4))
    assert kda.bwd_workspace_bytes(N, T, H, dk, dv) == exp
    # fp32 inputs (token form): states every 64 tokens, the ungated output,
    # per-slice partial sums and sub-chunk start states
    exp = (up((T // 64) * st) + up(th * dv * 4) + 3 * up(nsl * th * dk * 4)
           + up(nsl * th * 4) + up(N * H * nsl * 16 * dk * 8 * 4))
    assert kda.bwd_workspace_bytes(N, T, H, dk, dv, kda.KDA_F32) == exp
    out = ctypes.c_size_t(0)
    assert kda.lib().kda_bwd_workspace_bytes(None, ctypes.byref(out)) == NULLP


def test_bwd_rejects():
    s = good_shape()
    assert bwd(good_shape(dk=80)) == SHAPE
    assert bwd(good_shape(in_dtype=4)) == DTYPE
    for name in ["q", "k", "v", "a", "b", "cu", "dy", "dq", "dk", "dv", "da", "db"]:
        assert bwd(s, **{name: None}) == NULLP, name
    assert bwd(s, dgate=None) == NULLP                # a gate needs its gradient
    assert bwd(s, ws=None) == WS
    assert bwd(s, ws_bytes=16) == WS
    for name in ["q", "dy", "dq", "dgate", "ds0", "ws"]:
        assert bwd(s, **{name: GP.get(name, P.get(name)) + 8}) == MISAL, name
    assert bwd(s, dq=P["k"]) == ALIAS                 # gradient over an input
    assert bwd(s, dv=GP["dy"]) == ALIAS               # over the cotangent
    assert bwd(s, dk=GP["dq"] + 64) == ALIAS          # two gradients overlap
    assert bwd(s, ws=GP["ds0"]) == ALIAS              # workspace over an output
    assert bwd(good_shape(num_seqs=0, total_tokens=0)) == OK


def fwd_noalloc(shape, **over):
    args = dict(P)
    args.update(over)
    return kda.lib().kda_fwd_chunked_noalloc(
        ctypes.byref(shape) if shape is not None else None, args["q"], args["k"], args["v"],
        args["a"], args["b"], args["gate"], args["cu"], args["s0"], args["o"], args["sf"], None)


def test_noalloc_rejects_like_fwd():
    """The forward without a workspace validates its arguments as
    kda_fwd_chunked does, before anything is enqueued."""
    assert fwd_noalloc(None) == NULLP
    assert fwd_noalloc(good_shape(dk=96)) == SHAPE
    assert fwd_noalloc(good_shape(in_dtype=7)) == DTYPE
    for name in ["q", "k", "v", "a", "b", "o", "cu"]:
        assert fwd_noalloc(good_shape(), **{name: None}) == NULLP, name
    for name in ["q", "gate", "s0", "o", "sf"]:
        assert fwd_noalloc(good_shape(), **{name: P[name] + 8}) == MISAL, name
    assert fwd_noalloc(good_shape(), o=P["q"]) == ALIAS
    assert fwd_noalloc(good_shape(), sf=P["s0"] + 16) == ALIAS
    assert fwd_noalloc(good_shape(num_seqs=0, total_tokens=0)) == OK


@pytest.mark.parametrize("N,T,H,dk", [(1, 2 << 20, 96, 128), (1, 1 << 20, 120, 128),
                                      (3, 3_000_000, 40, 128)])
def test_noalloc_rejects_beyond_its_scratch(N, T, H, dk):
    """Two-pass shapes whose fixed parts (b transposed: 2 H T bytes; carried
    states: 4 N H dk dv bytes) plus 8 chunk records per (sequence, head)
    exceed the 256 MiB array: KDA_ERR_SCRATCH (no GPU touched)."""
    s = good_shape(num_seqs=N, total_tokens=T, num_heads=H, dk=dk)
    if not _uses_split(N, T, H, dk, 128):
        pytest.skip("fused-kernel shape: no scratch")
    far = {name: BASE + i * (1 << 39) for i, name in enumerate(P) if name != "ws_bytes"}
    assert fwd_noalloc(s, **far) == SCRATCH


def fwd_norm(shape, weight=BASE + 12 * (1 << 36), eps=1e-5, **over):
    args = dict(P)
    args.update(over)
    return kda.lib().kda_fwd_chunked_rmsnorm_gate(
        ctypes.byref(shape) if shape is not None else None, args["q"], args["k"], args["v"],
        args["a"], args["b"], args["gate"], args["cu"], args["s0"], weight, ctypes.c_float(eps),
        args["o"], args["sf"], args["ws"], args["ws_bytes"], None)


def test_fwd_rmsnorm_gate_rejects():
    assert fwd_norm(None) == NULLP
    assert fwd_norm(good_shape(dk=96)) == SHAPE
    assert fwd_norm(good_shape(), eps=-1.0) == SHAPE
    assert fwd_norm(good_shape(), eps=float("nan")) == SHAPE
    assert fwd_norm(good_shape(), eps=2.0) == SHAPE
    assert fwd_norm(good_shape(), weight=BASE + 12 * (1 << 36) + 4) == MISAL
    assert fwd_norm(good_shape(), weight=P["o"]) == ALIAS          # weight inside the output
    assert fwd_norm(good_shape(), o=P["q"]) == ALIAS
    assert fwd_norm(good_shape(), ws=None) == WS
    assert fwd_norm(good_shape(num_seqs=0, total_tokens=0)) == OK
