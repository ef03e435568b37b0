"""GPU parity of the layer operations around the core (short convolution ->
Swish -> L2 front, head-wise RMSNorm -> sigmoid gate back) against the fp64
layer oracle, through the C ABI, and of the whole KDA layer chain
(front on q and k, core without gate, RMSNorm gate) against the oracles
chained the same way.  Tolerances as for the core: max |gpu - ref| / RMS(ref)
<= 2e-2 for bf16 inputs, 1e-4 for fp32 inputs."""
import numpy as np
import pytest

import oracle
import synth
from oracle import layer
from tests import kda_cases as kc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import delta_rule_linear_kda_amd as kda  # noqa: E402


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _tol(dtype):
    return kc.TOL_F32 if dtype == synth.F32 else kc.TOL_BF16


def _conv_weights(H, d, W, seed=0):
    return synth.host_normal(synth.key(seed, "conv_w"), H * d, W, dtype=synth.F32,
                             std=0.5).reshape(H, d, W)


def _state(dtype, N, H, d, W, seed=0):
    return synth.host_normal(synth.key(seed, "conv_state"), N * H * d, W - 1,
                             dtype=dtype).reshape(N, H, d, W - 1)


LENS = [300, 1, 0, 77, 2, 130]


def _check_stored(got, ref, dtype):
    """The front's output is stored in the input dtype.  For bf16 the storage
    rounding alone (round to nearest even: at most 2^-8 of the value) reaches
    0.02 of RMS here (L2-normalised rows: elements up to ~0.9 against an RMS of
    1/sqrt(d)), so the bound is elementwise: the oracle's value up to that
    rounding plus 1e-6 for the fp32 arithmetic.  fp32 storage: 1e-4 of RMS."""
    if dtype == synth.BF16:
        bound = 2.0 ** -8 * np.abs(ref) + 1e-6
        worst = float(np.max(np.abs(got - ref) / bound))
        print(f"    worst |err| / (2^-8 |ref| + 1e-6) = {worst:.3f}", flush=True)
        assert worst <= 1.0
    else:
        assert kc.rel_err(got, ref) <= kc.TOL_F32


@pytest.mark.parametrize("dtype,d,W,with_state", [
    (synth.BF16, 128, 4, True), (synth.BF16, 128, 4, False), (synth.BF16, 64, 3, True),
    (synth.BF16, 128, 1, False), (synth.F32, 128, 4, True), (synth.F32, 64, 2, True)])
def test_shortconv_swish_l2(dtype, d, W, with_state):
    _require_gpu()
    H = 20  # two head groups, the second partly filled
    print(f"[case] shortconv dtype={dtype} d={d} W={W} state={with_state} lens={LENS}", flush=True)
    w = kc.custom_workload(synth.WORKLOADS[1 if dtype == synth.BF16 else 0], heads=H, dk=d, dv=d)
    T = sum(LENS)
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int64)
    x = kc.host_tokens(w, "q", T)
    wt = _conv_weights(H, d, W)
    st = _state(dtype, len(LENS), H, d, W) if with_state and W > 1 else None
    y, so = kda.shortconv_swish_l2(kc.to_torch(x), torch.from_numpy(wt).cuda(),
                                   torch.from_numpy(cu.astype(np.int32)).cuda(),
                                   kc.to_torch(st) if st is not None else None, want_state=True)
    torch.cuda.synchronize()
    y_ref, so_ref = layer.shortconv_swish_l2(kc.f64(x), wt, cu, kc.f64(st) if st is not None else None)
    y_np = y.float().cpu().numpy() if dtype == synth.BF16 else y.cpu().numpy()
    e = kc.rel_err(y_np, y_ref)
    print(f"    err y={e:.3e} (max |err| / RMS)", flush=True)
    assert np.all(np.isfinite(y_np))
    _check_stored(y_np, y_ref, dtype)
    if W > 1:  # the carried state is a copy of inputs: exact
        so_np = so.float().cpu().numpy() if dtype == synth.BF16 else so.cpu().numpy()
        np.testing.assert_array_equal(so_np.astype(np.float64), so_ref)


def test_shortconv_in_place_state_and_decode():
    """The carried state updated in place, then one token per sequence (the
    decode form) from it, against the oracle run over the concatenation."""
    _require_gpu()
    H, d, W = 4, 128, 4
    print("[case] shortconv in-place state + decode", flush=True)
    w = kc.custom_workload(synth.WORKLOADS[1], heads=H, dk=d, dv=d)
    lens = [5, 2, 0, 9]
    N, T = len(lens), sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = kc.host_tokens(w, "k", T)
    xd = kc.host_tokens(w, "k", N, step=1)  # one new token per sequence
    wt = _conv_weights(H, d, W, seed=1)
    st0 = _state(synth.BF16, N, H, d, W, seed=1)
    st = kc.to_torch(st0)
    wt_d = torch.from_numpy(wt).cuda()
    kda.shortconv_swish_l2(kc.to_torch(x), wt_d, torch.from_numpy(cu.astype(np.int32)).cuda(),
                           st, state_out=st)
    yd = kda.shortconv_swish_l2(kc.to_torch(xd), wt_d,
                                torch.arange(N + 1, dtype=torch.int32, device="cuda"), st,
                                state_out=st)[0]
    torch.cuda.synchronize()
    # oracle: each sequence followed by its decode token
    xx = np.concatenate([np.concatenate([kc.f64(x)[cu[n]:cu[n + 1]], kc.f64(xd)[n:n + 1]])
                         for n in range(N)])
    cu2 = np.concatenate([[0], np.cumsum([L + 1 for L in lens])])
    y_ref, s_ref = layer.shortconv_swish_l2(xx, wt, cu2, kc.f64(st0))
    _check_stored(yd.float().cpu().numpy(), y_ref[cu2[1:] - 1], synth.BF16)
    np.testing.assert_array_equal(st.float().cpu().numpy().astype(np.float64), s_ref)


@pytest.mark.parametrize("gdtype,dv,with_gate,with_w", [
    (synth.BF16, 128, True, True), (synth.BF16, 64, True, False), (synth.F32, 128, True, True),
    (synth.F32, 128, False, False)])
def test_rmsnorm_gate(gdtype, dv, with_gate, with_w):
    _require_gpu()
    T, H, eps = 333, 5, 1e-6
    print(f"[case] rmsnorm gate gdtype={gdtype} dv={dv} gate={with_gate} weight={with_w}",
          flush=True)
    o = synth.host_normal(synth.key(0, "o"), T * H, dv, dtype=synth.F32).reshape(T, H, dv)
    w = kc.custom_workload(synth.WORKLOADS[1 if gdtype == synth.BF16 else 0], heads=H, dv=dv)
    g = kc.host_tokens(w, "gate", T) if with_gate else None
    wt = (synth.host_normal(synth.key(0, "norm_w"), 1, dv, dtype=synth.F32, mean=1.0,
                            std=0.2)[0] if with_w else None)
    o_d = torch.from_numpy(o).cuda()
    y = kda.rmsnorm_gate(o_d, kc.to_torch(g) if g is not None else None,
                         torch.from_numpy(wt).cuda() if wt is not None else None, eps)
    y2 = kda.rmsnorm_gate(o_d.clone(), kc.to_torch(g) if g is not None else None,
                          torch.from_numpy(wt).cuda() if wt is not None else None, eps)
    o_in = o_d.clone()
    kda.rmsnorm_gate(o_in, kc.to_torch(g) if g is not None else None,
                     torch.from_numpy(wt).cuda() if wt is not None else None, eps, out=o_in)
    torch.cuda.synchronize()
    y_ref = layer.rmsnorm_gate(o, kc.f64(g) if g is not None else None, wt, eps)
    e = kc.rel_err(y.cpu().numpy(), y_ref)
    print(f"    err y={e:.3e}", flush=True)
    assert e <= kc.TOL_F32  # fp32 o, identical gate bits on both sides
    assert torch.equal(y, y2) and torch.equal(y, o_in)  # repeatable, and in place


def _round_bf16(x):
    """fp64 -> nearest-even bf16 (via fp32), back to fp64: the storage step
    between the front and the core when the layer runs on bf16 tensors."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    b = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("base", [1, 0])
def test_kda_layer_chain(base):
    """q, k through the front, the core without gate, then the RMSNorm gate,
    against the oracles chained the same way.  Each side runs its own chain
    (nothing the GPU produces reaches the oracle); with bf16 tensors both
    chains store the front's q, k in bf16 before the core.  The chain is
    ill-conditioned in q, k (Swish makes the keys strongly correlated, so a
    2^-8 change of k moves the state by several percent), which is why that
    storage step has to be the same on both sides."""
    _require_gpu()
    W0 = synth.WORKLOADS[base]
    w = kc.custom_workload(W0, heads=3, s0_std=0.02 if base else 0.5)
    lens = [300, 17, 0, 129]
    print(f"[case] layer chain {w.name} lens={lens}", flush=True)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = kc.host_inputs(w, T)
    s0 = kc.host_state(w, len(lens))
    wq = _conv_weights(w.heads, w.dk, 4, seed=2)
    wk = _conv_weights(w.heads, w.dk, 4, seed=3)
    nw = synth.host_normal(synth.key(1, "norm_w"), 1, w.dv, dtype=synth.F32, mean=1.0, std=0.2)[0]
    eps = 1e-6
    cu_d = torch.from_numpy(cu.astype(np.int32)).cuda()
    dev = {n: kc.to_torch(x[n]) for n in x}
    qf = kda.shortconv_swish_l2(dev["q"], torch.from_numpy(wq).cuda(), cu_d)
    kf = kda.shortconv_swish_l2(dev["k"], torch.from_numpy(wk).cuda(), cu_d)
    o, sf = kda.fwd_chunked(qf, kf, dev["v"], dev["a"], dev["b"], None, cu_d,
                            torch.from_numpy(s0).cuda() if s0 is not None else None)
    y = kda.rmsnorm_gate(o, dev["gate"], torch.from_numpy(nw).cuda(), eps)
    torch.cuda.synchronize()
    xr = {n: kc.f64(x[n]) for n in x}
    qr, _ = layer.shortconv_swish_l2(xr["q"], wq, cu)
    kr, _ = layer.shortconv_swish_l2(xr["k"], wk, cu)
    if W0.dtype == synth.BF16:
        qr, kr = _round_bf16(qr), _round_bf16(kr)
    o_ref, sf_ref = oracle.fwd(qr, kr, xr["v"], xr["a"], xr["b"], None, cu, s0)
    y_ref = layer.rmsnorm_gate(o_ref, xr["gate"], nw, eps)
    eo, ey = kc.rel_err(o.cpu().numpy(), o_ref), kc.rel_err(y.cpu().numpy(), y_ref)
    es = kc.rel_err(sf.cpu().numpy(), sf_ref)
    tol = _tol(W0.dtype)
    print(f"    err o={eo:.3e} y={ey:.3e} state={es:.3e} (tol {tol:.0e})", flush=True)
    assert eo <= tol and es <= tol and ey <= tol


# --- the forward with the head-wise RMSNorm before the gate ------------------
# path -> (base workload, heads, lens): the two-pass form's whole-head state
# pass applies the norm in its output stage (more than 32 pairs at dv = 128,
# fewer than the compute units); the other shapes run the forward, then the
# norm pass in place.
NORM_PATHS = {
    "fused_in_state_pass": (1, 40, [300, 17, 0, 129]),
    "state_pass_no_gate": (1, 40, [300, 17, 0, 129]),
    "fused_kernel": (1, 32, [256, 256, 130, 256]),
    "sliced_state_pass": (1, 3, [300, 17, 0, 129]),
    "fp32": (0, 2, [200, 0, 77]),
}


def norm_err(y, y_ref, o_ref):
    """Error of a normed output against the oracle chain, per row scaled by
    the row's conditioning: the norm divides each (token, head) row by its own
    RMS, so the forward's rounding (bounded against RMS(o)) reaches a row of y
    amplified by kappa = RMS(o) / rms(row).  Returns (max over elements of
    |y - y_ref| / (RMS(y_ref) max(1, kappa_row)), plain max |y - y_ref| /
    RMS(y_ref), fraction of rows with kappa > 4)."""
    y = np.asarray(y, dtype=np.float64)
    d = np.abs(y - y_ref)
    rms_y = np.sqrt(np.mean(y_ref ** 2))
    rms_o = np.sqrt(np.mean(o_ref ** 2))
    row = np.sqrt(np.mean(o_ref ** 2, axis=-1, keepdims=True))
    kappa = np.maximum(1.0, rms_o / np.maximum(row, 1e-300))
    return (float(np.max(d / (rms_y * kappa))), float(np.max(d) / rms_y),
            float(np.mean(kappa > 4.0)))


@pytest.mark.parametrize("path", list(NORM_PATHS))
@pytest.mark.parametrize("with_w", [True, False])
def test_fwd_rmsnorm_gate(path, with_w):
    """kda_fwd_chunked_rmsnorm_gate against the oracles chained: the forward
    without gate, then RMSNorm (weight, eps) and the sigmoid gate."""
    _require_gpu()
    base, H, lens = NORM_PATHS[path]
    W = synth.WORKLOADS[base]
    w = kc.custom_workload(W, heads=H, s0_std=0.02,
                           dk=128 if base else 64, dv=128 if base else 64)
    gate = path != "state_pass_no_gate"
    print(f"[case] fwd rmsnorm gate path={path} weight={with_w} H={H} lens={lens}", flush=True)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = kc.host_inputs(w, T)
    s0 = kc.host_state(w, len(lens))
    nw = (synth.host_normal(synth.key(0, "norm_w"), 1, w.dv, dtype=synth.F32, mean=1.0,
                            std=0.3)[0] if with_w else None)
    eps = 1e-5
    dev = {n: kc.to_torch(x[n]) for n in x}
    y, sf = kda.fwd_chunked_rmsnorm_gate(
        *(dev[n] if (n != "gate" or gate) else None for n in ("q", "k", "v", "a", "b", "gate")),
        torch.from_numpy(cu.astype(np.int32)).cuda(), torch.from_numpy(s0).cuda(),
        torch.from_numpy(nw).cuda() if nw is not None else None, eps)
    torch.cuda.synchronize()
    xr = {n: kc.f64(x[n]) for n in x}
    o_ref, sf_ref = oracle.fwd(xr["q"], xr["k"], xr["v"], xr["a"], xr["b"], None, cu,
                               s0.astype(np.float64))
    y_ref = layer.rmsnorm_gate(o_ref, xr["gate"] if gate else None, nw, eps)
    ey, plain, frac = norm_err(y.cpu().numpy(), y_ref, o_ref)
    es = kc.rel_err(sf.cpu().numpy(), sf_ref)
    tol = _tol(w.dtype)
    print(f"    err y={ey:.3e} (unscaled {plain:.3e}, rows with kappa > 4: {frac:.2%}) "
          f"state={es:.3e} (tol {tol:.0e})", flush=True)
    assert np.all(np.isfinite(y.cpu().numpy()))
    assert ey <= tol and es <= tol
    # the norm in the forward's output stage equals the forward followed by
    # the separate norm pass (the same fp32 o; only the order of the row sums
    # differs)
    cu_d = torch.from_numpy(cu.astype(np.int32)).cuda()
    o2, sf2 = kda.fwd_chunked(*(dev[n] for n in ("q", "k", "v", "a", "b")), None, cu_d,
                              torch.from_numpy(s0).cuda())
    y2 = kda.rmsnorm_gate(o2, dev["gate"] if gate else None,
                          torch.from_numpy(nw).cuda() if nw is not None else None, eps)
    torch.cuda.synchronize()
    e2 = kc.rel_err(y.cpu().numpy(), y2.cpu().numpy())
    print(f"    against the forward then the norm pass: {e2:.3e}", flush=True)
    assert e2 <= 1e-5 and torch.equal(sf, sf2)


def test_fwd_rmsnorm_gate_many_blocks():
    """The norm in the output stage of the two-pass form over several blocks
    (1 x 60,000 tokens x 96 heads): every row of 12 heads against the oracle
    chain, the oracle streamed."""
    _require_gpu()
    w = kc.custom_workload(synth.WORKLOADS[3], s0_std=0.02)
    T, H = 60_000, w.heads
    heads = [0, 7, 19, 31, 40, 52, 63, 71, 80, 88, 94, 95]
    print(f"[case] fwd rmsnorm gate many blocks T={T} H={H}", flush=True)
    dev = {n: synth.device_tokens(w, n, T) for n in synth.TOKEN_TENSORS}
    s0 = synth.device_state(w, 1)
    nw = synth.host_normal(synth.key(0, "norm_w"), 1, w.dv, dtype=synth.F32, mean=1.0,
                           std=0.3)[0]
    eps = 1e-5
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    y, sf = kda.fwd_chunked_rmsnorm_gate(*(dev[n] for n in ("q", "k", "v", "a", "b", "gate")),
                                         cu, s0, torch.from_numpy(nw).cuda(), eps)
    torch.cuda.synchronize()
    names = ("q", "k", "v", "a", "b", "gate")
    got, refs, o_refs = [], [], []

    def fetch(t0, t1):
        return {nm: kc.device_rows_f64(dev[nm], t0, t1, heads) for nm in names}

    def on_slice(t0, t1, o_ref):
        g = kc.device_rows_f64(dev["gate"], t0, t1, heads)
        got.append(y[t0:t1, heads].cpu().numpy())
        refs.append(layer.rmsnorm_gate(o_ref, g, nw, eps))
        o_refs.append(o_ref)

    s_ref = kc.oracle_stream(fetch, T, s0[0, heads].cpu().numpy()[None].astype(np.float64),
                             gate=False, on_slice=on_slice)
    ey, plain, frac = norm_err(np.concatenate(got), np.concatenate(refs),
                               np.concatenate(o_refs))
    es = kc.rel_err(sf[0, heads].cpu().numpy(), s_ref[0])
    print(f"    err y={ey:.3e} (unscaled {plain:.3e}, rows with kappa > 4: {frac:.2%}) "
          f"state={es:.3e}", flush=True)
    assert ey <= kc.TOL_BF16 and es <= kc.TOL_BF16
