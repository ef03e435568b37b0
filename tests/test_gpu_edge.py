"""The method's degenerate cases through every HIP forward path and decode,
element by element against the fp64 oracle (through the C ABI).

Cases (page "[Paper Review] Kimi K3...", section "Kimi Delta Attention
(KDA)"; the "Lower-bounded decay" paragraph bounds g below by -5, so the
cumulative log-decay of a 16-token tile lies in [-80, 0] and its column
factors reach e^80):
  a_pinf   decay logits +inf on every channel: g = -5 exactly, tile sums -80
  a_p8     decay logits +8 on every channel: g = -4.998, tile sums near -80
  a_mix    decay logits +-inf by sign: channels switch between g = -5 and
           g = 0 from token to token
  onehot   one-hot keys, distinct within each sequence (gated linear
           attention in closed form; pinned on the CPU)
  orth     orthonormal keys with beta = 1 (b = +inf) and g = 0 (a = -inf):
           causal linear attention (pinned on the CPU)
  big_s0   initial states ~ N(0, s^2) and values x s for s = 1e3, 1e5: the
           fp32 state must not be limited by a 16-bit operand's range (65504)
  mixed    initial states ~ N(0, 1e10) with values x 1e3 over 60,000 tokens:
           the first outputs are ~1000 times the later ones; checked for
           finite results, the final state, and the outputs after the first
           5,920 tokens (the state-path products carry fp16's relative
           precision of the state's current scale, so the transient's own
           rounding is ~3e-4 of its scale, which the whole sequence's RMS
           does not reflect)
Paths: the fused kernel (enough (sequence, head) pairs to fill the device),
the two-pass form in one block of records (64-column state slices; few and
many pairs), the two-pass form over several blocks of chunks with whole-head
state workgroups (1 x 60,000 tokens x 96 heads), the fp32 kernel, and
decode.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import kda_cases as kc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import delta_rule_linear_kda_amd as kda  # noqa: E402

W0, W1, W3, W4 = (synth.WORKLOADS[i] for i in (0, 1, 3, 4))
NAMES = ("q", "k", "v", "a", "b", "gate")
BF16_PINF, BF16_NINF = np.uint16(0x7F80), np.uint16(0xFF80)


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _const(arr, value):
    """An array like `arr` (fp32, or bf16 bit patterns) filled with value."""
    if arr.dtype == np.uint16:
        bits = np.array([value], dtype=np.float32).view(np.uint32)[0] >> 16
        return np.full_like(arr, np.uint16(bits))
    return np.full_like(arr, np.float32(value))


def _sign_inf(arr):
    """+inf where the value is >= 0, -inf where it is negative."""
    if arr.dtype == np.uint16:
        return np.where(arr & 0x8000, BF16_NINF, BF16_PINF).astype(np.uint16)
    return np.where(arr < 0, -np.inf, np.inf).astype(np.float32)


def _round_to(arr_f32, like):
    """fp32 values stored as `like` does (bf16 with round-to-nearest-even)."""
    if like.dtype == np.uint16:
        u = arr_f32.astype(np.float32).view(np.uint32).astype(np.uint64)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return arr_f32.astype(np.float32)


def apply_case(case, x, lens, dk, seed=5, v_scale=1e3):
    """Modify host inputs x in place for `case` (sequence lengths `lens`)."""
    rng = np.random.default_rng(seed)
    H = x["q"].shape[1]
    if case == "a_pinf":
        x["a"] = _const(x["a"], np.inf)
    elif case == "a_p8":
        x["a"] = _const(x["a"], 8.0)
    elif case == "a_mix":
        x["a"] = _sign_inf(x["a"])
    elif case in ("onehot", "orth"):
        k = np.zeros(x["k"].shape, dtype=np.float32)
        t0 = 0
        for L in lens:
            assert L <= dk
            for h in range(H):
                if case == "onehot":
                    c = rng.permutation(dk)[:L]
                    k[t0 + np.arange(L), h, c] = 1.0
                else:
                    qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
                    k[t0:t0 + L, h] = qm[:L]
            t0 += L
        x["k"] = _round_to(k, x["k"])
        if case == "orth":
            x["b"] = _const(x["b"], np.inf)
            x["a"] = _const(x["a"], -np.inf)
    elif case == "big_v":
        vf = synth.to_f64(x["v"]).astype(np.float32) * np.float32(v_scale)
        x["v"] = _round_to(vf, x["v"])
    else:
        raise ValueError(case)


# path -> (base workload, heads, sequence lengths, dk, dv)
PATHS = {
    "fused": (W1, 32, [128, 100, 77, 128], 128, 128),   # 128 pairs: two slices each fill 256 CUs
    "ct1": (W1, 3, [128, 57, 0, 100], 128, 128),       # 12 pairs: 64-column state slices
    "many": (W1, 12, [128, 100, 77, 128], 128, 128),   # 48 pairs, one block: 64-column slices
    "fp32": (W0, 2, [64, 50, 0, 64], 64, 64),
    "fp32_d128": (W0, 2, [128, 30], 128, 128),
}
CASES = ["a_pinf", "a_p8", "a_mix", "onehot", "orth"]


def run_small(path, case, s0_std=None):
    _require_gpu()
    base, H, lens, dk, dv = PATHS[path]
    w = kc.custom_workload(base, heads=H, dk=dk, dv=dv, s0_std=s0_std)
    print(f"[case] edge {case} path={path} H={H} lens={lens} s0_std={s0_std}", flush=True)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = kc.host_inputs(w, T)
    apply_case(case if case != "big_s0" else "big_v", x, lens, dk, v_scale=s0_std or 1.0)
    s0 = kc.host_state(w, len(lens)) if s0_std else None
    dev = {n: kc.to_torch(x[n]) for n in x}
    o, sf = kda.fwd_chunked(*(dev[n] for n in NAMES),
                            torch.from_numpy(cu.astype(np.int32)).cuda(),
                            torch.from_numpy(s0).cuda() if s0 is not None else None)
    torch.cuda.synchronize()
    o, sf = o.cpu().numpy(), sf.cpu().numpy()
    xr = {n: kc.f64(x[n]) for n in x}
    o_ref, sf_ref = oracle.fwd(*(xr[n] for n in NAMES), cu,
                               s0.astype(np.float64) if s0 is not None else None)
    eo, es = kc.rel_err(o, o_ref), kc.rel_err(sf, sf_ref)
    tol = kc.TOL_F32 if w.dtype == synth.F32 else kc.TOL_BF16
    print(f"    err o={eo:.3e} state={es:.3e} (tol {tol:.0e})", flush=True)
    if es > tol / 4:  # where the state's worst element sits
        i = np.unravel_index(np.argmax(np.abs(sf - sf_ref)), sf.shape)
        print(f"    worst state element {i}: gpu {sf[i]:.6e} ref {sf_ref[i]:.6e} "
              f"rms {np.sqrt(np.mean(sf_ref ** 2)):.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(sf))
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("case", CASES)
def test_edge_small(path, case):
    run_small(path, case)


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("s0_std", [1e3, 1e5])
def test_large_state_and_values(path, s0_std):
    """Initial states of std s and values x s for s = 1e3, 1e5 (the state
    and U exceed 65504, the largest fp16 value)."""
    run_small(path, "big_s0", s0_std=s0_std)


MULTI_T = 60_000
MULTI_HEADS = [0, 7, 19, 31, 40, 52, 63, 71, 80, 88, 94, 95]


@pytest.mark.parametrize("case", ["a_pinf", "a_p8", "a_mix", "big_s0", "mixed"])
def test_edge_multi_block(case):
    """The two-pass form over several blocks of chunks (1 x 60,000 tokens x
    96 heads: a quarter-size first block, then full blocks): every output
    row and the final state of 12 heads against the oracle over the whole
    sequence."""
    _require_gpu()
    w = kc.custom_workload(W3, s0_std=1e5 if case in ("big_s0", "mixed") else None)
    T, H = MULTI_T, w.heads
    ws = kda.fwd_workspace_bytes(1, T, H, w.dk, w.dv)
    print(f"[case] edge multi-block {case} T={T} H={H} workspace={ws}", flush=True)
    dev = {n: kc.device_tokens(w, n, T) for n in synth.TOKEN_TENSORS}
    if case == "a_pinf":
        dev["a"].fill_(float("inf"))
    elif case == "a_p8":
        dev["a"].fill_(8.0)
    elif case == "a_mix":
        dev["a"] = torch.where(dev["a"] < 0, float("-inf"), float("inf")).to(torch.bfloat16)
    else:
        dev["v"] = (dev["v"].float() * (1e5 if case == "big_s0" else 1e3)).to(torch.bfloat16)
    s0 = kc.device_state(w, 1)
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    o, sf = kda.fwd_chunked(*(dev[n] for n in NAMES), cu, s0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(sf).all())
    acc = kc.ErrAcc()

    def fetch(t0, t1):
        return {nm: kc.device_rows_f64(dev[nm], t0, t1, MULTI_HEADS) for nm in NAMES}


    per_slice = []
    skip = 5920 if case == "mixed" else 0  # the mixed case's transient (see above)

    def on_slice(t0, t1, o_ref):
        got = o[t0:t1, MULTI_HEADS].cpu().numpy()
        if t0 >= skip:
            acc.add(got, o_ref)
        per_slice.append((t0, float(np.abs(got - o_ref).max()), float(np.sqrt(np.mean(o_ref ** 2)))))

    s0_h = None if s0 is None else s0[0, MULTI_HEADS].cpu().numpy()[None].astype(np.float64)
    s_ref = kc.oracle_stream(fetch, T, s0_h, slice_tokens=5920, on_slice=on_slice)
    es = kc.rel_err(sf[0, MULTI_HEADS].cpu().numpy(), s_ref[0])
    print(f"    err o={acc.err():.3e} state={es:.3e}", flush=True)
    if acc.err() > kc.TOL_BF16 / 4:
        for t0, mx, rms in per_slice:
            print(f"      tokens from {t0}: max |diff| {mx:.3e}, slice rms {rms:.3e}", flush=True)
    assert acc.err() <= kc.TOL_BF16 and es <= kc.TOL_BF16


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
@pytest.mark.parametrize("case", CASES + ["big_s0"])
def test_edge_decode(dtype, case):
    """Decode steps under the same cases (one token per sequence per step;
    the key cases use one-hot / orthonormal keys within each step's batch)."""
    _require_gpu()
    w = kc.custom_workload(W4, num_seqs=6, heads=3, dtype=dtype,
                           s0_std=1e5 if case == "big_s0" else 0.02)
    N = w.num_seqs
    print(f"[case] edge decode {case} dtype={dtype}", flush=True)
    state = torch.from_numpy(kc.host_state(w, N)).cuda()
    s_ref = kc.host_state(w, N).astype(np.float64)
    tol = kc.TOL_F32 if dtype == synth.F32 else kc.TOL_BF16
    worst = 0.0
    for s in range(3):
        x = {n: kc.host_tokens(w, n, N, step=s) for n in synth.TOKEN_TENSORS}
        apply_case(case if case != "big_s0" else "big_v", x, [1] * N, w.dk, seed=s, v_scale=1e5)
        dev = {n: kc.to_torch(x[n]) for n in x}
        o = kda.decode_step(*(dev[n] for n in NAMES), state)
        o_ref = oracle.decode_step(*(kc.f64(x[n]) for n in NAMES), s_ref)
        worst = max(worst, kc.rel_err(o.cpu().numpy(), o_ref))
    es = kc.rel_err(state.cpu().numpy(), s_ref)
    print(f"    err o={worst:.3e} state={es:.3e}", flush=True)
    assert worst <= tol and es <= tol
