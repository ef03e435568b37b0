"""GPU parity of the backward (kda_bwd_chunked) against the fp64 oracle's
reverse-mode backward (itself pinned by finite differences), through the C
ABI, on the same seeded inputs: every gradient tensor within max |gpu - ref| /
RMS(ref) <= 2e-2 (bf16 inputs) or 1e-4 (fp32 inputs)."""
import numpy as np
import pytest

import oracle
import synth
from tests import kda_cases as kc
from tests.test_gpu_edge import apply_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import delta_rule_linear_kda_amd as kda  # noqa: E402


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cotangents(w, T, N, seed):
    dy = synth.host_normal(synth.key(seed, "o", 1), T * w.heads, w.dv,
                           dtype=synth.F32).reshape(T, w.heads, w.dv)
    dsf = synth.host_normal(synth.key(seed, "o", 2), N * w.heads * w.dk, w.dv, dtype=synth.F32,
                            std=0.1).reshape(N, w.heads, w.dk, w.dv)
    return dy, dsf


def run_bwd(w, lens, gate=True, with_s0=True, with_dsf=True, label="", case=None, v_scale=1.0,
            tol_over=None):
    _require_gpu()
    print(f"[case] bwd {label} {w.name} H={w.heads} dk={w.dk} dv={w.dv} lens={lens} "
          f"gate={gate} s0={with_s0} dsf={with_dsf} case={case}", flush=True)
    T, N = sum(lens), len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = kc.host_inputs(w, T)
    if case is not None:
        apply_case(case, x, lens, w.dk, v_scale=v_scale)
    s0 = kc.host_state(w, N) if with_s0 else None
    dy, dsf = _cotangents(w, T, N, seed=3)
    dev = {n: kc.to_torch(x[n]) for n in x}
    g = kda.bwd_chunked(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"],
                        dev["gate"] if gate else None,
                        torch.from_numpy(cu.astype(np.int32)).cuda(),
                        torch.from_numpy(s0).cuda() if s0 is not None else None,
                        torch.from_numpy(dy).cuda(),
                        torch.from_numpy(dsf).cuda() if with_dsf else None)
    torch.cuda.synchronize()
    xr = {n: kc.f64(x[n]) for n in x}
    ref = oracle.bwd(xr["q"], xr["k"], xr["v"], xr["a"], xr["b"], xr["gate"] if gate else None,
                     cu, s0, dy, dsf if with_dsf else None)
    tol = kc.TOL_F32 if w.dtype == synth.F32 else kc.TOL_BF16
    errs = {}
    for key in ("dq", "dk", "dv", "da", "db", "dgate", "ds0"):
        if ref[key] is None:
            assert g[key] is None
            continue
        got = g[key].cpu().numpy()
        assert np.all(np.isfinite(got)), key
        errs[key] = kc.rel_err(got, ref[key])
    print("    err " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" (tol {tol:.0e})",
          flush=True)
    for key, e in errs.items():
        assert e <= (tol_over or {}).get(key, tol), (key, e)
    return g


LENS = [130, 1, 0, 77, 64, 200]


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_bwd_bf16_head_dims(dk, dv):
    w = kc.custom_workload(synth.WORKLOADS[1], heads=2, dk=dk, dv=dv, s0_std=0.02)
    run_bwd(w, LENS, label=f"bf16 {dk}x{dv}")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_fp32(d):
    w = kc.custom_workload(synth.WORKLOADS[0], heads=2, dk=d, dv=d, s0_std=0.5)
    run_bwd(w, LENS, label=f"fp32 d{d}")


@pytest.mark.parametrize("gate,s0,dsf", [(False, False, False), (True, False, True),
                                         (False, True, False)])
def test_bwd_optional_arguments(gate, s0, dsf):
    w = kc.custom_workload(synth.WORKLOADS[1], heads=3, s0_std=0.02)
    run_bwd(w, [70, 129, 5], gate=gate, with_s0=s0, with_dsf=dsf, label="optional")


def test_bwd_repeatable():
    w = kc.custom_workload(synth.WORKLOADS[1], heads=2, s0_std=0.02)
    g1 = run_bwd(w, [100, 50], label="repeat 1")
    g2 = run_bwd(w, [100, 50], label="repeat 2")
    for key in ("dq", "dk", "dv", "da", "db", "dgate", "ds0"):
        assert torch.equal(g1[key], g2[key]), key


def test_bwd_full_workload_sampled():
    """The training-shaped workload the benchmark times (4 x 4096 tokens, 32
    heads, d = 128, bf16, zero initial state, device-generated inputs and dy):
    every gradient of three sampled (sequence, head) pairs, recomputed by the
    oracle from host-regenerated slices of the same streams."""
    _require_gpu()
    w = synth.WORKLOADS[1]
    T, H = sum(w.seq_lens()), w.heads
    cu = np.asarray(w.cu_seqlens(), dtype=np.int64)
    print(f"[case] bwd full {w.name} T={T} H={H}", flush=True)
    dev = {n: kc.device_tokens(w, n, T) for n in synth.TOKEN_TENSORS}
    dy = torch.empty((T, H, w.dv), dtype=torch.float32, device="cuda")
    synth.device_normal(dy.view(-1, w.dv), synth.key(w.seed, "o", 1))
    g = kda.bwd_chunked(dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], dev["gate"],
                        torch.from_numpy(cu.astype(np.int32)).cuda(), None, dy, None)
    torch.cuda.synchronize()
    for n, h in [(0, 0), (1, 17), (3, 31)]:
        t0, t1 = int(cu[n]), int(cu[n + 1])
        xs = {name: kc.f64(kc.host_head_slice(w, name, t0, t1, h))[:, None]
              for name in synth.TOKEN_TENSORS}
        dys = synth.host_normal(synth.key(w.seed, "o", 1), t1 - t0, w.dv, dtype=synth.F32,
                                row_stride=H * w.dv, base=(t0 * H + h) * w.dv)[:, None]
        ref = oracle.bwd(xs["q"], xs["k"], xs["v"], xs["a"], xs["b"], xs["gate"],
                         [0, t1 - t0], None, dys, None)
        errs = {}
        for key in ("dq", "dk", "dv", "da", "db", "dgate"):
            got = g[key][t0:t1, h].cpu().numpy()
            assert np.all(np.isfinite(got)), key
            errs[key] = kc.rel_err(got, ref[key][:, 0])
        print(f"    seq {n} head {h} err " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
              flush=True)
        for key, e in errs.items():
            assert e <= kc.TOL_BF16, (n, h, key, e)


# The decay edge cases of the "Lower-bounded decay" paragraph (tile sums at
# -80, factors e^80), one-hot and orthonormal keys, and large values over
# large initial states, through both backward forms.
EDGE_LENS = [128, 57, 0, 100]


# With every decay logit at +8 (alpha = 6.7e-3 per token) the gradient of the
# decay logits is a sum of read-out and erase terms of the chunk-start states
# that cancel to about 1/15 of their size, so da carries the recomputed
# states' error amplified about 15x: the bf16 forward's states are within
# about 3e-3 (fp16 operands on the state path), and an fp64 model of the
# chunked backward with 3e-3 relative noise on those states gives 4.6e-2.
# da is held to 1e-1 there; every other gradient to 2e-2.
DA_SATURATED_BF16 = 1e-1


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case", ["a_pinf", "a_p8", "a_mix", "onehot", "orth"])
def test_bwd_edge_cases(dtype, case):
    base = synth.WORKLOADS[1] if dtype == "bf16" else synth.WORKLOADS[0]
    w = kc.custom_workload(base, heads=2, dk=128, dv=128, s0_std=0.02)
    over = {"da": DA_SATURATED_BF16} if (dtype, case) == ("bf16", "a_p8") else None
    run_bwd(w, EDGE_LENS, label=f"edge {dtype}", case=case, tol_over=over)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bwd_large_state_and_values(dtype):
    """Initial states of std 1e3 and values x 1e3: the gradients' products
    keep fp32's exponent range."""
    base = synth.WORKLOADS[1] if dtype == "bf16" else synth.WORKLOADS[0]
    w = kc.custom_workload(base, heads=2, dk=128, dv=128, s0_std=1e3)
    run_bwd(w, EDGE_LENS, label=f"large {dtype}", case="big_v", v_scale=1e3)
