"""GPU parity of the long-context workload (1 x 1,048,576 tokens, H=96,
dk=dv=128, bf16 inputs, fp32 state and output) against the fp64 oracle, in
the launch configuration the benchmark times.

One forward over device-generated inputs serves every test of this module:
  * the first 4096 output rows of three heads (nothing earlier feeds them);
  * the last 4096 output rows and the final state of all 96 heads, from the
    oracle started at a zero state 8192 tokens before the end: the dropped
    start state's effect is below 1e-15 there by the forgetting bound pinned
    on the CPU (tests/test_oracle_pins.py, long-context tail window);
  * every output row and the final state of 8 heads over the whole sequence,
    the oracle streamed in 65,536-token slices with its state carried;
  * split invariance at full size (two halves with the state carried).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import kda_cases as kc
from tests.test_oracle_pins import TAIL_SKIP, TAIL_WINDOW

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import delta_rule_linear_kda_amd as kda  # noqa: E402

W3 = synth.WORKLOADS[3]
NAMES = ("q", "k", "v", "a", "b", "gate")


@pytest.fixture(scope="module")
def run():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = W3
    T, H = w.seq_lens()[0], w.heads
    print(f"[case] cfg3 forward T={T} H={H}", flush=True)
    dev = {n: kc.device_tokens(w, n, T) for n in synth.TOKEN_TENSORS}
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    o, sf = kda.fwd_chunked(*(dev[n] for n in NAMES), cu)
    torch.cuda.synchronize()
    yield dev, o, sf
    del dev, o, sf
    torch.cuda.empty_cache()


def _fetch(dev, heads):
    def f(t0, t1):
        x = {n: kc.device_rows_f64(dev[n], t0, t1, heads) for n in NAMES}
        return x
    return f


def test_cfg3_finite(run):
    _, o, sf = run
    assert bool(torch.isfinite(sf).all())
    for r0 in range(0, o.shape[0], 1 << 16):
        assert bool(torch.isfinite(o[r0:r0 + (1 << 16)]).all())


def test_cfg3_head_prefix(run):
    """Every output row of heads 0, 47, 95 over tokens [0, 4096); the device
    generator's bits equal the host generator's there."""
    dev, o, _ = run
    t_s = 4096
    for h in (0, 47, 95):
        x = {nm: kc.host_head_slice(W3, nm, 0, t_s, h) for nm in synth.TOKEN_TENSORS}
        for nm in synth.TOKEN_TENSORS:
            d = dev[nm][:t_s, h].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            np.testing.assert_array_equal(d.reshape(x[nm].shape), x[nm])
        xr = {nm: kc.f64(x[nm])[:, None] for nm in x}
        o_ref, _ = oracle.fwd(xr["q"], xr["k"], xr["v"], xr["a"], xr["b"], xr["gate"], [0, t_s])
        eo = kc.rel_err(o[:t_s, h].cpu().numpy(), o_ref[:, 0])
        print(f"    head {h}, tokens [0, {t_s}): err o={eo:.3e}", flush=True)
        assert eo <= kc.TOL_BF16


def test_cfg3_tail_all_heads(run):
    """The last 4096 output rows and the final state of all 96 heads against
    the oracle started from zero 8192 tokens before the end."""
    dev, o, sf = run
    T, H = o.shape[0], o.shape[1]
    t0 = T - TAIL_WINDOW
    heads = list(range(H))
    # the tail's bits come from the same generator as the host's
    xh = synth.host_head_slice(W3, "k", t0, t0 + 64, 95)
    d = dev["k"][t0:t0 + 64, 95].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(d, xh)
    x = _fetch(dev, heads)(t0, T)
    o_ref, s_ref = oracle.fwd(x["q"], x["k"], x["v"], x["a"], x["b"], x["gate"],
                              [0, TAIL_WINDOW])
    eo = kc.rel_err(o[T - (TAIL_WINDOW - TAIL_SKIP):].cpu().numpy(), o_ref[TAIL_SKIP:])
    es = kc.rel_err(sf.cpu().numpy(), s_ref)
    print(f"    tokens [{t0 + TAIL_SKIP}, {T}) all heads: err o={eo:.3e}; "
          f"final state all heads: err={es:.3e}", flush=True)
    assert eo <= kc.TOL_BF16 and es <= kc.TOL_BF16


FULL_HEADS = [0, 13, 27, 40, 54, 67, 81, 95]


@pytest.mark.slow
def test_cfg3_full_length_heads(run):
    """Every output row and the final state of 8 heads over all 1,048,576
    tokens, the oracle streamed in 65,536-token slices."""
    dev, o, sf = run
    T = o.shape[0]
    acc = kc.ErrAcc()

    def on_slice(t0, t1, o_ref):
        acc.add(o[t0:t1, FULL_HEADS].cpu().numpy(), o_ref)

    s_ref = kc.oracle_stream(_fetch(dev, FULL_HEADS), T, None, on_slice=on_slice)
    es = kc.rel_err(sf[0, FULL_HEADS].cpu().numpy(), s_ref[0])
    print(f"    heads {FULL_HEADS}, all {T} tokens: err o={acc.err():.3e} "
          f"final state={es:.3e}", flush=True)
    assert acc.err() <= kc.TOL_BF16 and es <= kc.TOL_BF16


def test_cfg3_split_invariance(run):
    """Running the two halves with the state carried reproduces the single
    run's second-half outputs and final state (to the bf16 bound)."""
    dev, o, sf = run
    T = o.shape[0]
    half = T // 2 + 13  # off the chunk grid
    cu1 = torch.tensor([0, half], dtype=torch.int32, device="cuda")
    cu2 = torch.tensor([0, T - half], dtype=torch.int32, device="cuda")
    o_a, s_a = kda.fwd_chunked(*(dev[n][:half] for n in NAMES), cu1)
    del o_a
    o_b, s_b = kda.fwd_chunked(*(dev[n][half:] for n in NAMES), cu2, s_a)
    torch.cuda.synchronize()
    eo = kc.rel_err_device(o_b, o[half:])
    es = kc.rel_err(s_b.cpu().numpy(), sf.cpu().numpy())
    print(f"    split at {half}: err o={eo:.3e} state={es:.3e}", flush=True)
    assert eo <= kc.TOL_BF16 and es <= kc.TOL_BF16
