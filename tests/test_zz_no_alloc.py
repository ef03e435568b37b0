"""kda_fwd_chunked_noalloc (the forward whose scratch is the library's fixed
device array) against kda_fwd_chunked (workspace from the caller) through
the C ABI: two calls in a row, the second on a smaller input, then four
4096-token sequences (one block of records for the regular call, blocks in
sequence in the fixed array), then a shape that needs no scratch at all.  Same tolerance as every bf16 comparison here
(2e-2 of the reference's RMS); where both entry points cut the work into the
same blocks the results are bitwise equal."""
import numpy as np
import pytest

import synth
from tests import kda_cases as kc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import delta_rule_linear_kda_amd as kda  # noqa: E402

NAMES = ("q", "k", "v", "a", "b", "gate")


def _inputs(w, lens):
    T = int(sum(lens))
    dev = {n: synth.device_tokens(w, n, T) for n in synth.TOKEN_TENSORS}
    s0 = synth.device_state(w, len(lens))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    return dev, s0, cu


def _check(w, lens, expect_bitwise):
    print(f"[case] noalloc H={w.heads} lens={lens}", flush=True)
    dev, s0, cu = _inputs(w, lens)
    T = int(sum(lens))
    ws = kda.fwd_workspace_bytes(len(lens), T, w.heads, w.dk, w.dv)
    o_ref, s_ref = kda.fwd_chunked(*(dev[n] for n in NAMES), cu, s0)
    o = torch.full_like(o_ref, float("nan"))
    sf = torch.full_like(s_ref, float("nan"))
    kda.fwd_chunked_noalloc(*(dev[n] for n in NAMES), cu, s0, out=o, final_state=sf)
    torch.cuda.synchronize()
    eo = kc.rel_err_device(o, o_ref)
    es = kc.rel_err(sf.cpu().numpy(), s_ref.cpu().numpy())
    same = bool(torch.equal(o, o_ref)) and bool(torch.equal(sf, s_ref))
    print(f"    workspace of the regular call {ws} B; err o={eo:.3e} state={es:.3e} "
          f"bitwise={same}", flush=True)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(sf).all())
    assert eo <= kc.TOL_BF16 and es <= kc.TOL_BF16
    if expect_bitwise:
        assert same


def test_noalloc_matches_fwd_chunked():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w3 = synth.WORKLOADS[3]
    # 1) the two-pass form over many small blocks inside the fixed array
    #    (the regular call runs 3 large ones)
    _check(synth.custom_workload(w3, s0_std=0.02), [60_000], expect_bitwise=False)
    # 2) a smaller input right after: one block on both sides
    _check(synth.custom_workload(w3, heads=12, s0_std=0.02), [700, 0, 301], expect_bitwise=True)
    # 3) four 4096-token sequences x 32 heads: one block of records for the
    #    regular call, blocks in sequence inside the fixed array
    _check(synth.custom_workload(synth.WORKLOADS[1], s0_std=0.02), [4096] * 4,
           expect_bitwise=False)
    # 4) a shape of the fused kernel (no scratch)
    _check(synth.custom_workload(synth.WORKLOADS[1], s0_std=0.02), [256, 256, 130, 256],
           expect_bitwise=True)


def test_noalloc_rejects_beyond_scratch():
    """A shape whose fixed parts alone exceed the array: KDA_ERR_SCRATCH."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = synth.custom_workload(synth.WORKLOADS[3], heads=96)
    T = 2 << 20  # b transposed alone is 2 H T = 384 MiB
    small = {n: torch.empty(0, dtype=torch.bfloat16, device="cuda") for n in NAMES}
    shape = kda.Shape(1, T, 96, 128, 128, kda.KDA_BF16, kda.KDA_F32)
    import ctypes
    far = 1 << 40  # never dereferenced: rejected before anything is enqueued
    rc = kda.lib().kda_fwd_chunked_noalloc(ctypes.byref(shape), *[far + i * (1 << 39) for i in
                                                                  range(10)], None)
    assert rc == 8, kda.status_str(rc)
    del small, w
