"""Pins for the oracle's backward (``oracle.bwd``), CPU only.

Every gradient is checked element by element against central finite
differences of the forward oracle (``oracle.fwd``, itself pinned in
test_oracle_pins.py): the loss is L = sum <dy, y> + <dS_final, S_final>,
each input element is moved by +-h in fp64, and (L+ - L-) / 2h must equal the
analytic gradient.  The backward shares no code with the forward (a separate
reverse-mode routine), so a dropped term, a sign or a transposed product in
any gradient fails here."""
import numpy as np
import pytest

import oracle


def _inputs(lens, H, dk, dv, seed, gate=True, s0=True):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    x = {"q": rng.standard_normal((T, H, dk)), "k": rng.standard_normal((T, H, dk)),
         "v": rng.standard_normal((T, H, dv)), "a": rng.standard_normal((T, H, dk)) - 2.0,
         "b": rng.standard_normal((T, H)),
         "gate": rng.standard_normal((T, H, dv)) if gate else None,
         "s0": rng.standard_normal((len(lens), H, dk, dv)) if s0 else None}
    dy = rng.standard_normal((T, H, dv))
    dsf = rng.standard_normal((len(lens), H, dk, dv))
    return x, dy, dsf


def _loss(x, cu, dy, dsf):
    o, sf = oracle.fwd(x["q"], x["k"], x["v"], x["a"], x["b"], x["gate"], cu, x["s0"],
                       nthreads=1)
    return float((dy * o).sum() + (dsf * sf).sum())


@pytest.mark.parametrize("gate,s0,with_dsf", [(True, True, True), (False, False, False),
                                              (True, False, True)])
def test_backward_matches_finite_differences(gate, s0, with_dsf):
    lens, H, dk, dv = [4, 0, 3], 2, 3, 2
    x, dy, dsf = _inputs(lens, H, dk, dv, seed=11, gate=gate, s0=s0)
    if not with_dsf:
        dsf = np.zeros_like(dsf)
    cu = np.concatenate([[0], np.cumsum(lens)])
    g = oracle.bwd(x["q"], x["k"], x["v"], x["a"], x["b"], x["gate"], cu, x["s0"], dy,
                   dsf if with_dsf else None, nthreads=1)
    grads = {"q": g["dq"], "k": g["dk"], "v": g["dv"], "a": g["da"], "b": g["db"],
             "gate": g["dgate"], "s0": g["ds0"]}
    h = 1e-6
    checked = 0
    for name, arr in x.items():
        if arr is None:
            continue
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = arr[idx]
            arr[idx] = keep + h
            lp = _loss(x, cu, dy, dsf)
            arr[idx] = keep - h
            lm = _loss(x, cu, dy, dsf)
            arr[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grads[name], fd, rtol=2e-5, atol=2e-7, err_msg=name)
        checked += fd.size
    assert checked > 100
    if not gate:
        assert g["dgate"] is None


def test_backward_zero_cotangent_is_zero():
    x, dy, dsf = _inputs([5], 1, 4, 3, seed=12)
    g = oracle.bwd(x["q"], x["k"], x["v"], x["a"], x["b"], x["gate"], [0, 5], x["s0"],
                   np.zeros_like(dy), None, nthreads=1)
    for key in ("dq", "dk", "dv", "da", "db", "dgate", "ds0"):
        assert np.all(g[key] == 0.0), key


def test_backward_linear_in_cotangent():
    """Gradients are linear in (dy, dS_final)."""
    x, dy, dsf = _inputs([6, 2], 2, 4, 3, seed=13)
    cu = [0, 6, 8]
    args = (x["q"], x["k"], x["v"], x["a"], x["b"], x["gate"], cu, x["s0"])
    g1 = oracle.bwd(*args, dy, dsf, nthreads=1)
    g2 = oracle.bwd(*args, 2.5 * dy, 2.5 * dsf, nthreads=1)
    for key in ("dq", "dk", "dv", "da", "db", "dgate", "ds0"):
        np.testing.assert_allclose(g2[key], 2.5 * g1[key], rtol=1e-12, atol=1e-14)
