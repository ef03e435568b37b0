"""Host-side checks of the seeded input generator (CPU only)."""
import numpy as np

import synth


def test_deterministic_and_sliceable():
    k = synth.key(0, "q")
    x = synth.host_normal(k, 64, 32, dtype=synth.F32)
    y = synth.host_normal(k, 64, 32, dtype=synth.F32)
    np.testing.assert_array_equal(x, y)
    # any sub-block regenerates from its element indices alone
    z = synth.host_normal(k, 10, 5, dtype=synth.F32, row_stride=32, base=3 * 32 + 7)
    np.testing.assert_array_equal(z, x[3:13, 7:12])


def test_streams_differ():
    a = synth.host_normal(synth.key(0, "q"), 4, 8, dtype=synth.F32)
    b = synth.host_normal(synth.key(0, "k"), 4, 8, dtype=synth.F32)
    c = synth.host_normal(synth.key(0, "q", step=1), 4, 8, dtype=synth.F32)
    d = synth.host_normal(synth.key(1, "q"), 4, 8, dtype=synth.F32)
    for other in (b, c, d):
        assert not np.any(a == other)


def test_normal_moments():
    x = synth.host_normal(synth.key(0, "v"), 2000, 500, dtype=synth.F32).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    # fourth moment of a normal is 3
    assert abs((x ** 4).mean() - 3.0) < 0.05
    y = synth.host_normal(synth.key(0, "s0"), 1000, 128, dtype=synth.F32, std=0.02)
    assert abs(y.std() - 0.02) < 2e-4


def test_bf16_is_round_to_nearest_even_of_f32():
    k = synth.key(0, "a")
    f = synth.host_normal(k, 500, 128, dtype=synth.F32, std=np.sqrt(3.0))
    h = synth.host_normal(k, 500, 128, dtype=synth.BF16, std=np.sqrt(3.0))
    u = f.view(np.uint32).astype(np.uint64)
    lower = (u >> 16) << 16
    rem = u - lower
    up = (rem > 0x8000) | ((rem == 0x8000) & (((u >> 16) & 1) == 1))
    expect = ((u >> 16) + up).astype(np.uint16)
    np.testing.assert_array_equal(h, expect)
    assert np.max(np.abs(synth.to_f64(h) - f) / np.abs(f)) <= 2.0 ** -8   # bf16 unit roundoff


def test_lengths_range():
    w = synth.WORKLOADS[2]
    lens = w.seq_lens()
    assert len(lens) == 16 and min(lens) >= 256 and max(lens) <= 16384
    assert w.seq_lens() == lens
    many = synth.uniform_ints(synth.key(5, "lengths"), 20000, 256, 16384)
    assert many.min() >= 256 and many.max() <= 16384
    small = synth.uniform_ints(synth.key(5, "lengths"), 5000, 256, 260)
    assert sorted(set(small.tolist())) == [256, 257, 258, 259, 260]
    counts = np.bincount(small - 256)
    assert counts.min() > 850 and counts.max() < 1150
