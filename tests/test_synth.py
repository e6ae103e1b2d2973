"""Host-side checks of the seeded input generator (CPU only)."""
import numpy as np
import pytest

from fft_long_convolution_libhyena_amd import synth


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000)).astype(np.float32)
    # include exact ties: mantissa low half equal to 0x8000
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(synth.round_to_bf16(x), want)
    bits = synth.bf16_bits(want)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(bits), want)


def test_generate_shapes_and_determinism():
    wl = synth.custom(2, 3, 64, 3, kind="onehot", seed=3)
    a, b = synth.generate(wl), synth.generate(wl)
    assert a.u_proj.shape == (2, 12, 64) and a.short_w.shape == (12, 3)
    assert a.h.shape == (2, 3, 64) and a.bias.shape == (2, 3)
    for f in ("u_proj", "short_w", "h", "bias"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    # one-hot inputs: each time step takes one of four columns of the random Linear
    for bb in range(2):
        assert len({tuple(a.u_proj[bb, :, t]) for t in range(64)}) <= 4


def test_filter_decay_envelope():
    wl = synth.custom(1, 4, 256, 2, seed=1)
    x = synth.generate(wl)
    # channel 0 decays slowest (alpha_lo), the last channel fastest (alpha_hi)
    tail = np.abs(x.h[0, :, 200:]).mean(axis=1)
    assert tail[0] > tail[-1]


def test_sample_rows():
    wl = synth.WORKLOADS["long64k"]
    rows = synth.sample_rows(wl, 10)
    assert rows[0] == 0 and rows[-1] == wl.B * wl.D - 1 and len(rows) == 10
    assert np.all(np.diff(rows) > 0)
