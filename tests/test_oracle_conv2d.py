"""Pins of the 2-D long-convolution oracle (one gated step on an H x W grid, input
zero-padded to the doubled grid, kernel given on the doubled grid), CPU only.

The direct sum and the FFT form agree; a causal separable kernel reduces to the
separately pinned 1-D causal convolution along each axis; a delta kernel gives the
gating closed form; shift kernels one step forward and one step back (the wrapped
offset) move the input by exactly one row or column with zeros entering at the
edge, which fixes the kernel's offset convention.
"""
import numpy as np
import pytest

import oracle


def _inputs(B=2, D=3, H=4, W=8, seed=0):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((B, D, H, W))
    g = rng.standard_normal((B, D, H, W))
    x = rng.standard_normal((B, D, H, W))
    k = rng.standard_normal((D, 2 * H, 2 * W))
    bias = rng.standard_normal(D)
    return v, g, x, k, bias


@pytest.mark.parametrize("H,W", [(1, 1), (2, 4), (4, 8), (8, 2)])
def test_direct_and_fft_agree(H, W):
    v, g, x, k, bias = _inputs(H=H, W=W, seed=H * 10 + W)
    a = oracle.conv2d_forward(v, k, bias, g, x, mode="direct")
    b = oracle.conv2d_forward(v, k, bias, g, x, mode="fft")
    assert np.allclose(a, b, rtol=1e-11, atol=1e-11)


def test_causal_separable_kernel_is_two_1d_causal_convolutions():
    rng = np.random.default_rng(1)
    B, D, H, W = 2, 2, 8, 16
    v = rng.standard_normal((B, D, H, W))
    a = rng.standard_normal((D, H))
    b = rng.standard_normal((D, W))
    k = np.zeros((D, 2 * H, 2 * W))
    k[:, :H, :W] = a[:, :, None] * b[:, None, :]
    y = oracle.conv2d_forward(v, k, np.zeros(D), mode="fft")
    want = np.empty_like(v)
    for bb in range(B):
        for d in range(D):
            cols = np.stack([oracle.causal_conv(v[bb, d, :, q], a[d], "direct") for q in range(W)], axis=1)
            want[bb, d] = np.stack([oracle.causal_conv(cols[p], b[d], "direct") for p in range(H)])
    assert np.allclose(y, want, rtol=1e-11, atol=1e-11)


def test_delta_kernel_gives_the_gating_closed_form():
    v, g, x, k, bias = _inputs(seed=2)
    k[:] = 0.0
    k[:, 0, 0] = 1.0
    y = oracle.conv2d_forward(v, k, bias, g, x, mode="direct")
    want = (1.0 + bias[None, :, None, None]) * v * g * x
    assert np.allclose(y, want, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("mode", ["direct", "fft"])
def test_shift_kernels_fix_the_offset_convention(mode):
    v, _, _, k, _ = _inputs(B=1, D=4, H=4, W=8, seed=3)
    H, W = 4, 8
    k[:] = 0.0
    k[0, 1, 0] = 1.0            # one row forward:  c[p] = v[p - 1]
    k[1, 2 * H - 1, 0] = 1.0    # one row back:     c[p] = v[p + 1]
    k[2, 0, 1] = 1.0            # one column forward
    k[3, 0, 2 * W - 1] = 1.0    # one column back
    c = oracle.conv2d_forward(v, k, np.zeros(4), mode=mode)[0]
    z = np.zeros_like(v[0, 0])
    fwd_r = z.copy(); fwd_r[1:] = v[0, 0, :-1]
    bwd_r = z.copy(); bwd_r[:-1] = v[0, 1, 1:]
    fwd_c = z.copy(); fwd_c[:, 1:] = v[0, 2, :, :-1]
    bwd_c = z.copy(); bwd_c[:, :-1] = v[0, 3, :, 1:]
    for got, want in zip(c, (fwd_r, bwd_r, fwd_c, bwd_c)):
        assert np.allclose(got, want, atol=1e-12)


def test_rejects_a_kernel_not_on_the_doubled_grid():
    v, g, x, k, bias = _inputs()
    with pytest.raises(ValueError):
        oracle.conv2d_forward(v, k[:, :4], bias)


# ---------------------------------------------------------------- circular mode

@pytest.mark.parametrize("H,W", [(1, 1), (2, 4), (4, 8), (8, 2), (3, 5)])
def test_circular_direct_and_fft_agree(H, W):
    v, g, x, _, bias = _inputs(H=H, W=W, seed=H * 7 + W)
    k = np.random.default_rng(H + W).standard_normal((v.shape[1], H, W))
    a = oracle.conv2d_forward(v, k, bias, g, x, mode="direct", circular=True)
    b = oracle.conv2d_forward(v, k, bias, g, x, mode="fft", circular=True)
    assert np.allclose(a, b, rtol=1e-11, atol=1e-11)


def test_circular_single_row_is_the_1d_circular_convolution():
    """H = 1: each image row is the separately pinned 1-D circular convolution."""
    v, _, _, _, _ = _inputs(H=1, W=16, seed=8)
    k = np.random.default_rng(9).standard_normal((v.shape[1], 1, 16))
    y = oracle.conv2d_forward(v, k, np.zeros(v.shape[1]), mode="direct", circular=True)
    for b in range(v.shape[0]):
        for d in range(v.shape[1]):
            assert np.allclose(y[b, d, 0], oracle.circular_conv(v[b, d, 0], k[d, 0], "direct"), rtol=1e-12,
                               atol=1e-12)


def test_circular_step_on_the_doubled_grid_is_the_zero_padded_step():
    """The zero-padded step is the circular step on the doubled grid of the padded
    image, truncated: this ties the two modes' kernel conventions together."""
    v, g, x, k, bias = _inputs(H=4, W=8, seed=10)
    B, D, H, W = v.shape
    pad = np.zeros((B, D, 2 * H, 2 * W))
    pad[:, :, :H, :W] = v * g
    xp = np.ones((B, D, 2 * H, 2 * W))
    xp[:, :, :H, :W] = x
    y = oracle.conv2d_forward(pad, k, bias, None, xp, mode="direct", circular=True)[:, :, :H, :W]
    want = oracle.conv2d_forward(v, k, bias, g, x, mode="direct")
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12)


def test_circular_shift_kernel_wraps_around():
    v, _, _, _, _ = _inputs(B=1, D=1, H=4, W=8, seed=11)
    k = np.zeros((1, 4, 8))
    k[0, 1, 0] = 1.0  # one row forward: the last row comes back as the first
    y = oracle.conv2d_forward(v, k, np.zeros(1), mode="fft", circular=True)
    assert np.allclose(y, np.roll(v, 1, axis=2), rtol=1e-12, atol=1e-12)
    k[:] = 0.0
    k[0, 0, 7] = 1.0  # one column back, wrapped
    y = oracle.conv2d_forward(v, k, np.zeros(1), mode="fft", circular=True)
    assert np.allclose(y, np.roll(v, -1, axis=3), rtol=1e-12, atol=1e-12)
