"""Pins of the 3-D long-convolution oracle (one gated step on an A x H x W grid,
input zero-padded to the doubled grid, kernel given on the doubled grid), CPU only.

The direct sum and the FFT form agree; a kernel with only its first depth slice
set is the 2-D step on every slice (the separately pinned 2-D oracle); a causal
separable kernel is three 1-D causal convolutions, one per axis; a delta kernel
gives the gating closed form; shift kernels one step forward and one step back
along each axis move the input by one step with zeros entering at the edge.
"""
import numpy as np
import pytest

import oracle


def _inputs(B=2, D=2, A=2, H=4, W=4, seed=0):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((B, D, A, H, W))
    g = rng.standard_normal((B, D, A, H, W))
    x = rng.standard_normal((B, D, A, H, W))
    k = rng.standard_normal((D, 2 * A, 2 * H, 2 * W))
    bias = rng.standard_normal(D)
    return v, g, x, k, bias


@pytest.mark.parametrize("A,H,W", [(1, 1, 1), (1, 2, 4), (2, 4, 2), (4, 2, 4), (3, 2, 2)])
def test_direct_and_fft_agree(A, H, W):
    v, g, x, k, bias = _inputs(A=A, H=H, W=W, seed=A * 100 + H * 10 + W)
    a = oracle.conv3d_forward(v, k, bias, g, x, mode="direct")
    b = oracle.conv3d_forward(v, k, bias, g, x, mode="fft")
    assert np.allclose(a, b, rtol=1e-11, atol=1e-11)


def test_first_slice_kernel_is_the_2d_step_on_every_slice():
    v, g, x, k, bias = _inputs(A=3, H=4, W=8, seed=3)
    k[:, 1:] = 0.0
    y = oracle.conv3d_forward(v, k, bias, g, x, mode="direct")
    for a in range(3):
        want = oracle.conv2d_forward(v[:, :, a], k[:, 0], bias, g[:, :, a], x[:, :, a], mode="direct")
        assert np.allclose(y[:, :, a], want, rtol=1e-12, atol=1e-12)


def test_causal_separable_kernel_is_three_1d_causal_convolutions():
    rng = np.random.default_rng(1)
    B, D, A, H, W = 1, 2, 4, 4, 8
    v = rng.standard_normal((B, D, A, H, W))
    fa, fh, fw = rng.standard_normal((D, A)), rng.standard_normal((D, H)), rng.standard_normal((D, W))
    k = np.zeros((D, 2 * A, 2 * H, 2 * W))
    k[:, :A, :H, :W] = fa[:, :, None, None] * fh[:, None, :, None] * fw[:, None, None, :]
    y = oracle.conv3d_forward(v, k, np.zeros(D), mode="fft")
    want = v.copy()
    for d in range(D):
        for axis, f in ((2, fa[d]), (3, fh[d]), (4, fw[d])):
            want[:, d] = np.apply_along_axis(lambda r: oracle.causal_conv(r, f, "direct"), axis - 1, want[:, d])
    assert np.allclose(y, want, rtol=1e-11, atol=1e-11)


def test_delta_kernel_gives_the_gating_closed_form():
    v, g, x, k, bias = _inputs(seed=2)
    k[:] = 0.0
    k[:, 0, 0, 0] = 1.0
    y = oracle.conv3d_forward(v, k, bias, g, x, mode="direct")
    want = (1.0 + bias[None, :, None, None, None]) * v * g * x
    assert np.allclose(y, want, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("mode", ["direct", "fft"])
@pytest.mark.parametrize("axis", [0, 1, 2])
def test_shift_kernels_move_the_input_by_one_step(mode, axis):
    v, _, _, k, _ = _inputs(B=1, D=1, A=4, H=4, W=4, seed=5)
    n = v.shape[2 + axis]
    for off, idx in ((1, 1), (-1, 2 * n - 1)):
        k[:] = 0.0
        pos = [0, 0, 0]
        pos[axis] = idx
        k[0, pos[0], pos[1], pos[2]] = 1.0
        y = oracle.conv3d_forward(v, k, np.zeros(1), mode=mode)
        want = np.zeros_like(v)
        src = [slice(None)] * 5
        dst = [slice(None)] * 5
        if off == 1:
            dst[2 + axis], src[2 + axis] = slice(1, None), slice(0, n - 1)
        else:
            dst[2 + axis], src[2 + axis] = slice(0, n - 1), slice(1, None)
        want[tuple(dst)] = v[tuple(src)]
        assert np.allclose(y, want, rtol=1e-12, atol=1e-12), (axis, off)


# ---------------------------------------------------------------- circular mode

@pytest.mark.parametrize("A,H,W", [(1, 1, 1), (2, 2, 4), (4, 2, 2), (3, 2, 5)])
def test_circular_direct_and_fft_agree(A, H, W):
    v, g, x, _, bias = _inputs(A=A, H=H, W=W, seed=A * 50 + H * 7 + W)
    k = np.random.default_rng(A + H + W).standard_normal((v.shape[1], A, H, W))
    a = oracle.conv3d_forward(v, k, bias, g, x, mode="direct", circular=True)
    b = oracle.conv3d_forward(v, k, bias, g, x, mode="fft", circular=True)
    assert np.allclose(a, b, rtol=1e-11, atol=1e-11)


def test_circular_first_slice_kernel_is_the_circular_2d_step_on_every_slice():
    v, g, x, _, bias = _inputs(A=3, H=4, W=8, seed=13)
    k = np.zeros((v.shape[1], 3, 4, 8))
    k[:, 0] = np.random.default_rng(14).standard_normal((v.shape[1], 4, 8))
    y = oracle.conv3d_forward(v, k, bias, g, x, mode="direct", circular=True)
    for a in range(3):
        want = oracle.conv2d_forward(v[:, :, a], k[:, 0], bias, g[:, :, a], x[:, :, a], mode="direct",
                                     circular=True)
        assert np.allclose(y[:, :, a], want, rtol=1e-12, atol=1e-12)


def test_circular_step_on_the_doubled_grid_is_the_zero_padded_step():
    v, g, x, k, bias = _inputs(A=2, H=4, W=4, seed=15)
    B, D, A, H, W = v.shape
    pad = np.zeros((B, D, 2 * A, 2 * H, 2 * W))
    pad[:, :, :A, :H, :W] = v * g
    y = oracle.conv3d_forward(pad, k, bias, mode="fft", circular=True)[:, :, :A, :H, :W] * x
    want = oracle.conv3d_forward(v, k, bias, g, x, mode="direct")
    assert np.allclose(y, want, rtol=1e-11, atol=1e-11)


def test_circular_depth_shift_wraps_around():
    v, _, _, _, _ = _inputs(B=1, D=1, A=4, H=2, W=4, seed=16)
    k = np.zeros((1, 4, 2, 4))
    k[0, 1, 0, 0] = 1.0
    y = oracle.conv3d_forward(v, k, np.zeros(1), mode="fft", circular=True)
    assert np.allclose(y, np.roll(v, 1, axis=2), rtol=1e-12, atol=1e-12)
