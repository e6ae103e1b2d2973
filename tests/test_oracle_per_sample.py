"""Pins of the per-sample forward and backward oracles (a filter set per input sample), CPU only.

The per-sample oracle is the pinned forward oracle applied sample by sample; what
needs pinning is that sample b meets exactly filters h[b]: equal filter sets reduce
it to the shared forward bit for bit, each sample's output ignores the other
samples' filters, permuting samples with their filters permutes the outputs, and a
delta filter set on one sample gives the closed form of that sample alone. The
per-sample backward is pinned as the adjoint of the per-sample forward (exact
linearity in each step's filters and, at order 2, in the shared bias) and, with
equal filter sets, against the pinned shared backward.
"""
import numpy as np
import pytest

import oracle
from fft_long_convolution_libhyena_amd import synth


def _case(B=3, D=4, L=64, N=3, seed=1):
    wl = synth.custom(B, D, L, N, seed=seed)
    return wl, synth.generate(wl), synth.per_sample_filters(wl)


@pytest.mark.parametrize("mode", ["direct", "fft"])
def test_equal_filter_sets_give_the_shared_forward(mode):
    wl, x, _ = _case()
    hb = np.repeat(x.h[None], wl.B, axis=0)
    a = oracle.forward_per_sample(x.u_proj, x.short_w, hb, x.bias, wl.order, mode=mode)
    b = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, wl.order, mode=mode)
    assert np.array_equal(a, b)


def test_a_sample_ignores_the_other_samples_filters():
    wl, x, hb = _case()
    y = oracle.forward_per_sample(x.u_proj, x.short_w, hb, x.bias, wl.order)
    hb2 = hb.copy()
    hb2[1] *= -3.0
    y2 = oracle.forward_per_sample(x.u_proj, x.short_w, hb2, x.bias, wl.order)
    assert np.array_equal(y[0], y2[0]) and np.array_equal(y[2], y2[2])
    assert not np.allclose(y[1], y2[1])


def test_permuting_samples_with_their_filters_permutes_outputs():
    wl, x, hb = _case(B=4)
    y = oracle.forward_per_sample(x.u_proj, x.short_w, hb, x.bias, wl.order)
    perm = np.array([2, 0, 3, 1])
    yp = oracle.forward_per_sample(x.u_proj[perm], x.short_w, hb[perm], x.bias, wl.order)
    assert np.array_equal(yp, y[perm])


def test_delta_filters_on_one_sample_give_the_gating_closed_form():
    # order 2, sample 1 has delta filters: y = x0 (1 + bias) x1 v on that sample only
    wl, x, hb = _case(B=2, D=3, L=32, N=2)
    hb[1] = 0.0
    hb[1, :, :, 0] = 1.0
    y = oracle.forward_per_sample(x.u_proj, x.short_w, hb, x.bias, 2, mode="direct")
    D, L = wl.D, wl.L
    uc = np.stack([oracle.short_conv_row(x.u_proj[1, c], x.short_w[c]) for c in range(3 * D)])
    want = uc[:D] * (1.0 + x.bias[0][:, None].astype(np.float64)) * uc[D:2 * D] * uc[2 * D:]
    assert np.allclose(y[1], want, rtol=1e-13, atol=1e-13)


def test_rejects_a_filter_set_count_that_is_not_B():
    wl, x, hb = _case()
    with pytest.raises(ValueError):
        oracle.forward_per_sample(x.u_proj, x.short_w, hb[:2], x.bias, wl.order)


# ---------------------------------------------------------------- backward

@pytest.mark.parametrize("N", [2, 3])
def test_per_sample_backward_is_the_adjoint_of_the_per_sample_forward(N):
    """y is linear in the filters of one step h[:, o] (everything else fixed), so
    <y(h + delta) - y(h), dy> = <delta, dh[:, o]> exactly, with y from the separately
    pinned per-sample forward; the perturbed filters are fp32 values (the oracle's
    input precision), so delta is exact. At order 2 the same holds for the shared
    bias, whose gradient sums the samples' contributions."""
    wl, x, hb = _case(B=3, D=3, L=32, N=N, seed=4)
    rng = np.random.default_rng(7)
    dy = rng.standard_normal((wl.B, wl.D, wl.L)).astype(np.float32)  # the oracle's input precision
    du, dw, dh, db = oracle.backward_per_sample(x.u_proj, x.short_w, hb, x.bias, dy, N, mode="direct")
    y0 = oracle.forward_per_sample(x.u_proj, x.short_w, hb, x.bias, N, mode="direct")
    for o in range(N - 1):
        h1 = hb.copy()
        h1[:, o] = (hb[:, o] + rng.standard_normal(hb[:, o].shape)).astype(np.float32)
        delta = h1.astype(np.float64) - hb.astype(np.float64)
        y1 = oracle.forward_per_sample(x.u_proj, x.short_w, h1, x.bias, N, mode="direct")
        assert np.isclose(np.sum((y1 - y0) * dy), np.sum(delta * dh), rtol=1e-9, atol=1e-9), o
    if N == 2:
        b1 = (x.bias + rng.standard_normal(x.bias.shape)).astype(np.float32)
        y2 = oracle.forward_per_sample(x.u_proj, x.short_w, hb, b1, N, mode="direct")
        d_b = b1.astype(np.float64) - x.bias.astype(np.float64)
        assert np.isclose(np.sum((y2 - y0) * dy), np.sum(d_b * db), rtol=1e-9, atol=1e-9)


def test_per_sample_backward_with_equal_sets_sums_to_the_shared_backward():
    wl, x, _ = _case(B=3, D=2, L=64, N=3, seed=5)
    dy = np.random.default_rng(8).standard_normal((wl.B, wl.D, wl.L))
    hb = np.repeat(x.h[None], wl.B, axis=0)
    du, dw, dh, db = oracle.backward_per_sample(x.u_proj, x.short_w, hb, x.bias, dy, wl.order)
    du0, dw0, dh0, db0 = oracle.backward(x.u_proj, x.short_w, x.h, x.bias, dy, wl.order)
    assert np.allclose(du, du0, rtol=1e-12, atol=1e-12)
    assert np.allclose(dw, dw0, rtol=1e-10, atol=1e-10)
    assert np.allclose(dh.sum(axis=0), dh0, rtol=1e-10, atol=1e-10)
    assert np.allclose(db, db0, rtol=1e-10, atol=1e-10)
