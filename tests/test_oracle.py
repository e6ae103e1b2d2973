"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a closed form, a brute-force
evaluation on tiny inputs, a library routine that computes the same special
case, an invariant of the method, or a hand-worked example under tests/golden.
"""
import json
import os

import numpy as np
import pytest

import oracle
from fft_long_convolution_libhyena_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- radix-2 FFT


@pytest.mark.parametrize("n", [1, 2, 4, 8, 64, 1024])
def test_fft_delta_is_all_ones(n):
    # closed form: the DFT of a unit impulse at t=0 is 1 at every frequency
    x = np.zeros(n, complex)
    x[0] = 1.0
    np.testing.assert_allclose(oracle.fft(x), np.ones(n), atol=1e-13)
    np.testing.assert_allclose(oracle.fft(x, inverse=True), np.ones(n), atol=1e-13)


@pytest.mark.parametrize("n,k0", [(8, 3), (64, 1), (256, 17), (1024, 1023)])
def test_fft_single_tone_is_spike(n, k0):
    # closed form: sum_t exp(2 pi i k0 t/n) exp(-2 pi i k t/n) = n * [k == k0]
    t = np.arange(n)
    x = np.exp(2j * np.pi * k0 * t / n)
    X = oracle.fft(x)
    want = np.zeros(n, complex)
    want[k0] = n
    np.testing.assert_allclose(X, want, atol=1e-9 * n)


@pytest.mark.parametrize("n", [2, 4, 16, 128])
def test_fft_matches_bruteforce_dft(n):
    # brute force: the O(n^2) DFT matrix written out
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n) + 1j * rng.standard_normal(n)
    jk = np.outer(np.arange(n), np.arange(n))
    F = np.exp(-2j * np.pi * jk / n)
    np.testing.assert_allclose(oracle.fft(x), F @ x, rtol=0, atol=1e-11 * n)
    np.testing.assert_allclose(oracle.fft(x, inverse=True), np.conj(F) @ x, rtol=0, atol=1e-11 * n)


@pytest.mark.parametrize("n", [32, 4096])
def test_fft_matches_numpy_and_parseval_and_roundtrip(n):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(n) + 1j * rng.standard_normal(n)
    X = oracle.fft(x)
    np.testing.assert_allclose(X, np.fft.fft(x), atol=1e-10 * np.sqrt(n))  # library special case
    assert abs(np.sum(np.abs(X) ** 2) / n - np.sum(np.abs(x) ** 2)) < 1e-9 * n  # Parseval
    np.testing.assert_allclose(oracle.fft(X, inverse=True) / n, x, atol=1e-12)  # round trip


def test_fft_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.fft(np.ones(12))


# ------------------------------------------------------- causal convolution


@pytest.mark.parametrize("L", [1, 2, 3, 5, 8, 31, 64, 100, 512])
def test_conv_direct_matches_toeplitz_and_numpy(L):
    rng = np.random.default_rng(L)
    v, h = rng.standard_normal(L), rng.standard_normal(L)
    got = oracle.causal_conv(v, h, mode="direct")
    # brute force: lower-triangular Toeplitz matrix T[t, s] = h[t - s]
    T = np.zeros((L, L))
    for t in range(L):
        T[t, : t + 1] = h[t::-1]
    np.testing.assert_allclose(got, T @ v, rtol=1e-12, atol=1e-12)
    # library special case: full linear convolution, first L samples
    np.testing.assert_allclose(got, np.convolve(v, h)[:L], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("L", [1, 2, 3, 4, 7, 16, 33, 128, 512, 1024])
def test_conv_fft_matches_direct(L):
    rng = np.random.default_rng(100 + L)
    v, h = rng.standard_normal(L), rng.standard_normal(L) * np.exp(-np.arange(L) / max(L, 1))
    d = oracle.causal_conv(v, h, mode="direct")
    f = oracle.causal_conv(v, h, mode="fft")
    assert np.max(np.abs(f - d)) <= 1e-12 * max(1.0, np.max(np.abs(d)))


def test_conv_is_causal_and_time_invariant():
    L = 64
    rng = np.random.default_rng(3)
    h = rng.standard_normal(L)
    delta = np.zeros(L)
    delta[5] = 1.0
    # impulse response: a shifted copy of h (shift invariance + causality)
    out = oracle.causal_conv(delta, h, mode="fft")
    np.testing.assert_allclose(out[:5], 0.0, atol=1e-13)
    np.testing.assert_allclose(out[5:], h[: L - 5], atol=1e-12)


# ------------------------------------------------------------- short conv


def test_short_conv_matches_torch_conv1d():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    C, L = 9, 37
    u = rng.standard_normal((2, C, L)).astype(np.float32)
    w = rng.standard_normal((C, 3)).astype(np.float32)
    ref = torch.nn.functional.conv1d(torch.from_numpy(u).double(), torch.from_numpy(w).double()[:, None, :],
                                     padding=2, groups=C)[..., :L].numpy()
    for b in range(2):
        for c in range(C):
            np.testing.assert_allclose(oracle.short_conv_row(u[b, c], w[c]), ref[b, c], rtol=1e-13, atol=1e-13)


def test_short_conv_tap_orientation():
    u = np.arange(1, 9, dtype=np.float32)
    np.testing.assert_array_equal(oracle.short_conv_row(u, np.array([0, 0, 1], np.float32)), u)
    want = np.concatenate([[0, 0], u[:-2]])  # taps [1,0,0] delay by two samples
    np.testing.assert_array_equal(oracle.short_conv_row(u, np.array([1, 0, 0], np.float32)), want)


# ---------------------------------------------------------- the full chain


@pytest.mark.parametrize("name", ["hand_worked_order2.json", "hand_worked_order3.json"])
@pytest.mark.parametrize("mode", ["direct", "fft"])
def test_chain_hand_worked_examples(name, mode):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    y = oracle.forward(np.array(g["u_proj"], np.float32), np.array(g["short_w"], np.float32),
                       np.array(g["h"], np.float32), np.array(g["bias"], np.float32), g["order"], mode=mode)
    np.testing.assert_allclose(y, np.array(g["y"], np.float64), rtol=0, atol=1e-12)


def _identity_taps(C):
    w = np.zeros((C, 3), np.float32)
    w[:, 2] = 1.0
    return w


@pytest.mark.parametrize("order", [2, 3, 4])
def test_chain_delta_filter_reduces_to_gating(order):
    # h[o] = delta: each step is v <- (1 + bias[o]) * v after its gate, so
    # y = x_0 * prod_{i>=1} x_i * v * prod_o (1 + bias[o])
    B, D, L, N = 2, 3, 40, order
    rng = np.random.default_rng(order)
    u = rng.standard_normal((B, (N + 1) * D, L)).astype(np.float32)
    w = rng.standard_normal(((N + 1) * D, 3)).astype(np.float32)
    h = np.zeros((N - 1, D, L), np.float32)
    h[:, :, 0] = 1.0
    bias = rng.standard_normal((N - 1, D)).astype(np.float32)
    y = oracle.forward(u, w, h, bias, N, mode="fft")
    uc = np.zeros((B, (N + 1) * D, L))
    for b in range(B):
        for c in range((N + 1) * D):
            uc[b, c] = oracle.short_conv_row(u[b, c], w[c])
    want = uc[:, N * D:] * np.prod(1.0 + bias.astype(np.float64), axis=0)[None, :, None]
    for i in range(N):
        want = want * uc[:, i * D:(i + 1) * D]
    np.testing.assert_allclose(y, want, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("a", [0.5, 0.9, -0.7])
def test_chain_geometric_filter_closed_form(a):
    # gates and v identically 1, h[t] = a^t, order 2:
    # y[t] = sum_{s<=t} a^s + bias = (1 - a^{t+1}) / (1 - a) + bias
    D, L = 2, 128
    u = np.ones((1, 3 * D, L), np.float32)
    w = _identity_taps(3 * D)
    t = np.arange(L)
    h = np.tile((a ** t).astype(np.float32), (1, D, 1))
    bias = np.array([[0.25, -1.5]], np.float32)
    y = oracle.forward(u, w, h, bias, 2, mode="fft")
    want = (1 - a ** (t + 1)) / (1 - a)
    for d in range(D):
        np.testing.assert_allclose(y[0, d], want + bias[0, d], rtol=1e-6, atol=1e-6)


def test_chain_is_causal():
    # perturbing u at t0 (every channel) leaves y[..., :t0] unchanged bit for bit
    wl = synth.custom(2, 4, 64, 3, seed=5)
    x = synth.generate(wl)
    y0 = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, 3, mode="direct")
    u2 = x.u_proj.copy()
    t0 = 29
    u2[:, :, t0] += 3.0
    y1 = oracle.forward(u2, x.short_w, x.h, x.bias, 3, mode="direct")
    np.testing.assert_array_equal(y1[..., :t0], y0[..., :t0])
    assert np.all(np.abs(y1[..., t0:t0 + 3] - y0[..., t0:t0 + 3]) > 0)


def test_chain_is_linear_in_v():
    # with the gate channels fixed, y is linear in the v chunk of u_proj
    wl = synth.custom(1, 3, 50, 2, seed=9)
    x = synth.generate(wl)
    D = wl.D
    rng = np.random.default_rng(1)
    va = rng.standard_normal((1, D, wl.L)).astype(np.float32)
    vb = rng.standard_normal((1, D, wl.L)).astype(np.float32)

    def run(vchunk):
        u = x.u_proj.copy()
        u[:, 2 * D:] = vchunk
        return oracle.forward(u, x.short_w, x.h, x.bias, 2, mode="direct")

    ya, yb = run(va), run(vb)
    ysum = run((2 * va.astype(np.float64) - 3 * vb).astype(np.float32))
    # 2*va - 3*vb is not exactly representable in fp32 in general; compare with tolerance
    np.testing.assert_allclose(ysum, 2 * ya - 3 * yb, rtol=1e-6, atol=1e-6 * np.max(np.abs(ya)))


def test_chain_zero_value_gives_zero_output():
    wl = synth.custom(1, 2, 32, 2, seed=2)
    x = synth.generate(wl)
    u = x.u_proj.copy()
    u[:, 2 * wl.D:] = 0
    assert not np.any(oracle.forward(u, x.short_w, x.h, x.bias, 2, mode="fft"))


def test_chain_fft_matches_direct_on_tiny_workload():
    wl = synth.WORKLOADS["tiny"]
    x = synth.generate(wl)
    rows = synth.sample_rows(wl, 16)
    d = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, wl.order, mode="direct", rows=rows)
    f = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, wl.order, mode="fft", rows=rows)
    assert oracle.rel_l2(f, d) < 1e-13


def test_chain_row_subset_matches_full():
    wl = synth.custom(3, 5, 48, 3, seed=4)
    x = synth.generate(wl)
    full = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, 3)
    rows = [0, 7, 14]
    sub = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, 3, rows=rows)
    flat = full.reshape(-1, wl.L)
    np.testing.assert_array_equal(sub, flat[rows])


def test_chain_rejects_bad_shapes():
    wl = synth.custom(1, 2, 16, 2)
    x = synth.generate(wl)
    with pytest.raises(ValueError):
        oracle.forward(x.u_proj, x.short_w, x.h, x.bias, 3)


# ------------------------------------------------------------ the comparison


def test_rel_l2_hand_computed_values():
    # every expected value is worked by hand from the definition ||g - r|| / ||r||
    assert oracle.rel_l2(np.array([1.0, 2.0, 2.0]), np.array([1.0, 2.0, 2.0])) == 0.0
    # g - r = (0, 2, 2): norm sqrt(8); ||r|| = 1
    assert oracle.rel_l2(np.array([1.0, 2.0, 2.0]), np.array([1.0, 0.0, 0.0])) == pytest.approx(np.sqrt(8.0), rel=1e-15)
    # the same pair swapped: ||r|| is now 3, so the value is sqrt(8)/3, not sqrt(8)
    assert oracle.rel_l2(np.array([1.0, 0.0, 0.0]), np.array([1.0, 2.0, 2.0])) == pytest.approx(np.sqrt(8.0) / 3.0,
                                                                                               rel=1e-15)
    # a 2-D pair reduces over every element: diff ((0,-1),(-1,0)) has norm sqrt(2); ||r|| = 2
    assert oracle.rel_l2(np.array([[1.0, 0.0], [0.0, 1.0]]), np.ones((2, 2))) == pytest.approx(np.sqrt(2.0) / 2.0,
                                                                                              rel=1e-15)
    # a scaled result: g = (1 + eps) r gives exactly eps
    r = np.array([3.0, -4.0])
    assert oracle.rel_l2(1.25 * r, r) == pytest.approx(0.25, rel=1e-15)


def test_rel_l2_zero_reference_gives_absolute_norm():
    # ||r|| = 0: the absolute error ||g|| is returned (3-4-5 triangle)
    assert oracle.rel_l2(np.array([3.0, 4.0]), np.zeros(2)) == pytest.approx(5.0, rel=1e-15)
    assert oracle.rel_l2(np.zeros(4), np.zeros(4)) == 0.0


def test_rel_l2_widens_the_result_to_fp64():
    # an fp32 result is compared at its exact float32 value, not re-rounded
    g = np.array([1.0 + 2.0 ** -20], dtype=np.float32)
    assert oracle.rel_l2(g, np.array([1.0])) == pytest.approx(2.0 ** -20, rel=1e-12)


@pytest.mark.parametrize("gs,rs", [((2, 3), (3,)), ((3, 1), (3,)), ((3,), (1,)), ((4, 4), (2, 8))])
def test_rel_l2_rejects_shape_mismatch(gs, rs):
    # a mis-shaped result must fail, never broadcast against the reference
    with pytest.raises(ValueError):
        oracle.rel_l2(np.ones(gs), np.ones(rs))
