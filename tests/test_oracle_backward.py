"""Pins of the fp64 backward oracle against things other than itself (CPU only).

The forward is linear in each of these argument groups when the others are held
fixed: one long filter h[o], one bias row bias[o], the short-conv taps of one
channel group (rows i*D .. i*D+D-1 of short_w), and one channel group of u_proj.
So for a perturbation delta of one group, <y(theta + delta) - y(theta), dy> equals
<delta, grad> exactly (up to fp64 rounding), with y from the separately pinned
forward oracle. A second, independent pin differentiates a plain float64 torch
formulation of the same forward with autograd.
"""
import numpy as np
import pytest

import oracle


def _inputs(B, D, L, N, seed):
    rng = np.random.default_rng(seed)
    C = (N + 1) * D
    u = rng.standard_normal((B, C, L)).astype(np.float32)
    w = (rng.standard_normal((C, 3)) / np.sqrt(3)).astype(np.float32)
    t = np.arange(L)
    h = (rng.standard_normal((N - 1, D, L)) * np.exp(-3.0 * t / L)).astype(np.float32)
    bias = rng.standard_normal((N - 1, D)).astype(np.float32)
    dy = rng.standard_normal((B, D, L)).astype(np.float32)
    return u, w, h, bias, dy


def _perturb(a, rng, scale=0.25):
    """a + delta rounded to fp32, and the exact delta that rounding leaves."""
    a2 = (a.astype(np.float64) + scale * rng.standard_normal(a.shape)).astype(np.float32)
    return a2, a2.astype(np.float64) - a.astype(np.float64)


def _dot(a, b):
    return float(np.sum(np.asarray(a, np.float64) * np.asarray(b, np.float64)))


@pytest.mark.parametrize("order", [2, 3, 4])
@pytest.mark.parametrize("mode", ["direct", "fft"])
def test_backward_directional_identities(order, mode):
    B, D, L, N = 2, 3, 16, order
    u, w, h, bias, dy = _inputs(B, D, L, N, seed=10 + order)
    y0 = oracle.forward(u, w, h, bias, N, mode="direct")
    du, dw, dh, db = oracle.backward(u, w, h, bias, dy, N, mode=mode)
    rng = np.random.default_rng(99)
    checks = []
    for o in range(N - 1):
        h2 = h.copy()
        h2[o], dlt = _perturb(h[o], rng)
        y1 = oracle.forward(u, w, h2, bias, N, mode="direct")
        checks.append((f"h[{o}]", _dot(y1 - y0, dy), _dot(dlt, dh[o])))
        b2 = bias.copy()
        b2[o], dlt = _perturb(bias[o], rng)
        y1 = oracle.forward(u, w, h, b2, N, mode="direct")
        checks.append((f"bias[{o}]", _dot(y1 - y0, dy), _dot(dlt, db[o])))
    for i in range(N + 1):
        sl = slice(i * D, (i + 1) * D)
        w2 = w.copy()
        w2[sl], dlt = _perturb(w[sl], rng)
        y1 = oracle.forward(u, w2, h, bias, N, mode="direct")
        checks.append((f"w group {i}", _dot(y1 - y0, dy), _dot(dlt, dw[sl])))
        u2 = u.copy()
        u2[:, sl], dlt = _perturb(u[:, sl], rng)
        y1 = oracle.forward(u2, w, h, bias, N, mode="direct")
        checks.append((f"u group {i}", _dot(y1 - y0, dy), _dot(dlt, du[:, sl])))
    for name, lhs, rhs in checks:
        assert abs(lhs - rhs) <= 1e-9 * (1.0 + abs(lhs)), (name, lhs, rhs)


def _torch_forward(torch, u, w, h, bias, N):
    """The forward written with plain float64 torch ops: Conv1d for the short filter,
    an explicit lower-triangular Toeplitz product for the long convolution."""
    B, C, L = u.shape
    D = C // (N + 1)
    uc = torch.nn.functional.conv1d(u, w.unsqueeze(1), padding=2, groups=C)[..., :L]
    xs = [uc[:, i * D:(i + 1) * D] for i in range(N)]
    v = uc[:, N * D:]
    idx = torch.arange(L)
    lag = idx[:, None] - idx[None, :]  # t - s
    for o in range(N - 1):
        v = v * xs[N - 1 - o]
        hk = h[o]  # [D, L]
        T = torch.where(lag >= 0, hk[:, lag.clamp(min=0)], torch.zeros((), dtype=hk.dtype))  # [D, L, L]
        c = torch.einsum("dts,bds->bdt", T, v)
        v = c + bias[o][None, :, None] * v
    return v * xs[0]


@pytest.mark.parametrize("order", [2, 3])
def test_backward_matches_torch_autograd(order):
    torch = pytest.importorskip("torch")
    B, D, L, N = 2, 2, 12, order
    u, w, h, bias, dy = _inputs(B, D, L, N, seed=30 + order)
    tu, tw, th, tb = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (u, w, h, bias))
    y = _torch_forward(torch, tu, tw, th, tb, N)
    np.testing.assert_allclose(y.detach().numpy(), oracle.forward(u, w, h, bias, N, mode="direct"), atol=1e-11)
    gu, gw, gh, gb = torch.autograd.grad(y, (tu, tw, th, tb), grad_outputs=torch.tensor(dy, dtype=torch.float64))
    du, dw, dh, db = oracle.backward(u, w, h, bias, dy, N, mode="direct")
    for got, want in ((du, gu), (dw, gw), (dh, gh), (db, gb)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-10, atol=1e-10)


def test_backward_delta_filter_closed_form():
    # h = unit impulse, identity taps: y = (1 + bias) v x1 x0 pointwise, so
    # du_v = (1+b) dy x1 x0, du_x1 = (1+b) dy v x0, du_x0 = (1+b) dy v x1,
    # dbias = sum dy v x1 x0, dh[0] = sum_b dy x0 (v x1) and dh[tau] = sum_t dy[t] x0[t] g[t-tau].
    B, D, L, N = 2, 2, 8, 2
    u, _, _, bias, dy = _inputs(B, D, L, N, seed=5)
    C = 3 * D
    w = np.zeros((C, 3), np.float32)
    w[:, 2] = 1.0
    h = np.zeros((1, D, L), np.float32)
    h[0, :, 0] = 1.0
    x0, x1, v = (u[:, i * D:(i + 1) * D].astype(np.float64) for i in range(3))
    g = v * x1
    dyd = dy.astype(np.float64)
    s = 1.0 + bias[0].astype(np.float64)[None, :, None]
    du, dw, dh, db = oracle.backward(u, w, h, bias, dy, N, mode="direct")
    np.testing.assert_allclose(du[:, 2 * D:], s * dyd * x1 * x0, atol=1e-12)
    np.testing.assert_allclose(du[:, D:2 * D], s * dyd * v * x0, atol=1e-12)
    np.testing.assert_allclose(du[:, :D], s * dyd * v * x1, atol=1e-12)
    np.testing.assert_allclose(db[0], np.sum(dyd * x0 * g, axis=(0, 2)), atol=1e-12)
    a = dyd * x0
    want = np.zeros((D, L))
    for tau in range(L):
        want[:, tau] = np.sum(a[:, :, tau:] * g[:, :, :L - tau], axis=(0, 2))
    np.testing.assert_allclose(dh[0], want, atol=1e-12)
    # dw[:, 2] (the tap on u[t]) is sum_t duc[t] u[t]; duc of v is (1+b) dy x1 x0
    np.testing.assert_allclose(dw[2 * D:, 2], np.sum(s * dyd * x1 * x0 * v, axis=(0, 2)), atol=1e-11)


@pytest.mark.parametrize("L", [1, 2, 5, 16, 100, 256])
def test_corr_is_the_adjoint_of_conv(L):
    # <conv(v, k), a> = <v, corr(a, k)> for all v, a: the defining property
    rng = np.random.default_rng(L)
    v, k, a = (rng.standard_normal(L) for _ in range(3))
    for mode in ("direct", "fft"):
        lhs = _dot(oracle.causal_conv(v, k, mode="direct"), a)
        rhs = _dot(v, oracle.causal_corr(a, k, mode=mode))
        assert abs(lhs - rhs) <= 1e-11 * (1 + abs(lhs))
    # and matches numpy's full correlation restricted to non-negative lags
    full = np.correlate(a, k, mode="full")  # full[n] = sum_m a[m+n-(L-1)] k[m]
    np.testing.assert_allclose(oracle.causal_corr(a, k, mode="direct"), full[L - 1:], atol=1e-11)


def test_backward_fft_matches_direct():
    B, D, L, N = 2, 4, 64, 3
    u, w, h, bias, dy = _inputs(B, D, L, N, seed=77)
    a = oracle.backward(u, w, h, bias, dy, N, mode="direct")
    b = oracle.backward(u, w, h, bias, dy, N, mode="fft")
    for x, y in zip(a, b):
        assert oracle.rel_l2(y, x) < 1e-12


def test_backward_rejects_bad_shapes():
    u, w, h, bias, dy = _inputs(1, 2, 8, 2, seed=1)
    with pytest.raises(ValueError):
        oracle.backward(u, w, h, bias, dy[:, :1], 2)
    with pytest.raises(ValueError):
        oracle.backward(u, w[:-1], h, bias, dy, 2)
