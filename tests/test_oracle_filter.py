"""Pins of the fp64 implicit-filter oracle (HyenaDNA walkthrough, section 2.2,
HyenaFilter: positional embedding -> Linear/Sin stack -> Linear without bias ->
exponential modulation -> the [L, (N-1)*D] to [N-1][D][L] reshape), CPU only.

Closed forms fix each stage on its own: a stack whose hidden units are all exactly
one leaves only the output weights, the modulation and the layout; identity weights
expose the positional features one by one; a one-unit stack is a nested sine
written out by hand; linearity in the output weights and the modulation ratio hold
for any parameters; and an independent float64 torch module (nn.Linear layers and
a Sin module) agrees on random parameters.
"""
import math
import types

import numpy as np
import pytest

import oracle


def _params(E, W, M, C, seed, s=1.0):
    rng = np.random.default_rng(seed)
    K = (E - 1) // 2
    return types.SimpleNamespace(
        band_freq=np.arange(1, K + 1, dtype=np.float64) * 1.5,
        w_in=rng.standard_normal((W, E)) / np.sqrt(E), b_in=rng.standard_normal(W),
        w_inner=rng.standard_normal((M, W, W)) / np.sqrt(W), b_inner=rng.standard_normal((M, W)),
        sin_freq=np.full(W, s) + 0.1 * rng.standard_normal(W),
        w_out=rng.standard_normal((C, W)) / np.sqrt(W), alpha=np.linspace(0.3, 30.0, C))


@pytest.mark.parametrize("order,E,M", [(2, 3, 0), (3, 5, 2), (4, 3, 1)])
def test_unit_hidden_layers_leave_layout_and_modulation(order, E, M):
    # every hidden unit is sin(s * pi / (2 s)) = 1, so h[o][d][tau] = sum_j w_out[c][j]
    # times exp(-alpha_c tau / L) with c = o*D + d
    D, L, W = 3, 32, 4
    C = (order - 1) * D
    s = np.array([1.7, 0.6, 2.2, 1.0])
    p = types.SimpleNamespace(band_freq=np.arange(1, (E - 1) // 2 + 1, dtype=np.float64),
                              w_in=np.zeros((W, E)), b_in=np.pi / (2 * s), w_inner=np.zeros((M, W, W)),
                              b_inner=np.tile(np.pi / (2 * s), (M, 1)), sin_freq=s,
                              w_out=np.repeat((np.arange(C) + 1.0)[:, None] / W, W, axis=1),
                              alpha=np.linspace(-1.0, 5.0, C))
    h = oracle.implicit_filter(L, D, order, p)
    assert h.shape == (order - 1, D, L)
    for o in range(order - 1):
        for d in range(D):
            c = o * D + d
            for tau in range(L):
                want = (c + 1) * math.exp(-p.alpha[c] * tau / L)
                assert abs(h[o, d, tau] - want) <= 1e-12 * abs(want)


@pytest.mark.parametrize("E", [3, 5, 7])
def test_identity_weights_expose_positional_features(E):
    # W = E, identity input weights, no inner layers, unit Sin frequency, identity
    # output weights, no modulation: channel c is sin(z_c)
    L, K = 64, (E - 1) // 2
    f = np.array([1.0, 2.5, 7.0])[:K]
    p = types.SimpleNamespace(band_freq=f, w_in=np.eye(E), b_in=np.zeros(E), w_inner=np.zeros((0, E, E)),
                              b_inner=np.zeros((0, E)), sin_freq=np.ones(E), w_out=np.eye(E), alpha=np.zeros(E))
    h = oracle.implicit_filter(L, E, 2, p)[0]
    for tau in range(L):
        t = tau / L
        z = [t] + [math.sin(2 * math.pi * f[k] * t) for k in range(K)] + \
            [math.cos(2 * math.pi * f[k] * t) for k in range(K)]
        for c in range(E):
            assert abs(h[c, tau] - math.sin(z[c])) <= 1e-14


def test_one_unit_stack_is_a_nested_sine():
    a, b0, c1, d1, c2, d2, s, g, al = 1.3, -0.4, 0.8, 0.25, -1.6, 0.7, 2.1, -0.9, 3.0
    p = types.SimpleNamespace(band_freq=np.array([2.0]), w_in=np.array([[a, 0.0, 0.0]]), b_in=np.array([b0]),
                              w_inner=np.array([[[c1]], [[c2]]]), b_inner=np.array([[d1], [d2]]),
                              sin_freq=np.array([s]), w_out=np.array([[g]]), alpha=np.array([al]))
    L = 16
    h = oracle.implicit_filter(L, 1, 2, p)[0, 0]
    for tau in range(L):
        t = tau / L
        want = g * math.sin(s * (c2 * math.sin(s * (c1 * math.sin(s * (a * t + b0)) + d1)) + d2)) * math.exp(-al * t)
        assert abs(h[tau] - want) <= 1e-14


def test_linear_in_output_weights_and_modulation_ratio():
    D, L, N, E, W, M = 5, 128, 3, 5, 8, 2
    C = (N - 1) * D
    p = _params(E, W, M, C, seed=1)
    q = _params(E, W, M, C, seed=2)
    h1 = oracle.implicit_filter(L, D, N, p)
    p2 = types.SimpleNamespace(**{**vars(p), "w_out": q.w_out})
    p12 = types.SimpleNamespace(**{**vars(p), "w_out": p.w_out + q.w_out})
    h2 = oracle.implicit_filter(L, D, N, p2)
    h12 = oracle.implicit_filter(L, D, N, p12)
    assert np.max(np.abs(h12 - h1 - h2)) <= 1e-12 * np.max(np.abs(h12))
    p0 = types.SimpleNamespace(**{**vars(p), "alpha": np.zeros(C)})
    h0 = oracle.implicit_filter(L, D, N, p0).reshape(C, L)
    t = np.arange(L) / L
    ratio = np.exp(-np.outer(p.alpha, t))
    assert np.max(np.abs(h1.reshape(C, L) - h0 * ratio)) <= 1e-13 * np.max(np.abs(h0))


@pytest.mark.parametrize("E,W,M,order", [(3, 16, 2, 2), (5, 8, 0, 3), (7, 4, 3, 2)])
def test_matches_float64_torch_module(E, W, M, order):
    torch = pytest.importorskip("torch")
    D, L = 4, 64
    C = (order - 1) * D
    p = _params(E, W, M, C, seed=E * 10 + M)
    f64 = torch.float64

    class Sin(torch.nn.Module):
        def __init__(self, freq):
            super().__init__()
            self.freq = torch.nn.Parameter(torch.tensor(freq, dtype=f64))

        def forward(self, x):
            return torch.sin(self.freq * x)

    act = Sin(p.sin_freq)
    layers = [torch.nn.Linear(E, W, dtype=f64), act]
    for _ in range(M):
        layers += [torch.nn.Linear(W, W, dtype=f64), act]
    layers.append(torch.nn.Linear(W, C, bias=False, dtype=f64))
    net = torch.nn.Sequential(*layers)
    with torch.no_grad():
        net[0].weight.copy_(torch.tensor(p.w_in))
        net[0].bias.copy_(torch.tensor(p.b_in))
        for m in range(M):
            net[2 + 2 * m].weight.copy_(torch.tensor(p.w_inner[m]))
            net[2 + 2 * m].bias.copy_(torch.tensor(p.b_inner[m]))
        net[-1].weight.copy_(torch.tensor(p.w_out))
        t = torch.arange(L, dtype=f64) / L
        ang = 2 * torch.pi * t[:, None] * torch.tensor(p.band_freq)[None, :]
        z = torch.cat([t[:, None], torch.sin(ang), torch.cos(ang)], dim=1)
        k = net(z) * torch.exp(-t[:, None] * torch.tensor(p.alpha)[None, :])  # [L, (N-1)*D]
        want = k.T.reshape(order - 1, D, L).numpy()
    got = oracle.implicit_filter(L, D, order, p)
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def test_rejects_output_weights_of_the_wrong_size():
    p = _params(3, 4, 1, 5, seed=3)
    with pytest.raises(ValueError):
        oracle.implicit_filter(16, 3, 2, p)  # needs (2 - 1) * 3 = 3 output rows, has 5
