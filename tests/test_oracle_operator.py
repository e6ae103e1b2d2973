"""Pins of the fp64 operator oracle (projections around the hot path), CPU only.

The projections are library matrix products; what needs pinning is how they are
wired around the path: the layouts and rearranges, which projection output is a
gate and which the value, and the biases. An independent float64 torch module
(nn.Linear in and out, the short Conv1d, an explicit Toeplitz long convolution)
fixes all of it; special cases pin the rearranges and the output bias alone.
"""
import numpy as np
import pytest

import oracle


def _params(B, D, L, N, seed):
    rng = np.random.default_rng(seed)
    C = (N + 1) * D
    x = rng.standard_normal((B, L, D)).astype(np.float32)
    w_in = (rng.standard_normal((C, D)) / np.sqrt(D)).astype(np.float32)
    b_in = rng.standard_normal(C).astype(np.float32)
    short_w = (rng.standard_normal((C, 3)) / np.sqrt(3)).astype(np.float32)
    t = np.arange(L)
    h = (rng.standard_normal((N - 1, D, L)) * np.exp(-2.0 * t / L)).astype(np.float32)
    bias = rng.standard_normal((N - 1, D)).astype(np.float32)
    w_out = (rng.standard_normal((D, D)) / np.sqrt(D)).astype(np.float32)
    b_out = rng.standard_normal(D).astype(np.float32)
    return x, w_in, b_in, short_w, h, bias, w_out, b_out


def _torch_operator(torch, x, w_in, b_in, short_w, h, bias, w_out, b_out, N):
    B, L, D = x.shape
    C = (N + 1) * D
    lin_in = torch.nn.Linear(D, C, dtype=torch.float64)
    lin_out = torch.nn.Linear(D, D, dtype=torch.float64)
    with torch.no_grad():
        lin_in.weight.copy_(torch.tensor(w_in, dtype=torch.float64))
        lin_in.bias.copy_(torch.tensor(b_in, dtype=torch.float64))
        lin_out.weight.copy_(torch.tensor(w_out, dtype=torch.float64))
        lin_out.bias.copy_(torch.tensor(b_out, dtype=torch.float64))
        u = lin_in(torch.tensor(x, dtype=torch.float64)).transpose(1, 2)  # b l c -> b c l
        uc = torch.nn.functional.conv1d(u, torch.tensor(short_w, dtype=torch.float64).unsqueeze(1), padding=2,
                                        groups=C)[..., :L]
        xs = [uc[:, i * D:(i + 1) * D] for i in range(N)]
        v = uc[:, N * D:]
        idx = torch.arange(L)
        lag = idx[:, None] - idx[None, :]
        for o in range(N - 1):
            v = v * xs[N - 1 - o]
            hk = torch.tensor(h[o], dtype=torch.float64)
            T = torch.where(lag >= 0, hk[:, lag.clamp(min=0)], torch.zeros((), dtype=torch.float64))
            v = torch.einsum("dts,bds->bdt", T, v) + torch.tensor(bias[o], dtype=torch.float64)[None, :, None] * v
        y = v * xs[0]
        return lin_out(y.transpose(1, 2)).numpy()


@pytest.mark.parametrize("order", [2, 3])
def test_operator_matches_torch_module(order):
    torch = pytest.importorskip("torch")
    p = _params(2, 3, 16, order, seed=order)
    want = _torch_operator(torch, *p, order)
    got = oracle.operator_forward(*p, order, mode="direct")
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)


def test_operator_with_identity_projections_is_the_path():
    # w_in stacks N+1 identities (each channel group copies x) with b_in = 0, and
    # w_out = I, b_out = 0: the operator is the path on u_proj = x^T repeated
    B, D, L, N = 2, 4, 32, 2
    x, _, _, short_w, h, bias, _, _ = _params(B, D, L, N, seed=9)
    w_in = np.tile(np.eye(D, dtype=np.float32), (N + 1, 1))
    out = oracle.operator_forward(x, w_in, np.zeros((N + 1) * D, np.float32), short_w, h, bias,
                                  np.eye(D, dtype=np.float32), np.zeros(D, np.float32), N, mode="direct")
    u_proj = np.tile(x.transpose(0, 2, 1), (1, N + 1, 1))
    y = oracle.forward(u_proj, short_w, h, bias, N, mode="direct")
    np.testing.assert_allclose(out, y.transpose(0, 2, 1), atol=1e-12)


def test_operator_output_bias_alone():
    # zero short-conv taps make every gate zero, so y = 0 and out = b_out everywhere
    B, D, L, N = 2, 3, 8, 2
    x, w_in, b_in, short_w, h, bias, w_out, b_out = _params(B, D, L, N, seed=4)
    out = oracle.operator_forward(x, w_in, b_in, np.zeros_like(short_w), h, bias, w_out, b_out, N, mode="direct")
    np.testing.assert_allclose(out, np.broadcast_to(b_out.astype(np.float64), (B, L, D)), atol=0)


def test_operator_input_bias_enters_before_the_short_conv():
    # with x = 0 the activation is the constant b_in; with identity taps the gates
    # and value are constants and the output follows in closed form
    B, D, L, N = 1, 2, 8, 2
    _, w_in, b_in, _, _, bias, w_out, b_out = _params(B, D, L, N, seed=5)
    short_w = np.zeros(((N + 1) * D, 3), np.float32)
    short_w[:, 2] = 1.0
    h = np.zeros((1, D, L), np.float32)
    h[0, :, 0] = 1.0  # delta filter: conv(v, h) = v
    out = oracle.operator_forward(np.zeros((B, L, D), np.float32), w_in, b_in, short_w, h, bias, w_out, b_out, N,
                                  mode="direct")
    bi = b_in.astype(np.float64)
    y = bi[2 * D:] * bi[D:2 * D] * (1 + bias[0].astype(np.float64)) * bi[:D]  # v x1 (1 + bias) x0, per channel
    want = w_out.astype(np.float64) @ y + b_out
    np.testing.assert_allclose(out, np.broadcast_to(want, (B, L, D)), rtol=1e-12, atol=1e-12)
