"""Pins of the circular-mode backward oracle, CPU only.

The circular correlation is pinned by the transpose of the circulant matrix
built entry by entry. The gradients are pinned by central finite differences of
an fp64 forward of the circular chain (every gradient, on random directions), by
the direct and FFT forms agreeing, by the delta-filter case, where a circular and
a causal step coincide, reducing to the (separately pinned) causal backward
oracle for du, dshort_w and dbias, and by per-sample filter sets that are all
equal reproducing the shared gradients.
"""
import numpy as np
import pytest

import oracle


def test_circular_corr_is_the_transposed_circulant():
    rng = np.random.default_rng(3)
    for S in (1, 2, 5, 16):
        a, k = rng.standard_normal(S), rng.standard_normal(S)
        M = np.zeros((S, S))  # circular_conv(v, k) = M @ v
        for t in range(S):
            for s in range(S):
                M[t, (t - s) % S] += k[s]
        for mode in ("direct", "fft"):
            assert np.allclose(oracle.circular_corr(a, k, mode), M.T @ a, rtol=1e-12, atol=1e-12)


def _inputs(B, D, S, N, seed):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((B, (N + 1) * D, S)).astype(np.float32)
    w = (rng.standard_normal(((N + 1) * D, 3)) / np.sqrt(3)).astype(np.float32)
    h = rng.standard_normal((N - 1, D, S)).astype(np.float32)
    b = rng.standard_normal((N - 1, D)).astype(np.float32)
    dy = rng.standard_normal((B, D, S)).astype(np.float32)
    return u, w, h, b, dy


def _forward64(u, w, h, b, N):
    """The circular chain in fp64 for finite differences: causal short conv, then
    v <- v x_{N-1-o}; v <- circular_conv(v, h_o) + b_o v; y = v x_0."""
    B, C, S = u.shape
    D = C // (N + 1)
    uc = np.zeros((B, C, S))
    for j in range(3):  # uc[t] += w_j u[t - 2 + j]
        sh = 2 - j
        uc[:, :, sh:] += w[None, :, j, None] * u[:, :, :S - sh]
    x = [uc[:, i * D:(i + 1) * D] for i in range(N)]
    v = uc[:, N * D:]
    for o in range(N - 1):
        v = v * x[N - 1 - o]
        v = oracle.circular_conv(v, h[o][None], "direct") + b[o][None, :, None] * v
    return v * x[0]


@pytest.mark.parametrize("N", [2, 3, 4])
def test_gradients_match_finite_differences(N):
    B, D, S = 2, 3, 16
    u, w, h, b, dy = _inputs(B, D, S, N, seed=10 + N)
    grads = oracle.backward_circular(u, w, h, b, dy, N, mode="direct")
    base = {"u": u.astype(np.float64), "w": w.astype(np.float64), "h": h.astype(np.float64),
            "b": b.astype(np.float64)}
    rng = np.random.default_rng(20 + N)
    eps = 1e-6
    for name, g in zip("uwhb", grads):
        for _ in range(2):
            d = rng.standard_normal(base[name].shape)
            hi = dict(base)
            lo = dict(base)
            hi[name] = base[name] + eps * d
            lo[name] = base[name] - eps * d
            fd = (np.sum(_forward64(hi["u"], hi["w"], hi["h"], hi["b"], N) * dy)
                  - np.sum(_forward64(lo["u"], lo["w"], lo["h"], lo["b"], N) * dy)) / (2 * eps)
            assert np.sum(g * d) == pytest.approx(fd, rel=1e-6, abs=1e-8), name


def test_direct_and_fft_forms_agree():
    u, w, h, b, dy = _inputs(3, 4, 64, 3, seed=5)
    for x, y in zip(oracle.backward_circular(u, w, h, b, dy, 3, mode="direct"),
                    oracle.backward_circular(u, w, h, b, dy, 3, mode="fft")):
        assert np.allclose(x, y, rtol=1e-10, atol=1e-10)


def test_delta_filters_reduce_to_the_causal_backward():
    # with h = delta every step is the same circular or causal, so the gradients of
    # the inputs, the short-conv taps and the biases are those of the causal chain
    N, B, D, S = 3, 2, 4, 32
    u, w, _, b, dy = _inputs(B, D, S, N, seed=7)
    h = np.zeros((N - 1, D, S), dtype=np.float32)
    h[:, :, 0] = 1.0
    cdu, cdw, _, cdb = oracle.backward_circular(u, w, h, b, dy, N)
    du, dw, _, db = oracle.backward(u, w, h, b, dy, N, mode="direct")
    assert np.allclose(cdu, du, rtol=1e-9, atol=1e-9)
    assert np.allclose(cdw, dw, rtol=1e-9, atol=1e-9)
    assert np.allclose(cdb, db, rtol=1e-9, atol=1e-9)


def test_equal_per_sample_sets_give_the_shared_gradients():
    N, B, D, S = 2, 3, 2, 16
    u, w, h, b, dy = _inputs(B, D, S, N, seed=9)
    du, dw, dh, db = oracle.backward_circular(u, w, h, b, dy, N)
    pdu, pdw, pdh, pdb = oracle.backward_circular_per_sample(u, w, np.broadcast_to(h, (B,) + h.shape), b, dy, N)
    assert np.allclose(pdu, du, atol=1e-10) and np.allclose(pdw, dw, atol=1e-10)
    assert np.allclose(pdh.sum(axis=0), dh, atol=1e-10) and np.allclose(pdb, db, atol=1e-10)
