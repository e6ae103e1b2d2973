"""The device transforms on their own, through hyena_filter_spectrum (the forward
transform of the zero-padded filter, the same transform code the forward runs on
the gated input), checked against closed forms of the discrete Fourier transform
rather than against another FFT:

* a unit impulse at t = 0 has every bin equal to 1;
* an impulse at t = s has bins exp(-2 pi i k s / 2L) (the shift theorem);
* Parseval: sum_t h[t]^2 = (|H_0|^2 + |H_L|^2 + 2 sum_{0<k<L} |H_k|^2) / 2L;
* linearity: the spectrum of a*h1 + h2 is a*H1 + H2.

Both paths (the LDS transform and the four-step passes) at sizes from the
smallest plan to 2^20.
"""
import numpy as np
import pytest

from tests._hy import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fft_long_convolution_libhyena_amd import load_library

    load_library()
    yield


def _bins(h, path):
    """Bins 0..L of the 2L-point transform of each zero-padded filter row of h [1, D, L],
    decoded from the plan's spectrum layout (scale 1/(4L); slot 0 = (bin 0, bin L);
    the four-step layout stores bin k1 + L1*k2 at [k1][k2])."""
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    _, D, L = h.shape
    with Plan(L, D, 2, "f32", path) as p:
        assert p.path == path
        spec = p.spectrum(torch.from_numpy(np.ascontiguousarray(h, np.float32)).cuda())
        torch.cuda.synchronize()
        s = spec.cpu().numpy().view(np.complex64).reshape(D, L).astype(np.complex128) * (4 * L)
    if path == "fourstep":
        log = L.bit_length() - 1
        L1 = 1 << min(log // 2, 9)
        s = s.reshape(D, L1, L // L1).transpose(0, 2, 1).reshape(D, L)
    out = np.empty((D, L + 1), np.complex128)
    out[:, 1:L] = s[:, 1:L]
    out[:, 0] = s[:, 0].real
    out[:, L] = s[:, 0].imag
    return out


SIZES = [(16, "lds"), (1024, "lds"), (16384, "lds"), (256, "fourstep"), (65536, "fourstep"),
         (1 << 20, "fourstep")]


@pytest.mark.parametrize("L,path", SIZES)
def test_impulses(L, path):
    shifts = [0, 1, L // 3, L - 1]
    h = np.zeros((1, len(shifts), L), np.float32)
    for i, s in enumerate(shifts):
        h[0, i, s] = 1.0
    H = _bins(h, path)
    k = np.arange(L + 1)
    err = 0.0
    for i, s in enumerate(shifts):
        want = np.exp(-2j * np.pi * k * s / (2 * L))
        err = max(err, np.abs(H[i] - want).max())
    say(f"[transform] impulses L={L} {path}: max |H - closed form| {err:.2e}")
    assert np.abs(H[0] - 1.0).max() < 1e-6  # the impulse at 0 meets no twiddle
    assert err < 2e-5 * max(1.0, np.log2(L) / 10)


@pytest.mark.parametrize("L,path", SIZES)
def test_parseval_and_linearity(L, path):
    rng = np.random.default_rng(L + len(path))
    h1 = rng.standard_normal((1, 2, L)).astype(np.float32)
    h2 = rng.standard_normal((1, 2, L)).astype(np.float32)
    a = np.float32(0.75)  # exact in fp32, so a*h1 + h2 is formed exactly enough
    mix = (a * h1 + h2).astype(np.float32)
    H1, H2, Hm = _bins(h1, path), _bins(h2, path), _bins(mix, path)
    energy_t = (h1[0].astype(np.float64) ** 2).sum(axis=1)
    energy_f = (np.abs(H1[:, 0]) ** 2 + np.abs(H1[:, L]) ** 2 + 2 * (np.abs(H1[:, 1:L]) ** 2).sum(axis=1)) / (2 * L)
    pe = np.abs(energy_f / energy_t - 1).max()
    lin = np.linalg.norm(Hm - (float(a) * H1 + H2)) / np.linalg.norm(Hm)
    say(f"[transform] L={L} {path}: Parseval rel {pe:.2e}, linearity rel {lin:.2e}")
    assert pe < 1e-5
    assert lin < 2e-6
