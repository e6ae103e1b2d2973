"""The binding's debugging switches on the GPU: HYENA_FORCE_PATH sends plans that ask
for automatic selection down the named path (parity against the oracle there), and
HYENA_DEBUG_SYNC changes no result."""
import numpy as np
import pytest

import oracle
from fft_long_convolution_libhyena_amd import synth
from tests._hy import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fft_long_convolution_libhyena_amd import load_library

    load_library()
    yield


def _forward(x):
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = x.wl
    t = to_device(x)
    with Plan(wl.L, wl.D, wl.order, wl.dtype) as p:
        y = p.forward(t["u"], t["w"], p.spectrum(t["h"]), t["bias"])
        torch.cuda.synchronize()
        return p.path, y.double().cpu().numpy()


@pytest.mark.parametrize("forced,L", [("fourstep", 1024), ("partitioned", 16384), ("lds", 16384)])
def test_force_path(monkeypatch, forced, L):
    wl = synth.custom(2, 3, L, 3, seed=L + len(forced))
    x = synth.generate(wl)
    monkeypatch.setenv("HYENA_FORCE_PATH", forced)
    used, y = _forward(x)
    err = oracle.rel_l2(y, oracle.forward(x.u_proj, x.short_w, x.h, x.bias, wl.order))
    say(f"[debug] HYENA_FORCE_PATH={forced} L={L}: path {used}, rel_l2 {err:.2e}")
    assert used == forced and err <= 1e-4


def test_debug_sync_changes_nothing(monkeypatch):
    wl = synth.custom(2, 4, 4096, 2, seed=17)
    x = synth.generate(wl)
    _, y0 = _forward(x)
    monkeypatch.setenv("HYENA_DEBUG_SYNC", "1")
    _, y1 = _forward(x)
    assert np.array_equal(y0, y1)
