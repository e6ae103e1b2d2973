"""GPU parity of the partitioned path (HYENA_PATH_PARTITIONED: the causal long
convolution with the filter cut into blocks of 4096 taps, windows of 8192 samples)
against the fp64 oracle.

Bounds as for the other paths: relative L2 1e-4 for fp32 I/O, 1e-2 for bf16 I/O.
The shapes cover every block count the path serves (2 to 32 blocks, both pass 2
groupings), orders 2 to 4 (the gated output of a step carried through the
workspace), ragged D, B > 1 and chunking by a small workspace.
"""
import numpy as np
import pytest

import oracle
from fft_long_convolution_libhyena_amd import synth
from tests._hy import say, to_device

pytestmark = pytest.mark.gpu

Q = 4096


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fft_long_convolution_libhyena_amd import load_library

    load_library()
    yield


def _forward(x, workspace_rows=None, repeat=1):
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = x.wl
    t = to_device(x)
    outs = []
    with Plan(wl.L, wl.D, wl.order, wl.dtype, "partitioned") as p:
        assert p.path == "partitioned"
        spec = p.spectrum(t["h"])
        ws = None
        if workspace_rows is not None:
            per_row = (8 + (4 if wl.order > 2 else 0)) * wl.L
            ws = torch.empty(workspace_rows * per_row, dtype=torch.uint8, device=t["u"].device)
        for _ in range(repeat):
            outs.append(p.forward(t["u"], t["w"], spec, t["bias"], workspace=ws))
        torch.cuda.synchronize()
    return outs


CASES = [
    # B, D, L, order, dtype: 2 blocks (pass 2 pairs), 4..32 blocks (groups of four)
    (1, 3, 8192, 2, "f32"),
    (2, 3, 16384, 2, "f32"),
    (1, 5, 16384, 3, "bf16"),
    (2, 2, 32768, 3, "f32"),
    (1, 3, 65536, 2, "f32"),
    (2, 2, 65536, 2, "bf16"),
    (1, 2, 65536, 4, "f32"),
    (1, 2, 131072, 2, "f32"),
]


@pytest.mark.parametrize("B,D,L,order,dtype", CASES)
def test_partitioned_matches_oracle(B, D, L, order, dtype):
    wl = synth.custom(B, D, L, order, dtype, seed=L % 97 + 10 * D + order)
    x = synth.generate(wl)
    say(f"[partitioned] {wl.describe()}")
    y, = _forward(x)
    got = y.float().cpu().numpy().astype(np.float64)
    ref = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, order)
    err = oracle.rel_l2(got, ref)
    bound = 1e-2 if dtype == "bf16" else 1e-4
    # per output block: a wrong window or filter block shows in its own block
    blk = got.reshape(B * D, L // Q, Q) - ref.reshape(B * D, L // Q, Q)
    per = np.linalg.norm(blk, axis=2) / np.maximum(np.linalg.norm(ref.reshape(B * D, L // Q, Q), axis=2), 1e-30)
    say(f"   rel_l2 {err:.3e}, worst block {per.max():.2e}")
    assert np.all(np.isfinite(got))
    assert err <= bound
    assert per.max() <= 10 * bound


@pytest.mark.parametrize("name", ["long64k", "long64k_o3"])
def test_partitioned_workload_channels(name):
    """long64k at orders 2 and 3, all of L, on three channels."""
    wl = synth.WORKLOADS[name]
    x = synth.channel_subset(synth.generate(wl), [0, 383, wl.D - 1])
    say(f"[partitioned] {name} channels [0, 383, {wl.D - 1}]")
    y, = _forward(x)
    err = oracle.rel_l2(y.float().cpu().numpy().astype(np.float64),
                        oracle.forward(x.u_proj, x.short_w, x.h, x.bias, wl.order))
    say(f"   rel_l2 {err:.3e}")
    assert err <= 1e-4


@pytest.mark.parametrize("order,rows", [(2, 1), (3, 3)])
def test_partitioned_chunked_workspace_is_bit_identical(order, rows):
    """A workspace of one or three rows runs the rows in chunks; every row's
    arithmetic is the same, so the output must not change at all."""
    wl = synth.custom(2, 5, 16384, order, seed=31 + order)
    x = synth.generate(wl)
    full, again = _forward(x, repeat=2)
    small, = _forward(x, workspace_rows=rows)
    assert bool((full == again).all()), "two calls differ"
    assert bool((full == small).all()), "chunked run differs"


def test_partitioned_agrees_with_fourstep():
    """Two evaluations of the same convolution: both within the fp32 bound of the
    oracle and of each other."""
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = synth.custom(1, 4, 65536, 3, seed=44)
    x = synth.generate(wl)
    t = to_device(x)
    ys = {}
    for path in ("fourstep", "partitioned"):
        with Plan(wl.L, wl.D, wl.order, "f32", path) as p:
            ys[path] = p.forward(t["u"], t["w"], p.spectrum(t["h"]), t["bias"]).double().cpu().numpy()
            torch.cuda.synchronize()
    ref = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, wl.order)
    e4, ep = oracle.rel_l2(ys["fourstep"], ref), oracle.rel_l2(ys["partitioned"], ref)
    say(f"[partitioned] vs oracle {ep:.2e}, four-step vs oracle {e4:.2e}")
    assert ep <= 1e-4 and e4 <= 1e-4
    assert oracle.rel_l2(ys["partitioned"], ys["fourstep"]) <= 2e-4


def test_partitioned_spectrum_matches_numpy_rfft():
    """The plan's spectrum: for every filter, the 8192-point real FFT of each
    4096-tap block zero-padded, bins 0..4096 with slot 0 = (bin 0, bin 4096),
    scaled by 1/(4*4096)."""
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = synth.custom(1, 3, 32768, 3, seed=5)
    x = synth.generate(wl)
    P = wl.L // Q
    with Plan(wl.L, wl.D, wl.order, "f32", "partitioned") as p:
        assert p.spectrum_bytes() == 8 * (wl.order - 1) * wl.D * wl.L
        s = p.spectrum(torch.from_numpy(x.h).cuda())
        torch.cuda.synchronize()
        got = s.cpu().numpy().view(np.complex64).reshape(wl.order - 1, wl.D, P, Q).astype(np.complex128) * (4 * Q)
    blocks = x.h.astype(np.float64).reshape(wl.order - 1, wl.D, P, Q)
    want = np.fft.rfft(np.concatenate([blocks, np.zeros_like(blocks)], -1), axis=-1)  # Q + 1 bins
    full = np.empty_like(want)
    full[..., 1:Q] = got[..., 1:Q]
    full[..., 0] = got[..., 0].real
    full[..., Q] = got[..., 0].imag
    err = np.linalg.norm(full - want) / np.linalg.norm(want)
    say(f"[partitioned] block spectra rel_l2 {err:.3e}")
    assert err < 2e-6


def test_partitioned_per_sample():
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = synth.custom(3, 2, 16384, 3, seed=9)
    x = synth.generate(wl)
    hb = synth.per_sample_filters(wl)
    t = to_device(x)
    with Plan(wl.L, wl.D, wl.order, "f32", "partitioned") as p:
        y = p.forward_per_sample(t["u"], t["w"], p.spectrum_batched(torch.from_numpy(hb).cuda()), t["bias"])
        torch.cuda.synchronize()
    ref = oracle.forward_per_sample(x.u_proj, x.short_w, hb, x.bias, wl.order)
    err = oracle.rel_l2(y.double().cpu().numpy(), ref)
    say(f"[partitioned] per-sample rel_l2 {err:.3e}")
    assert err <= 1e-4


def test_partitioned_plan_limits_and_errors():
    import ctypes

    import torch

    from fft_long_convolution_libhyena_amd import HyenaError, Plan, load_library
    from fft_long_convolution_libhyena_amd.binding import FLAG_CIRCULAR, PATH_PARTITIONED

    lib = load_library()
    h = ctypes.c_void_p()
    for L in (4096, 1 << 18):  # fewer than two blocks; more than 32
        assert lib.hyena_plan_create_path(ctypes.byref(h), L, 4, 2, 0, PATH_PARTITIONED) == 2
    assert lib.hyena_plan_create_ex(ctypes.byref(h), 65536, 4, 2, 0, PATH_PARTITIONED, FLAG_CIRCULAR) == 2
    wl = synth.custom(1, 2, 8192, 3, seed=4)
    x = synth.generate(wl)
    t = to_device(x)
    with Plan(8192, 2, 3, "f32", "partitioned") as p:
        assert p.workspace_bytes(1) == 2 * 12 * 8192  # both rows, window spectra + a step's output
        assert p.backward_workspace_bytes(1) == 0
        spec = p.spectrum(t["h"])
        with pytest.raises(HyenaError) as e:  # less than one row
            p.forward(t["u"], t["w"], spec, t["bias"],
                      workspace=torch.empty(12 * 8192 - 16, dtype=torch.uint8, device=t["u"].device))
        assert e.value.status == 3
        g = torch.zeros((1, 2, 8192), dtype=torch.float32, device=t["u"].device)
        with pytest.raises(HyenaError) as e:
            p.backward(t["u"], t["w"], spec, t["bias"], g,
                       workspace=torch.empty(1024, dtype=torch.uint8, device=t["u"].device))
        assert e.value.status == 2
