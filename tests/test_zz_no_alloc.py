"""hyena_forward_noalloc (no workspace, no allocation) through the C ABI against
hyena_forward with its workspace: the same bits on two calls in a row, the
second with a smaller batch, and sampled rows within the parity bound of the
oracle. Marked gpu; needs an MI355X."""
import ctypes

import numpy as np
import pytest

import oracle
from fft_long_convolution_libhyena_amd import synth
from tests._hy import say, to_device, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fft_long_convolution_libhyena_amd import load_library

    load_library()
    yield


def _call_noalloc(p, t, y):
    import torch

    st = p.lib.hyena_forward_noalloc(p.handle, int(t["u"].shape[0]), t["u"].data_ptr(), t["w"].data_ptr(),
                                     t["spec"].data_ptr(), t["bias"].data_ptr(), y.data_ptr(),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, f"hyena_forward_noalloc returned {st}"


def _call_forward(p, t, y):
    import torch

    B = int(t["u"].shape[0])
    need = p.workspace_bytes(B)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    st = p.lib.hyena_forward(p.handle, B, t["u"].data_ptr(), t["w"].data_ptr(), t["spec"].data_ptr(),
                             t["bias"].data_ptr(), y.data_ptr(), ws.data_ptr() if need else None, need,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, f"hyena_forward returned {st}"
    return ws


@pytest.mark.parametrize("Bs,D,L,order,dtype,path", [
    ((2, 1), 96, 65536, 2, "f32", "fourstep"),    # pipelined launches over the scratch array's 42-row chunks
    ((3, 2), 16, 65536, 3, "bf16", "fourstep"),   # chunk by chunk (order 3)
    ((2, 1), 12, 1 << 20, 2, "f32", "fourstep"),  # 8 MiB rows: 8 rows per chunk
    ((2, 1), 10, 16384, 2, "f32", "partitioned"),
    ((4, 3), 8, 4096, 3, "f32", "lds"),           # no scratch on the LDS path
])
def test_noalloc_matches_forward(Bs, D, L, order, dtype, path):
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    with Plan(L, D, order, dtype, path) as p:
        for i, B in enumerate(Bs):  # the second call has a smaller input
            wl = synth.custom(B, D, L, order, dtype=dtype, seed=7 * B + D + i)
            x = synth.generate(wl)
            say(f"[noalloc] call {i}: {wl.describe()} path={path}")
            t = to_device(x)
            t["spec"] = p.spectrum(t["h"])
            y_na = torch.full((B, D, L), float("nan"), dtype=p.io_dtype, device="cuda")
            _call_noalloc(p, t, y_na)
            y_ref = torch.empty((B, D, L), dtype=p.io_dtype, device="cuda")
            _call_forward(p, t, y_ref)
            torch.cuda.synchronize()
            assert bool((y_na == y_ref).all()), "no-alloc forward differs from hyena_forward"
            rows = synth.sample_rows(wl, 4)
            ref = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, order, rows=rows)
            got = y_na.float().cpu().numpy().astype(np.float64).reshape(-1, L)[rows]
            err = oracle.rel_l2(got, ref)
            say(f"   equal to hyena_forward; rel_l2 vs oracle {err:.3e}")
            assert err <= tol(wl)
