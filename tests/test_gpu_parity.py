"""GPU parity of libhyena against the fp64 oracle (marked gpu; needs an MI355X).

Every call goes through the C ABI (ctypes binding). Floating-point outputs are
compared with the relative L2 bound of the parity contract: 1e-4 for fp32 I/O
and 1e-2 for bf16 I/O (fp32 arithmetic inside).
"""
import numpy as np
import pytest

import oracle
from fft_long_convolution_libhyena_amd import synth
from tests._hy import run, say, to_device, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fft_long_convolution_libhyena_amd import load_library

    load_library()  # raises if the HIP library was not built
    yield


def _check(x, path="auto", rows=None, mode="fft", label=""):
    wl = x.wl
    say(f"[parity] {label or wl.name}: {wl.describe()} path={path}")
    y, used, _ = run(x, path)
    if rows is None:
        ref = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, wl.order, mode=mode)
        got = y
    else:
        ref = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, wl.order, mode=mode, rows=rows)
        got = y.reshape(-1, wl.L)[rows]
    assert np.all(np.isfinite(got)), "non-finite output"
    err = oracle.rel_l2(got, ref)
    say(f"   path={used} rel_l2={err:.3e} (bound {tol(wl):.0e})")
    assert err <= tol(wl), f"rel L2 {err:.3e} exceeds {tol(wl):.0e}"
    # no single row may be far off either (a wrong row hides easily in a global norm)
    g2, r2 = got.reshape(-1, wl.L), ref.reshape(-1, wl.L)
    row_err = np.linalg.norm(g2 - r2, axis=1) / np.maximum(np.linalg.norm(r2, axis=1), 1e-30)
    assert row_err.max() <= 10 * tol(wl), f"worst row rel L2 {row_err.max():.3e}"
    return used, err


# ------------------------------------------------------------ spectrum layout


@pytest.mark.parametrize("L,path", [(16, "lds"), (1024, "lds"), (16384, "lds"), (256, "fourstep"),
                                    (4096, "fourstep"), (65536, "fourstep")])
def test_spectrum_matches_numpy_rfft(L, path):
    """hyena_filter_spectrum vs numpy's real FFT of the zero-padded filter (library special case)."""
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = synth.custom(1, 3, L, 3, seed=L)
    x = synth.generate(wl)
    say(f"[spectrum] L={L} path={path}")
    with Plan(L, wl.D, wl.order, "f32", path) as p:
        spec = p.spectrum(torch.from_numpy(x.h).cuda())
        torch.cuda.synchronize()
        s = spec.cpu().numpy().view(np.complex64).reshape(wl.order - 1, wl.D, L).astype(np.complex128)
        used = p.path
    s *= 4 * L  # stored spectra carry an exact 2^-(log2 L + 2) scale
    want = np.fft.rfft(np.concatenate([x.h.astype(np.float64), np.zeros_like(x.h, np.float64)], -1), axis=-1)
    if used == "lds":
        got = s.copy()
    else:
        from fft_long_convolution_libhyena_amd import binding  # noqa: F401

        # four-step layout: [k1][k2] holds bin k1 + L1*k2
        log = L.bit_length() - 1
        l1 = min(log // 2, 9)
        L1, L2 = 1 << l1, 1 << (log - l1)
        got = s.reshape(wl.order - 1, wl.D, L1, L2).transpose(0, 1, 3, 2).reshape(wl.order - 1, wl.D, L)
    full = np.empty_like(want)
    full[..., 1:L] = got[..., 1:L]
    full[..., 0] = got[..., 0].real
    full[..., L] = got[..., 0].imag
    err = np.linalg.norm(full - want) / np.linalg.norm(want)
    say(f"   rel_l2={err:.3e}")
    assert err < 2e-6


# -------------------------------------------------------------- small grids


SMALL = [
    # (B, D, L, order, dtype, path)
    (1, 1, 16, 2, "f32", "lds"),
    (1, 3, 32, 2, "f32", "lds"),
    (2, 5, 64, 3, "f32", "lds"),
    (1, 13, 128, 2, "f32", "lds"),
    (3, 4, 256, 4, "f32", "lds"),
    (1, 9, 512, 2, "bf16", "lds"),
    (2, 8, 2048, 3, "f32", "lds"),
    (1, 6, 4096, 2, "bf16", "lds"),
    (1, 2, 8192, 2, "f32", "lds"),
    (1, 3, 16384, 3, "f32", "lds"),
    (1, 3, 256, 2, "f32", "fourstep"),
    (2, 5, 512, 3, "f32", "fourstep"),
    (1, 4, 1024, 2, "bf16", "fourstep"),
    (1, 3, 2048, 4, "f32", "fourstep"),
    (2, 3, 4096, 2, "f32", "fourstep"),
    (1, 2, 8192, 3, "f32", "fourstep"),
    (1, 2, 16384, 2, "f32", "fourstep"),
    # orders 5 to 8: every order the plan accepts runs through the forward kernels
    (1, 3, 1024, 5, "f32", "lds"),
    (2, 2, 1024, 6, "bf16", "lds"),
    (1, 2, 1024, 7, "f32", "lds"),
    (1, 2, 1024, 8, "f32", "lds"),
    (1, 2, 16384, 5, "f32", "lds"),
    (1, 2, 16384, 8, "f32", "lds"),
    (1, 2, 16384, 8, "bf16", "lds"),
    (1, 3, 4096, 5, "f32", "fourstep"),
    (1, 2, 4096, 6, "f32", "fourstep"),
    (2, 2, 4096, 7, "bf16", "fourstep"),
    (1, 2, 4096, 8, "f32", "fourstep"),
    (1, 2, 65536, 5, "f32", "fourstep"),
    (1, 1, 65536, 8, "f32", "fourstep"),
]


@pytest.mark.parametrize("B,D,L,order,dtype,path", SMALL)
def test_parity_small(B, D, L, order, dtype, path):
    wl = synth.custom(B, D, L, order, dtype=dtype, seed=L + D + order)
    x = synth.generate(wl)
    used, _ = _check(x, path, mode="direct" if L <= 1024 else "fft",
                     label=f"small B={B} D={D} L={L} N={order} {dtype} {path}")
    assert used == path


def test_fourstep_and_lds_agree():
    wl = synth.custom(2, 4, 4096, 3, seed=77)
    x = synth.generate(wl)
    say("[paths] LDS vs four-step at L=4096")
    a, pa, _ = run(x, "lds")
    b, pb, _ = run(x, "fourstep")
    assert (pa, pb) == ("lds", "fourstep")
    assert oracle.rel_l2(a, b) < 2e-6


# ----------------------------------------------------------- the workloads


def test_workload_tiny_full():
    x = synth.generate(synth.WORKLOADS["tiny"])
    _check(x, mode="direct")


def test_workload_dna_small_full():
    x = synth.generate(synth.WORKLOADS["dna_small"])
    used, _ = _check(x)
    assert used == "lds"


def test_workload_lm125m_sampled():
    wl = synth.WORKLOADS["lm125m"]
    x = synth.generate(wl)
    used, _ = _check(x, rows=synth.sample_rows(wl, 384))
    assert used == "lds"


@pytest.mark.parametrize("name,nrows", [("long64k_o3", 24), ("long64k", 24), ("dna_1m", 6)])
def test_workload_long_sampled(name, nrows):
    wl = synth.WORKLOADS[name]
    x = synth.generate(wl)
    used, _ = _check(x, rows=synth.sample_rows(wl, nrows))
    assert used == "fourstep"


# -------------------------------------------------------------- invariants


def test_deterministic_bitwise():
    wl = synth.custom(2, 16, 8192, 3, seed=5)
    x = synth.generate(wl)
    say("[determinism] L=8192 and L=65536")
    _, _, outs = run(x, repeat=2)
    assert bool((outs[0] == outs[1]).all())
    wl2 = synth.custom(1, 8, 65536, 2, seed=6)
    _, _, outs2 = run(synth.generate(wl2), repeat=2)
    assert bool((outs2[0] == outs2[1]).all())


@pytest.mark.parametrize("path", ["lds", "fourstep"])
def test_delta_filter_reduces_to_gating(path):
    """h = delta: y = x_0 * x_1 * v * (1 + bias), independent of the FFT."""
    wl = synth.custom(2, 6, 1024, 2, seed=8)
    x = synth.generate(wl)
    x.h[:] = 0
    x.h[:, :, 0] = 1
    say(f"[delta] path={path}")
    y, _, _ = run(x, path)
    D = wl.D
    want = np.empty_like(y)
    for b in range(wl.B):
        for d in range(D):
            xs = [oracle.short_conv_row(x.u_proj[b, i * D + d], x.short_w[i * D + d]) for i in range(3)]
            want[b, d] = xs[0] * xs[1] * xs[2] * (1.0 + float(x.bias[0, d]))
    assert oracle.rel_l2(y, want) < 1e-5


@pytest.mark.parametrize("path", ["lds", "fourstep"])
def test_causal_up_to_rounding(path):
    wl = synth.custom(1, 4, 2048, 3, seed=9)
    x = synth.generate(wl)
    say(f"[causality] path={path}")
    y0, _, _ = run(x, path)
    t0 = 1001
    x.u_proj[:, :, t0] += 5.0
    y1, _, _ = run(x, path)
    scale = np.abs(y0).max()
    # outputs before t0 move only by transform rounding; the perturbation itself
    # changes every channel's output from t0 on
    assert np.abs(y1[..., :t0] - y0[..., :t0]).max() < 1e-5 * scale
    moved = np.abs(y1[..., t0:] - y0[..., t0:]).max(axis=-1)
    assert np.all(moved > 1e-2 * np.abs(y0[..., t0:]).max(axis=-1))


def test_edge_zero_value_branch():
    wl = synth.custom(1, 4, 512, 2, seed=10)
    x = synth.generate(wl)
    x.u_proj[:, 2 * wl.D:] = 0
    say("[edge] zero value branch")
    y, _, _ = run(x)
    assert not np.any(y)


# ------------------------------------------------------------------ errors


def test_error_paths_on_device():
    import ctypes

    import torch

    from fft_long_convolution_libhyena_amd import HyenaError, Plan

    wl = synth.custom(1, 4, 65536, 2, seed=11)
    x = synth.generate(wl)
    t = to_device(x)
    say("[errors] workspace / shapes")
    with Plan(wl.L, wl.D, 2) as p:
        spec = p.spectrum(t["h"])
        y = torch.empty((1, wl.D, wl.L), device="cuda")
        lib = p.lib
        small = torch.empty(8 * wl.L - 16, dtype=torch.uint8, device="cuda")
        st = lib.hyena_forward(p.handle, 1, t["u"].data_ptr(), t["w"].data_ptr(), spec.data_ptr(),
                               t["bias"].data_ptr(), y.data_ptr(), small.data_ptr(), small.numel(), None)
        assert st == 3  # HYENA_ERR_WORKSPACE
        st = lib.hyena_forward(p.handle, 1, t["u"].data_ptr(), t["w"].data_ptr(), spec.data_ptr(),
                               t["bias"].data_ptr(), y.data_ptr(), None, 0, None)
        assert st == 3
        st = lib.hyena_forward(p.handle, 0, t["u"].data_ptr(), t["w"].data_ptr(), spec.data_ptr(),
                               t["bias"].data_ptr(), y.data_ptr(), None, 0, None)
        assert st == 1  # B < 1
        st = lib.hyena_forward(p.handle, 1, t["u"].data_ptr() + 4, t["w"].data_ptr(), spec.data_ptr(),
                               t["bias"].data_ptr(), y.data_ptr(), None, 0, None)
        assert st == 1  # misaligned
        with pytest.raises(ValueError):
            p.forward(t["u"][:, :-1].contiguous(), t["w"], spec, t["bias"])
        # a workspace of exactly one row still works (one row per launch)
        one = torch.empty(8 * wl.L, dtype=torch.uint8, device="cuda")
        y1 = p.forward(t["u"], t["w"], spec, t["bias"], workspace=one)
        y2 = p.forward(t["u"], t["w"], spec, t["bias"])
        torch.cuda.synchronize()
        assert bool((y1 == y2).all())
    h = ctypes.c_void_p()
    from fft_long_convolution_libhyena_amd import load_library

    lib = load_library()
    assert lib.hyena_plan_create_path(ctypes.byref(h), 1 << 15, 4, 2, 0, 1) == 2  # LDS path too long
    assert lib.hyena_plan_create_path(ctypes.byref(h), 128, 4, 2, 0, 2) == 2  # four-step too short
    assert lib.hyena_plan_create_path(ctypes.byref(h), 65536, 4, 2, 0, 3) == 1  # path value 3 is unused
    with pytest.raises(HyenaError):
        Plan(1000, 4, 2)


# ------------------------------------------------- chunking of the four-step


@pytest.mark.parametrize("B,D,L,dtype,circular,ws_rows", [
    (1, 100, 65536, "f32", False, 32),    # 4 pipelined chunks of 32 rows, the last one of 4
    (2, 70, 65536, "bf16", False, 48),    # 3 chunks, ragged
    (1, 40, 131072, "f32", False, 32),    # the 256 x 512 split, 2 chunks
    (1, 37, 131072, "f32", True, 32),     # circular: a 65536-point transform
])
def test_pipelined_chunks_match_sequential_and_oracle(B, D, L, dtype, circular, ws_rows):
    """Order-2 four-step forwards run as pipelined launches when the workspace holds
    three tile slots; a one-row workspace runs chunk by chunk. Both must give the
    same bits, and sampled rows must match the oracle."""
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = synth.custom(B, D, L, 2, dtype=dtype, seed=D + L % 1000)
    x = synth.generate(wl)
    t = to_device(x)
    say(f"[pipelined] B={B} D={D} L={L} {dtype} circular={circular} chunk rows={ws_rows}")
    with Plan(L, D, 2, dtype, "fourstep", circular=circular) as p:
        spec = p.spectrum(t["h"])
        T = L // 2 if circular else L  # complex points per row's tile
        ws = torch.empty(3 * ws_rows * 8 * T, dtype=torch.uint8, device="cuda")
        y_pipe = p.forward(t["u"], t["w"], spec, t["bias"], workspace=ws)
        one = torch.empty(8 * T, dtype=torch.uint8, device="cuda")
        y_seq = p.forward(t["u"], t["w"], spec, t["bias"], workspace=one)
        timed = p.forward_timed(t["u"], t["w"], spec, t["bias"], torch.empty_like(y_pipe), workspace=ws)
        torch.cuda.synchronize()
    assert timed["pipe"] > 0 and timed["pass_a"] == 0  # the pipelined launches ran
    assert bool((y_pipe == y_seq).all()), "pipelined and sequential chunks differ"
    rows = synth.sample_rows(wl, 6)
    got = y_pipe.float().cpu().numpy().astype(np.float64).reshape(-1, L)[rows]
    if circular:
        ref = oracle.forward_circular(x.u_proj, x.short_w, x.h, x.bias, 2).reshape(-1, L)[rows]
    else:
        ref = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, 2, rows=rows)
    err = oracle.rel_l2(got, ref)
    say(f"   rel_l2={err:.3e}")
    assert err <= tol(wl)


# ---------------------------------------------------------- fused path


@pytest.mark.skip(reason="the fused persistent path was removed from the library: its first two runs on "
                         "MI355X did not finish (the second with time-bounded waits), a CPU emulation of its "
                         "ticket/counter logic completed, and the cause was never shown; the pipelined launches "
                         "(k_fs_pipe) replace it with no cross-workgroup waits")
@pytest.mark.parametrize("B,D", [(1, 1), (1, 13), (2, 24), (1, 96)])
def test_fused_path_parity(B, D):
    """The persistent single-launch four-step (order 2, L = 65536) against the oracle,
    including fewer rows than XCDs; its bounded waits must never expire."""
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = synth.custom(B, D, 65536, 2, seed=100 + D)
    x = synth.generate(wl)
    t = to_device(x)
    say(f"[fused] B={B} D={D}")
    with Plan(wl.L, wl.D, 2, "f32", "fused") as p:
        spec = p.spectrum(t["h"])
        ws = torch.empty(p.workspace_bytes(B), dtype=torch.uint8, device="cuda")
        say("   first forward")
        y = p.forward(t["u"], t["w"], spec, t["bias"], workspace=ws)
        torch.cuda.synchronize()
        say(f"   done; bounded-wait error flag {p.fused_check(ws)}")
        assert p.fused_check(ws) == 0
        y2 = p.forward(t["u"], t["w"], spec, t["bias"], workspace=ws)
        torch.cuda.synchronize()
        assert p.fused_check(ws) == 0
    rows = synth.sample_rows(wl, 8)
    ref = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, 2, rows=rows)
    got = y.cpu().numpy().astype(np.float64).reshape(-1, wl.L)[rows]
    err = oracle.rel_l2(got, ref)
    say(f"   rel_l2={err:.3e}")
    assert err <= 1e-4
    assert bool((y == y2).all())
