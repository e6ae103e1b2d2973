"""GPU parity of the gated 2-D long convolution (hyena_plan2d_create,
hyena_filter_spectrum2d, hyena_conv2d_forward) against the fp64 oracle.

Bounds: relative L2 1e-4 for fp32 I/O, 1e-2 for bf16 I/O (the 1-D contract's),
each image within 10x of it.
"""
import numpy as np
import pytest

import oracle
from fft_long_convolution_libhyena_amd import synth
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


def _dev(a, dtype):
    import torch

    t = torch.from_numpy(a).cuda()
    return t.to(torch.bfloat16).contiguous() if dtype == "bf16" else t


def _run(inp, B, D, H, W, dtype, use_g, use_x, ws_bytes=None, repeat=1):
    import torch

    from fft_long_convolution_libhyena_amd import Plan2D

    outs = []
    with Plan2D(H, W, D, dtype) as p:
        spec = p.spectrum(torch.from_numpy(inp.k).cuda())
        v = _dev(inp.v, dtype)
        g = _dev(inp.g, dtype) if use_g else None
        x = _dev(inp.x, dtype) if use_x else None
        bias = torch.from_numpy(inp.bias).cuda()
        ws = None if ws_bytes is None else torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        for _ in range(repeat):
            outs.append(p.forward(v, spec, bias, g=g, x=x, workspace=ws))
        torch.cuda.synchronize()
    return outs


CASES = [
    # B, D, H, W, dtype, pre-gate, post-gate, centred kernel
    (1, 2, 16, 32, "f32", True, True, True),      # the smallest plan
    (2, 3, 32, 64, "f32", False, False, False),   # causal kernel, no gates
    (1, 4, 64, 32, "bf16", True, True, True),
    (2, 2, 128, 128, "f32", True, False, True),
    (1, 2, 512, 32, "f32", False, True, True),    # the tallest plan
    (1, 2, 16, 512, "f32", True, True, False),    # the widest plan
    (1, 3, 256, 256, "f32", True, True, True),
    (2, 2, 64, 256, "bf16", True, False, True),
]


@pytest.mark.parametrize("B,D,H,W,dtype,use_g,use_x,centred", CASES)
def test_conv2d_matches_oracle(B, D, H, W, dtype, use_g, use_x, centred):
    inp = synth.conv2d_inputs(B, D, H, W, dtype, seed=H + W + D, centred=centred)
    (y,) = _run(inp, B, D, H, W, dtype, use_g, use_x)
    ref = oracle.conv2d_forward(inp.v, inp.k, inp.bias, inp.g if use_g else None, inp.x if use_x else None)
    got = y.float().cpu().numpy().astype(np.float64)
    err = oracle.rel_l2(got, ref)
    per = max(oracle.rel_l2(got[b, d], ref[b, d]) for b in range(B) for d in range(D))
    bound = 1e-2 if dtype == "bf16" else 1e-4
    say(f"[conv2d] B={B} D={D} {H}x{W} {dtype} g={use_g} x={use_x} centred={centred}: "
        f"rel_l2 {err:.3e} worst image {per:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= bound and per <= 10 * bound


@pytest.mark.parametrize("H,W", [(16, 32), (64, 128), (256, 64)])
def test_spectrum2d_matches_numpy_rfft2(H, W):
    import torch

    from fft_long_convolution_libhyena_amd import Plan2D

    D = 3
    inp = synth.conv2d_inputs(1, D, H, W, seed=7)
    with Plan2D(H, W, D) as p:
        spec = p.spectrum(torch.from_numpy(inp.k).cuda())
        torch.cuda.synchronize()
        s = spec.cpu().numpy().view(np.complex64).reshape(D, 2 * H, W + 1).astype(np.complex128)
    s *= 8.0 * H * W  # stored with the scale 1 / (4 * 2H * W)
    want = np.fft.rfft2(inp.k.astype(np.float64))
    err = np.linalg.norm(s - want) / np.linalg.norm(want)
    say(f"[conv2d spectrum] {H}x{W}: rel_l2 {err:.3e}")
    assert err < 2e-6


def test_conv2d_chunking_and_determinism():
    """One image per launch gives the same bits as all images at once, and two calls agree."""
    B, D, H, W = 2, 3, 64, 64
    inp = synth.conv2d_inputs(B, D, H, W, seed=11)
    a, b = _run(inp, B, D, H, W, "f32", True, True, repeat=2)
    (c,) = _run(inp, B, D, H, W, "f32", True, True, ws_bytes=8 * H * W)
    assert bool((a == b).all()) and bool((a == c).all())


def test_conv2d_error_paths():
    import torch

    from fft_long_convolution_libhyena_amd import HyenaError, Plan2D

    with pytest.raises(HyenaError) as e:
        Plan2D(64, 1024, 2)
    assert e.value.status == 2
    inp = synth.conv2d_inputs(1, 2, 32, 32, seed=1)
    with Plan2D(32, 32, 2) as p:
        spec = p.spectrum(torch.from_numpy(inp.k).cuda())
        v = torch.from_numpy(inp.v).cuda()
        bias = torch.from_numpy(inp.bias).cuda()
        with pytest.raises(HyenaError) as e:
            p.forward(v, spec, bias, workspace=torch.empty(8 * 32 * 32 - 256, dtype=torch.uint8, device="cuda"))
        assert e.value.status == 3
        with pytest.raises(ValueError):
            p.forward(v[:, :1].contiguous(), spec, bias)
        with pytest.raises(ValueError):
            p.spectrum(torch.from_numpy(inp.k[:, :32]).contiguous().cuda())


def _kernel_sets(B, D, dims, seed, nd):
    """B seeded kernel sets [B, D, *doubled grid] (sample b drawn with seed + b)."""
    make = synth.conv2d_inputs if nd == 2 else synth.conv3d_inputs
    return np.stack([make(1, D, *dims, seed=seed + b).k for b in range(B)])


@pytest.mark.parametrize("B,D,H,W,dtype", [(3, 2, 32, 64, "f32"), (2, 3, 64, 32, "bf16")])
def test_conv2d_per_sample_matches_oracle(B, D, H, W, dtype):
    """A kernel set per sample (input-dependent kernels): image (b, d) uses kernel
    d of sample b."""
    import torch

    from fft_long_convolution_libhyena_amd import Plan2D

    inp = synth.conv2d_inputs(B, D, H, W, dtype, seed=21)
    kb = _kernel_sets(B, D, (H, W), 300, 2)
    with Plan2D(H, W, D, dtype) as p:
        spec = p.spectrum_batched(torch.from_numpy(kb).cuda())
        y = p.forward_per_sample(_dev(inp.v, dtype), spec, torch.from_numpy(inp.bias).cuda(),
                                 g=_dev(inp.g, dtype), x=_dev(inp.x, dtype))
        torch.cuda.synchronize()
    ref = np.concatenate([oracle.conv2d_forward(inp.v[b:b + 1], kb[b], inp.bias, inp.g[b:b + 1], inp.x[b:b + 1])
                          for b in range(B)])
    got = y.float().cpu().numpy().astype(np.float64)
    err = oracle.rel_l2(got, ref)
    per = [oracle.rel_l2(got[b], ref[b]) for b in range(B)]
    bound = 1e-2 if dtype == "bf16" else 1e-4
    say(f"[conv2d per-sample] B={B} D={D} {H}x{W} {dtype}: rel_l2 {err:.3e}, per sample {max(per):.2e}")
    assert err <= bound and max(per) <= 10 * bound


def test_conv2d_equal_kernel_sets_reproduce_the_shared_step():
    import torch

    from fft_long_convolution_libhyena_amd import Plan2D

    B, D, H, W = 3, 2, 32, 32
    inp = synth.conv2d_inputs(B, D, H, W, seed=22)
    kb = np.repeat(inp.k[None], B, axis=0)
    with Plan2D(H, W, D) as p:
        v, g, x = (torch.from_numpy(a).cuda() for a in (inp.v, inp.g, inp.x))
        bias = torch.from_numpy(inp.bias).cuda()
        a = p.forward_per_sample(v, p.spectrum_batched(torch.from_numpy(kb).cuda()), bias, g=g, x=x)
        b = p.forward(v, p.spectrum(torch.from_numpy(inp.k).cuda()), bias, g=g, x=x)
        torch.cuda.synchronize()
        with pytest.raises(ValueError):  # one spectrum is too small for B = 3
            p.forward_per_sample(v, p.spectrum(torch.from_numpy(inp.k).cuda()), bias)
    assert bool((a == b).all())


CIRC_CASES = [
    # B, D, H, W, dtype: the smallest circular plan, non-square, bf16, the largest axes
    (1, 2, 32, 64, "f32"),
    (2, 2, 64, 128, "f32"),
    (1, 3, 128, 64, "bf16"),
    (1, 1, 1024, 64, "f32"),
    (1, 1, 32, 1024, "f32"),
]


@pytest.mark.parametrize("B,D,H,W,dtype", CIRC_CASES)
def test_conv2d_circular_matches_oracle(B, D, H, W, dtype):
    """Circular plans (periodic grid, kernel on the grid itself) against the
    circular oracle; the zero-padded result differs by far more than the bound."""
    import torch

    from fft_long_convolution_libhyena_amd import Plan2D

    inp = synth.conv2d_inputs(B, D, H, W, dtype, seed=H + W + 3)
    kc = np.ascontiguousarray(inp.k[:, :H, :W])  # a kernel on the H x W grid
    with Plan2D(H, W, D, dtype, circular=True) as p:
        assert p.spectrum_bytes() == 8 * D * H * (W // 2 + 1)
        y = p.forward(_dev(inp.v, dtype), p.spectrum(torch.from_numpy(kc).cuda()), torch.from_numpy(inp.bias).cuda(),
                      g=_dev(inp.g, dtype), x=_dev(inp.x, dtype))
        torch.cuda.synchronize()
    ref = oracle.conv2d_forward(inp.v, kc, inp.bias, inp.g, inp.x, circular=True)
    got = y.float().cpu().numpy().astype(np.float64)
    err = oracle.rel_l2(got, ref)
    bound = 1e-2 if dtype == "bf16" else 1e-4
    kz = np.zeros((D, 2 * H, 2 * W), np.float32)
    kz[:, :H, :W] = kc
    gap = oracle.rel_l2(oracle.conv2d_forward(inp.v, kz, inp.bias, inp.g, inp.x), ref)
    say(f"[conv2d circular] B={B} D={D} {H}x{W} {dtype}: rel_l2 {err:.3e} (zero-padded differs by {gap:.1e})")
    assert err <= bound and gap > 10 * bound


def test_conv2d_circular_spectrum_matches_numpy_rfft2():
    import torch

    from fft_long_convolution_libhyena_amd import Plan2D

    D, H, W = 2, 64, 128
    k = synth.conv2d_inputs(1, D, H, W, seed=4).k[:, :H, :W].copy()
    with Plan2D(H, W, D, circular=True) as p:
        s = p.spectrum(torch.from_numpy(k).cuda())
        torch.cuda.synchronize()
        s = s.cpu().numpy().view(np.complex64).reshape(D, H, W // 2 + 1).astype(np.complex128) * (2.0 * H * W)
    want = np.fft.rfft2(k.astype(np.float64))
    assert np.linalg.norm(s - want) / np.linalg.norm(want) < 2e-6
