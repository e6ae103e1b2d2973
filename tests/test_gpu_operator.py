"""GPU parity of the whole operator forward (hyena_operator_forward: in_proj GEMM,
the hot path, out_proj GEMM) against the fp64 operator oracle. Bounds: relative
L2 1e-4 for fp32 plans; 1e-2 for bf16 plans, whose GEMM operands and u_proj are
bf16 as in a bf16 module."""
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


def _run(wl, path="auto", timed=False):
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    x = synth.generate(wl)
    p = synth.operator_params(wl)
    dev = torch.device("cuda", 0)
    io = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    def dv(a, dt=io):
        return torch.from_numpy(a).to(dev).to(dt).contiguous()

    with Plan(wl.L, wl.D, wl.order, wl.dtype, path) as plan:
        spec = plan.spectrum(dv(x.h, torch.float32))
        args = (dv(p.x), dv(p.w_in), dv(p.b_in), dv(x.short_w, torch.float32), spec, dv(x.bias, torch.float32),
                dv(p.w_out), dv(p.b_out))
        out = plan.operator_forward(*args)
        ms = plan.operator_forward_timed(*args, out=torch.empty_like(out)) if timed else None
        torch.cuda.synchronize()
        used = plan.path
    return x, p, out.float().cpu().numpy().astype(np.float64), used, ms


CASES = [
    (2, 16, 256, 2, "f32", "auto"),
    (1, 24, 1024, 3, "f32", "auto"),
    (2, 8, 4096, 2, "f32", "fourstep"),
    (2, 32, 2048, 2, "bf16", "auto"),
    (1, 16, 32768, 2, "f32", "auto"),
    (1, 64, 8192, 4, "bf16", "auto"),
    # bf16 with D a multiple of 64: the fused matrix-core in_proj + short conv
    (3, 64, 1024, 2, "bf16", "auto"),      # five 252-step tiles per sequence, the last one partial
    (3, 128, 128, 2, "bf16", "auto"),      # out_proj: one time tile per sequence, half of it past L
    (2, 320, 512, 3, "bf16", "auto"),      # C = 1280: five full channel tiles
    (1, 192, 65536, 2, "bf16", "auto"),    # C = 576: a partial channel tile; four-step path
    # hipBLASLt in_proj with b_in as one more inner-dimension term: widths whose padded
    # inner dimension (D + 1 rounded up to 8) holds zeros after the bias term
    (2, 5, 512, 2, "f32", "auto"),         # inner dimension 8: five values, the bias term, two zeros
    (1, 12, 1024, 3, "bf16", "auto"),      # inner dimension 16 (bf16 below the matrix-core width)
]


@pytest.mark.parametrize("B,D,L,order,dtype,path", CASES)
def test_operator_parity(B, D, L, order, dtype, path):
    wl = synth.custom(B, D, L, order, dtype, seed=D + order)
    say(f"[operator] {wl.describe()} path={path}")
    x, p, got, used, _ = _run(wl, path)
    ref = oracle.operator_forward(p.x, p.w_in, p.b_in, x.short_w, x.h, x.bias, p.w_out, p.b_out, order)
    err = oracle.rel_l2(got, ref)
    bound = 1e-2 if dtype == "bf16" else 1e-4
    say(f"   path={used} rel_l2={err:.3e} (bound {bound:.0e})")
    assert np.all(np.isfinite(got)) and err <= bound


def test_operator_lm125m_width_one_sequence():
    """The lm125m operator shape (D = 768, L = 8192, bf16) for one sequence, in full."""
    base = synth.WORKLOADS["lm125m"]
    wl = synth.custom(1, base.D, base.L, base.order, base.dtype, kind=base.kind, seed=base.seed)
    x, p, got, used, ms = _run(wl, timed=True)
    ref = oracle.operator_forward(p.x, p.w_in, p.b_in, x.short_w, x.h, x.bias, p.w_out, p.b_out, wl.order)
    err = oracle.rel_l2(got, ref)
    say(f"[operator] lm125m width, B=1: rel_l2={err:.3e}, stage ms {ms}")
    assert err <= 1e-2
    assert ms["total"] > 0 and ms["in_proj"] > 0 and ms["path"] > 0 and ms["out_proj"] > 0


def test_operator_reuses_state_across_batch_sizes():
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    for B in (2, 1, 3):
        wl = synth.custom(B, 8, 512, 2, seed=B)
        x, p, got, _, _ = _run(wl)
        ref = oracle.operator_forward(p.x, p.w_in, p.b_in, x.short_w, x.h, x.bias, p.w_out, p.b_out, 2)
        assert oracle.rel_l2(got, ref) <= 1e-4
    # one plan, two batch sizes in a row (descriptors rebuilt in between)
    wl = synth.custom(3, 8, 512, 2, seed=11)
    x = synth.generate(wl)
    p = synth.operator_params(wl)
    dev = torch.device("cuda", 0)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    with Plan(512, 8, 2, "f32") as plan:
        spec = plan.spectrum(f(x.h))
        for B in (3, 1):
            out = plan.operator_forward(f(p.x[:B]), f(p.w_in), f(p.b_in), f(x.short_w), spec, f(x.bias),
                                        f(p.w_out), f(p.b_out))
            ref = oracle.operator_forward(p.x[:B], p.w_in, p.b_in, x.short_w, x.h, x.bias, p.w_out, p.b_out, 2)
            assert oracle.rel_l2(out.cpu().numpy(), ref) <= 1e-4


def test_operator_fused_inproj_every_time_step():
    """Per time step over all sequences and channels: the fused in_proj writes tiles of
    254 steps that each recompute two steps of history, so a wrong seam would show
    in single time steps that a global norm hides."""
    wl = synth.custom(2, 128, 2048, 2, "bf16", seed=5)
    x, p, got, used, _ = _run(wl)
    ref = oracle.operator_forward(p.x, p.w_in, p.b_in, x.short_w, x.h, x.bias, p.w_out, p.b_out, 2)
    per_t = np.linalg.norm(got - ref, axis=(0, 2)) / np.linalg.norm(ref, axis=(0, 2))
    say(f"[operator] fused in_proj: worst time step rel_l2 {per_t.max():.3e} at t={int(per_t.argmax())}")
    assert per_t.max() <= 2e-2
    assert oracle.rel_l2(got, ref) <= 1e-2


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 16)])
def test_operator_tune_keeps_results(dtype, D):
    """hyena_operator_tune picks among hipBLASLt's candidates; the results stay within
    the parity bound afterwards."""
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = synth.custom(2, D, 1024, 2, dtype, seed=9)
    x = synth.generate(wl)
    p = synth.operator_params(wl)
    io = torch.bfloat16 if dtype == "bf16" else torch.float32
    dv = lambda a, dt=io: torch.from_numpy(a).cuda().to(dt).contiguous()  # noqa: E731
    with Plan(wl.L, wl.D, 2, dtype) as plan:
        spec = plan.spectrum(dv(x.h, torch.float32))
        args = (dv(p.x), dv(p.w_in), dv(p.b_in), dv(x.short_w, torch.float32), spec, dv(x.bias, torch.float32),
                dv(p.w_out), dv(p.b_out))
        plan.operator_tune(*args)
        out = plan.operator_forward(*args)
        torch.cuda.synchronize()
    ref = oracle.operator_forward(p.x, p.w_in, p.b_in, x.short_w, x.h, x.bias, p.w_out, p.b_out, 2)
    err = oracle.rel_l2(out.float().cpu().numpy().astype(np.float64), ref)
    say(f"[operator] after tuning ({dtype}): rel_l2={err:.3e}")
    assert err <= (1e-2 if dtype == "bf16" else 1e-4)
