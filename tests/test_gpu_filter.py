"""GPU parity of the implicit filter generator (hyena_implicit_filter) against the
fp64 oracle, and of the chain filter -> spectrum -> forward.

The bound is the fp32 contract's relative L2 of 1e-4 over each filter tensor, with
every channel row within 10x of it; the kernel's arithmetic (positional features
rounded once from fp64, an fp32 Linear/Sin stack of at most a few dozen terms per
sum, fp32 exp) stays near 1e-7.
"""
import types

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


def _device_mlp(p):
    import torch

    return types.SimpleNamespace(**{k: torch.from_numpy(np.ascontiguousarray(v, np.float32)).cuda()
                                    for k, v in vars(p).items()})


def _gpu_filter(wl, p, repeat=1):
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    dp = _device_mlp(p)
    with Plan(wl.L, wl.D, wl.order, "f32") as plan:
        outs = [plan.implicit_filter(dp) for _ in range(repeat)]
        torch.cuda.synchronize()
    return outs


def _compare(got, ref, label):
    err = oracle.rel_l2(got, ref)
    rows = got.reshape(-1, got.shape[-1])
    rrows = ref.reshape(-1, ref.shape[-1])
    row = np.linalg.norm(rows - rrows, axis=1) / np.maximum(np.linalg.norm(rrows, axis=1), 1e-300)
    say(f"[filter] {label}: rel_l2={err:.3e} worst row {row.max():.3e}")
    assert np.all(np.isfinite(got))
    assert err <= 1e-4
    assert row.max() <= 1e-3


CASES = [
    # L, D, order, emb_dim, width, num_inner, Sin frequency
    (16, 3, 2, 3, 8, 0, 1.0),       # L below one 64-step tile
    (256, 5, 3, 5, 16, 2, 1.0),
    (1024, 64, 2, 3, 16, 2, 1.0),   # the tiny workload's plan
    (2048, 24, 3, 7, 64, 3, 0.5),
    (4096, 7, 4, 9, 32, 1, 2.0),
    (8192, 768, 2, 3, 16, 2, 1.0),  # the lm125m plan
]


@pytest.mark.parametrize("L,D,order,E,W,M,w", CASES)
def test_filter_matches_oracle(L, D, order, E, W, M, w):
    wl = synth.custom(1, D, L, order, seed=L + D)
    p = synth.filter_mlp(wl, emb_dim=E, width=W, num_inner=M, w=w)
    got = _gpu_filter(wl, p)[0].cpu().numpy().astype(np.float64)
    _compare(got, oracle.implicit_filter(L, D, order, p), f"L={L} D={D} N={order} E={E} W={W} M={M} w={w}")


def test_filter_long64k_plan_in_full():
    wl = synth.WORKLOADS["long64k"]
    p = synth.filter_mlp(wl)
    got = _gpu_filter(wl, p)[0].cpu().numpy().astype(np.float64)
    _compare(got, oracle.implicit_filter(wl.L, wl.D, wl.order, p), "long64k plan (D=768, L=65536)")


def test_filter_dna_1m_plan_sampled_channels():
    """L = 2^20 with a wide MLP; channels are independent, so the oracle runs on 12
    sampled rows of w_out / alpha."""
    wl = synth.WORKLOADS["dna_1m"]
    p = synth.filter_mlp(wl, emb_dim=5, width=64, num_inner=2)
    got = _gpu_filter(wl, p)[0].cpu().numpy().astype(np.float64).reshape(-1, wl.L)
    cs = np.unique(np.r_[0, wl.D - 1, np.random.default_rng(7).choice(wl.D, 10, replace=False)])
    sub = types.SimpleNamespace(**{**vars(p), "w_out": p.w_out[cs], "alpha": p.alpha[cs]})
    ref = oracle.implicit_filter(wl.L, len(cs), 2, sub).reshape(-1, wl.L)
    _compare(got[cs], ref, f"dna_1m plan, channels {list(cs)}")


@pytest.mark.parametrize("L,D,order,path", [(4096, 8, 3, "lds"), (65536, 4, 2, "fourstep")])
def test_filter_spectrum_forward_chain(L, D, order, path):
    """The generated filters feed hyena_filter_spectrum and hyena_forward unchanged:
    the output matches the forward oracle run on the oracle's filters."""
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = synth.custom(2, D, L, order, seed=5)
    x = synth.generate(wl)
    p = synth.filter_mlp(wl, emb_dim=5, width=32, num_inner=2)
    t = to_device(x)
    with Plan(L, D, order, "f32", path) as plan:
        h = plan.implicit_filter(_device_mlp(p))
        y = plan.forward(t["u"], t["w"], plan.spectrum(h), t["bias"])
        torch.cuda.synchronize()
        assert plan.path == path
    h_ref = oracle.implicit_filter(L, D, order, p)
    ref = oracle.forward(x.u_proj, x.short_w, h_ref.astype(np.float32), x.bias, order)
    err = oracle.rel_l2(y.cpu().numpy().astype(np.float64), ref)
    say(f"[filter] chain {path} L={L} D={D} N={order}: rel_l2={err:.3e}")
    assert err <= 1e-4


def test_filter_is_deterministic():
    wl = synth.custom(1, 40, 2048, 3, seed=9)
    a, b = _gpu_filter(wl, synth.filter_mlp(wl, emb_dim=7, width=32), repeat=2)
    assert bool((a == b).all())


def test_filter_error_paths():
    import torch

    from fft_long_convolution_libhyena_amd import HyenaError, Plan

    wl = synth.custom(1, 4, 1024, 2, seed=1)
    with Plan(1024, 4, 2, "f32") as plan:
        with pytest.raises(HyenaError) as e:  # width 12 is not built
            plan.implicit_filter(_device_mlp(synth.filter_mlp(wl, width=12)))
        assert e.value.status == 2
        p = _device_mlp(synth.filter_mlp(wl, num_inner=0))
        with pytest.raises(ValueError):  # w_out rows must be (N-1)*D
            plan.implicit_filter(types.SimpleNamespace(**{**vars(p), "w_out": p.w_out[:3].contiguous()}))
        with pytest.raises(ValueError):
            plan.implicit_filter(p, out=torch.empty((1, 4, 512), device="cuda"))
