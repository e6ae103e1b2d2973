"""GPU parity of the backward (hyena_backward, both paths) against the fp64 oracle.

Every gradient (du_proj, dshort_w, dh, dbias) is compared with the oracle's by
relative L2: 1e-4 when u_proj/dy/du are fp32, and for bf16 I/O 1e-2 on du_proj
(rounded to bf16 on output) and 1e-4 on the fp32 parameter gradients, which the
kernel sums in fp32 from the same bf16 input values the oracle receives.
"""
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


def _run_backward(x, dy, repeat=1, path="lds"):
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = x.wl
    t = to_device(x)
    dev = t["u"].device
    g = torch.from_numpy(dy).to(dev)
    if wl.dtype == "bf16":
        g = g.to(torch.bfloat16)
    outs = []
    with Plan(wl.L, wl.D, wl.order, wl.dtype, path) as p:
        spec = p.spectrum(t["h"])
        for _ in range(repeat):
            outs.append(p.backward(t["u"], t["w"], spec, t["bias"], g.contiguous()))
        torch.cuda.synchronize()
    return outs


def _compare(x, dy, label, mode="fft", path="lds"):
    wl = x.wl
    say(f"[backward] {label}: {wl.describe()} path={path}")
    (du, dw, dh, db), = _run_backward(x, dy, path=path)
    ref = oracle.backward(x.u_proj, x.short_w, x.h, x.bias, dy, wl.order, mode=mode)
    got = [a.float().cpu().numpy().astype(np.float64) for a in (du, dw, dh, db)]
    bounds = [1e-2 if wl.dtype == "bf16" else 1e-4, 1e-4, 1e-4, 1e-4]
    for name, g, r, bound in zip(("du_proj", "dshort_w", "dh", "dbias"), got, ref, bounds):
        assert np.all(np.isfinite(g)), f"{name}: non-finite values"
        err = oracle.rel_l2(g, r)
        say(f"   {name:9s} rel_l2={err:.3e} (bound {bound:.0e})")
        assert err <= bound, f"{name}: rel L2 {err:.3e} exceeds {bound:.0e}"
    # per-channel check of du: a wrong channel hides easily in a global norm
    g2 = got[0].reshape(-1, wl.L)
    r2 = ref[0].reshape(-1, wl.L)
    row = np.linalg.norm(g2 - r2, axis=1) / np.maximum(np.linalg.norm(r2, axis=1), 1e-30)
    assert row.max() <= 10 * bounds[0], f"worst du row rel L2 {row.max():.3e}"


SMALL = [
    # B, D, L, order, dtype: every LDS size class, E = 16 and 32, orders 2..8, ragged D
    (1, 1, 16, 2, "f32"),
    (2, 3, 32, 3, "f32"),
    (3, 5, 64, 2, "f32"),
    (2, 4, 256, 4, "f32"),
    (2, 7, 1024, 2, "f32"),
    (1, 3, 2048, 5, "f32"),
    (2, 4, 4096, 2, "f32"),
    (2, 3, 8192, 2, "f32"),
    (2, 2, 16384, 2, "f32"),
    (1, 2, 16384, 3, "f32"),
    (2, 2, 512, 8, "f32"),
    (2, 5, 1024, 2, "bf16"),
    (2, 3, 8192, 3, "bf16"),
]


@pytest.mark.parametrize("B,D,L,order,dtype", SMALL)
def test_backward_small_shapes(B, D, L, order, dtype):
    wl = synth.custom(B, D, L, order, dtype, seed=B * 1000 + D * 10 + order)
    x = synth.generate(wl)
    _compare(x, synth.upstream_grad(wl), f"small {B}x{D}x{L} N={order} {dtype}",
             mode="direct" if L <= 256 else "fft")


@pytest.mark.parametrize("name,nch", [("lm125m", 3), ("dna_small", 3), ("tiny", 64)])
def test_backward_workload_channels(name, nch):
    """Full-size rows of a workload (every b, all of L) on sampled channels: channels
    are independent, so the oracle runs on the channel subset while the GPU runs the
    subset too at the workload's B, L and dtype."""
    wl = synth.WORKLOADS[name]
    x = synth.generate(wl)
    ds = np.unique(np.r_[0, wl.D - 1, np.random.default_rng(5).choice(wl.D, size=max(nch - 2, 0), replace=False)])
    xs = synth.channel_subset(x, ds[:nch])
    dy = synth.upstream_grad(xs.wl)
    _compare(xs, dy, f"{name} channels {list(ds[:nch])}")


FOURSTEP = [
    # the four-step path: the smallest split, ragged D, bf16, the default four-step
    # sizes (32768, 65536), the largest split; orders 2, 3, 4 and 8
    (2, 3, 256, 2, "f32"),
    (2, 3, 256, 3, "f32"),
    (1, 5, 4096, 2, "f32"),
    (2, 3, 1024, 4, "f32"),
    (1, 2, 512, 8, "f32"),
    (3, 2, 8192, 2, "bf16"),
    (2, 2, 8192, 3, "bf16"),
    (2, 2, 32768, 2, "f32"),
    (1, 2, 32768, 3, "f32"),
    (1, 2, 65536, 2, "bf16"),
    (1, 1, 1 << 20, 2, "f32"),
    (1, 1, 1 << 18, 3, "f32"),
]


@pytest.mark.parametrize("B,D,L,order,dtype", FOURSTEP)
def test_backward_fourstep_shapes(B, D, L, order, dtype):
    wl = synth.custom(B, D, L, order, dtype, seed=B * 100 + D + L % 97 + order)
    x = synth.generate(wl)
    _compare(x, synth.upstream_grad(wl), f"four-step {B}x{D}x{L} N={order} {dtype}",
             mode="direct" if L <= 512 else "fft", path="fourstep")


@pytest.mark.parametrize("name", ["long64k", "long64k_o3"])
def test_backward_fourstep_workload_channels(name):
    """long64k at orders 2 and 3 on sampled channels: all of L."""
    wl = synth.WORKLOADS[name]
    x = synth.generate(wl)
    xs = synth.channel_subset(x, [0, 383, wl.D - 1])
    _compare(xs, synth.upstream_grad(xs.wl), f"{name} channels [0, 383, 767]", path="fourstep")


@pytest.mark.parametrize("order", [2, 3])
def test_backward_fourstep_is_deterministic(order):
    wl = synth.custom(2, 3, 1024, order, seed=8)
    x = synth.generate(wl)
    dy = synth.upstream_grad(wl)
    a, b = _run_backward(x, dy, repeat=2, path="fourstep")
    for ta, tb in zip(a, b):
        assert bool((ta == tb).all()), "two backward calls differ"


def test_backward_is_deterministic():
    wl = synth.custom(3, 6, 4096, 3, seed=21)
    x = synth.generate(wl)
    dy = synth.upstream_grad(wl)
    a, b = _run_backward(x, dy, repeat=2)
    for ta, tb in zip(a, b):
        assert bool((ta == tb).all()), "two backward calls differ"


def test_backward_zero_upstream_gives_zero():
    wl = synth.custom(2, 4, 2048, 2, seed=3)
    x = synth.generate(wl)
    (du, dw, dh, db), = _run_backward(x, np.zeros((wl.B, wl.D, wl.L), np.float32))
    for t in (du, dw, dh, db):
        assert float(t.abs().max()) == 0.0


def test_backward_rejects_small_workspaces():
    import torch

    from fft_long_convolution_libhyena_amd import HyenaError, Plan

    wl = synth.custom(1, 2, 1024, 2, seed=4)
    x = synth.generate(wl)
    t = to_device(x)
    g = torch.zeros((1, 2, 1024), dtype=torch.float32, device=t["u"].device)
    with Plan(1024, 2, 2, "f32", "fourstep") as p:
        spec = p.spectrum(t["h"])
        with pytest.raises(HyenaError) as e:
            p.backward(t["u"], t["w"], spec, t["bias"], g, workspace=torch.empty(16, dtype=torch.uint8,
                                                                             device=g.device))
        assert e.value.status == 3  # HYENA_ERR_WORKSPACE
    with Plan(1024, 2, 2, "f32", "lds") as p:
        spec = p.spectrum(t["h"])
        small = torch.empty(p.backward_workspace_bytes(1) - 256, dtype=torch.uint8, device=g.device)
        with pytest.raises(HyenaError) as e:
            p.backward(t["u"], t["w"], spec, t["bias"], g, workspace=small)
        assert e.value.status == 3  # HYENA_ERR_WORKSPACE


def _run_backward_per_sample(x, hb, dy, path):
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = x.wl
    t = to_device(x)
    g = torch.from_numpy(dy).to(t["u"].device)
    if wl.dtype == "bf16":
        g = g.to(torch.bfloat16)
    with Plan(wl.L, wl.D, wl.order, wl.dtype, path) as p:
        spec = p.spectrum_batched(torch.from_numpy(hb).to(g.device))
        out = p.backward_per_sample(t["u"], t["w"], spec, t["bias"], g.contiguous())
        torch.cuda.synchronize()
    return out


PER_SAMPLE = [
    # B, D, L, order, dtype, path: both paths, orders 2..4, ragged D, bf16 I/O
    (3, 3, 256, 2, "f32", "lds"),
    (3, 3, 1024, 2, "f32", "lds"),
    (2, 5, 4096, 3, "f32", "lds"),
    (2, 3, 8192, 3, "bf16", "lds"),
    (2, 2, 16384, 4, "f32", "lds"),
    (3, 3, 256, 2, "f32", "fourstep"),
    (3, 3, 1024, 3, "f32", "fourstep"),
    (2, 3, 8192, 4, "bf16", "fourstep"),
    (2, 2, 32768, 3, "f32", "fourstep"),
    (2, 1, 1 << 18, 2, "f32", "fourstep"),
]


@pytest.mark.parametrize("B,D,L,order,dtype,path", PER_SAMPLE)
def test_backward_per_sample_matches_oracle(B, D, L, order, dtype, path):
    """hyena_backward_per_sample against the oracle's per-sample backward: every
    gradient by relative L2, and each sample's filter gradient dh[b] on its own,
    since a sample reading another sample's spectrum would hide in the global norm."""
    wl = synth.custom(B, D, L, order, dtype, seed=B * 31 + D + L % 89 + order)
    x = synth.generate(wl)
    hb = synth.per_sample_filters(wl)
    dy = synth.upstream_grad(wl)
    say(f"[backward per-sample] {wl.describe()} path={path}")
    got = [a.float().cpu().numpy().astype(np.float64) for a in _run_backward_per_sample(x, hb, dy, path)]
    ref = oracle.backward_per_sample(x.u_proj, x.short_w, hb, x.bias, dy, order,
                                     mode="direct" if L <= 256 else "fft")
    bounds = [1e-2 if dtype == "bf16" else 1e-4, 1e-4, 1e-4, 1e-4]
    for name, g, r, bound in zip(("du_proj", "dshort_w", "dh", "dbias"), got, ref, bounds):
        assert np.all(np.isfinite(g)), f"{name}: non-finite values"
        err = oracle.rel_l2(g, r)
        say(f"   {name:9s} rel_l2={err:.3e} (bound {bound:.0e})")
        assert err <= bound, f"{name}: rel L2 {err:.3e} exceeds {bound:.0e}"
    per = [oracle.rel_l2(got[2][b], ref[2][b]) for b in range(B)]
    say(f"   dh per sample {', '.join(f'{e:.2e}' for e in per)}")
    assert max(per) <= 1e-4


@pytest.mark.parametrize("path,L,order", [("lds", 2048, 3), ("fourstep", 4096, 3), ("fourstep", 1024, 2)])
def test_backward_per_sample_equal_sets_match_shared(path, L, order):
    """With every sample given the shared filters, du_proj and dshort_w are the shared
    backward's bit for bit (the same arithmetic on the same spectra), the per-sample
    filter gradients sum to the shared one, and dbias agrees to rounding."""
    import torch

    wl = synth.custom(3, 4, L, order, seed=77 + order)
    x = synth.generate(wl)
    dy = synth.upstream_grad(wl)
    same = np.ascontiguousarray(np.repeat(x.h[None], wl.B, axis=0))
    du, dw, dh, db = _run_backward_per_sample(x, same, dy, path)
    (du0, dw0, dh0, db0), = _run_backward(x, dy, path=path)
    assert bool((du == du0).all()) and bool((dw == dw0).all())
    e_dh = oracle.rel_l2(dh.double().sum(0).cpu().numpy(), dh0.double().cpu().numpy())
    e_db = oracle.rel_l2(db.double().cpu().numpy(), db0.double().cpu().numpy())
    say(f"[backward per-sample] equal sets, {path} L={L} N={order}: sum dh vs shared {e_dh:.2e}, dbias {e_db:.2e}")
    assert e_dh <= 1e-5 and e_db <= 1e-5
    torch.cuda.synchronize()


def test_backward_per_sample_workspace_and_errors():
    import torch

    from fft_long_convolution_libhyena_amd import HyenaError, Plan

    wl = synth.custom(2, 2, 1024, 2, seed=6)
    x = synth.generate(wl)
    t = to_device(x)
    g = torch.zeros((2, 2, 1024), dtype=torch.float32, device=t["u"].device)
    hb = torch.from_numpy(synth.per_sample_filters(wl)).to(g.device)
    with Plan(1024, 2, 2, "f32", "fourstep") as p:
        assert p.backward_workspace_bytes(2, per_sample=True) > p.backward_workspace_bytes(2)
        spec = p.spectrum_batched(hb)
        small = torch.empty(p.backward_workspace_bytes(2), dtype=torch.uint8, device=g.device)
        with pytest.raises(HyenaError) as e:  # the shared backward's workspace is too small here
            p.backward_per_sample(t["u"], t["w"], spec, t["bias"], g, workspace=small)
        assert e.value.status == 3
        with pytest.raises(ValueError):  # one spectrum where two are needed
            p.backward_per_sample(t["u"], t["w"], p.spectrum(t["h"]), t["bias"], g)
    with Plan(1024, 2, 2, "f32", "lds") as p:
        assert p.backward_workspace_bytes(2, per_sample=True) == p.backward_workspace_bytes(2)
        du, dw, dh, db = p.backward_per_sample(t["u"], t["w"], p.spectrum_batched(hb), t["bias"], g)
        torch.cuda.synchronize()
        assert tuple(dh.shape) == (2, 1, 2, 1024)
        for a in (du, dw, dh, db):
            assert float(a.abs().max()) == 0.0


@pytest.mark.parametrize("name", ["lm125m", "long64k"])
def test_backward_full_workload_sampled_channels(name):
    """The whole workload through hyena_backward in the launch configuration the
    benchmark times (all B*D rows, the default workspace); the oracle runs on three
    sampled channels, whose gradients (every channel group of du_proj, their taps,
    filters and biases) depend on those channels alone."""
    wl = synth.WORKLOADS[name]
    x = synth.generate(wl)
    dy = synth.upstream_grad(wl)
    say(f"[backward] full {name}: {wl.describe()}")
    (du, dw, dh, db), = _run_backward(x, dy, path="auto")
    N, D, L = wl.order, wl.D, wl.L
    ds = [0, D // 2 + 1, D - 1]
    xs = synth.channel_subset(x, ds)
    ref = oracle.backward(xs.u_proj, xs.short_w, xs.h, xs.bias, np.ascontiguousarray(dy[:, ds]), N)
    idx = [i * D + d for i in range(N + 1) for d in ds]
    got = [du.float().cpu().numpy()[:, idx].astype(np.float64), dw.cpu().numpy()[idx].astype(np.float64),
           dh.cpu().numpy()[:, ds].astype(np.float64), db.cpu().numpy()[:, ds].astype(np.float64)]
    bounds = [1e-2 if wl.dtype == "bf16" else 1e-4, 1e-4, 1e-4, 1e-4]
    for nm, g, r, bound in zip(("du_proj", "dshort_w", "dh", "dbias"), got, ref, bounds):
        err = oracle.rel_l2(g, r)
        say(f"   {nm:9s} rel_l2={err:.3e} (bound {bound:.0e})")
        assert np.all(np.isfinite(g)) and err <= bound, (nm, err)
