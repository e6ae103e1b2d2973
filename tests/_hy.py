"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
library through its binding, and compare with the oracle."""
import sys

import numpy as np

from fft_long_convolution_libhyena_amd import synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(x: synth.Inputs):
    import torch

    dev = torch.device("cuda", 0)
    u = torch.from_numpy(x.u_proj).to(dev)
    if x.wl.dtype == "bf16":
        u = u.to(torch.bfloat16)  # exact: the values are already bf16
    return dict(u=u.contiguous(), w=torch.from_numpy(x.short_w).to(dev), h=torch.from_numpy(x.h).to(dev),
                bias=torch.from_numpy(x.bias).to(dev))


def run(x: synth.Inputs, path: str = "auto", repeat: int = 1):
    """Plan + spectrum + forward; returns (y as float64 numpy, plan path, list of y tensors)."""
    import torch

    from fft_long_convolution_libhyena_amd import Plan

    wl = x.wl
    t = to_device(x)
    outs = []
    with Plan(wl.L, wl.D, wl.order, wl.dtype, path) as p:
        spec = p.spectrum(t["h"])
        for _ in range(repeat):
            outs.append(p.forward(t["u"], t["w"], spec, t["bias"]))
        torch.cuda.synchronize()
        path_used = p.path
    y = outs[0].float().cpu().numpy().astype(np.float64)
    return y, path_used, outs


def tol(wl) -> float:
    # relative L2 bound of the parity contract: 1e-4 for fp32 I/O, 1e-2 for bf16 I/O
    return 1e-2 if wl.dtype == "bf16" else 1e-4
