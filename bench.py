#!/usr/bin/env python3
"""Throughput of the Hyena operator forward hot path (libhyena) on one MI355X.

One step = one hyena_forward over one batch of a workload: short conv + split,
the order-N gated chain of FFT long convolutions with bias skip, and the final
gate, all in libhyena's HIP kernels; inputs and the filter spectrum are
resident in HBM before timing starts (the spectrum is made once per plan and
timed separately).

Prints ONE JSON line:
  value            channel-tokens/s = B*D*L / t_step
  roofline         the dominant kernel against the 8 TB/s HBM peak (algorithmic bytes)
  cpu_baseline     the fp64 oracle on the host cores, over a bounded sample of rows
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "channel-tokens/s (B·D·L/s) and % HBM peak, Hyena op fwd at L=64K order 2"
HBM_PEAK_GBS = 8000.0
VALU_F32_PEAK_TFLOPS = 157.3  # published: 256 CUs x 128 fp32 lanes/clk (packed) x 2 (FMA) x 2.4 GHz
# The kernels are built without packed fp32 instructions, so the vector rate they
# can reach is half the published one: 256 CUs x 64 fp32 lanes/clk x 2 (FMA) x 2.4 GHz.
VALU_F32_UNPACKED_TFLOPS = 78.6
# flop per byte above which a kernel is priced against the vector-ALU roof instead of HBM
RIDGE_FLOP_PER_BYTE = VALU_F32_UNPACKED_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
# rows per chunk of the pipelined four-step forward (mirrors the library's rule)
PIPE_ROWS, PIPE_MIN_ROWS = 128, 32


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def io_bytes(wl) -> int:
    return 2 if wl.dtype == "bf16" else 4


def alg_bytes_forward(wl) -> int:
    """One read of u_proj, one write of y, one read of the fp32 filter spectrum
    (bins 0..L of each (o, d)) and of the small parameters."""
    s = io_bytes(wl)
    B, D, L, N = wl.B, wl.D, wl.L, wl.order
    return (s * B * (N + 1) * D * L + s * B * D * L + 8 * (N - 1) * D * (L + 1)
            + 4 * (N + 1) * D * 3 + 4 * (N - 1) * D)


def alg_flops_forward(wl) -> float:
    """Algorithmic flops of one forward: per (b, d) and step a real forward and a real
    inverse FFT of size 2L at 2.5 n log2 n each, the complex product (6 per bin) and
    the bias skip (2 per point); per (b, d) the gates (N per point) and the width-3
    conv of the N+1 channels (5 per point)."""
    B, D, L, N = wl.B, wl.D, wl.L, wl.order
    per_step = 10.0 * L * math.log2(2 * L) + 6.0 * (L + 1) + 2.0 * L
    return B * D * ((N - 1) * per_step + N * L + 5.0 * (N + 1) * L)


def roofline(kernel: str, launches: int, launch_ms: float, bytes_per_launch: float, flops_per_launch: float,
             traffic=None, step_traffic=None, step_alg_bytes=None) -> dict:
    """The roofline object of one kernel: HBM-bound (algorithmic bytes per launch
    against 8 TB/s) when its algorithmic intensity is at or below the ridge of the
    unpacked fp32 vector rate and HBM, else ALU-bound (algorithmic flops against
    78.6 TFLOP/s). `traffic` is the measured HBM bytes per launch and
    `step_traffic` per step, both from committed counter summaries, or None."""
    sec = launch_ms * 1e-3
    intensity = flops_per_launch / bytes_per_launch
    if intensity > RIDGE_FLOP_PER_BYTE:
        achieved, peak, unit, bound = flops_per_launch / sec / 1e12, VALU_F32_UNPACKED_TFLOPS, "TFLOP/s", "alu"
    else:
        achieved, peak, unit, bound = bytes_per_launch / sec / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    out = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
           "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel,
           "alg_bytes_per_launch": int(bytes_per_launch), "alg_flops_per_launch": int(flops_per_launch),
           "flop_per_byte": round(intensity, 2), "ridge_flop_per_byte": round(RIDGE_FLOP_PER_BYTE, 2),
           "launch_ms": round(launch_ms, 5), "launches_per_step": launches,
           "step_traffic": step_traffic}
    if step_traffic is not None and step_alg_bytes:
        out["step_traffic_over_alg"] = round(step_traffic / step_alg_bytes, 3)
    return out


def pipe_chunk_rows(rows: int, ws_bytes: int, tile_bytes: int) -> int:
    """Rows per chunk of a pipelined order-2 four-step forward with this workspace
    (three tile slots), or 0 when the library runs the chunks one by one."""
    R = min(PIPE_ROWS, ws_bytes // (3 * tile_bytes), rows)
    return R if R >= min(rows, PIPE_MIN_ROWS) else 0


def device_copy_gbs(torch, dev, nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Bandwidth of a plain device-to-device copy of nbytes (read + write counted),
    the median of reps copies timed with HIP events: the practical HBM ceiling."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        ev0.record()
        b.copy_(a)
        ev1.record()
        torch.cuda.synchronize()
        ts.append(ev0.elapsed_time(ev1))
    del a, b
    return 2 * nbytes / (float(np.median(ts)) * 1e-3) / 1e9


def alg_bytes_backward(wl) -> int:
    """One read of u_proj, dy, the filter spectrum and the small parameters; one
    write of du_proj, dh, dbias and dshort_w."""
    s = io_bytes(wl)
    B, D, L, N = wl.B, wl.D, wl.L, wl.order
    return (2 * s * B * (N + 1) * D * L + s * B * D * L + 8 * (N - 1) * D * (L + 1) + 4 * (N - 1) * D * L
            + 2 * (4 * (N + 1) * D * 3 + 4 * (N - 1) * D))


def alg_bytes_pass(wl, family: str) -> int:
    """Bytes each four-step pass must move by design, per forward (all rows):
    pass A reads two u_proj rows and writes the L-point complex tile; pass B
    reads the tile and the spectrum and writes the tile; pass C reads the tile
    and, for the last step, one gate row and writes y (earlier steps also read
    the next gate row and write the tile again)."""
    s = io_bytes(wl)
    B, D, L, N = wl.B, wl.D, wl.L, wl.order
    rows = B * D
    tile = 8 * L
    if family == "pass_a":
        return rows * (2 * s * L + tile)
    if family == "pass_b":
        return (N - 1) * (rows * (2 * tile) + 8 * D * L)
    if family == "pass_c":
        return (N - 1) * rows * (tile + s * L) + rows * s * L + (N - 2) * rows * tile
    raise ValueError(family)


def alg_bytes_part(wl, family: str) -> int:
    """Bytes each pass of the partitioned path must move by design, per forward
    (all rows): pass 1 reads the step's input (two u_proj rows at the first step,
    the previous step's fp32 output after it) and writes the window spectra (8L
    per row); pass 2 reads the window spectra, the filter block spectra (8L per
    channel and step) and one gate row, and writes y (last step) or the fp32
    input of the next step."""
    s = io_bytes(wl)
    B, D, L, N = wl.B, wl.D, wl.L, wl.order
    rows = B * D
    if family == "pass_1":
        return rows * (2 * s * L + 8 * L) + (N - 2) * rows * (4 * L + 8 * L)
    if family == "pass_2":
        return (N - 1) * (rows * (8 * L + s * L) + 8 * D * L) + rows * s * L + (N - 2) * rows * 4 * L
    raise ValueError(family)


# the sources each kernel family is compiled from, including the host code that
# sizes its launches (chunking, grids)
_CSRC = os.path.join(ROOT, "fft_long_convolution_libhyena_amd", "csrc")
KERNEL_SOURCES = {
    "lds": ["fft_core.hpp", "pair.hpp", "kernels.hpp", "plan.hpp", "lds_path.hpp", "lds_path_a.hip",
            "lds_path_b.hip", "lds_path_c.hip", "lds_path_d.hip", "hyena_api.hip"],
    "fourstep": ["fft_core.hpp", "pair.hpp", "kernels.hpp", "plan.hpp", "fourstep.hpp", "fourstep.hip",
                 "hyena_api.hip"],
    "backward": ["fft_core.hpp", "pair.hpp", "kernels.hpp", "plan.hpp", "backward.hpp", "lds_backward.hpp",
                 "lds_backward_a.hip", "lds_backward_b.hip", "lds_backward_c.hip", "lds_backward_d.hip",
                 "lds_backward_e.hip", "lds_backward_f.hip", "hyena_backward.hip"],
    "fs_backward": ["fft_core.hpp", "pair.hpp", "kernels.hpp", "plan.hpp", "backward.hpp", "fourstep.hpp",
                    "fourstep_backward.hip", "hyena_backward.hip"],
    "filter": ["plan.hpp", "implicit_filter.hip"],
    "conv2d": ["fft_core.hpp", "pair.hpp", "fourstep.hpp", "kernels.hpp", "plan.hpp", "tables.hpp", "conv_nd.hpp",
               "conv2d.hip"],
    "conv3d": ["fft_core.hpp", "pair.hpp", "fourstep.hpp", "kernels.hpp", "plan.hpp", "tables.hpp", "conv_nd.hpp",
               "conv3d.hip"],
    "partitioned": ["fft_core.hpp", "pair.hpp", "kernels.hpp", "plan.hpp", "partitioned.hip", "hyena_api.hip"],
    "operator": ["kernels.hpp", "inproj.hip", "outproj.hpp", "outproj.hip", "hyena_operator.hip"],
    "synthesis": ["plan.hpp", "kernel_synthesis.hip"],
}


def kernel_family(kernel: str) -> str:
    if kernel.startswith(("k_inproj", "k_outproj", "operator")):
        return "operator"
    if kernel.startswith("k_kernel_synthesis"):
        return "synthesis"
    if kernel.startswith("k_implicit_filter"):
        return "filter"
    if kernel.startswith("k_c3"):
        return "conv3d"
    if kernel.startswith("k_c2"):
        return "conv2d"
    if kernel.startswith("fs_backward"):
        return "fs_backward"
    if kernel.startswith("k_lds_bwd"):
        return "backward"
    if kernel.startswith("k_part"):
        return "partitioned"
    return "lds" if kernel.startswith("k_lds") else "fourstep"


def kernel_sources_hash(kernel: str) -> str:
    """Hash of the sources `kernel` is built from; counter summaries record it."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel_family(kernel)]:
        with open(os.path.join(_CSRC, name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, already scaled by the copy calibration), or None when
    there is no summary or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("sources_sha256") != kernel_sources_hash(kernel):
        return None
    try:
        return int(float(kv["fetch_bytes_per_dispatch"]) + float(kv["write_bytes_per_dispatch"]))
    except (KeyError, ValueError):
        return None


def measured_step_traffic(kernel: str, workload: str):
    """HBM bytes of one whole forward (every kernel it launches) from the committed
    counter summary of `kernel`, or None (see measured_traffic)."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.txt")
    if measured_traffic(kernel, workload) is None:
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("step_bytes:"):
                return int(float(line.split(":", 1)[1]))
    return None


def cpu_baseline(x, wl, budget_s: float):
    """The oracle (fp64 FFT mode) on a bounded, seeded sample of (b, d) rows."""
    import oracle
    from fft_long_convolution_libhyena_amd import synth

    threads = oracle.max_threads()
    n = max(1, min(wl.B * wl.D, 2 * threads))
    rows = synth.sample_rows(wl, n, seed=99)
    t0 = time.perf_counter()
    oracle.forward(x.u_proj, x.short_w, x.h, x.bias, wl.order, mode="fft", rows=rows)
    dt = time.perf_counter() - t0
    if dt < budget_s / 4 and n < wl.B * wl.D:
        n = int(min(wl.B * wl.D, max(n + 1, n * budget_s / max(dt, 1e-3) * 0.8)))
        rows = synth.sample_rows(wl, n, seed=99)
        t0 = time.perf_counter()
        oracle.forward(x.u_proj, x.short_w, x.h, x.bias, wl.order, mode="fft", rows=rows)
        dt = time.perf_counter() - t0
    res = {"value": len(rows) * wl.L / dt, "unit": "channel-tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{len(rows)} of {wl.B * wl.D} (b,d) rows of the same inputs, fp64 radix-2 FFT "
                     f"convolution, OpenMP over rows, {dt:.1f} s wall"}
    if wl.L <= 1024:
        # small enough for the O(L^2) definition itself: timed on the whole input as well
        t0 = time.perf_counter()
        oracle.forward(x.u_proj, x.short_w, x.h, x.bias, wl.order, mode="direct")
        dd = time.perf_counter() - t0
        res["direct"] = {"value": wl.B * wl.D * wl.L / dd, "unit": "channel-tokens/s", "cores": threads,
                         "sample": f"all {wl.B * wl.D} rows, fp64 direct O(L^2) convolution, {dd:.2f} s wall"}
    return res


def cpu_baseline_backward(x, wl, budget_s: float, hb=None):
    """The fp64 backward oracle (FFT mode) on a bounded, seeded sample of channels
    (all b and t of each); channels are independent, so this is a smaller instance.
    With per-sample filters hb [B, N-1, D, L], the per-sample backward oracle."""
    import oracle
    from fft_long_convolution_libhyena_amd import synth

    threads = oracle.max_threads()
    rng = np.random.default_rng(99)
    n = max(1, min(wl.D, threads))
    while True:
        ds = np.sort(rng.choice(wl.D, size=n, replace=False))
        xs = synth.channel_subset(x, ds)
        dy = synth.upstream_grad(xs.wl)
        t0 = time.perf_counter()
        if hb is None:
            oracle.backward(xs.u_proj, xs.short_w, xs.h, xs.bias, dy, wl.order, mode="fft")
        else:
            oracle.backward_per_sample(xs.u_proj, xs.short_w, np.ascontiguousarray(hb[:, :, ds]), xs.bias, dy,
                                       wl.order, mode="fft")
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or n >= wl.D:
            break
        n = int(min(wl.D, max(n + 1, n * budget_s / max(dt, 1e-3) * 0.8)))
    return {"value": wl.B * n * wl.L / dt, "unit": "channel-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {wl.D} channels (all {wl.B} batch rows, all L) of the same inputs, fp64 radix-2 "
                      f"FFT backward{' with a filter set per sample' if hb is not None else ''}, OpenMP over "
                      f"channels, {dt:.1f} s wall"}


def bench_backward(args, wl, x, torch, Plan, per_sample=False):
    """hyena_backward, or with per_sample hyena_backward_per_sample (a filter set per
    sample: B spectra read, B filter gradients written); with --circular on a
    circular plan (circular correlations, L/2 + 1 spectrum bins per filter)."""
    from fft_long_convolution_libhyena_amd import synth

    circ = bool(getattr(args, "circular", False))
    dev = torch.device("cuda", 0)
    iot = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    u = torch.from_numpy(x.u_proj).to(dev).to(iot).contiguous()
    w = torch.from_numpy(x.short_w).to(dev)
    h = torch.from_numpy(x.h).to(dev)
    bias = torch.from_numpy(x.bias).to(dev)
    dy = torch.from_numpy(synth.upstream_grad(wl)).to(dev).to(iot).contiguous()
    plan = Plan(wl.L, wl.D, wl.order, wl.dtype, circular=circ)
    hb = synth.per_sample_filters(wl) if per_sample else None
    spec = plan.spectrum_batched(torch.from_numpy(hb).to(dev)) if per_sample else plan.spectrum(h)
    N, D, L, B = wl.order, wl.D, wl.L, wl.B
    ws = torch.empty(plan.backward_workspace_bytes(B, per_sample), dtype=torch.uint8, device=dev)
    outs = (torch.empty((B, (N + 1) * D, L), dtype=iot, device=dev),
            torch.empty(((N + 1) * D, 3), dtype=torch.float32, device=dev),
            torch.empty(((B,) if per_sample else ()) + (N - 1, D, L), dtype=torch.float32, device=dev),
            torch.empty((N - 1, D), dtype=torch.float32, device=dev))
    log(f"[bench] backward workspace {ws.numel() / 2**20:.1f} MiB")

    def step():
        plan.backward(u, w, spec, bias, dy, *outs, workspace=ws, per_sample=per_sample)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for rep in range(args.reps):
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            step()
        ev1.record()
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / args.steps)
        log(f"[bench] rep {rep}: {times[-1] * 1e3:.1f} us/step")
    ms = float(np.median(times))
    nbytes = alg_bytes_backward(wl)
    spec_bins = L // 2 + 1 if circ else L + 1  # spectrum bins per filter
    if circ:
        nbytes -= 8 * (N - 1) * D * (L + 1 - spec_bins)
    if per_sample:  # B filter spectra read and B filter gradients written instead of one each
        nbytes += (B - 1) * (N - 1) * D * (8 * spec_bins + 4 * L)
    # the step's kernels taken together: k_lds_bwd_rows + k_lds_bwd_finish on the LDS
    # path, the launches of the four-step backward ("fs_backward") otherwise
    bk = "k_lds_bwd_rows" if plan.path == "lds" else "fs_backward"
    achieved = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "channel-tokens/s (B·D·L/s) and % HBM peak, Hyena op backward (gradients of u_proj, short_w, "
                  "h, bias)" + (" with a filter set per sample" if per_sample else "")
                  + (", circular plan" if circ else ""),
        "value": B * D * L / (ms * 1e-3), "unit": "channel-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if wl.dtype == "f32" else "bf16-io/f32",
        "data": f"synthetic seeded ({wl.kind} activations, N(0,1) upstream gradient"
                f"{', per-sample exponentially decaying random filters' if per_sample else ''})",
        "config": {"workload": wl.name, "B": B, "D": D, "L": L, "order": N, "io_dtype": wl.dtype,
                   "path": plan.path, "pass": ("backward_per_sample" if per_sample else "backward")
                   + ("_circular" if circ else "")},
        # the whole backward step (two launches on the LDS path, nine on the
        # four-step path) against its algorithmic bytes
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     # the whole step's HBM bytes (every launch of one backward step)
                     "traffic": measured_step_traffic(bk, wl.name + ("_per_sample" if per_sample else "")
                                                      + ("_circular" if circ else "")),
                     "kernel": bk,
                     "alg_bytes_per_launch": nbytes, "launch_ms": round(ms, 5), "launches_per_step": 1},
    }
    if args.check:
        import oracle

        ds = [0, D // 2, D - 1]
        xs = synth.channel_subset(x, ds)
        g = synth.upstream_grad(wl)[:, ds]
        if circ and per_sample:
            ref = oracle.backward_circular_per_sample(xs.u_proj, xs.short_w, np.ascontiguousarray(hb[:, :, ds]),
                                                      xs.bias, g, N)
        elif circ:
            ref = oracle.backward_circular(xs.u_proj, xs.short_w, xs.h, xs.bias, g, N)
        elif per_sample:
            ref = oracle.backward_per_sample(xs.u_proj, xs.short_w, np.ascontiguousarray(hb[:, :, ds]), xs.bias, g, N)
        else:
            ref = oracle.backward(xs.u_proj, xs.short_w, xs.h, xs.bias, g, N)
        got = outs[0].float().cpu().numpy().reshape(B, N + 1, D, L)[:, :, ds].reshape(B, -1, L)
        out["check_rel_l2_du"] = oracle.rel_l2(got, ref[0])
        out["check_rel_l2_dh"] = oracle.rel_l2(outs[2].double().cpu().numpy()[..., ds, :], ref[2])
        log(f"[bench] oracle check on channels {ds}: du rel_l2 {out['check_rel_l2_du']:.3e}, "
            f"dh rel_l2 {out['check_rel_l2_dh']:.3e}")
    if not args.no_cpu_baseline and not circ:
        log("[bench] cpu baseline (backward oracle) ...")
        out["cpu_baseline"] = cpu_baseline_backward(x, wl, args.cpu_budget, hb)
    print(json.dumps(out), flush=True)
    plan.close()


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def cpu_baseline_operator(x, p, wl, budget_s: float):
    """The fp64 operator oracle on the first L' tokens of every sequence (the path is
    causal, so those outputs need only those inputs), L' a power of two sized to
    about the time budget."""
    import oracle

    threads = oracle.max_threads()
    Lp = min(wl.L, 1024)
    while True:
        t0 = time.perf_counter()
        oracle.operator_forward(p.x[:, :Lp], p.w_in, p.b_in, x.short_w, x.h[:, :, :Lp], x.bias, p.w_out, p.b_out,
                                wl.order, mode="fft")
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or Lp >= wl.L:
            break
        Lp = min(wl.L, Lp * 2)
    return {"value": wl.B * Lp / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the first {Lp} of {wl.L} tokens of all {wl.B} sequences (causal: exact for those tokens), "
                      f"fp64 numpy projections + fp64 FFT path, {dt:.1f} s wall"}


def bench_operator(args, wl, x, torch, Plan):
    from fft_long_convolution_libhyena_amd import synth

    dev = torch.device("cuda", 0)
    iot = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    p = synth.operator_params(wl)

    def dv(a, dt=iot):
        return torch.from_numpy(a).to(dev).to(dt).contiguous()

    plan = Plan(wl.L, wl.D, wl.order, wl.dtype)
    spec = plan.spectrum(dv(x.h, torch.float32))
    N, D, L, B = wl.order, wl.D, wl.L, wl.B
    C = (N + 1) * D
    args_ = (dv(p.x), dv(p.w_in), dv(p.b_in), dv(x.short_w, torch.float32), spec, dv(x.bias, torch.float32),
             dv(p.w_out), dv(p.b_out))
    out = torch.empty((B, L, D), dtype=iot, device=dev)
    ws = torch.empty(plan.operator_workspace_bytes(B), dtype=torch.uint8, device=dev)
    log(f"[bench] operator workspace {ws.numel() / 2**20:.1f} MiB, path={plan.path}")
    t0 = time.perf_counter()
    plan.operator_tune(*args_, out=out, workspace=ws)  # once per plan, outside the timed region
    tune_ms = (time.perf_counter() - t0) * 1e3
    for _ in range(args.warmup):
        plan.operator_forward(*args_, out=out, workspace=ws)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for rep in range(args.reps):
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            plan.operator_forward(*args_, out=out, workspace=ws)
        ev1.record()
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / args.steps)
        log(f"[bench] rep {rep}: {times[-1] * 1e3:.1f} us/step")
    ms = float(np.median(times))
    stage = {}
    nt = max(3, min(args.steps, 10))
    for _ in range(nt):
        for k, v in plan.operator_forward_timed(*args_, out=out, workspace=ws).items():
            stage[k] = stage.get(k, 0.0) + v / nt
    log(f"[bench] stage ms: {json.dumps({k: round(v, 4) for k, v in stage.items()})}")
    flops = {"in_proj": 2.0 * B * L * D * C, "out_proj": 2.0 * B * L * D * D}
    dom = max(("in_proj", "path", "out_proj"), key=lambda k: stage[k])
    # the stages' share of the timed region (events around each stage add fence time)
    dom_ms = ms * stage[dom] / max(stage["in_proj"] + stage["path"] + stage["out_proj"], 1e-9)
    if dom == "path":
        nbytes = alg_bytes_forward(wl)
        roof = {"bound": "hbm", "achieved": round(nbytes / (dom_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "kernel": "hyena_forward", "alg_bytes_per_launch": nbytes}
        roof["frac"] = round(roof["achieved"] / HBM_PEAK_GBS, 4)
    else:
        peak = MFMA_PEAK_TFLOPS[wl.dtype]
        tf = flops[dom] / (dom_ms * 1e-3) / 1e12
        fused = dom == "in_proj" and wl.dtype == "bf16" and D % 64 == 0
        kname = "k_inproj_conv3 (matrix-core in_proj with b_in and the short conv)" if fused else \
            f"hipBLASLt GEMM ({dom})"
        roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tf / peak, 4), "kernel": kname, "alg_flops_per_launch": flops[dom]}
    roof.update({"traffic": None, "launch_ms": round(dom_ms, 5), "launches_per_step": 1,
                 "stage_ms": {k: round(v, 4) for k, v in stage.items()}})
    res = {
        "metric": "tokens/s (B·L/s), Hyena operator forward with in/out projections",
        "value": B * L / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if wl.dtype == "f32" else "bf16",
        "data": f"synthetic seeded ({wl.kind} activations, N(0,1/D) projection weights)",
        "config": {"workload": wl.name, "B": B, "D": D, "L": L, "order": N, "io_dtype": wl.dtype,
                   "path": plan.path, "pass": "operator"},
        "roofline": roof,
        "tune_ms": round(tune_ms, 1),
    }
    if args.check:
        import oracle

        # the first tokens of the first sequence: the operator is causal, so they
        # depend on those tokens alone
        Lp = min(L, 1024)
        ref = oracle.operator_forward(p.x[:1, :Lp], p.w_in, p.b_in, x.short_w, x.h[:, :, :Lp], x.bias, p.w_out,
                                      p.b_out, N)
        res["check_rel_l2"] = oracle.rel_l2(out[:1, :Lp].double().cpu().numpy(), ref)
        log(f"[bench] oracle check on the first {Lp} tokens of sequence 0: rel_l2 {res['check_rel_l2']:.3e}")
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (operator oracle) ...")
        res["cpu_baseline"] = cpu_baseline_operator(x, p, wl, args.cpu_budget)
    print(json.dumps(res), flush=True)
    plan.close()


def cpu_baseline_filter(p, wl, budget_s: float):
    """The fp64 implicit-filter oracle on a seeded subset of the output channels (rows
    of w_out and alpha; channels are independent), all L time steps, the subset
    doubled until it takes about a quarter of the time budget."""
    import types

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    C = (wl.order - 1) * wl.D
    n = min(C, 8)
    rng = np.random.default_rng(11)
    while True:
        cs = np.sort(rng.choice(C, size=n, replace=False))
        sub = types.SimpleNamespace(**{**vars(p), "w_out": p.w_out[cs], "alpha": p.alpha[cs]})
        t0 = time.perf_counter()
        oracle.implicit_filter(wl.L, n, 2, sub)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or n >= C:
            break
        n = min(C, n * 2)
    return {"value": n * wl.L / dt, "unit": "filter taps/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {C} filter channels, all {wl.L} time steps, fp64 numpy (BLAS threads), {dt:.1f} s wall"}


def bench_filter(args, wl, torch, Plan):
    """hyena_implicit_filter for the workload's plan with the walkthrough's default
    HyenaFilter shape (emb_dim 3, MLP width 16, two inner layers); the spectrum of the
    generated filters is timed beside it."""
    import types

    from fft_long_convolution_libhyena_amd import synth

    dev = torch.device("cuda", 0)
    p = synth.filter_mlp(wl)
    dp = types.SimpleNamespace(**{k: torch.from_numpy(v).to(dev).contiguous() for k, v in vars(p).items()})
    plan = Plan(wl.L, wl.D, wl.order, wl.dtype)
    N, D, L = wl.order, wl.D, wl.L
    C = (N - 1) * D
    h = torch.empty((N - 1, D, L), dtype=torch.float32, device=dev)
    spec = torch.empty(plan.spectrum_bytes(), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        plan.implicit_filter(dp, out=h)
        plan.spectrum(h, out=spec)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        times = []
        for rep in range(args.reps):
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(args.steps):
                fn()
            ev1.record()
            torch.cuda.synchronize()
            times.append(ev0.elapsed_time(ev1) / args.steps)
        return float(np.median(times))

    ms = timed(lambda: plan.implicit_filter(dp, out=h))
    spec_ms = timed(lambda: plan.spectrum(h, out=spec))
    log(f"[bench] implicit filter {ms * 1e3:.1f} us, spectrum of its output {spec_ms * 1e3:.1f} us")
    W, E, M = p.width, p.emb_dim, p.num_inner
    # written filters plus the parameters read once
    nbytes = 4 * C * L + 4 * (p.band_freq.size + p.w_in.size + p.b_in.size + p.w_inner.size + p.b_inner.size
                               + p.sin_freq.size + p.w_out.size + p.alpha.size)
    achieved = nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "filter taps/s ((N-1)·D·L/s), implicit long-filter generation (positional embedding, Sin MLP, "
                  "exponential modulation)",
        "value": C * L / (ms * 1e-3), "unit": "filter taps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic seeded filter parameters (N(0,1/fan_in) weights, log-spaced alpha)",
        "config": {"workload": wl.name, "D": D, "L": L, "order": N, "emb_dim": E, "width": W, "num_inner": M,
                   "pass": "implicit_filter"},
        "spectrum_ms": round(spec_ms, 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("k_implicit_filter", wl.name),
                     "kernel": "k_implicit_filter", "alg_bytes_per_launch": nbytes, "launch_ms": round(ms, 5),
                     "launches_per_step": 1},
    }
    if args.check:
        import oracle

        got = h.cpu().numpy().astype(np.float64).reshape(C, L)
        cs = np.array([0, C // 2, C - 1])
        sub = types.SimpleNamespace(**{**vars(p), "w_out": p.w_out[cs], "alpha": p.alpha[cs]})
        res["check_rel_l2"] = oracle.rel_l2(got[cs], oracle.implicit_filter(L, 3, 2, sub).reshape(3, L))
        log(f"[bench] oracle check on channels {list(cs)}: rel_l2 {res['check_rel_l2']:.3e}")
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (implicit filter oracle) ...")
        res["cpu_baseline"] = cpu_baseline_filter(p, wl, args.cpu_budget)
    print(json.dumps(res), flush=True)
    plan.close()


def bench_synthesis(args, wl, torch, Plan):
    """hyena_kernel_synthesis: per-sample filters for the workload's plan (B samples,
    (N-1)*D kernels on a causal axis of L points; width 16, two layers, 16 control
    values); the per-sample spectra of its output are timed beside it."""
    import types

    import oracle
    from fft_long_convolution_libhyena_amd import kernel_synthesis, synth

    dev = torch.device("cuda", 0)
    N, D, L, B = wl.order, wl.D, wl.L, wl.B
    C, W, M, Z = (N - 1) * D, 16, 2, 16
    p = synth.synthesis_params((L,), (False,), C, width=W, layers=M, zdim=Z, seed=wl.seed)
    z = synth.synthesis_controls(B, Z, seed=wl.seed)
    dp = types.SimpleNamespace(**{k: (torch.from_numpy(v).to(dev).contiguous() if isinstance(v, np.ndarray) else v)
                                  for k, v in vars(p).items()})
    zd = torch.from_numpy(z).to(dev)
    k = torch.empty((B, C, L), dtype=torch.float32, device=dev)
    plan = Plan(L, D, N, wl.dtype)
    spec = torch.empty(B * plan.spectrum_bytes(), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        kernel_synthesis(dp, zd, out=k)
        plan.spectrum_batched(k.view(B, N - 1, D, L), out=spec)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        times = []
        for _ in range(args.reps):
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(args.steps):
                fn()
            ev1.record()
            torch.cuda.synchronize()
            times.append(ev0.elapsed_time(ev1) / args.steps)
        return float(np.median(times))

    ms = timed(lambda: kernel_synthesis(dp, zd, out=k))
    spec_ms = timed(lambda: plan.spectrum_batched(k.view(B, N - 1, D, L), out=spec))
    log(f"[bench] kernel synthesis {ms * 1e3:.1f} us, per-sample spectra of its output {spec_ms * 1e3:.1f} us")
    outs = B * C * L
    params = sum(v.size for v in vars(p).values() if isinstance(v, np.ndarray))
    nbytes = 4 * outs + 4 * params + 4 * z.size
    # per output value: the output layer (2W), the window (4 per axis + 2); per point and
    # sample the sine layers (2 W fan_in + 4 per unit), shared by the C kernels
    flops = outs * (2 * W + 4 + 2) + B * L * (W * (2 * 1 + 4) + (M - 1) * W * (2 * W + 4))
    res = {
        "metric": "kernel values/s (B·C·L/s), input-dependent kernel synthesis (FiLM-modulated SIREN times a "
                  "Gaussian window)",
        "value": outs / (ms * 1e-3), "unit": "kernel values/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic seeded synthesis parameters and N(0,1) control vectors",
        "config": {"workload": wl.name, "B": B, "D": D, "L": L, "order": N, "kernels": C, "width": W, "layers": M,
                   "zdim": Z, "pass": "kernel_synthesis"},
        "spectrum_ms": round(spec_ms, 5),
        "roofline": roofline("k_kernel_synthesis", 1, ms, nbytes, flops),
    }
    if args.check:
        cs = np.array([0, C // 2, C - 1])
        sub = types.SimpleNamespace(**{**vars(p), "w_out": p.w_out[cs], "b_out": p.b_out[cs],
                                       "win_mu": p.win_mu[cs], "win_sigma": p.win_sigma[cs]})
        got = k.cpu().numpy().astype(np.float64)[:, cs]
        res["check_rel_l2"] = oracle.rel_l2(got, oracle.kernel_synthesis(sub, z))
        log(f"[bench] oracle check on kernels {list(cs)}: rel_l2 {res['check_rel_l2']:.3e}")
    if not args.no_cpu_baseline:
        n = 1
        while True:
            t0 = time.perf_counter()
            oracle.kernel_synthesis(p, z[:n])
            dt = time.perf_counter() - t0
            if dt >= args.cpu_budget / 4 or n >= B:
                break
            n = int(min(B, max(n + 1, n * args.cpu_budget / max(dt, 1e-3) * 0.8)))
        res["cpu_baseline"] = {"value": n * C * L / dt, "unit": "kernel values/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} of {B} samples (all kernels and points), fp64 numpy, {dt:.1f} s wall"}
    print(json.dumps(res), flush=True)
    plan.close()


def _per_sample_rows(x, hb, wl, rows):
    """The per-sample oracle on flat rows b*D + d (sorted): each sample's rows with its own filters."""
    import oracle

    out = []
    for b in range(wl.B):
        ds = [int(r) - b * wl.D for r in rows if int(r) // wl.D == b]
        if ds:
            out.append(oracle.forward(x.u_proj[b:b + 1], x.short_w, hb[b], x.bias, wl.order, mode="fft", rows=ds))
    return np.concatenate(out, axis=0)


def bench_per_sample(args, wl, x, torch, Plan):
    """hyena_forward_per_sample: the workload with a filter set per sample (B spectra
    read, one per sample), against its algorithmic bytes."""
    import oracle
    from fft_long_convolution_libhyena_amd import synth

    dev = torch.device("cuda", 0)
    iot = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    u = torch.from_numpy(x.u_proj).to(dev).to(iot).contiguous()
    w = torch.from_numpy(x.short_w).to(dev)
    bias = torch.from_numpy(x.bias).to(dev)
    hb = synth.per_sample_filters(wl)
    plan = Plan(wl.L, wl.D, wl.order, wl.dtype)
    spec = plan.spectrum_batched(torch.from_numpy(hb).to(dev))
    B, D, L, N = wl.B, wl.D, wl.L, wl.order
    ws_bytes = plan.workspace_bytes(B)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    y = torch.empty((B, D, L), dtype=iot, device=dev)
    for _ in range(args.warmup):
        plan.forward_per_sample(u, w, spec, bias, y, ws)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for rep in range(args.reps):
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            plan.forward_per_sample(u, w, spec, bias, y, ws)
        ev1.record()
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / args.steps)
        log(f"[bench] rep {rep}: {times[-1] * 1e3:.1f} us/step")
    ms = float(np.median(times))
    # as the shared forward, with B filter spectra instead of one
    nbytes = alg_bytes_forward(wl) + 8 * (B - 1) * (N - 1) * D * (L + 1)
    achieved = nbytes / (ms * 1e-3) / 1e9
    lds = plan.path == "lds"
    dom = "k_lds_forward" if lds else "four-step passes (whole step)"
    out = {
        "metric": "channel-tokens/s (B·D·L/s) and % HBM peak, Hyena op fwd with a filter set per sample",
        "value": B * D * L / (ms * 1e-3), "unit": "channel-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if wl.dtype == "f32" else "bf16-io/f32",
        "data": f"synthetic seeded ({wl.kind} activations, per-sample exponentially decaying random filters)",
        "config": {"workload": wl.name, "B": B, "D": D, "L": L, "order": N, "io_dtype": wl.dtype,
                   "path": plan.path, "pass": "forward_per_sample"},
        "hbm_frac_forward": round(achieved / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(dom, wl.name + "_per_sample") if lds else None,
                     "kernel": dom, "alg_bytes_per_launch": nbytes, "launch_ms": round(ms, 5),
                     "launches_per_step": 1},
    }
    if args.check:
        rows = synth.sample_rows(wl, 8)
        got = y.float().cpu().numpy().reshape(-1, L)[rows]
        out["check_rel_l2"] = oracle.rel_l2(got, _per_sample_rows(x, hb, wl, rows))
        log(f"[bench] oracle check on {len(rows)} rows: rel_l2 {out['check_rel_l2']:.3e}")
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (per-sample oracle) ...")
        threads = oracle.max_threads()
        n = max(1, min(B * D, 2 * threads))
        while True:
            rows = synth.sample_rows(wl, n, seed=99)
            t0 = time.perf_counter()
            _per_sample_rows(x, hb, wl, rows)
            dt = time.perf_counter() - t0
            if dt >= args.cpu_budget / 4 or n >= B * D:
                break
            n = int(min(B * D, max(n + 1, n * args.cpu_budget / max(dt, 1e-3) * 0.8)))
        out["cpu_baseline"] = {"value": len(rows) * L / dt, "unit": "channel-tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"{len(rows)} of {B * D} (b,d) rows, each with its sample's filters, "
                                         f"fp64 radix-2 FFT convolution, OpenMP over rows, {dt:.1f} s wall"}
    print(json.dumps(out), flush=True)
    plan.close()


def bench_circular(args, wl, x, torch, Plan):
    """hyena_forward on a circular plan (HYENA_FLAG_CIRCULAR: circular long
    convolution of the L samples, an L-point real transform), against its
    algorithmic bytes (the spectrum holds L/2 + 1 bins per filter)."""
    import oracle
    from fft_long_convolution_libhyena_amd import synth

    dev = torch.device("cuda", 0)
    iot = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    u = torch.from_numpy(x.u_proj).to(dev).to(iot).contiguous()
    w = torch.from_numpy(x.short_w).to(dev)
    bias = torch.from_numpy(x.bias).to(dev)
    plan = Plan(wl.L, wl.D, wl.order, wl.dtype, circular=True)
    spec = plan.spectrum(torch.from_numpy(x.h).to(dev))
    B, D, L, N = wl.B, wl.D, wl.L, wl.order
    ws_bytes = plan.workspace_bytes(B)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    y = torch.empty((B, D, L), dtype=iot, device=dev)
    for _ in range(args.warmup):
        plan.forward(u, w, spec, bias, y, ws)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for rep in range(args.reps):
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            plan.forward(u, w, spec, bias, y, ws)
        ev1.record()
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / args.steps)
        log(f"[bench] rep {rep}: {times[-1] * 1e3:.1f} us/step")
    ms = float(np.median(times))
    s = io_bytes(wl)
    nbytes = (s * B * (N + 1) * D * L + s * B * D * L + 8 * (N - 1) * D * (L // 2 + 1)
              + 4 * (N + 1) * D * 3 + 4 * (N - 1) * D)
    achieved = nbytes / (ms * 1e-3) / 1e9
    lds = plan.path == "lds"
    dom = "k_lds_forward" if lds else "four-step passes (whole step)"
    out = {
        "metric": "channel-tokens/s (B·D·L/s) and % HBM peak, Hyena op fwd with circular long convolutions",
        "value": B * D * L / (ms * 1e-3), "unit": "channel-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if wl.dtype == "f32" else "bf16-io/f32",
        "data": f"synthetic seeded ({wl.kind} activations, exponentially decaying random filters)",
        "config": {"workload": wl.name, "B": B, "D": D, "L": L, "order": N, "io_dtype": wl.dtype,
                   "path": plan.path, "pass": "forward_circular"},
        "hbm_frac_forward": round(achieved / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(dom, wl.name + "_circular") if lds else None,
                     "kernel": dom, "alg_bytes_per_launch": nbytes, "launch_ms": round(ms, 5),
                     "launches_per_step": 1},
    }
    if args.check:
        ds = [0, D // 2, D - 1]
        xs = synth.channel_subset(x, ds)
        ref = oracle.forward_circular(xs.u_proj, xs.short_w, xs.h, xs.bias, N)
        got = y.float().cpu().numpy()[:, ds]
        out["check_rel_l2"] = oracle.rel_l2(got, ref)
        log(f"[bench] oracle check on channels {ds}: rel_l2 {out['check_rel_l2']:.3e}")
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (circular oracle) ...")
        rng = np.random.default_rng(99)
        n = 1
        while True:
            ds = np.sort(rng.choice(D, size=n, replace=False))
            xs = synth.channel_subset(x, ds)
            t0 = time.perf_counter()
            oracle.forward_circular(xs.u_proj, xs.short_w, xs.h, xs.bias, N)
            dt = time.perf_counter() - t0
            if dt >= args.cpu_budget / 4 or n >= D:
                break
            n = int(min(D, max(n + 1, n * args.cpu_budget / max(dt, 1e-3) * 0.8)))
        out["cpu_baseline"] = {"value": B * n * L / dt, "unit": "channel-tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} of {D} channels at every b and t, fp64 numpy (one thread), "
                                         f"{dt:.1f} s wall"}
    print(json.dumps(out), flush=True)
    plan.close()


def bench_convnd(args, torch, nd: int):
    """hyena_conv2d_forward / hyena_conv3d_forward: one gated N-d long-convolution
    step on a 256 x 256 grid (2-D) or a 32 x 32 x 64 grid (3-D) -- 65536 tokens per
    channel, as in long64k -- of 768 channels, both gates, a centred kernel; against
    its algorithmic bytes (v, g, x read once, y written once, the kernel spectrum
    read once)."""
    import oracle
    from fft_long_convolution_libhyena_amd import Plan2D, Plan3D, synth

    B, D = 1, 768
    dims = (256, 256) if nd == 2 else (32, 32, 64)
    circ = bool(args.circular)
    dev = torch.device("cuda", 0)
    if nd == 2:
        inp = synth.conv2d_inputs(B, D, *dims, seed=3)
        plan = Plan2D(*dims, D, circular=circ)
        base_fn = oracle.conv2d_forward
    else:
        inp = synth.conv3d_inputs(B, D, *dims, seed=3)
        plan = Plan3D(*dims, D, circular=circ)
        base_fn = oracle.conv3d_forward
    if circ:  # a kernel on the grid itself: the leading corner of the doubled-grid draw
        inp.k = np.ascontiguousarray(inp.k[(slice(None),) + tuple(slice(0, n) for n in dims)])

    def ref_fn(*a):
        return base_fn(*a, circular=circ)

    spec = plan.spectrum(torch.from_numpy(inp.k).to(dev))
    v, g, x = (torch.from_numpy(a).to(dev) for a in (inp.v, inp.g, inp.x))
    bias = torch.from_numpy(inp.bias).to(dev)
    y = torch.empty_like(v)
    ws = torch.empty(plan.workspace_bytes(B), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        plan.forward(v, spec, bias, g=g, x=x, y=y, workspace=ws)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for rep in range(args.reps):
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            plan.forward(v, spec, bias, g=g, x=x, y=y, workspace=ws)
        ev1.record()
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / args.steps)
        log(f"[bench] rep {rep}: {times[-1] * 1e3:.1f} us/step")
    ms = float(np.median(times))
    pts = int(np.prod(dims))
    if circ:
        spec_bins = int(np.prod(dims[:-1])) * (dims[-1] // 2 + 1)
    else:
        spec_bins = int(np.prod([2 * n for n in dims[:-1]])) * (dims[-1] + 1)
    nbytes = 4 * 4 * B * D * pts + 8 * D * spec_bins + 4 * D
    achieved = nbytes / (ms * 1e-3) / 1e9
    grid = "x".join(str(n) for n in dims)
    names = "B·D·H·W" if nd == 2 else "B·D·A·H·W"
    out = {
        "metric": f"channel-tokens/s ({names}/s) and % HBM peak, gated {nd}-D long convolution "
                  + ("(circular)" if circ else "(grid doubled)"),
        "value": B * D * pts / (ms * 1e-3), "unit": "channel-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic seeded (N(0,1) grids and gates, centred decaying random kernels)",
        "config": {"workload": f"conv{nd}d {grid}" + (" circular" if circ else ""), "B": B, "D": D,
                   "grid": list(dims), "pass": f"conv{nd}d_forward"},
        "hbm_frac_forward": round(achieved / HBM_PEAK_GBS, 4),
        # traffic: the committed counter summary of the zero-padded step (all launches of one step)
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if circ else measured_traffic(f"k_c{nd}_conv{nd}d", grid),
                     "kernel": f"{nd}-D passes (whole step)", "alg_bytes_per_launch": nbytes,
                     "launch_ms": round(ms, 5), "launches_per_step": 1},
    }
    if args.check:
        ds = [0, D // 2, D - 1]
        ref = ref_fn(inp.v[:, ds], inp.k[ds], inp.bias[ds], inp.g[:, ds], inp.x[:, ds])
        out["check_rel_l2"] = oracle.rel_l2(y.cpu().numpy()[:, ds], ref)
        log(f"[bench] oracle check on channels {ds}: rel_l2 {out['check_rel_l2']:.3e}")
    if not args.no_cpu_baseline:
        n = 4
        while True:
            ds = list(range(n))
            t0 = time.perf_counter()
            ref_fn(inp.v[:, ds], inp.k[ds], inp.bias[ds], inp.g[:, ds], inp.x[:, ds])
            dt = time.perf_counter() - t0
            if dt >= args.cpu_budget / 4 or n >= D:
                break
            n = int(min(D, max(n + 1, n * args.cpu_budget / max(dt, 1e-3) * 0.8)))
        out["cpu_baseline"] = {"value": B * n * pts / dt, "unit": "channel-tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} of {D} channels, fp64 numpy rfftn (one thread), {dt:.1f} s wall"}
    print(json.dumps(out), flush=True)
    plan.close()


# ------------------------------------------------------------ profile summaries

def _csv_rows(d: str, suffix: str):
    """Rows of every rocprofv3 csv file under directory d whose name ends with suffix."""
    import csv
    import glob

    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {d}")
    return rows


def _short_name(name: str) -> str:
    """'void hy::k_fs_row<8, 8, 0>(...)' -> 'k_fs_row<8, 8, 0>'; namespaces inside the
    template arguments go too ('k_cnd_row<8, 0, hy::PairMap2, false>' -> '... PairMap2 ...')."""
    n = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").strip()
    head, lt, rest = n.partition("<")
    return head.split("hy::")[-1] + lt + rest.replace("hy::", "")


def _is_forward_kernel(short: str) -> bool:
    """Kernels one forward launches (not the once-per-plan spectrum kernels)."""
    base, _, targs = short.partition("<")
    a = [t.strip() for t in targs.rstrip(">").split(",")] if targs else []
    if base in ("k_fs_pipe", "k_lds_forward", "k_fs_colinv", "k_part_fwd", "k_part_inv"):
        return True
    if base == "k_fs_colfwd":
        return len(a) > 3 and a[3] == "0"
    if base == "k_fs_row":
        return len(a) > 2 and a[2] == "0"
    return False


def _is_backward_kernel(short: str) -> bool:
    """Kernels one backward launches (the forward recompute's column pass included)."""
    base, _, targs = short.partition("<")
    a = [t.strip() for t in targs.rstrip(">").split(",")] if targs else []
    if base == "k_fs_colfwd":
        return len(a) > 3 and a[3] == "0"
    return base.startswith(("k_fs_row_bwd", "k_fs_colinv_bwd", "k_fs_dh_col", "k_fs_bwd_", "k_fs_dbias",
                            "k_lds_bwd"))


def _calibration():
    kv = {}
    with open(os.path.join(ROOT, "profiles", "copy_calibration_1GiB.txt")) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    return float(kv["fetch_scale"]), float(kv["write_scale"])


def summarize_pmc(args):
    """Counter summary (profiles/pmc_<kernel>_<workload>.txt) from a FETCH_SIZE run and
    a WRITE_SIZE run of `bench.py --profile-forwards F`: per-dispatch HBM bytes of the
    dominant kernel and the bytes of one whole forward, scaled by the copy calibration."""
    from fft_long_convolution_libhyena_amd import synth

    fdir, wdir = args.summarize_pmc
    fs, ws = _calibration()
    per = {}
    for d, cname, key in ((fdir, "FETCH_SIZE", "fetch"), (wdir, "WRITE_SIZE", "write")):
        for r in _csv_rows(d, "counter_collection.csv"):
            if r.get("Counter_Name") != cname:
                continue
            k = _short_name(r["Kernel_Name"])
            e = per.setdefault(k, {"fetch": [], "write": []})
            e[key].append(float(r["Counter_Value"]))
    F = args.forwards
    kern = args.kernel
    # a family name stands for every kernel of one step: k_fs_passes, k_part_passes
    # (the forward); fs_backward, k_lds_bwd_rows (the backward); k_c2_conv2d, k_c3_conv3d
    # (the N-d step: its kernels run at least once per step, the spectrum's once per plan)
    family = kern in ("k_fs_passes", "k_part_passes", "fs_backward", "k_lds_bwd_rows", "k_c2_conv2d",
                      "k_c3_conv3d")
    if kern in ("fs_backward", "k_lds_bwd_rows"):
        member = _is_backward_kernel
    elif kern in ("k_c2_conv2d", "k_c3_conv3d"):
        def member(k):
            e = per[k]
            return k.startswith(("k_c2_", "k_c3_", "k_cnd_")) and max(len(e["fetch"]), len(e["write"])) >= F
    else:
        # the forward's kernels, and the kernel itself when it is not one (the filter's)
        def member(k):
            return _is_forward_kernel(k) or k.split("<")[0] == kern
    dom = [k for k in per if (member(k) if family else k.split("<")[0] == kern)]
    if not dom:
        raise SystemExit(f"kernel {kern} not in the counters: {sorted(per)}")
    wl = synth.WORKLOADS.get(args.workload)
    label = getattr(args, "label", "") or args.workload
    what = getattr(args, "what", "") or (f"{wl.name} ({wl.describe()})" if wl else label)
    if getattr(args, "alg_bytes", 0):
        alg = args.alg_bytes
    elif wl is None:
        raise SystemExit("--alg-bytes is needed for a workload that is not one of the synthetic workloads")
    else:
        alg = alg_bytes_backward(wl) if kern in ("fs_backward", "k_lds_bwd_rows") else alg_bytes_forward(wl)
    step = 0.0
    lines = []
    for k in sorted(per, key=lambda k: -sum(per[k]["fetch"])):
        e = per[k]
        fb = sum(e["fetch"]) * 1024 * fs
        wb = sum(e["write"]) * 1024 * ws
        n = max(len(e["fetch"]), len(e["write"]))
        fwd = member(k)
        if fwd:
            step += (fb + wb) / F
        lines.append(f"#   {k}: dispatches {n}, fetch {fb / max(n, 1):.0f}, write {wb / max(n, 1):.0f} bytes per dispatch"
                     + ("" if fwd else " (not part of the step)"))
    d0 = dom[0] if not family else ", ".join(sorted(dom))
    fe_all = [v for k in dom for v in per[k]["fetch"]]
    wr_all = [v for k in dom for v in per[k]["write"]]
    nd = max(len(fe_all), len(wr_all))
    fk = sum(fe_all) / len(fe_all)
    wk = sum(wr_all) / len(wr_all)
    if kern in ("k_c2_conv2d", "k_c3_conv3d"):  # a dispatch of the N-d step is the whole step
        nd, fk, wk = F, sum(fe_all) / F, sum(wr_all) / F
    cmd = args.command or ""
    out = [f"# rocprofv3 HBM byte counters per dispatch: {kern} on {what}",
           "# commands (from the repository root):"]
    out += [f"#   {c.strip()}" for c in cmd.split(";;") if c.strip()]
    out += ["# scaled with the factors of copy_calibration_1GiB.txt; the kernels of one step (forward or backward) summed over "
            f"{F} steps give step_bytes",
            f"kernel: {kern}", f"instance: {d0}", f"workload: {label}",
            f"sources_sha256: {kernel_sources_hash(kern)}", f"dispatches: {nd}",
            f"fetch_size_kib_per_dispatch: {fk:.1f}", f"write_size_kib_per_dispatch: {wk:.1f}",
            f"fetch_scale: {fs:.4f}", f"write_scale: {ws:.4f}",
            f"fetch_bytes_per_dispatch: {fk * 1024 * fs:.0f}", f"write_bytes_per_dispatch: {wk * 1024 * ws:.0f}",
            f"step_bytes: {step:.0f}", f"alg_bytes_per_step: {alg}", f"step_traffic_over_alg: {step / alg:.3f}",
            "# every kernel of the run (scaled bytes per dispatch):"] + lines
    print("\n".join(out))


def summarize_sq(args):
    """Instruction-counter summary (profiles/sq_<kernel>_<workload>.txt) from one
    rocprofv3 --pmc run of `bench.py --profile-forwards F` with SQ counters: every
    counter of the forward's kernels summed over the run, per forward and per
    channel-token (b, d, t) point. SQ_INSTS_* count wave instructions (64 lanes)."""
    from fft_long_convolution_libhyena_amd import synth

    wl = synth.WORKLOADS[args.workload]
    tot = {}
    disp = {}
    for r in _csv_rows(args.summarize_sq, "counter_collection.csv"):
        k = _short_name(r["Kernel_Name"])
        if not _is_forward_kernel(k):
            continue
        tot[r["Counter_Name"]] = tot.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        disp[k] = disp.get(k, 0) + 1
    F = args.forwards
    pts = wl.B * wl.D * wl.L
    cmd = args.command or ""
    out = [f"# rocprofv3 SQ counters: {args.kernel} on {wl.name} ({wl.describe()})",
           "# command (from the repository root):"]
    out += [f"#   {c.strip()}" for c in cmd.split(";;") if c.strip()]
    out += [f"# kernel sources sha256[:16]: {kernel_sources_hash(args.kernel)}",
            f"# forward kernels and counter rows: {dict(sorted(disp.items()))}; {F} forwards; "
            f"{pts} channel-token points per forward",
            "# wave instructions (64 lanes each) per forward, and lane instructions per point (x 64 / points)",
            f"{'counter':28s} {'per_forward':>16s} {'lane_instr_per_point':>22s}"]
    for name in sorted(tot):
        pf = tot[name] / F
        per = pf * 64 / pts if name.startswith("SQ_INSTS") else float("nan")
        out.append(f"{name:28s} {pf:16.0f} {per:22.2f}")
    if args.note:
        out.append(f"# {args.note}")
    print("\n".join(out))


def summarize_trace(args):
    """Kernel-trace summary (profiles/trace_<kernel>_<workload>.txt) from a
    `rocprofv3 --kernel-trace --stats` run."""
    from fft_long_convolution_libhyena_amd import synth

    rows = _csv_rows(args.summarize_trace, "kernel_stats.csv")
    wl = synth.WORKLOADS.get(args.workload)
    what = getattr(args, "what", "") or (f"{wl.name} ({wl.describe()})" if wl else
                                         (getattr(args, "label", "") or args.workload))
    cmd = args.command or ""
    out = [f"# rocprofv3 kernel-trace statistics: {args.kernel} on {what}",
           "# command (from the repository root):"]
    out += [f"#   {c.strip()}" for c in cmd.split(";;") if c.strip()]
    out += [f"# kernel sources sha256[:16]: {kernel_sources_hash(args.kernel)}",
            f"{'kernel':60s} {'calls':>7s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0))):
        out.append(f"{_short_name(r['Name'])[:60]:60s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                   f"{float(r['Percentage']):6.2f}")
    if args.note:
        out.append(f"# {args.note}")
    print("\n".join(out))


def profile_forwards(args, wl, x, torch, Plan):
    """Plan, spectrum and exactly args.profile_forwards forwards, for counter runs."""
    dev = torch.device("cuda", 0)
    u = torch.from_numpy(x.u_proj).to(dev)
    if wl.dtype == "bf16":
        u = u.to(torch.bfloat16)
    plan = Plan(wl.L, wl.D, wl.order, wl.dtype, args.path)
    spec = plan.spectrum(torch.from_numpy(x.h).to(dev))
    w, bias = torch.from_numpy(x.short_w).to(dev), torch.from_numpy(x.bias).to(dev)
    ws_bytes = int(args.workspace_mb * 2 ** 20) if args.workspace_mb > 0 else plan.workspace_bytes(wl.B)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    y = torch.empty((wl.B, wl.D, wl.L), dtype=plan.io_dtype, device=dev)
    torch.cuda.synchronize()
    for i in range(args.profile_forwards):
        plan.forward(u, w, spec, bias, y, ws)
        torch.cuda.synchronize()
        log(f"[profile] forward {i + 1} of {args.profile_forwards} done")
    plan.close()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long64k")
    ap.add_argument("--reps", type=int, default=5, help="timed repetitions of --steps; the median is reported")
    ap.add_argument("--workspace-mb", type=float, default=0.0,
                    help="four-step / partitioned workspace (0 = the library's recommendation)")
    ap.add_argument("--path", default="auto", choices=["auto", "lds", "fourstep", "partitioned"],
                    help="kernel family of the forward plan")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the oracle comparison of sampled outputs (run by default, after the timed region)")
    ap.add_argument("--operator", action="store_true",
                    help="time hyena_operator_forward (in_proj GEMM + the path + out_proj GEMM) instead")
    ap.add_argument("--backward", action="store_true",
                    help="time hyena_backward instead of the forward")
    ap.add_argument("--conv2d", action="store_true",
                    help="time hyena_conv2d_forward (gated 2-D long convolution, 256 x 256 x 768) instead")
    ap.add_argument("--conv3d", action="store_true",
                    help="time hyena_conv3d_forward (gated 3-D long convolution, 32 x 32 x 64 x 768) instead")
    ap.add_argument("--circular", action="store_true",
                    help="time hyena_forward on a circular plan (circular long convolutions) instead; with "
                         "--conv2d or --conv3d, a circular N-d plan")
    ap.add_argument("--per-sample", action="store_true",
                    help="time hyena_forward_per_sample (a filter set per sample) instead; with --backward, "
                         "hyena_backward_per_sample")
    ap.add_argument("--filter", action="store_true",
                    help="time hyena_implicit_filter (the long filters of the workload's plan) instead")
    ap.add_argument("--synthesis", action="store_true",
                    help="time hyena_kernel_synthesis (per-sample filters of the workload's plan) instead")
    ap.add_argument("--profile-forwards", type=int, default=0,
                    help="run plan, spectrum and exactly this many forwards, then exit (for counter runs)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print a counter summary from rocprofv3 FETCH_SIZE and WRITE_SIZE csv output")
    ap.add_argument("--summarize-sq", metavar="DIR",
                    help="print an instruction-counter summary from rocprofv3 SQ counter csv output")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a kernel-trace summary from rocprofv3 --kernel-trace --stats csv output")
    ap.add_argument("--kernel", default="k_fs_pipe", help="kernel a summary is about")
    ap.add_argument("--forwards", type=int, default=5, help="forwards in the profiled run (--summarize-pmc)")
    ap.add_argument("--command", default="", help="the profiling commands, ';;'-separated, for the summary header")
    ap.add_argument("--note", default="", help="a closing note line for a trace summary")
    ap.add_argument("--label", default="", help="workload label of a summary (default: --workload), e.g. "
                    "long64k_per_sample or 256x256")
    ap.add_argument("--what", default="", help="what a summary covers, for its first line (default: the "
                    "workload's description)")
    ap.add_argument("--alg-bytes", type=int, default=0,
                    help="algorithmic bytes of one step for a counter summary (default: the forward's or "
                         "backward's of --workload)")
    args = ap.parse_args()
    args.check = not args.no_check
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_trace:
        summarize_trace(args)
        return
    if args.summarize_sq:
        summarize_sq(args)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} (WORLD_SIZE={world}) is not supported; "
              "the path shards over channels with no exchange (see the design notes), run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from fft_long_convolution_libhyena_amd import Plan, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.conv2d or args.conv3d:  # with --circular: a circular N-d plan
        bench_convnd(args, torch, 2 if args.conv2d else 3)
        return
    wl = synth.WORKLOADS[args.workload]
    log(f"[bench] workload {wl.name}: {wl.describe()}")
    if args.filter:
        bench_filter(args, wl, torch, Plan)
        return
    if args.synthesis:
        bench_synthesis(args, wl, torch, Plan)
        return
    t0 = time.perf_counter()
    x = synth.generate(wl)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")
    if args.operator:
        bench_operator(args, wl, x, torch, Plan)
        return
    if args.backward:
        bench_backward(args, wl, x, torch, Plan, per_sample=args.per_sample)
        return
    if args.per_sample:
        bench_per_sample(args, wl, x, torch, Plan)
        return
    if args.circular:
        bench_circular(args, wl, x, torch, Plan)
        return
    if args.profile_forwards > 0:
        profile_forwards(args, wl, x, torch, Plan)
        return
    dev = torch.device("cuda", 0)
    u = torch.from_numpy(x.u_proj).to(dev)
    if wl.dtype == "bf16":
        u = u.to(torch.bfloat16)
    u = u.contiguous()
    w = torch.from_numpy(x.short_w).to(dev)
    h = torch.from_numpy(x.h).to(dev)
    bias = torch.from_numpy(x.bias).to(dev)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    plan = Plan(wl.L, wl.D, wl.order, wl.dtype, args.path)  # host set-up and the twiddle tables
    torch.cuda.synchronize()
    plan_ms = (time.perf_counter() - t0) * 1e3
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spec = plan.spectrum(h)  # first call: allocates the buffer and loads the kernels
    torch.cuda.synchronize()
    ev0.record()
    plan.spectrum(h, out=spec)
    ev1.record()
    torch.cuda.synchronize()
    spectrum_ms = ev0.elapsed_time(ev1)
    ws_bytes = int(args.workspace_mb * 2 ** 20) if args.workspace_mb > 0 else plan.workspace_bytes(wl.B)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    y = torch.empty((wl.B, wl.D, wl.L), dtype=plan.io_dtype, device=dev)
    log(f"[bench] path={plan.path} spectrum {spectrum_ms:.3f} ms workspace {ws_bytes / 2**20:.1f} MiB")

    for _ in range(args.warmup):
        plan.forward(u, w, spec, bias, y, ws)
    torch.cuda.synchronize()

    times = []
    for rep in range(args.reps):
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            plan.forward(u, w, spec, bias, y, ws)
        ev1.record()
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1) / args.steps)
        log(f"[bench] rep {rep}: {times[-1] * 1e3:.1f} us/step")
    ms = float(np.median(times))
    value = wl.B * wl.D * wl.L / (ms * 1e-3)
    fwd_bytes = alg_bytes_forward(wl)
    hbm_frac = fwd_bytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9)
    valu_frac = alg_flops_forward(wl) / (ms * 1e-3) / (VALU_F32_PEAK_TFLOPS * 1e12)
    copy_gbs = device_copy_gbs(torch, dev)
    log(f"[bench] device copy {copy_gbs:.0f} GB/s")

    # per-kernel durations, HIP events on the library's stream around every launch
    fam_ms = {}
    nt = max(3, min(args.steps, 10))
    for _ in range(nt):
        r = plan.forward_timed(u, w, spec, bias, y, ws)
        for k, v in r.items():
            fam_ms[k] = fam_ms.get(k, 0.0) + v / nt
    log(f"[bench] per-forward kernel-family ms: {json.dumps({k: round(v, 4) for k, v in fam_ms.items()})}")
    fwd_flops = alg_flops_forward(wl)
    rows = wl.B * wl.D
    dominant = None
    if plan.path == "lds":
        # the step is this one launch: the timed region itself gives its duration
        # (events around a single launch add their own fence time)
        kernel, launches, kms = "k_lds_forward", 1, ms
    elif fam_ms.get("pipe", 0.0) > 0:
        # pipelined four-step: every launch runs the three passes on three chunks, so
        # the forward's algorithmic bytes spread over its launches
        # (the launches follow each other with no gap, so the timed region divided by
        # the launch count is the average launch; events around each launch would add
        # their own fence time)
        T = wl.L // 2 if getattr(plan, "circular", False) else wl.L
        R = pipe_chunk_rows(rows, ws_bytes, 8 * T)
        launches = math.ceil(rows / R) + 2 * wl.order - 2
        kernel, kms = "k_fs_pipe", ms / launches
    else:
        # several kernel families: the forward's algorithmic bytes over all its launches;
        # the slowest family is reported on its own under "dominant_kernel"
        if plan.path == "partitioned":
            fams = {"pass_a": "k_part_fwd", "pass_b": "k_part_inv"}
            per_row = 8 * wl.L + (4 * wl.L if wl.order > 2 else 0)
            chunk = max(1, min(rows, ws_bytes // per_row))
            nper = {"pass_a": wl.order - 1, "pass_b": wl.order - 1}
            design = lambda f: alg_bytes_part(wl, {"pass_a": "pass_1", "pass_b": "pass_2"}[f])  # noqa: E731
        else:
            fams = {"pass_a": "k_fs_colfwd", "pass_b": "k_fs_row", "pass_c": "k_fs_colinv"}
            chunk = max(1, min(rows, (ws_bytes // (8 * wl.L)) if ws_bytes else rows))
            nper = {"pass_a": 1, "pass_b": wl.order - 1, "pass_c": wl.order - 1}
            design = lambda f: alg_bytes_pass(wl, f)  # noqa: E731
        nch = math.ceil(rows / chunk)
        launches = nch * sum(nper.values())
        kernel = "k_part_passes" if plan.path == "partitioned" else "k_fs_passes"  # every launch of the forward
        kms = sum(fam_ms[f] for f in fams) / launches
        fam = max(fams, key=lambda k: fam_ms[k])
        dl = nch * nper[fam]
        dominant = {"kernel": fams[fam], "launches_per_step": dl, "launch_ms": round(fam_ms[fam] / dl, 5),
                    "design_bytes_per_launch": int(design(fam) / dl),
                    "design_frac": round(design(fam) / (fam_ms[fam] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(fams[fam], wl.name)}
    per_launch = measured_traffic(kernel, wl.name)
    step_traffic = measured_step_traffic(kernel, wl.name)
    roof = roofline(kernel, launches, kms, fwd_bytes / launches, fwd_flops / launches, per_launch, step_traffic,
                    fwd_bytes)
    if dominant:
        roof["kernels"] = list(fams.values())
        roof["dominant_kernel"] = dominant

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "channel-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.dtype == "f32" else "bf16-io/f32",
        "data": f"synthetic seeded ({wl.kind} activations, exponentially decaying random filters)",
        "config": {"workload": wl.name, "B": wl.B, "D": wl.D, "L": wl.L, "order": wl.order,
                   "io_dtype": wl.dtype, "path": plan.path},
        "hbm_frac_forward": round(hbm_frac, 4),
        "alg_bytes_per_step": fwd_bytes,
        # the same step against the measured copy bandwidth and the fp32 vector peak
        "copy_gbs": round(copy_gbs, 1),
        "copy_frac_forward": round(fwd_bytes / (ms * 1e-3) / 1e9 / copy_gbs, 4),
        "alg_flops_per_step": int(alg_flops_forward(wl)),
        "valu_frac_forward": round(valu_frac, 4),
        "plan_ms": round(plan_ms, 3),
        "spectrum_ms": round(spectrum_ms, 4),
        "roofline": roof,
    }

    if not args.no_check:
        import oracle

        rows = synth.sample_rows(wl, 8)
        ref = oracle.forward(x.u_proj, x.short_w, x.h, x.bias, wl.order, rows=rows)
        got = y.float().cpu().numpy().reshape(-1, wl.L)[rows]
        out["check_rel_l2"] = oracle.rel_l2(got, ref)
        log(f"[bench] oracle check on {len(rows)} rows: rel_l2 {out['check_rel_l2']:.3e}")

    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(x, wl, args.cpu_budget)
    print(json.dumps(out), flush=True)
    plan.close()


if __name__ == "__main__":
    main()
