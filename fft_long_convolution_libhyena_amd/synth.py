"""Seeded synthetic inputs for the Hyena operator forward hot path.

This module only draws random numbers and lays them out; it holds none of the
operator's arithmetic (no short convolution, no gating, no transform).  Both the
fp64 oracle and the HIP library consume exactly the arrays produced here.

Shapes follow the operator as written in the HyenaDNA walkthrough (page "HyenaDNA
model architecture", section 2.1, HyenaOperator code): ``u_proj`` is the
in-projected activation after the (B, L, D) -> (B, D, L) transpose, of shape
[B, (N+1)*D, L]; the long filters are ``k`` rearranged to [N-1, D, L]; the
long-filter bias is [N-1, D] (HyenaFilter code, section 2.2: ``torch.randn``
initialisation); the short depthwise Conv1d weight is [(N+1)*D, 3].

Distributions (the pages give no data; these stand in for the language-model and
genome workloads they describe):
  * ``normal`` activations: u_proj ~ N(0, 1).
  * ``onehot`` activations: 4-symbol tokens (nucleotides) drawn uniformly, then a
    random bias-free Linear(4 -> (N+1)*D) with N(0, 1) weights, i.e. a column
    lookup ``u_proj[b, :, t] = W[:, tok[b, t]]``.
  * short conv weights ~ N(0, 1/3) (variance 1/3).
  * h[o, d, t] = N(0, 1) * exp(-alpha_d * t / L), alpha_d log-spaced over
    [alpha_lo, alpha_hi] across channels and shared across o.
  * bias[o, d] ~ N(0, 1).
Draw order: activations (tokens then W for ``onehot``), short weights, filter
noise, bias.  bf16 activations are drawn in fp32 and rounded to bf16 with
round-to-nearest-even; the rounded values are the input to both sides.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    D: int
    L: int
    order: int
    dtype: str  # "f32" or "bf16": dtype of u_proj and y only
    kind: str  # "normal" or "onehot"
    alpha_lo: float
    alpha_hi: float
    seed: int

    @property
    def channels(self) -> int:
        return (self.order + 1) * self.D

    def describe(self) -> str:
        return (f"B={self.B} D={self.D} L={self.L} order={self.order} "
                f"{self.dtype} {self.kind}")


# The operator shapes of the workloads: a tiny case, HyenaDNA-small, Hyena-LM-125M,
# a 64K long-context operator (order 3, and the same shape at order 2) and HyenaDNA-1M.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 64, 1024, 2, "f32", "normal", 0.3, 30.0, 0),
    "dna_small": Workload("dna_small", 4, 256, 16384, 2, "f32", "onehot", 0.3, 30.0, 1),
    "lm125m": Workload("lm125m", 8, 768, 8192, 2, "bf16", "normal", 0.3, 30.0, 2),
    "long64k_o3": Workload("long64k_o3", 1, 768, 65536, 3, "f32", "normal", 0.3, 30.0, 3),
    "long64k": Workload("long64k", 1, 768, 65536, 2, "f32", "normal", 0.3, 30.0, 3),
    "dna_1m": Workload("dna_1m", 1, 256, 1048576, 2, "f32", "onehot", 0.03, 30.0, 4),
}


def custom(B: int, D: int, L: int, order: int, dtype: str = "f32",
           kind: str = "normal", seed: int = 0, alpha_lo: float = 0.3,
           alpha_hi: float = 30.0, name: str = "custom") -> Workload:
    return Workload(name, B, D, L, order, dtype, kind, alpha_lo, alpha_hi, seed)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    out = (rounded << 16).astype(np.uint32)
    return out.view(np.float32).reshape(x.shape)


def bf16_bits(x_bf16_values: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already exactly representable in bf16."""
    x = np.ascontiguousarray(x_bf16_values, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


@dataclasses.dataclass
class Inputs:
    """Host copies of one workload's inputs (all fp32; bf16 u_proj holds bf16 values)."""
    wl: Workload
    u_proj: np.ndarray  # [B, (N+1)D, L] float32
    short_w: np.ndarray  # [(N+1)D, 3] float32
    h: np.ndarray  # [N-1, D, L] float32
    bias: np.ndarray  # [N-1, D] float32


def _alphas(D: int, lo: float, hi: float) -> np.ndarray:
    if D == 1:
        return np.array([lo], dtype=np.float64)
    return lo * (hi / lo) ** (np.arange(D, dtype=np.float64) / (D - 1))


def generate(wl: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw one workload's inputs from numpy's PCG64 with the given (or the workload's) seed."""
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    B, D, L, N = wl.B, wl.D, wl.L, wl.order
    C = (N + 1) * D
    if wl.kind == "normal":
        u = rng.standard_normal((B, C, L), dtype=np.float32)
    elif wl.kind == "onehot":
        tok = rng.integers(0, 4, size=(B, L))
        W = rng.standard_normal((C, 4), dtype=np.float32)
        u = np.empty((B, C, L), dtype=np.float32)
        for b in range(B):
            u[b] = W[:, tok[b]]
    else:
        raise ValueError(f"unknown input kind {wl.kind!r}")
    if wl.dtype == "bf16":
        u = round_to_bf16(u)
    elif wl.dtype != "f32":
        raise ValueError(f"unknown dtype {wl.dtype!r}")
    short_w = (rng.standard_normal((C, 3), dtype=np.float32)
               * np.float32(1.0 / np.sqrt(3.0))).astype(np.float32)
    noise = rng.standard_normal((N - 1, D, L), dtype=np.float32)
    alpha = _alphas(D, wl.alpha_lo, wl.alpha_hi)
    t = np.arange(L, dtype=np.float64) / L
    decay = np.exp(-alpha[:, None] * t[None, :]).astype(np.float32)  # [D, L]
    h = (noise * decay[None, :, :]).astype(np.float32)
    bias = rng.standard_normal((N - 1, D), dtype=np.float32)
    return Inputs(wl, np.ascontiguousarray(u), np.ascontiguousarray(short_w),
                  np.ascontiguousarray(h), np.ascontiguousarray(bias))


def per_sample_filters(wl: Workload, seed: Optional[int] = None) -> np.ndarray:
    """Seeded long filters for every sample, h [B, N-1, D, L] fp32, drawn like the
    shared filters of ``generate`` (N(0, 1) noise times exp(-alpha_d t / L)) from
    their own PCG64 stream (seed + 4000)."""
    rng = np.random.Generator(np.random.PCG64((wl.seed if seed is None else seed) + 4000))
    B, D, L, N = wl.B, wl.D, wl.L, wl.order
    noise = rng.standard_normal((B, N - 1, D, L), dtype=np.float32)
    alpha = _alphas(D, wl.alpha_lo, wl.alpha_hi)
    t = np.arange(L, dtype=np.float64) / L
    decay = np.exp(-alpha[:, None] * t[None, :]).astype(np.float32)  # [D, L]
    return np.ascontiguousarray((noise * decay[None, None]).astype(np.float32))


def upstream_grad(wl: Workload, seed: Optional[int] = None) -> np.ndarray:
    """A seeded upstream gradient dy [B, D, L] ~ N(0, 1) for the backward, drawn from its
    own PCG64 stream (seed + 1000 by default) and rounded to bf16 for bf16 workloads."""
    rng = np.random.Generator(np.random.PCG64((wl.seed if seed is None else seed) + 1000))
    dy = rng.standard_normal((wl.B, wl.D, wl.L), dtype=np.float32)
    return np.ascontiguousarray(round_to_bf16(dy) if wl.dtype == "bf16" else dy)


@dataclasses.dataclass
class OperatorParams:
    x: np.ndarray      # [B, L, D] float32 (bf16 values for bf16 workloads)
    w_in: np.ndarray   # [(N+1)D, D]
    b_in: np.ndarray   # [(N+1)D]
    w_out: np.ndarray  # [D, D]
    b_out: np.ndarray  # [D]


def operator_params(wl: Workload, seed: Optional[int] = None) -> OperatorParams:
    """Seeded module input and projection parameters for the whole operator:
    x ~ N(0, 1); weights ~ N(0, 1/D) (the variance of PyTorch's default Linear
    initialisation scale); biases ~ N(0, 1/D). Drawn from their own PCG64 stream
    (seed + 2000); rounded to bf16 for bf16 workloads (the rounded values feed
    both sides)."""
    rng = np.random.Generator(np.random.PCG64((wl.seed if seed is None else seed) + 2000))
    B, D, L, C = wl.B, wl.D, wl.L, (wl.order + 1) * wl.D
    sd = np.float32(1.0 / np.sqrt(D))
    x = rng.standard_normal((B, L, D), dtype=np.float32)
    w_in = rng.standard_normal((C, D), dtype=np.float32) * sd
    b_in = rng.standard_normal(C, dtype=np.float32) * sd
    w_out = rng.standard_normal((D, D), dtype=np.float32) * sd
    b_out = rng.standard_normal(D, dtype=np.float32) * sd
    arrs = [x, w_in, b_in, w_out, b_out]
    if wl.dtype == "bf16":
        arrs = [round_to_bf16(a) for a in arrs]
    return OperatorParams(*[np.ascontiguousarray(a, dtype=np.float32) for a in arrs])


@dataclasses.dataclass
class FilterMLP:
    """Parameters of the implicit long-filter generator (HyenaDNA walkthrough,
    section 2.2, HyenaFilter): positional bands, the Linear / Sin stack, the output
    Linear without bias and the exponential modulation rates. With
    E = emb_dim, K = (E-1)/2, W = width, M = num_inner and C = (N-1)*D:"""
    band_freq: np.ndarray  # [K] frequencies of the positional sine/cosine bands
    w_in: np.ndarray       # [W, E]
    b_in: np.ndarray       # [W]
    w_inner: np.ndarray    # [M, W, W]
    b_inner: np.ndarray    # [M, W]
    sin_freq: np.ndarray   # [W] frequency of the Sin activation (shared by all its uses)
    w_out: np.ndarray      # [C, W]
    alpha: np.ndarray      # [C] modulation rates, channel c = o*D + d

    @property
    def emb_dim(self) -> int:
        return int(self.w_in.shape[1])

    @property
    def width(self) -> int:
        return int(self.w_in.shape[0])

    @property
    def num_inner(self) -> int:
        return int(self.w_inner.shape[0])


def filter_mlp(wl: Workload, emb_dim: int = 3, width: int = 16, num_inner: int = 2, w: float = 1.0,
               seed: Optional[int] = None) -> FilterMLP:
    """Seeded parameters of the implicit filter for a workload's plan (D, order),
    defaulting to the walkthrough's HyenaFilter defaults (emb_dim 3, MLP width 16,
    two inner layers, Sin frequency w = 1). Band k (k = 1..K) has frequency k;
    Linear weights and biases ~ N(0, 1/fan_in); alpha_d log-spaced over the
    workload's [alpha_lo, alpha_hi] and shared across o. Drawn from their own PCG64
    stream (seed + 3000)."""
    if emb_dim < 3 or emb_dim % 2 == 0:
        raise ValueError("emb_dim must be odd and at least 3")
    rng = np.random.Generator(np.random.PCG64((wl.seed if seed is None else seed) + 3000))
    E, W, M = emb_dim, width, num_inner
    C = (wl.order - 1) * wl.D
    K = (E - 1) // 2
    band = np.arange(1, K + 1, dtype=np.float32)
    w_in = rng.standard_normal((W, E), dtype=np.float32) * np.float32(1.0 / np.sqrt(E))
    b_in = rng.standard_normal(W, dtype=np.float32) * np.float32(1.0 / np.sqrt(E))
    w_inner = rng.standard_normal((M, W, W), dtype=np.float32) * np.float32(1.0 / np.sqrt(W))
    b_inner = rng.standard_normal((M, W), dtype=np.float32) * np.float32(1.0 / np.sqrt(W))
    sin_freq = np.full(W, w, dtype=np.float32)
    w_out = rng.standard_normal((C, W), dtype=np.float32) * np.float32(1.0 / np.sqrt(W))
    alpha = np.tile(_alphas(wl.D, wl.alpha_lo, wl.alpha_hi), wl.order - 1).astype(np.float32)
    arrs = [band, w_in, b_in, w_inner, b_inner, sin_freq, w_out, alpha]
    return FilterMLP(*[np.ascontiguousarray(a, dtype=np.float32) for a in arrs])


@dataclasses.dataclass
class SynthParams:
    """Parameters of the input-dependent kernel synthesis (a FiLM-modulated
    coordinate SIREN times a Gaussian window), all fp32. A = len(grid) axes,
    W hidden units, M layers, Z control values, C output kernels."""
    grid: tuple          # kernel grid size per axis (axis 0 slowest)
    signed: tuple        # per axis: True for signed (wrapped) offsets, False for causal ones
    w_first: np.ndarray  # [W, A]
    w_hidden: np.ndarray  # [M-1, W, W]
    b_layer: np.ndarray  # [M, W]
    omega: np.ndarray    # [M, W] sine frequencies
    film_g: np.ndarray   # [M, W, Z]  gamma = film_g z + film_gb
    film_gb: np.ndarray  # [M, W]
    film_b: np.ndarray   # [M, W, Z]  beta = film_b z + film_bb
    film_bb: np.ndarray  # [M, W]
    w_out: np.ndarray    # [C, W]
    b_out: np.ndarray    # [C]
    win_mu: np.ndarray   # [C, A] window centres (coordinate units)
    win_sigma: np.ndarray  # [C, A] window widths (coordinate units)


def synthesis_params(grid, signed, channels: int, width: int = 16, layers: int = 2, zdim: int = 8,
                     seed: int = 0) -> SynthParams:
    """Seeded synthesis parameters. SIREN-style draws: first layer U(-1/A, 1/A),
    hidden layers U(-sqrt(6/W)/omega, sqrt(6/W)/omega) per unit, biases U(-1/fan_in,
    1/fan_in); the sine frequencies come in blocks of units with frequencies 1, 4,
    12 and 30 (the multi-frequency initialisation); FiLM maps near the identity
    (gamma = 1 + 0.1 N(0,1) z-terms, beta = 0.1 N(0,1) z-terms); output weights
    N(0, 1/W); window centres U(0, 0.3) on causal axes and U(-0.3, 0.3) on signed
    ones, widths U(0.15, 0.6). Drawn from their own PCG64 stream (seed + 5000)."""
    grid = tuple(int(n) for n in grid)
    signed = tuple(bool(x) for x in signed)
    if not 1 <= len(grid) <= 3 or len(signed) != len(grid):
        raise ValueError("1 to 3 axes, one signed flag per axis")
    rng = np.random.Generator(np.random.PCG64(seed + 5000))
    A, W, M, Z, C = len(grid), width, layers, zdim, channels
    blocks = np.array([1.0, 4.0, 12.0, 30.0])
    omega = np.tile(blocks[(np.arange(W) * len(blocks)) // W], (M, 1))
    w_first = rng.uniform(-1.0 / A, 1.0 / A, (W, A))
    lim = np.sqrt(6.0 / W) / omega[1:, :, None]
    w_hidden = rng.uniform(-1.0, 1.0, (M - 1, W, W)) * lim
    b_layer = np.concatenate([rng.uniform(-1.0 / A, 1.0 / A, (1, W)), rng.uniform(-1.0 / W, 1.0 / W, (M - 1, W))])
    film_g = 0.1 * rng.standard_normal((M, W, Z))
    film_gb = np.ones((M, W))
    film_b = 0.1 * rng.standard_normal((M, W, Z))
    film_bb = np.zeros((M, W))
    w_out = rng.standard_normal((C, W)) / np.sqrt(W)
    b_out = 0.1 * rng.standard_normal(C)
    lo = np.array([-0.3 if sg else 0.0 for sg in signed])
    win_mu = lo + rng.uniform(0.0, 1.0, (C, A)) * (0.3 - lo)
    win_sigma = rng.uniform(0.15, 0.6, (C, A))
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)  # noqa: E731
    return SynthParams(grid, signed, f32(w_first), f32(w_hidden), f32(b_layer), f32(omega), f32(film_g),
                       f32(film_gb), f32(film_b), f32(film_bb), f32(w_out), f32(b_out), f32(win_mu),
                       f32(win_sigma))


def synthesis_controls(B: int, zdim: int, seed: int = 0) -> np.ndarray:
    """Per-sample control vectors z [B, Z] ~ N(0, 1), fp32 (seed + 6000)."""
    rng = np.random.Generator(np.random.PCG64(seed + 6000))
    return rng.standard_normal((B, zdim), dtype=np.float32)


@dataclasses.dataclass
class Conv2dInputs:
    """Inputs of one gated 2-D long-convolution step (all fp32; bf16 values for bf16)."""
    v: np.ndarray     # [B, D, H, W]
    g: np.ndarray     # [B, D, H, W] pre-gate
    x: np.ndarray     # [B, D, H, W] post-gate
    k: np.ndarray     # [D, 2H, 2W] kernel on the doubled grid
    bias: np.ndarray  # [D]


def conv2d_inputs(B: int, D: int, H: int, W: int, dtype: str = "f32", seed: int = 0,
                  centred: bool = True) -> Conv2dInputs:
    """Seeded inputs for the 2-D step: v, g, x ~ N(0, 1); a kernel k[d][i][j] =
    N(0, 1) * exp(-alpha_d * r / max(H, W)) with r the length of the offset the
    doubled-grid position stands for (negative offsets in the upper rows and
    columns when ``centred``; otherwise zero outside [0, H) x [0, W), a causal
    kernel), alpha_d log-spaced over [0.3, 30]; bias ~ N(0, 1). Drawn from one
    PCG64 stream; the activations are rounded to bf16 for bf16 (those values feed
    both sides)."""
    rng = np.random.Generator(np.random.PCG64(seed + 5000))
    v = rng.standard_normal((B, D, H, W), dtype=np.float32)
    g = rng.standard_normal((B, D, H, W), dtype=np.float32)
    x = rng.standard_normal((B, D, H, W), dtype=np.float32)
    noise = rng.standard_normal((D, 2 * H, 2 * W), dtype=np.float32)
    bias = rng.standard_normal(D, dtype=np.float32)
    di = np.arange(2 * H)
    dj = np.arange(2 * W)
    if centred:
        di = np.where(di < H, di, di - 2 * H)
        dj = np.where(dj < W, dj, dj - 2 * W)
    r = np.sqrt(di[:, None].astype(np.float64) ** 2 + dj[None, :].astype(np.float64) ** 2) / max(H, W)
    alpha = _alphas(D, 0.3, 30.0)
    k = noise * np.exp(-alpha[:, None, None] * r[None]).astype(np.float32)
    if not centred:
        k[:, H:, :] = 0.0
        k[:, :, W:] = 0.0
    arrs = [v, g, x]
    if dtype == "bf16":
        arrs = [round_to_bf16(a) for a in arrs]
    return Conv2dInputs(*[np.ascontiguousarray(a, dtype=np.float32) for a in arrs + [k, bias]])


@dataclasses.dataclass
class Conv3dInputs:
    """Inputs of one gated 3-D long-convolution step (all fp32; bf16 values for bf16)."""
    v: np.ndarray     # [B, D, A, H, W]
    g: np.ndarray     # [B, D, A, H, W] pre-gate
    x: np.ndarray     # [B, D, A, H, W] post-gate
    k: np.ndarray     # [D, 2A, 2H, 2W] kernel on the doubled grid
    bias: np.ndarray  # [D]


def conv3d_inputs(B: int, D: int, A: int, H: int, W: int, dtype: str = "f32", seed: int = 0,
                  centred: bool = True) -> Conv3dInputs:
    """Seeded inputs for the 3-D step, drawn as for ``conv2d_inputs`` with one more
    axis: v, g, x ~ N(0, 1); k = N(0, 1) * exp(-alpha_d * r / max(A, H, W)), r the
    length of the offset each doubled-grid position stands for (centred: the upper
    half of every axis holds negative offsets; otherwise a causal kernel, zero
    outside [0, A) x [0, H) x [0, W)); bias ~ N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed + 6000))
    v = rng.standard_normal((B, D, A, H, W), dtype=np.float32)
    g = rng.standard_normal((B, D, A, H, W), dtype=np.float32)
    x = rng.standard_normal((B, D, A, H, W), dtype=np.float32)
    noise = rng.standard_normal((D, 2 * A, 2 * H, 2 * W), dtype=np.float32)
    bias = rng.standard_normal(D, dtype=np.float32)
    offs = []
    for n in (A, H, W):
        o = np.arange(2 * n)
        offs.append(np.where(o < n, o, o - 2 * n) if centred else o)
    r = np.sqrt(offs[0][:, None, None].astype(np.float64) ** 2 + offs[1][None, :, None] ** 2
                + offs[2][None, None, :] ** 2) / max(A, H, W)
    alpha = _alphas(D, 0.3, 30.0)
    k = noise * np.exp(-alpha[:, None, None, None] * r[None]).astype(np.float32)
    if not centred:
        k[:, A:] = 0.0
        k[:, :, H:] = 0.0
        k[:, :, :, W:] = 0.0
    arrs = [v, g, x]
    if dtype == "bf16":
        arrs = [round_to_bf16(a) for a in arrs]
    return Conv3dInputs(*[np.ascontiguousarray(a, dtype=np.float32) for a in arrs + [k, bias]])


def channel_subset(x: Inputs, ds) -> Inputs:
    """The inputs restricted to channels ds of every channel group (gates, value,
    filters, biases): the hot path treats channels independently, so a subset is a
    smaller instance of the same problem."""
    wl = x.wl
    ds = np.asarray(ds, dtype=np.int64)
    N, D = wl.order, wl.D
    cols = np.concatenate([i * D + ds for i in range(N + 1)])
    sub = dataclasses.replace(wl, name=wl.name + f"[{len(ds)}ch]", D=int(len(ds)))
    return Inputs(sub, np.ascontiguousarray(x.u_proj[:, cols]), np.ascontiguousarray(x.short_w[cols]),
                  np.ascontiguousarray(x.h[:, ds]), np.ascontiguousarray(x.bias[:, ds]))


def sample_rows(wl: Workload, count: int, seed: int = 12345) -> np.ndarray:
    """A seeded, sorted sample of flat row indices b*D + d (always includes the first and last)."""
    total = wl.B * wl.D
    if count >= total:
        return np.arange(total, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(seed))
    picks = set(rng.choice(total, size=max(count - 2, 0), replace=False).tolist())
    picks.update({0, total - 1})
    return np.array(sorted(picks), dtype=np.int64)
