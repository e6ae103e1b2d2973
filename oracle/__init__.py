"""fp64 CPU oracle for the Hyena operator forward hot path, its backward, the whole
operator and the implicit filter generator (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product (the HIP library and its binding) never does.

The path's arithmetic lives in ``hyena_oracle.c`` (plain C, fp64, OpenMP over
rows), which this wrapper calls with numpy arrays; see that file's header for the
passages of the pages each step follows and the readings taken where the pages
are silent.  The operator's projections and the implicit filter generator are
written here in numpy fp64 (their docstrings cite their passages and readings).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hyena_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (fp64, -O2, OpenMP). Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER
        f32p, f64p, i64p = P(ctypes.c_float), P(ctypes.c_double), P(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.oracle_short_conv_row.argtypes = [f32p, f32p, i64, f64p]
        lib.oracle_short_conv_row.restype = None
        lib.oracle_causal_conv_direct.argtypes = [f64p, f64p, i64, f64p]
        lib.oracle_causal_conv_direct.restype = None
        lib.oracle_causal_conv_fft.argtypes = [f64p, f64p, i64, f64p]
        lib.oracle_causal_conv_fft.restype = None
        lib.oracle_fft.argtypes = [f64p, f64p, i64, ctypes.c_int]
        lib.oracle_fft.restype = ctypes.c_int
        lib.oracle_hyena_forward.argtypes = [i64, i64, i64, ctypes.c_int, f32p, f64p, f32p, f32p, f32p,
                                             i64p, i64, f64p, ctypes.c_int, ctypes.c_int]
        lib.oracle_hyena_forward.restype = ctypes.c_int
        lib.oracle_causal_corr_direct.argtypes = [f64p, f64p, i64, f64p]
        lib.oracle_causal_corr_direct.restype = None
        lib.oracle_causal_corr_fft.argtypes = [f64p, f64p, i64, f64p]
        lib.oracle_causal_corr_fft.restype = None
        lib.oracle_hyena_backward.argtypes = [i64, i64, i64, ctypes.c_int, f32p, f32p, f32p, f32p, f32p,
                                              f64p, f64p, f64p, f64p, ctypes.c_int, ctypes.c_int]
        lib.oracle_hyena_backward.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def fft(x: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Unscaled radix-2 DFT of a complex vector (sign -1 forward, +1 inverse)."""
    x = np.asarray(x, dtype=np.complex128)
    re = np.ascontiguousarray(x.real, dtype=np.float64).copy()
    im = np.ascontiguousarray(x.imag, dtype=np.float64).copy()
    rc = _load().oracle_fft(_ptr(re, ctypes.c_double), _ptr(im, ctypes.c_double), re.size,
                            1 if inverse else -1)
    if rc != 0:
        raise ValueError("length must be a power of two")
    return re + 1j * im


def short_conv_row(u: np.ndarray, w3: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(u, dtype=np.float32)
    w3 = np.ascontiguousarray(w3, dtype=np.float32)
    out = np.empty(u.size, dtype=np.float64)
    _load().oracle_short_conv_row(_ptr(u, ctypes.c_float), _ptr(w3, ctypes.c_float), u.size,
                                  _ptr(out, ctypes.c_double))
    return out


def causal_conv(v: np.ndarray, h: np.ndarray, mode: str = "fft") -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    h = np.ascontiguousarray(h, dtype=np.float64)
    if v.size != h.size:
        raise ValueError("v and h must have the same length")
    out = np.empty(v.size, dtype=np.float64)
    fn = _load().oracle_causal_conv_fft if mode == "fft" else _load().oracle_causal_conv_direct
    fn(_ptr(v, ctypes.c_double), _ptr(h, ctypes.c_double), v.size, _ptr(out, ctypes.c_double))
    return out


def causal_corr(a: np.ndarray, k: np.ndarray, mode: str = "fft") -> np.ndarray:
    """corr(a, k)[t] = sum_{s >= t} k[s - t] a[s]: the adjoint of v -> conv(v, k)."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    if a.size != k.size:
        raise ValueError("a and k must have the same length")
    out = np.empty(a.size, dtype=np.float64)
    fn = _load().oracle_causal_corr_fft if mode == "fft" else _load().oracle_causal_corr_direct
    fn(_ptr(a, ctypes.c_double), _ptr(k, ctypes.c_double), a.size, _ptr(out, ctypes.c_double))
    return out


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def forward(u_proj: np.ndarray, short_w: np.ndarray, h: np.ndarray, bias: np.ndarray,
            order: int, mode: str = "fft", rows: Optional[Sequence[int]] = None,
            threads: int = 0) -> np.ndarray:
    """Hyena operator forward hot path in fp64.

    u_proj [B,(N+1)D,L], short_w [(N+1)D,3], h [N-1,D,L], bias [N-1,D] (parameters
    taken as fp32 values; u_proj as fp32 values, or used as is when it is float64).
    Returns y as float64, [B,D,L] when ``rows`` is None, otherwise [len(rows), L]
    for the flat rows b*D + d.
    """
    if np.asarray(u_proj).dtype == np.float64:
        u = None
        u64 = np.ascontiguousarray(u_proj)
    else:
        u = np.ascontiguousarray(u_proj, dtype=np.float32)
        u64 = None
    shape_src = u if u is not None else u64
    w = np.ascontiguousarray(short_w, dtype=np.float32)
    hh = np.ascontiguousarray(h, dtype=np.float32)
    bb = np.ascontiguousarray(bias, dtype=np.float32)
    B, C, L = shape_src.shape
    N = int(order)
    if C % (N + 1):
        raise ValueError("u_proj channel count must be (order+1)*D")
    D = C // (N + 1)
    if w.shape != (C, 3) or hh.shape != (N - 1, D, L) or bb.shape != (N - 1, D):
        raise ValueError("parameter shapes do not match u_proj")
    if rows is None:
        out = np.empty((B, D, L), dtype=np.float64)
        rp, nr = None, 0
    else:
        ra = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((ra.size, L), dtype=np.float64)
        rp, nr = _ptr(ra, ctypes.c_int64), ra.size
    up = _ptr(u, ctypes.c_float) if u is not None else None
    u64p = _ptr(u64, ctypes.c_double) if u64 is not None else None
    rc = _load().oracle_hyena_forward(B, D, L, N, up, u64p, _ptr(w, ctypes.c_float),
                                      _ptr(hh, ctypes.c_float), _ptr(bb, ctypes.c_float), rp, nr,
                                      _ptr(out, ctypes.c_double), 0 if mode == "direct" else 1,
                                      int(threads))
    if rc != 0:
        raise ValueError("oracle_hyena_forward rejected its arguments")
    return out


def circular_conv(v: np.ndarray, h: np.ndarray, mode: str = "fft") -> np.ndarray:
    """Circular convolution along the last axis in fp64: out[t] = sum_{s<L} h[s]
    v[(t - s) mod L] (the HyenaND summary's circular boundary mode, for periodic
    data). ``direct`` is that sum written out; ``fft`` multiplies numpy real FFTs of
    length L (no zero padding) and inverts."""
    v = np.asarray(v, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    L = v.shape[-1]
    if mode == "direct":
        idx = (np.arange(L)[:, None] - np.arange(L)[None, :]) % L  # [t, s] -> (t - s) mod L
        return np.einsum("...s,...ts->...t", h, v[..., idx])
    return np.fft.irfft(np.fft.rfft(v, axis=-1) * np.fft.rfft(h, axis=-1), n=L, axis=-1)


def forward_circular(u_proj: np.ndarray, short_w: np.ndarray, h: np.ndarray, bias: np.ndarray, order: int,
                     mode: str = "fft") -> np.ndarray:
    """The hot path with circular long convolutions in fp64 (HyenaDNA walkthrough,
    section 2.1, the gated recurrence; HyenaND summary, circular boundary handling):
    the short conv keeps its causal zero padding (``short_conv_row``), then for
    o = 0..N-2: v = v * x_{N-1-o}; v = circular_conv(v, h[o]) + bias[o] * v; and
    y = v * x_0. Returns [B, D, L] float64."""
    u = np.asarray(u_proj, dtype=np.float32)
    B, C, L = u.shape
    N = int(order)
    D = C // (N + 1)
    w = np.asarray(short_w, dtype=np.float32)
    uc = np.empty((B, C, L), dtype=np.float64)
    for b in range(B):
        for c in range(C):
            uc[b, c] = short_conv_row(u[b, c], w[c])
    x = [uc[:, i * D:(i + 1) * D] for i in range(N)]
    v = uc[:, N * D:]
    hh = np.asarray(h, dtype=np.float32).astype(np.float64)
    bb = np.asarray(bias, dtype=np.float32).astype(np.float64)
    for o in range(N - 1):
        v = v * x[N - 1 - o]
        v = circular_conv(v, hh[o][None], mode=mode) + bb[o][None, :, None] * v
    return v * x[0]


def circular_corr(a: np.ndarray, k: np.ndarray, mode: str = "fft") -> np.ndarray:
    """Circular correlation along the last axis in fp64: out[t] = sum_{s<S}
    k[(s - t) mod S] a[s], the adjoint of v -> circular_conv(v, k) (and of
    k -> circular_conv(v, k) with v in the role of k). ``direct`` writes the sum
    out; ``fft`` multiplies a's real FFT by the conjugate of k's and inverts."""
    a = np.asarray(a, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    S = a.shape[-1]
    if mode == "direct":
        idx = (np.arange(S)[None, :] - np.arange(S)[:, None]) % S  # [t, s] -> (s - t) mod S
        return np.einsum("...s,...ts->...t", a, k[..., idx])
    return np.fft.irfft(np.fft.rfft(a, axis=-1) * np.conj(np.fft.rfft(k, axis=-1)), n=S, axis=-1)


def backward_circular(u_proj: np.ndarray, short_w: np.ndarray, h: np.ndarray, bias: np.ndarray, dy: np.ndarray,
                      order: int, mode: str = "fft"):
    """Gradients of ``forward_circular`` in fp64 for upstream gradient dy [B,D,S]
    (the chain rule of the gated recurrence, HyenaDNA walkthrough section 2.1, with
    the circular long convolution of the HyenaND summary's boundary handling):
    dv_{N-1} = dy * x_0, dx_0 = dy * v_{N-1}; for o = N-2 .. 0 with a = dv_{o+1}:
    dg_o = circular_corr(a, h_o) + bias_o * a, dh_o = sum_b circular_corr(a, g_o),
    dbias_o = sum_b sum_t a g_o, dx_{N-1-o} = dg_o * v_o, dv_o = dg_o * x_{N-1-o};
    then the causal short conv's transpose du[s] = sum_j w_j duc[s + 2 - j] (duc = 0
    past the end) and dw_j = sum_t duc[t] u[t - 2 + j] for every channel.
    Returns (du_proj [B,(N+1)D,S], dshort_w [(N+1)D,3], dh [N-1,D,S], dbias [N-1,D])."""
    u = np.asarray(u_proj, dtype=np.float32).astype(np.float64)
    w = np.asarray(short_w, dtype=np.float32).astype(np.float64)
    hh = np.asarray(h, dtype=np.float32).astype(np.float64)
    bb = np.asarray(bias, dtype=np.float32).astype(np.float64)
    g_up = np.asarray(dy, dtype=np.float32).astype(np.float64)
    B, C, S = u.shape
    N = int(order)
    if C % (N + 1):
        raise ValueError("u_proj channel count must be (order+1)*D")
    D = C // (N + 1)
    if w.shape != (C, 3) or hh.shape != (N - 1, D, S) or bb.shape != (N - 1, D) or g_up.shape != (B, D, S):
        raise ValueError("parameter shapes do not match u_proj")
    # the short conv (causal, zero before t = 0): uc[t] = sum_j w_j u[t - 2 + j]
    upad = np.concatenate([np.zeros((B, C, 2)), u], axis=-1)
    uc = sum(w[None, :, j, None] * upad[:, :, j:j + S] for j in range(3))
    x = [uc[:, i * D:(i + 1) * D] for i in range(N)]
    vs = [uc[:, N * D:]]
    gs = []
    for o in range(N - 1):
        g = vs[o] * x[N - 1 - o]
        gs.append(g)
        vs.append(circular_conv(g, hh[o][None], mode=mode) + bb[o][None, :, None] * g)
    duc = np.zeros((B, C, S))
    duc[:, 0:D] = g_up * vs[N - 1]
    a = g_up * x[0]
    dh = np.zeros((N - 1, D, S))
    db = np.zeros((N - 1, D))
    for o in range(N - 2, -1, -1):
        dh[o] = circular_corr(a, gs[o], mode=mode).sum(axis=0)
        db[o] = (a * gs[o]).sum(axis=(0, 2))
        dg = circular_corr(a, hh[o][None], mode=mode) + bb[o][None, :, None] * a
        gi = N - 1 - o
        duc[:, gi * D:(gi + 1) * D] += dg * vs[o]
        a = dg * x[gi]
    duc[:, N * D:] = a
    # the short conv's transpose and its taps' gradients
    dpad = np.concatenate([duc, np.zeros((B, C, 2))], axis=-1)
    du = sum(w[None, :, j, None] * dpad[:, :, 2 - j:2 - j + S] for j in range(3))
    dw = np.stack([(duc * upad[:, :, j:j + S]).sum(axis=(0, 2)) for j in range(3)], axis=1)
    return du, dw, dh, db


def backward_circular_per_sample(u_proj: np.ndarray, short_w: np.ndarray, h: np.ndarray, bias: np.ndarray,
                                 dy: np.ndarray, order: int, mode: str = "fft"):
    """``backward_circular`` with a filter set per sample (h [B, N-1, D, S]): sample b
    through its own filters; the shared parameters' gradients summed over the samples.
    Returns (du_proj, dshort_w, dh [B,N-1,D,S], dbias)."""
    u = np.asarray(u_proj)
    hb = np.asarray(h)
    g = np.asarray(dy)
    parts = [backward_circular(u[b:b + 1], short_w, hb[b], bias, g[b:b + 1], order, mode=mode)
             for b in range(u.shape[0])]
    return (np.concatenate([p[0] for p in parts], axis=0), np.sum([p[1] for p in parts], axis=0),
            np.stack([p[2] for p in parts]), np.sum([p[3] for p in parts], axis=0))


def conv2d_forward(v: np.ndarray, k: np.ndarray, bias: np.ndarray, g: Optional[np.ndarray] = None,
                   x: Optional[np.ndarray] = None, mode: str = "fft", circular: bool = False) -> np.ndarray:
    """One gated 2-D long-convolution step in fp64 (HyenaND summary, methodology:
    global convolution on the native N-d grid, evaluated by N-d FFT, the input
    zero-padded to double the grid in every dimension for the non-circular mode).
    v, g, x [B, D, H, W]; k [D, 2H, 2W], the kernel on the doubled grid (row i >= H
    and column j >= W hold the offsets i - 2H, j - 2W, so causal and centred kernels
    are both expressible); bias [D]. With s = v * g (s = v when g is None):
      c[p, q] = sum_{i < 2H, j < 2W} k[i, j] s_pad[(p - i) mod 2H, (q - j) mod 2W],
    p < H, q < W, s_pad being s zero-padded to 2H x 2W; y = (c + bias * s) * x (no
    factor when x is None). ``direct`` is that sum written out; ``fft`` multiplies
    numpy's rfft2 of the padded input and of the kernel and inverts.
    ``circular`` (the summary's boundary handling for periodic systems): no padding,
    k [D, H, W] on the grid itself, c[p, q] = sum_{i < H, j < W} k[i, j]
    s[(p - i) mod H, (q - j) mod W].
    Returns [B, D, H, W] float64."""
    s = np.asarray(v, dtype=np.float64)
    if g is not None:
        s = s * np.asarray(g, dtype=np.float64)
    B, D, H, W = s.shape
    kk = np.asarray(k, dtype=np.float64)
    if circular:
        if kk.shape != (D, H, W):
            raise ValueError("k must be [D, H, W] for a circular step")
        if mode == "direct":
            c = np.zeros((B, D, H, W))
            for i in range(H):
                for j in range(W):
                    c += kk[None, :, i, j, None, None] * np.roll(s, (i, j), axis=(2, 3))
        else:
            c = np.fft.irfft2(np.fft.rfft2(s) * np.fft.rfft2(kk)[None], s=(H, W))
    elif kk.shape != (D, 2 * H, 2 * W):
        raise ValueError("k must be [D, 2H, 2W]")
    elif mode == "direct":
        sp = np.zeros((B, D, 2 * H, 2 * W))
        sp[:, :, :H, :W] = s
        c = np.zeros((B, D, H, W))
        for i in range(2 * H):
            for j in range(2 * W):
                # shifted copy: entry (p, q) holds s_pad[(p - i) mod 2H, (q - j) mod 2W]
                sh = np.roll(np.roll(sp, i, axis=2), j, axis=3)[:, :, :H, :W]
                c += kk[None, :, i, j, None, None] * sh
    else:
        S = np.fft.rfft2(s, s=(2 * H, 2 * W))
        Kh = np.fft.rfft2(kk)
        c = np.fft.irfft2(S * Kh[None], s=(2 * H, 2 * W))[:, :, :H, :W]
    y = c + np.asarray(bias, dtype=np.float64)[None, :, None, None] * s
    if x is not None:
        y = y * np.asarray(x, dtype=np.float64)
    return y


def conv3d_forward(v: np.ndarray, k: np.ndarray, bias: np.ndarray, g: Optional[np.ndarray] = None,
                   x: Optional[np.ndarray] = None, mode: str = "fft", circular: bool = False) -> np.ndarray:
    """One gated 3-D long-convolution step in fp64: ``conv2d_forward`` with one more
    grid axis (HyenaND summary, methodology: global convolution on the native N-d
    grid by an N-d FFT, the input zero-padded to double the grid in every dimension
    for the non-circular mode). v, g, x [B, D, A, H, W]; k [D, 2A, 2H, 2W] on the
    doubled grid (index >= the axis length holds the negative offset, as in 2-D);
    bias [D]. With s = v * g:
      c[a, p, q] = sum_{l < 2A, i < 2H, j < 2W} k[l, i, j]
                   s_pad[(a - l) mod 2A, (p - i) mod 2H, (q - j) mod 2W],
    a < A, p < H, q < W; y = (c + bias * s) * x. ``direct`` is that sum written out;
    ``fft`` multiplies numpy's rfftn of the padded input and of the kernel.
    ``circular``: no padding, k [D, A, H, W] on the grid itself, every index taken
    modulo its own axis length.
    Returns [B, D, A, H, W] float64."""
    s = np.asarray(v, dtype=np.float64)
    if g is not None:
        s = s * np.asarray(g, dtype=np.float64)
    B, D, A, H, W = s.shape
    kk = np.asarray(k, dtype=np.float64)
    if circular:
        if kk.shape != (D, A, H, W):
            raise ValueError("k must be [D, A, H, W] for a circular step")
        if mode == "direct":
            c = np.zeros((B, D, A, H, W))
            for l in range(A):
                for i in range(H):
                    for j in range(W):
                        c += kk[None, :, l, i, j, None, None, None] * np.roll(s, (l, i, j), axis=(2, 3, 4))
        else:
            c = np.fft.irfftn(np.fft.rfftn(s, axes=(2, 3, 4)) * np.fft.rfftn(kk, axes=(1, 2, 3))[None],
                              s=(A, H, W), axes=(2, 3, 4))
    elif kk.shape != (D, 2 * A, 2 * H, 2 * W):
        raise ValueError("k must be [D, 2A, 2H, 2W]")
    elif mode == "direct":
        sp = np.zeros((B, D, 2 * A, 2 * H, 2 * W))
        sp[:, :, :A, :H, :W] = s
        c = np.zeros((B, D, A, H, W))
        for l in range(2 * A):
            for i in range(2 * H):
                for j in range(2 * W):
                    sh = np.roll(sp, (l, i, j), axis=(2, 3, 4))[:, :, :A, :H, :W]
                    c += kk[None, :, l, i, j, None, None, None] * sh
    else:
        S = np.fft.rfftn(s, s=(2 * A, 2 * H, 2 * W), axes=(2, 3, 4))
        Kh = np.fft.rfftn(kk, axes=(1, 2, 3))
        c = np.fft.irfftn(S * Kh[None], s=(2 * A, 2 * H, 2 * W), axes=(2, 3, 4))[:, :, :A, :H, :W]
    y = c + np.asarray(bias, dtype=np.float64)[None, :, None, None, None] * s
    if x is not None:
        y = y * np.asarray(x, dtype=np.float64)
    return y


def forward_per_sample(u_proj: np.ndarray, short_w: np.ndarray, h: np.ndarray, bias: np.ndarray, order: int,
                       mode: str = "fft", threads: int = 0) -> np.ndarray:
    """The hot path with a filter set per sample (input-dependent long convolutions,
    HyenaND summary, methodology: the kernel is conditioned on the whole input
    sample): sample b of u_proj [B, (N+1)D, L] runs through ``forward`` with the
    filters h[b] of h [B, N-1, D, L]; short_w and bias are shared. Returns
    [B, D, L] float64."""
    u = np.asarray(u_proj)
    hb = np.asarray(h)
    if hb.ndim != 4 or hb.shape[0] != u.shape[0]:
        raise ValueError("h must be [B, N-1, D, L] with the B of u_proj")
    return np.concatenate([forward(u[b:b + 1], short_w, hb[b], bias, order, mode=mode, threads=threads)
                           for b in range(u.shape[0])], axis=0)


def backward(u_proj: np.ndarray, short_w: np.ndarray, h: np.ndarray, bias: np.ndarray, dy: np.ndarray,
             order: int, mode: str = "fft", threads: int = 0):
    """Gradients of the hot path in fp64 for upstream gradient dy [B,D,L].

    Returns (du_proj [B,(N+1)D,L], dshort_w [(N+1)D,3], dh [N-1,D,L], dbias [N-1,D]),
    all float64; every input is taken as fp32 values.
    """
    u = np.ascontiguousarray(u_proj, dtype=np.float32)
    w = np.ascontiguousarray(short_w, dtype=np.float32)
    hh = np.ascontiguousarray(h, dtype=np.float32)
    bb = np.ascontiguousarray(bias, dtype=np.float32)
    g = np.ascontiguousarray(dy, dtype=np.float32)
    B, C, L = u.shape
    N = int(order)
    if C % (N + 1):
        raise ValueError("u_proj channel count must be (order+1)*D")
    D = C // (N + 1)
    if w.shape != (C, 3) or hh.shape != (N - 1, D, L) or bb.shape != (N - 1, D) or g.shape != (B, D, L):
        raise ValueError("parameter shapes do not match u_proj")
    du = np.empty((B, C, L), dtype=np.float64)
    dw = np.empty((C, 3), dtype=np.float64)
    dh = np.empty((N - 1, D, L), dtype=np.float64)
    db = np.empty((N - 1, D), dtype=np.float64)
    d64 = ctypes.c_double
    rc = _load().oracle_hyena_backward(B, D, L, N, _ptr(u, ctypes.c_float), _ptr(w, ctypes.c_float),
                                       _ptr(hh, ctypes.c_float), _ptr(bb, ctypes.c_float),
                                       _ptr(g, ctypes.c_float), _ptr(du, d64), _ptr(dw, d64), _ptr(dh, d64),
                                       _ptr(db, d64), 0 if mode == "direct" else 1, int(threads))
    if rc != 0:
        raise ValueError("oracle_hyena_backward rejected its arguments")
    return du, dw, dh, db


def backward_per_sample(u_proj: np.ndarray, short_w: np.ndarray, h: np.ndarray, bias: np.ndarray, dy: np.ndarray,
                        order: int, mode: str = "fft", threads: int = 0):
    """Gradients of ``forward_per_sample`` (a filter set per sample, HyenaND summary,
    methodology): sample b runs through ``backward`` with its own filters h[b] of
    h [B, N-1, D, L]; the shared parameters' gradients are summed over the samples.
    Returns (du_proj [B,(N+1)D,L], dshort_w [(N+1)D,3], dh [B,N-1,D,L], dbias [N-1,D])."""
    u = np.asarray(u_proj)
    hb = np.asarray(h)
    g = np.asarray(dy)
    if hb.ndim != 4 or hb.shape[0] != u.shape[0]:
        raise ValueError("h must be [B, N-1, D, L] with the B of u_proj")
    parts = [backward(u[b:b + 1], short_w, hb[b], bias, g[b:b + 1], order, mode=mode, threads=threads)
             for b in range(u.shape[0])]
    du = np.concatenate([p[0] for p in parts], axis=0)
    dw = np.sum([p[1] for p in parts], axis=0)
    dh = np.stack([p[2] for p in parts])
    db = np.sum([p[3] for p in parts], axis=0)
    return du, dw, dh, db


def operator_forward(x: np.ndarray, w_in: np.ndarray, b_in: np.ndarray, short_w: np.ndarray, h: np.ndarray,
                     bias: np.ndarray, w_out: np.ndarray, b_out: np.ndarray, order: int, mode: str = "fft",
                     threads: int = 0) -> np.ndarray:
    """The whole operator forward in fp64 (HyenaDNA walkthrough, section 2.1,
    HyenaOperator.forward): u = in_proj(x) = x w_in^T + b_in on x [B, L, D]; the
    (B, L, D) -> (B, D, L) transpose; the hot path (``forward``); the (B, D, L) -> (B, L, D)
    rearrange; out_proj = y w_out^T + b_out. The projections are numpy matrix
    products in fp64. Returns [B, L, D] float64."""
    x64 = np.asarray(x, dtype=np.float64)
    u = x64 @ np.asarray(w_in, np.float64).T + np.asarray(b_in, np.float64)  # [B, L, (N+1)D]
    u_proj = np.ascontiguousarray(u.transpose(0, 2, 1))                      # [B, (N+1)D, L]
    y = forward(u_proj, short_w, h, bias, order, mode=mode, threads=threads)  # [B, D, L]
    return y.transpose(0, 2, 1) @ np.asarray(w_out, np.float64).T + np.asarray(b_out, np.float64)


def positional_embedding(L: int, band_freq: np.ndarray):
    """The positional features of the implicit filter (HyenaDNA walkthrough, section
    2.2: PositionalEmbedding gives every time step sine/cosine bands plus a linear time
    term; emb_dim odd, (emb_dim - 1)/2 bands). The pages give no formula; reading
    taken: t = tau / L for tau = 0..L-1 and z[tau] = (t, sin(2 pi f_k t) for each band
    k, then cos(2 pi f_k t) for each band k), with the band frequencies f_k an input.
    Returns (z [L, 1 + 2K], t [L]) in float64."""
    f = np.asarray(band_freq, dtype=np.float64).reshape(-1)
    t = np.arange(L, dtype=np.float64) / L
    ang = 2.0 * np.pi * t[:, None] * f[None, :]
    z = np.concatenate([t[:, None], np.sin(ang), np.cos(ang)], axis=1)
    return z, t


def implicit_filter(L: int, D: int, order: int, p) -> np.ndarray:
    """The implicit long filters h [N-1, D, L] in float64 (HyenaDNA walkthrough,
    section 2.2, the HyenaFilter module and its filter method).

    With z(tau) the positional embedding of step tau and t = tau / L:
        a_0     = sin(f * (W_in z + b_in))
        a_m     = sin(f * (W_m a_{m-1} + b_m)),   m = 1 .. num_inner
        g_c     = (W_out a_last)_c                (no bias)
        h[c, tau] = g_c * exp(-alpha_c * t)
    for the (N-1)*D output channels c = o*D + d, which are laid out as h[o][d][tau]
    (section 2.1 reshapes the time-major filter into that order).  Readings taken
    where the formulas are absent: the activation is an elementwise sine of the
    pre-activation scaled by a per-unit frequency vector f, one vector for every
    layer (the walkthrough builds a single activation object and reuses it after
    each linear layer); the modulation's t is the embedding's t.  `p` carries the
    fields of synth.FilterMLP."""
    z, t = positional_embedding(L, p.band_freq)
    freq = np.asarray(p.sin_freq, np.float64)
    a = np.sin(freq * (z @ np.asarray(p.w_in, np.float64).T + np.asarray(p.b_in, np.float64)))
    for m in range(np.asarray(p.w_inner).shape[0]):
        a = np.sin(freq * (a @ np.asarray(p.w_inner[m], np.float64).T + np.asarray(p.b_inner[m], np.float64)))
    g = a @ np.asarray(p.w_out, np.float64).T
    h = g * np.exp(-np.outer(t, np.asarray(p.alpha, np.float64)))
    C = (order - 1) * D
    if h.shape != (L, C):
        raise ValueError(f"w_out has {h.shape[1]} rows, the plan needs (order-1)*D = {C}")
    return np.ascontiguousarray(h.T.reshape(order - 1, D, L))


def synthesis_coords(grid, signed) -> np.ndarray:
    """Coordinates of the points of a kernel grid, [P, A] float64 with the points in
    row-major order (axis 0 slowest). Reading taken (the HyenaND summary, method,
    kernel parametrisation, defines the kernel on a continuous coordinate grid but
    gives no mapping): index j of a causal axis of n points sits at c = j / n in
    [0, 1); a signed axis of n points holds the offsets j for j < n/2 and j - n
    above (the wrapped layout of a kernel on a doubled or periodic grid), at
    c = 2 * offset / n in [-1, 1)."""
    axes = []
    for n, sg in zip(grid, signed):
        j = np.arange(n, dtype=np.float64)
        if sg:
            off = np.where(j < n // 2, j, j - n)
            axes.append(2.0 * off / n)
        else:
            axes.append(j / n)
    mesh = np.meshgrid(*axes, indexing="ij")
    return np.stack([m.reshape(-1) for m in mesh], axis=1)


def kernel_synthesis(p, z: np.ndarray) -> np.ndarray:
    """Input-dependent kernels K [B, C, *grid] in float64 (HyenaND summary, method:
    input-dependent kernels through registers and FiLM, kernel synthesis, kernel
    parametrisation): K_b = w(c) * f(c; z_b) at every grid coordinate c, where f is
    a coordinate SIREN whose layers are modulated by FiLM from the sample's control
    vector z_b, and w is a Gaussian window per output kernel.

    With h_0 = c and, for layers l = 0 .. M-1 (W_0 = w_first, W_l = w_hidden[l-1]):
        a_l     = W_l h_l + b_l
        gamma_l = G_l z_b + g_l,   beta_l = E_l z_b + e_l
        h_{l+1} = sin(omega_l * (gamma_l * a_l + beta_l))
    f = W_out h_M + b_out, and for kernel k
        w_k(c)  = exp(-1/2 sum_i ((c_i - mu_{k,i}) / sigma_{k,i})^2).
    Readings taken where the summary gives no formula: the SIREN activation is
    sin(omega * x) with a frequency per hidden unit (the multi-frequency
    initialisation gives blocks of units different frequencies); FiLM scales and
    shifts the pre-activation inside the sine, with gamma and beta affine in z per
    layer; the output layer is affine with no sine; the window is an axis-aligned
    Gaussian per output kernel; z_b is given (the register tokens and their softmax
    pooling belong to the model around the operator). `p` carries the fields of
    synth.SynthParams; z is [B, Z]."""
    c = synthesis_coords(p.grid, p.signed)
    z = np.asarray(z, np.float64)
    M = np.asarray(p.b_layer).shape[0]
    f64 = lambda a: np.asarray(a, np.float64)  # noqa: E731
    mu, sigma = f64(p.win_mu), f64(p.win_sigma)
    win = np.exp(-0.5 * np.sum(((c[:, None, :] - mu[None]) / sigma[None]) ** 2, axis=2))  # [P, C]
    C = mu.shape[0]
    out = np.empty((z.shape[0], C) + tuple(p.grid))
    for b in range(z.shape[0]):
        h = c
        for layer in range(M):
            Wl = f64(p.w_first) if layer == 0 else f64(p.w_hidden)[layer - 1]
            a = h @ Wl.T + f64(p.b_layer)[layer]
            gamma = f64(p.film_g)[layer] @ z[b] + f64(p.film_gb)[layer]
            beta = f64(p.film_b)[layer] @ z[b] + f64(p.film_bb)[layer]
            h = np.sin(f64(p.omega)[layer] * (gamma * a + beta))
        f = h @ f64(p.w_out).T + f64(p.b_out)  # [P, C]
        out[b] = (win * f).T.reshape((C,) + tuple(p.grid))
    return out


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_2 / ||ref||_2 over every element, with got widened to fp64.

    The two arrays must have the same shape (no broadcasting: a mis-shaped result
    raises instead of being compared against a stretched reference).  With an
    all-zero reference the absolute norm ||got||_2 is returned."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"rel_l2: shape {g.shape} of the result differs from the reference's {r.shape}")
    den = float(np.linalg.norm(r.ravel()))
    num = float(np.linalg.norm((g - r).ravel()))
    return num / den if den > 0 else num
