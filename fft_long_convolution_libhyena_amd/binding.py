"""Thin ctypes binding over libhyena's C ABI (include/hyena.h).

Only argument marshalling happens here: shapes and dtypes are checked, torch
tensors supply device pointers and the current HIP stream, and every step of
the hot path runs in the library's HIP kernels. There is no fallback: if
libhyena.so is missing or no GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhyena.so")

HYENA_F32, HYENA_BF16 = 0, 1
PATH_AUTO, PATH_LDS, PATH_FOURSTEP, PATH_PARTITIONED = 0, 1, 2, 4
STATUS = {0: "HYENA_OK", 1: "HYENA_ERR_INVALID_ARG", 2: "HYENA_ERR_UNSUPPORTED",
          3: "HYENA_ERR_WORKSPACE", 4: "HYENA_ERR_DEVICE"}
_PATHS = {"auto": PATH_AUTO, "lds": PATH_LDS, "fourstep": PATH_FOURSTEP, "partitioned": PATH_PARTITIONED}
_DTYPES = {"f32": HYENA_F32, "bf16": HYENA_BF16}

# every symbol include/hyena.h declares
FLAG_CIRCULAR = 1  # HYENA_FLAG_CIRCULAR

EXPORTS = ("hyena_plan_create", "hyena_plan_create_path", "hyena_plan_create_ex", "hyena_plan_destroy", "hyena_plan_path",
           "hyena_spectrum_bytes", "hyena_workspace_bytes", "hyena_filter_spectrum", "hyena_forward",
           "hyena_forward_timed", "hyena_backward_workspace_bytes", "hyena_backward",
           "hyena_backward_per_sample_workspace_bytes", "hyena_backward_per_sample",
           "hyena_operator_workspace_bytes", "hyena_operator_forward", "hyena_operator_forward_timed", "hyena_operator_tune",
           "hyena_implicit_filter", "hyena_filter_spectrum_batched", "hyena_forward_per_sample",
           "hyena_plan2d_create", "hyena_plan2d_destroy", "hyena_spectrum2d_bytes", "hyena_workspace2d_bytes",
           "hyena_filter_spectrum2d", "hyena_conv2d_forward", "hyena_plan3d_create", "hyena_plan3d_destroy",
           "hyena_spectrum3d_bytes", "hyena_workspace3d_bytes", "hyena_filter_spectrum3d", "hyena_conv3d_forward",
           "hyena_filter_spectrum2d_batched", "hyena_conv2d_forward_per_sample", "hyena_filter_spectrum3d_batched",
           "hyena_conv3d_forward_per_sample", "hyena_plan2d_create_ex", "hyena_plan3d_create_ex",
           "hyena_forward_noalloc", "hyena_kernel_synthesis", "hyena_status_string")


class FilterMLPStruct(ctypes.Structure):
    """hyena_filter_mlp_t: sizes, then device pointers of the filter generator's
    parameters (see include/hyena.h)."""
    _fields_ = [("emb_dim", ctypes.c_int64), ("width", ctypes.c_int64), ("num_inner", ctypes.c_int64),
                ("band_freq", ctypes.c_void_p), ("w_in", ctypes.c_void_p), ("b_in", ctypes.c_void_p),
                ("w_inner", ctypes.c_void_p), ("b_inner", ctypes.c_void_p), ("sin_freq", ctypes.c_void_p),
                ("w_out", ctypes.c_void_p), ("alpha", ctypes.c_void_p)]


class SynthParamsStruct(ctypes.Structure):
    """hyena_synth_params_t: sizes, then device pointers of the kernel-synthesis
    parameters (see include/hyena.h)."""
    _fields_ = [("axes", ctypes.c_int64), ("grid", ctypes.c_int64 * 3), ("signed_axes", ctypes.c_uint32),
                ("width", ctypes.c_int64), ("layers", ctypes.c_int64), ("zdim", ctypes.c_int64),
                ("channels", ctypes.c_int64)] + [(n, ctypes.c_void_p) for n in (
                    "w_first", "w_hidden", "b_layer", "omega", "film_g", "film_gb", "film_b", "film_bb", "w_out",
                    "b_out", "win_mu", "win_sigma")]


class HyenaError(RuntimeError):
    def __init__(self, call: str, status: int, detail: str = ""):
        self.status = status
        super().__init__(f"{call} failed: {STATUS.get(status, status)}" + (f" ({detail})" if detail else ""))


def _env_flag(name: str) -> bool:
    return os.environ.get(name, "") not in ("", "0")


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libhyena.so and declare its signatures (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libhyena is not built ({p} is missing); run __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    ci = ctypes.c_int
    lib.hyena_plan_create.argtypes = [ctypes.POINTER(vp), i64, i64, ci, ci]
    lib.hyena_plan_create.restype = ci
    lib.hyena_plan_create_path.argtypes = [ctypes.POINTER(vp), i64, i64, ci, ci, ci]
    lib.hyena_plan_create_path.restype = ci
    lib.hyena_plan_create_ex.argtypes = [ctypes.POINTER(vp), i64, i64, ci, ci, ci, ctypes.c_uint32]
    lib.hyena_plan_create_ex.restype = ci
    lib.hyena_plan_destroy.argtypes = [vp]
    lib.hyena_plan_destroy.restype = ci
    lib.hyena_plan_path.argtypes = [vp]
    lib.hyena_plan_path.restype = ci
    lib.hyena_spectrum_bytes.argtypes = [vp]
    lib.hyena_spectrum_bytes.restype = sz
    lib.hyena_workspace_bytes.argtypes = [vp, i64]
    lib.hyena_workspace_bytes.restype = sz
    lib.hyena_filter_spectrum.argtypes = [vp, vp, vp, vp]
    lib.hyena_filter_spectrum.restype = ci
    lib.hyena_forward.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hyena_forward.restype = ci
    lib.hyena_filter_spectrum_batched.argtypes = [vp, i64, vp, vp, vp]
    lib.hyena_filter_spectrum_batched.restype = ci
    lib.hyena_forward_per_sample.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hyena_forward_per_sample.restype = ci
    lib.hyena_kernel_synthesis.argtypes = [ctypes.POINTER(SynthParamsStruct), i64, vp, vp, vp]
    lib.hyena_kernel_synthesis.restype = ci
    lib.hyena_forward_noalloc.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp]
    lib.hyena_forward_noalloc.restype = ci
    lib.hyena_forward_timed.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, sz, vp, ctypes.POINTER(ctypes.c_float)]
    lib.hyena_forward_timed.restype = ci
    lib.hyena_backward_workspace_bytes.argtypes = [vp, i64]
    lib.hyena_backward_workspace_bytes.restype = sz
    lib.hyena_backward.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hyena_backward.restype = ci
    lib.hyena_backward_per_sample_workspace_bytes.argtypes = [vp, i64]
    lib.hyena_backward_per_sample_workspace_bytes.restype = sz
    lib.hyena_backward_per_sample.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hyena_backward_per_sample.restype = ci
    lib.hyena_operator_workspace_bytes.argtypes = [vp, i64]
    lib.hyena_operator_workspace_bytes.restype = sz
    lib.hyena_operator_forward.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hyena_operator_forward.restype = ci
    lib.hyena_operator_tune.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hyena_operator_tune.restype = ci
    lib.hyena_operator_forward_timed.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                                 ctypes.POINTER(ctypes.c_float)]
    lib.hyena_operator_forward_timed.restype = ci
    lib.hyena_implicit_filter.argtypes = [vp, ctypes.POINTER(FilterMLPStruct), vp, vp]
    lib.hyena_implicit_filter.restype = ci
    lib.hyena_plan2d_create.argtypes = [ctypes.POINTER(vp), i64, i64, i64, ci]
    lib.hyena_plan2d_create.restype = ci
    lib.hyena_plan2d_destroy.argtypes = [vp]
    lib.hyena_plan2d_destroy.restype = ci
    lib.hyena_spectrum2d_bytes.argtypes = [vp]
    lib.hyena_spectrum2d_bytes.restype = sz
    lib.hyena_workspace2d_bytes.argtypes = [vp, i64]
    lib.hyena_workspace2d_bytes.restype = sz
    lib.hyena_filter_spectrum2d.argtypes = [vp, vp, vp, vp]
    lib.hyena_filter_spectrum2d.restype = ci
    lib.hyena_conv2d_forward.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hyena_conv2d_forward.restype = ci
    lib.hyena_plan3d_create.argtypes = [ctypes.POINTER(vp), i64, i64, i64, i64, ci]
    lib.hyena_plan3d_create.restype = ci
    lib.hyena_plan3d_destroy.argtypes = [vp]
    lib.hyena_plan3d_destroy.restype = ci
    lib.hyena_spectrum3d_bytes.argtypes = [vp]
    lib.hyena_spectrum3d_bytes.restype = sz
    lib.hyena_workspace3d_bytes.argtypes = [vp, i64]
    lib.hyena_workspace3d_bytes.restype = sz
    lib.hyena_filter_spectrum3d.argtypes = [vp, vp, vp, vp]
    lib.hyena_filter_spectrum3d.restype = ci
    lib.hyena_conv3d_forward.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hyena_conv3d_forward.restype = ci
    lib.hyena_plan2d_create_ex.argtypes = [ctypes.POINTER(vp), i64, i64, i64, ci, ctypes.c_uint32]
    lib.hyena_plan2d_create_ex.restype = ci
    lib.hyena_plan3d_create_ex.argtypes = [ctypes.POINTER(vp), i64, i64, i64, i64, ci, ctypes.c_uint32]
    lib.hyena_plan3d_create_ex.restype = ci
    for nd in ("2d", "3d"):
        getattr(lib, f"hyena_filter_spectrum{nd}_batched").argtypes = [vp, i64, vp, vp, vp]
        getattr(lib, f"hyena_filter_spectrum{nd}_batched").restype = ci
        getattr(lib, f"hyena_conv{nd}_forward_per_sample").argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        getattr(lib, f"hyena_conv{nd}_forward_per_sample").restype = ci
    lib.hyena_status_string.argtypes = [ci]
    lib.hyena_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(call: str, st: int) -> None:
    """Raise HyenaError for a failed call. With HYENA_DEBUG_SYNC set (debugging
    only), every call that queued work is also followed by a device
    synchronisation, so that an asynchronous kernel error is reported against the
    call that launched it (as HYENA_ERR_DEVICE) instead of a later one."""
    if st != 0:
        raise HyenaError(call, st)
    if _env_flag("HYENA_DEBUG_SYNC"):
        import torch

        if torch.cuda.is_available():
            try:
                torch.cuda.synchronize()
            except RuntimeError as e:
                raise HyenaError(call, 4, f"after synchronisation: {e}") from e


def _stream_handle(torch, device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def kernel_synthesis(params, z, out=None):
    """hyena_kernel_synthesis: the input-dependent kernels of B samples.
    `params` has the fields of synth.SynthParams as fp32 device tensors (grid and
    signed as tuples); z is [B, Z] fp32 on the device. Returns k [B, C, *grid]."""
    import torch

    lib = load_library()
    z = z.contiguous()
    B, Z = int(z.shape[0]), int(z.shape[1])
    grid = tuple(int(n) for n in params.grid)
    A = len(grid)
    C, W = int(params.w_out.shape[0]), int(params.w_out.shape[1])
    M = int(params.b_layer.shape[0])
    dev = z.device
    want = {"w_first": (W, A), "w_hidden": (M - 1, W, W), "b_layer": (M, W), "omega": (M, W), "film_g": (M, W, Z),
            "film_gb": (M, W), "film_b": (M, W, Z), "film_bb": (M, W), "w_out": (C, W), "b_out": (C,),
            "win_mu": (C, A), "win_sigma": (C, A)}
    ptrs = {}
    for name, shape in want.items():
        t = getattr(params, name)
        if tuple(t.shape) != shape or t.dtype != torch.float32 or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp32 device tensor of shape {shape}")
        ptrs[name] = t.data_ptr() if t.numel() else None
    if z.dtype != torch.float32:
        raise ValueError("z must be fp32")
    if out is None:
        out = torch.empty((B, C) + grid, dtype=torch.float32, device=dev)
    if tuple(out.shape) != (B, C) + grid or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor [B, C, *grid]")
    st = SynthParamsStruct()
    st.axes, st.width, st.layers, st.zdim, st.channels = A, W, M, Z, C
    for i in range(3):
        st.grid[i] = grid[i] if i < A else 1
    st.signed_axes = sum(1 << i for i, sg in enumerate(params.signed) if sg)
    for name, ptr in ptrs.items():
        setattr(st, name, ptr)
    _check("hyena_kernel_synthesis",
           lib.hyena_kernel_synthesis(ctypes.byref(st), B, z.data_ptr(), out.data_ptr(), _stream_handle(torch, dev)))
    return out


class Plan:
    """A libhyena plan: fixed L, D, order and I/O dtype ("f32" or "bf16")."""

    def __init__(self, L: int, D: int, order: int, dtype: str = "f32", path: str = "auto",
                 circular: bool = False):
        """path "auto" lets the library choose; the environment variable
        HYENA_FORCE_PATH (lds, fourstep or partitioned) overrides that choice for
        plans created with path "auto" (a debugging switch, e.g. to run the four-step
        passes at sizes the LDS kernel would take)."""
        import torch  # device memory and streams only

        if path == "auto" and os.environ.get("HYENA_FORCE_PATH"):
            path = os.environ["HYENA_FORCE_PATH"]

        self._torch = torch
        self.lib = load_library()
        self.L, self.D, self.order, self.dtype = int(L), int(D), int(order), dtype
        self.circular = bool(circular)
        if dtype not in _DTYPES or path not in _PATHS:
            raise ValueError(f"dtype must be one of {list(_DTYPES)}, path one of {list(_PATHS)}")
        self.device = torch.device("cuda", torch.cuda.current_device())
        h = ctypes.c_void_p()
        _check("hyena_plan_create_ex",
               self.lib.hyena_plan_create_ex(ctypes.byref(h), self.L, self.D, self.order, _DTYPES[dtype],
                                             _PATHS[path], FLAG_CIRCULAR if self.circular else 0))
        self.handle = h
        self.path = {PATH_LDS: "lds", PATH_FOURSTEP: "fourstep",
                     PATH_PARTITIONED: "partitioned"}[self.lib.hyena_plan_path(h)]

    @property
    def io_dtype(self):
        return self._torch.bfloat16 if self.dtype == "bf16" else self._torch.float32

    def spectrum_bytes(self) -> int:
        return int(self.lib.hyena_spectrum_bytes(self.handle))

    def workspace_bytes(self, B: int) -> int:
        return int(self.lib.hyena_workspace_bytes(self.handle, int(B)))

    def _need(self, t, name, shape, dtype):
        torch = self._torch
        if not isinstance(t, torch.Tensor) or t.device != self.device:
            raise ValueError(f"{name} must be a tensor on {self.device}")
        if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                             f"got {t.dtype} {tuple(t.shape)}")

    def spectrum(self, h, out=None):
        """hyena_filter_spectrum: h [N-1, D, L] fp32 -> opaque uint8 device buffer."""
        torch = self._torch
        N, D, L = self.order, self.D, self.L
        self._need(h, "h", (N - 1, D, L), torch.float32)
        if out is None:
            out = torch.empty(self.spectrum_bytes(), dtype=torch.uint8, device=self.device)
        elif out.numel() * out.element_size() < self.spectrum_bytes():
            raise ValueError("spectrum buffer too small")
        _check("hyena_filter_spectrum",
               self.lib.hyena_filter_spectrum(self.handle, h.data_ptr(), out.data_ptr(),
                                              _stream_handle(torch, self.device)))
        return out

    def implicit_filter(self, mlp, out=None):
        """hyena_implicit_filter: the plan's long filters h [N-1, D, L] fp32 from the
        filter generator's parameters. `mlp` has the fields of synth.FilterMLP as
        contiguous fp32 tensors on the plan's device (band_freq [K], w_in [W, E],
        b_in [W], w_inner [M, W, W], b_inner [M, W], sin_freq [W], w_out [C, W],
        alpha [C])."""
        torch = self._torch
        N, D, L = self.order, self.D, self.L
        C = (N - 1) * D
        W, E = (int(v) for v in mlp.w_in.shape)
        M = int(mlp.w_inner.shape[0])
        K = (E - 1) // 2
        for name, shape in (("band_freq", (K,)), ("w_in", (W, E)), ("b_in", (W,)), ("w_inner", (M, W, W)),
                            ("b_inner", (M, W)), ("sin_freq", (W,)), ("w_out", (C, W)), ("alpha", (C,))):
            self._need(getattr(mlp, name), name, shape, torch.float32)
        if out is None:
            out = torch.empty((N - 1, D, L), dtype=torch.float32, device=self.device)
        self._need(out, "h", (N - 1, D, L), torch.float32)
        ptr = lambda t: t.data_ptr() if t.numel() else None  # noqa: E731
        st = FilterMLPStruct(E, W, M, ptr(mlp.band_freq), ptr(mlp.w_in), ptr(mlp.b_in), ptr(mlp.w_inner),
                             ptr(mlp.b_inner), ptr(mlp.sin_freq), ptr(mlp.w_out), ptr(mlp.alpha))
        _check("hyena_implicit_filter",
               self.lib.hyena_implicit_filter(self.handle, ctypes.byref(st), out.data_ptr(),
                                              _stream_handle(torch, self.device)))
        return out

    def spectrum_batched(self, h, out=None):
        """hyena_filter_spectrum_batched: per-sample filters h [B, N-1, D, L] fp32 ->
        B spectra in one opaque uint8 device buffer."""
        torch = self._torch
        N, D, L = self.order, self.D, self.L
        if h.dim() != 4:
            raise ValueError("h must be [B, N-1, D, L]")
        B = int(h.shape[0])
        self._need(h, "h", (B, N - 1, D, L), torch.float32)
        if out is None:
            out = torch.empty(B * self.spectrum_bytes(), dtype=torch.uint8, device=self.device)
        elif out.numel() * out.element_size() < B * self.spectrum_bytes():
            raise ValueError("spectrum buffer too small")
        _check("hyena_filter_spectrum_batched",
               self.lib.hyena_filter_spectrum_batched(self.handle, B, h.data_ptr(), out.data_ptr(),
                                                      _stream_handle(torch, self.device)))
        return out

    def forward_per_sample(self, u_proj, short_w, spec, bias, y=None, workspace=None):
        """hyena_forward_per_sample: as forward, with spec holding one spectrum per
        sample (from spectrum_batched)."""
        return self.forward(u_proj, short_w, spec, bias, y, workspace, per_sample=True)

    def forward(self, u_proj, short_w, spec, bias, y=None, workspace=None, per_sample=False):
        """hyena_forward: u_proj [B,(N+1)D,L], short_w [(N+1)D,3], bias [N-1,D] -> y [B,D,L]."""
        torch = self._torch
        N, D, L = self.order, self.D, self.L
        if u_proj.dim() != 3:
            raise ValueError("u_proj must be [B, (N+1)*D, L]")
        B = int(u_proj.shape[0])
        self._need(u_proj, "u_proj", (B, (N + 1) * D, L), self.io_dtype)
        self._need(short_w, "short_w", ((N + 1) * D, 3), torch.float32)
        self._need(bias, "bias", (N - 1, D), torch.float32)
        nspec = B if per_sample else 1
        if spec.device != self.device or spec.numel() * spec.element_size() < nspec * self.spectrum_bytes():
            raise ValueError("spec must come from Plan.spectrum (spectrum_batched for per-sample filters) "
                             "of an equal plan")
        if y is None:
            y = torch.empty((B, D, L), dtype=self.io_dtype, device=self.device)
        self._need(y, "y", (B, D, L), self.io_dtype)
        ws_ptr, ws_bytes = 0, 0
        need = self.workspace_bytes(B)
        if need:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        fn, name = ((self.lib.hyena_forward_per_sample, "hyena_forward_per_sample") if per_sample
                    else (self.lib.hyena_forward, "hyena_forward"))
        _check(name, fn(self.handle, B, u_proj.data_ptr(), short_w.data_ptr(), spec.data_ptr(), bias.data_ptr(),
                        y.data_ptr(), ws_ptr or None, ws_bytes, _stream_handle(torch, self.device)))
        return y

    def forward_noalloc(self, u_proj, short_w, spec, bias, y):
        """hyena_forward_noalloc: as forward into a caller-given y, with no workspace
        and no allocation (the library's per-device scratch array holds the tiles;
        calls that overlap on one GPU race)."""
        torch = self._torch
        N, D, L = self.order, self.D, self.L
        B = int(u_proj.shape[0])
        self._need(u_proj, "u_proj", (B, (N + 1) * D, L), self.io_dtype)
        self._need(short_w, "short_w", ((N + 1) * D, 3), torch.float32)
        self._need(bias, "bias", (N - 1, D), torch.float32)
        self._need(y, "y", (B, D, L), self.io_dtype)
        if spec.device != self.device or spec.numel() * spec.element_size() < self.spectrum_bytes():
            raise ValueError("spec must come from Plan.spectrum of an equal plan")
        _check("hyena_forward_noalloc",
               self.lib.hyena_forward_noalloc(self.handle, B, u_proj.data_ptr(), short_w.data_ptr(), spec.data_ptr(),
                                              bias.data_ptr(), y.data_ptr(), _stream_handle(torch, self.device)))
        return y

    def forward_timed(self, u_proj, short_w, spec, bias, y, workspace=None):
        """hyena_forward_timed: runs one forward (synchronously) and returns the
        per-kernel-family milliseconds {"lds", "pass_a", "pass_b", "pass_c", "total",
        "pipe"} ("pipe": the pipelined four-step launches, each running all three
        passes on consecutive chunks)."""
        torch = self._torch
        B = int(u_proj.shape[0])
        ws_ptr, ws_bytes = 0, 0
        if self.workspace_bytes(B):
            if workspace is None:
                workspace = torch.empty(self.workspace_bytes(B), dtype=torch.uint8, device=self.device)
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        ms = (ctypes.c_float * 6)()
        _check("hyena_forward_timed",
               self.lib.hyena_forward_timed(self.handle, B, u_proj.data_ptr(), short_w.data_ptr(),
                                            spec.data_ptr(), bias.data_ptr(), y.data_ptr(), ws_ptr or None,
                                            ws_bytes, _stream_handle(torch, self.device), ms))
        return dict(zip(("lds", "pass_a", "pass_b", "pass_c", "total", "pipe"), [float(v) for v in ms]))

    def backward_workspace_bytes(self, B: int, per_sample: bool = False) -> int:
        fn = self.lib.hyena_backward_per_sample_workspace_bytes if per_sample else self.lib.hyena_backward_workspace_bytes
        return int(fn(self.handle, int(B)))

    def backward_per_sample(self, u_proj, short_w, spec, bias, dy, du=None, dw=None, dh=None, dbias=None,
                            workspace=None):
        """hyena_backward_per_sample: as backward, with spec holding one spectrum per
        sample (from spectrum_batched) and dh [B,N-1,D,L] one filter gradient per sample."""
        return self.backward(u_proj, short_w, spec, bias, dy, du, dw, dh, dbias, workspace, per_sample=True)

    def backward(self, u_proj, short_w, spec, bias, dy, du=None, dw=None, dh=None, dbias=None, workspace=None,
                 per_sample=False):
        """hyena_backward: gradients (du_proj [B,(N+1)D,L] io dtype, dshort_w [(N+1)D,3],
        dh [N-1,D,L], dbias [N-1,D] fp32) of the forward for upstream gradient dy [B,D,L]."""
        torch = self._torch
        N, D, L = self.order, self.D, self.L
        if u_proj.dim() != 3:
            raise ValueError("u_proj must be [B, (N+1)*D, L]")
        B = int(u_proj.shape[0])
        self._need(u_proj, "u_proj", (B, (N + 1) * D, L), self.io_dtype)
        self._need(short_w, "short_w", ((N + 1) * D, 3), torch.float32)
        self._need(bias, "bias", (N - 1, D), torch.float32)
        self._need(dy, "dy", (B, D, L), self.io_dtype)
        nspec = B if per_sample else 1
        if spec.device != self.device or spec.numel() * spec.element_size() < nspec * self.spectrum_bytes():
            raise ValueError("spec must come from Plan.spectrum (spectrum_batched for per-sample filters) "
                             "of an equal plan")
        f32 = torch.float32
        dh_shape = (B, N - 1, D, L) if per_sample else (N - 1, D, L)
        du = torch.empty((B, (N + 1) * D, L), dtype=self.io_dtype, device=self.device) if du is None else du
        dw = torch.empty(((N + 1) * D, 3), dtype=f32, device=self.device) if dw is None else dw
        dh = torch.empty(dh_shape, dtype=f32, device=self.device) if dh is None else dh
        dbias = torch.empty((N - 1, D), dtype=f32, device=self.device) if dbias is None else dbias
        self._need(du, "du", (B, (N + 1) * D, L), self.io_dtype)
        self._need(dw, "dw", ((N + 1) * D, 3), f32)
        self._need(dh, "dh", dh_shape, f32)
        self._need(dbias, "dbias", (N - 1, D), f32)
        need = self.backward_workspace_bytes(B, per_sample)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        name = "hyena_backward_per_sample" if per_sample else "hyena_backward"
        _check(name,
               getattr(self.lib, name)(self.handle, B, u_proj.data_ptr(), short_w.data_ptr(), spec.data_ptr(),
                                       bias.data_ptr(), dy.data_ptr(), du.data_ptr(), dw.data_ptr(), dh.data_ptr(),
                                       dbias.data_ptr(), ws_ptr, ws_bytes, _stream_handle(torch, self.device)))
        return du, dw, dh, dbias

    def operator_workspace_bytes(self, B: int) -> int:
        return int(self.lib.hyena_operator_workspace_bytes(self.handle, int(B)))

    def _operator_args(self, x, w_in, b_in, short_w, spec, bias, w_out, b_out, out, workspace):
        torch = self._torch
        N, D, L = self.order, self.D, self.L
        if x.dim() != 3:
            raise ValueError("x must be [B, L, D]")
        B = int(x.shape[0])
        io = self.io_dtype
        self._need(x, "x", (B, L, D), io)
        self._need(w_in, "w_in", ((N + 1) * D, D), io)
        self._need(b_in, "b_in", ((N + 1) * D,), io)
        self._need(w_out, "w_out", (D, D), io)
        self._need(b_out, "b_out", (D,), io)
        self._need(short_w, "short_w", ((N + 1) * D, 3), torch.float32)
        self._need(bias, "bias", (N - 1, D), torch.float32)
        if spec.device != self.device or spec.numel() * spec.element_size() < self.spectrum_bytes():
            raise ValueError("spec must come from Plan.spectrum of an equal plan")
        if out is None:
            out = torch.empty((B, L, D), dtype=io, device=self.device)
        self._need(out, "out", (B, L, D), io)
        if workspace is None:
            workspace = torch.empty(self.operator_workspace_bytes(B), dtype=torch.uint8, device=self.device)
        return B, out, workspace

    def operator_forward(self, x, w_in, b_in, short_w, spec, bias, w_out, b_out, out=None, workspace=None):
        """hyena_operator_forward: x [B,L,D] -> out [B,L,D] through in_proj, the hot path and out_proj."""
        B, out, ws = self._operator_args(x, w_in, b_in, short_w, spec, bias, w_out, b_out, out, workspace)
        _check("hyena_operator_forward",
               self.lib.hyena_operator_forward(self.handle, B, x.data_ptr(), w_in.data_ptr(), b_in.data_ptr(),
                                               short_w.data_ptr(), spec.data_ptr(), bias.data_ptr(),
                                               w_out.data_ptr(), b_out.data_ptr(), out.data_ptr(), ws.data_ptr(),
                                               ws.numel(), _stream_handle(self._torch, self.device)))
        return out

    def operator_tune(self, x, w_in, b_in, short_w, spec, bias, w_out, b_out, out=None, workspace=None):
        """hyena_operator_tune: times the projection GEMMs' candidate kernels on these
        buffers and keeps the fastest for later calls (blocking; `out` is scratch)."""
        B, out, ws = self._operator_args(x, w_in, b_in, short_w, spec, bias, w_out, b_out, out, workspace)
        _check("hyena_operator_tune",
               self.lib.hyena_operator_tune(self.handle, B, x.data_ptr(), w_in.data_ptr(), b_in.data_ptr(),
                                            short_w.data_ptr(), spec.data_ptr(), bias.data_ptr(), w_out.data_ptr(),
                                            b_out.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(),
                                            _stream_handle(self._torch, self.device)))

    def operator_forward_timed(self, x, w_in, b_in, short_w, spec, bias, w_out, b_out, out, workspace=None):
        """hyena_operator_forward_timed: one synchronous call; returns milliseconds
        {"in_proj", "path", "out_proj", "total"}."""
        B, out, ws = self._operator_args(x, w_in, b_in, short_w, spec, bias, w_out, b_out, out, workspace)
        ms = (ctypes.c_float * 4)()
        _check("hyena_operator_forward_timed",
               self.lib.hyena_operator_forward_timed(self.handle, B, x.data_ptr(), w_in.data_ptr(),
                                                     b_in.data_ptr(), short_w.data_ptr(), spec.data_ptr(),
                                                     bias.data_ptr(), w_out.data_ptr(), b_out.data_ptr(),
                                                     out.data_ptr(), ws.data_ptr(), ws.numel(),
                                                     _stream_handle(self._torch, self.device), ms))
        return dict(zip(("in_proj", "path", "out_proj", "total"), [float(v) for v in ms]))

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            self.lib.hyena_plan_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class _GridPlan:
    """Shared body of the N-d plans (Plan2D, Plan3D): the grid dims, D channels,
    I/O dtype "f32" or "bf16"; the C calls are hyena_plan{2d,3d}_create, ... ."""
    _SFX = ""

    def __init__(self, dims, D: int, dtype: str = "f32", circular: bool = False):
        import torch

        self._torch = torch
        self.lib = load_library()
        self.dims, self.D, self.dtype = tuple(int(n) for n in dims), int(D), dtype
        self.circular = bool(circular)
        if dtype not in _DTYPES:
            raise ValueError(f"dtype must be one of {list(_DTYPES)}")
        self.device = torch.device("cuda", torch.cuda.current_device())
        h = ctypes.c_void_p()
        name = f"hyena_plan{self._SFX}_create_ex"
        _check(name, getattr(self.lib, name)(ctypes.byref(h), *self.dims, self.D, _DTYPES[dtype],
                                             FLAG_CIRCULAR if self.circular else 0))
        self.handle = h

    def kernel_shape(self):
        """Per-channel kernel grid: the doubled grid, or the grid itself when circular."""
        return tuple(self.dims) if self.circular else tuple(2 * n for n in self.dims)

    def _fn(self, stem, tail=""):
        return getattr(self.lib, f"hyena_{stem}{self._SFX}{tail}")

    @property
    def io_dtype(self):
        return self._torch.bfloat16 if self.dtype == "bf16" else self._torch.float32

    def spectrum_bytes(self) -> int:
        return int(self._fn("spectrum", "_bytes")(self.handle))

    def workspace_bytes(self, B: int) -> int:
        return int(self._fn("workspace", "_bytes")(self.handle, int(B)))

    def _need(self, t, name, shape, dtype):
        Plan._need(self, t, name, shape, dtype)

    def spectrum(self, k, out=None):
        """hyena_filter_spectrum{2d,3d}: k [D, *kernel grid] fp32 -> opaque uint8 device buffer."""
        torch = self._torch
        self._need(k, "k", (self.D, *self.kernel_shape()), torch.float32)
        if out is None:
            out = torch.empty(self.spectrum_bytes(), dtype=torch.uint8, device=self.device)
        elif out.numel() * out.element_size() < self.spectrum_bytes():
            raise ValueError("spectrum buffer too small")
        _check(f"hyena_filter_spectrum{self._SFX}",
               self._fn("filter_spectrum")(self.handle, k.data_ptr(), out.data_ptr(),
                                           _stream_handle(torch, self.device)))
        return out

    def spectrum_batched(self, k, out=None):
        """hyena_filter_spectrum{2d,3d}_batched: k [B, D, *doubled grid] fp32 (a kernel
        set per sample) -> B spectra in one uint8 device buffer."""
        torch = self._torch
        if k.dim() != 2 + len(self.dims):
            raise ValueError("k must be [B, D, *doubled grid]")
        B = int(k.shape[0])
        self._need(k, "k", (B, self.D, *self.kernel_shape()), torch.float32)
        if out is None:
            out = torch.empty(B * self.spectrum_bytes(), dtype=torch.uint8, device=self.device)
        elif out.numel() * out.element_size() < B * self.spectrum_bytes():
            raise ValueError("spectrum buffer too small")
        _check(f"hyena_filter_spectrum{self._SFX}_batched",
               self._fn("filter_spectrum", "_batched")(self.handle, B, k.data_ptr(), out.data_ptr(),
                                                       _stream_handle(torch, self.device)))
        return out

    def forward_per_sample(self, v, spec, bias, g=None, x=None, y=None, workspace=None):
        """hyena_conv{2d,3d}_forward_per_sample: as forward, with spec holding one
        spectrum per sample (from spectrum_batched)."""
        return self.forward(v, spec, bias, g, x, y, workspace, per_sample=True)

    def forward(self, v, spec, bias, g=None, x=None, y=None, workspace=None, per_sample=False):
        """hyena_conv{2d,3d}_forward: v (and the optional gates g, x) [B, D, *grid] -> y."""
        torch = self._torch
        if v.dim() != 2 + len(self.dims):
            raise ValueError(f"v must be [B, D, {', '.join(str(n) for n in self.dims)}]")
        B = int(v.shape[0])
        shape = (B, self.D, *self.dims)
        self._need(v, "v", shape, self.io_dtype)
        for name, t in (("g", g), ("x", x)):
            if t is not None:
                self._need(t, name, shape, self.io_dtype)
        self._need(bias, "bias", (self.D,), torch.float32)
        nspec = B if per_sample else 1
        if spec.device != self.device or spec.numel() * spec.element_size() < nspec * self.spectrum_bytes():
            raise ValueError(f"spec must come from {type(self).__name__}.spectrum (spectrum_batched for a kernel "
                             "set per sample) of an equal plan")
        if y is None:
            y = torch.empty(shape, dtype=self.io_dtype, device=self.device)
        self._need(y, "y", shape, self.io_dtype)
        if workspace is None:
            workspace = torch.empty(self.workspace_bytes(B), dtype=torch.uint8, device=self.device)
        name = f"hyena_conv{self._SFX}_forward" + ("_per_sample" if per_sample else "")
        _check(name,
               getattr(self.lib, name)(
                   self.handle, B, v.data_ptr(), g.data_ptr() if g is not None else None,
                   x.data_ptr() if x is not None else None, spec.data_ptr(), bias.data_ptr(), y.data_ptr(),
                   workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                   _stream_handle(torch, self.device)))
        return y

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            getattr(self.lib, f"hyena_plan{self._SFX}_destroy")(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class Plan2D(_GridPlan):
    """A 2-D plan: H x W images of D channels (hyena_plan2d_create; the gated 2-D
    long convolution of include/hyena.h)."""
    _SFX = "2d"

    def __init__(self, H: int, W: int, D: int, dtype: str = "f32", circular: bool = False):
        self.H, self.W = int(H), int(W)
        super().__init__((H, W), D, dtype, circular)


class Plan3D(_GridPlan):
    """A 3-D plan: A x H x W volumes of D channels (hyena_plan3d_create; the gated
    3-D long convolution of include/hyena.h)."""
    _SFX = "3d"

    def __init__(self, A: int, H: int, W: int, D: int, dtype: str = "f32", circular: bool = False):
        self.A, self.H, self.W = int(A), int(H), int(W)
        super().__init__((A, H, W), D, dtype, circular)
