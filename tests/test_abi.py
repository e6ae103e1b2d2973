"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before touching a device. No compute
call is made here."""
import ctypes
import os
import re
import subprocess

import pytest

from fft_long_convolution_libhyena_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hyena.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from fft_long_convolution_libhyena_amd import build

        build.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hyena_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (hyena_\w+)", out))
    for name in declared_functions():
        assert name in exported, f"{name} is declared in hyena.h but not exported"
        getattr(lib, name)


def test_status_strings(lib):
    for code in range(5):
        s = lib.hyena_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.hyena_status_string(99) == b"unknown status"


def test_null_plan_queries(lib):
    assert lib.hyena_plan_destroy(None) == 0
    assert lib.hyena_spectrum_bytes(None) == 0
    assert lib.hyena_workspace_bytes(None, 4) == 0
    assert lib.hyena_plan_path(None) == binding.PATH_AUTO


def _create(lib, L, D, order, dtype=0, path=0):
    h = ctypes.c_void_p()
    st = lib.hyena_plan_create_path(ctypes.byref(h), L, D, order, dtype, path)
    if st == 0:
        lib.hyena_plan_destroy(h)
    return st, h


@pytest.mark.parametrize("L,D,order,dtype,path,want", [
    (1024, 0, 2, 0, 0, 1),        # D < 1
    (1024, 4, 1, 0, 0, 1),        # order < 2
    (0, 4, 2, 0, 0, 1),           # L < 1
    (1024, 4, 2, 7, 0, 1),        # bad dtype
    (1024, 4, 2, 0, 9, 1),        # bad path
    (1000, 4, 2, 0, 0, 2),        # L not a power of two
    (8, 4, 2, 0, 0, 2),           # L below 16
    (1 << 21, 4, 2, 0, 0, 2),     # L above 2^20
    (1024, 4, 9, 0, 0, 2),        # order above 8
    (1 << 15, 4, 2, 0, 1, 2),     # LDS path beyond 16384
    (128, 4, 2, 0, 2, 2),         # four-step below 256
    (65536, 4, 2, 0, 3, 1),       # path value 3 is unused
])
def test_plan_argument_errors_before_any_device_call(lib, L, D, order, dtype, path, want):
    st, h = _create(lib, L, D, order, dtype, path)
    assert st == want
    assert h.value is None  # *out untouched on failure


def test_plan_create_null_out(lib):
    assert lib.hyena_plan_create(None, 1024, 4, 2, 0) == 1


def test_forward_and_spectrum_reject_null_plan(lib):
    assert lib.hyena_forward(None, 1, 16, 16, 16, 16, 16, None, 0, None) == 1
    assert lib.hyena_filter_spectrum(None, 16, 16, None) == 1


def test_operator_rejects_null_plan(lib):
    assert lib.hyena_operator_workspace_bytes(None, 1) == 0
    assert lib.hyena_operator_forward(None, 1, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 1 << 20, None) == 1


def test_backward_rejects_null_plan(lib):
    assert lib.hyena_backward_workspace_bytes(None, 1) == 0
    assert lib.hyena_backward(None, 1, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 1 << 20, None) == 1
    assert lib.hyena_backward_per_sample_workspace_bytes(None, 1) == 0
    assert lib.hyena_backward_per_sample(None, 1, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 1 << 20, None) == 1


def test_implicit_filter_rejects_null_arguments(lib):
    from fft_long_convolution_libhyena_amd.binding import FilterMLPStruct

    st = FilterMLPStruct(3, 16, 0, 16, 16, 16, None, None, 16, 16, 16)
    assert lib.hyena_implicit_filter(None, ctypes.byref(st), 16, None) == 1
    assert lib.hyena_implicit_filter(None, None, 16, None) == 1


def test_conv2d_entry_points_reject_bad_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.hyena_plan2d_create(None, 64, 64, 4, 0) == 1
    assert lib.hyena_plan2d_create(ctypes.byref(h), 0, 64, 4, 0) == 1
    assert lib.hyena_plan2d_create(ctypes.byref(h), 64, 64, 4, 5) == 1     # bad dtype
    assert lib.hyena_plan2d_create(ctypes.byref(h), 48, 64, 4, 0) == 2     # H not a power of two
    assert lib.hyena_plan2d_create(ctypes.byref(h), 8, 64, 4, 0) == 2      # H below 16
    assert lib.hyena_plan2d_create(ctypes.byref(h), 64, 16, 4, 0) == 2     # W below 32
    assert lib.hyena_plan2d_create(ctypes.byref(h), 64, 1024, 4, 0) == 2   # W above 512
    assert h.value is None
    assert lib.hyena_plan2d_destroy(None) == 0
    assert lib.hyena_spectrum2d_bytes(None) == 0 and lib.hyena_workspace2d_bytes(None, 1) == 0
    assert lib.hyena_filter_spectrum2d(None, 16, 16, None) == 1
    assert lib.hyena_conv2d_forward(None, 1, 16, None, None, 16, 16, 16, 16, 1 << 20, None) == 1


def test_conv3d_entry_points_reject_bad_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.hyena_plan3d_create(None, 32, 32, 32, 4, 0) == 1
    assert lib.hyena_plan3d_create(ctypes.byref(h), 32, 0, 32, 4, 0) == 1
    assert lib.hyena_plan3d_create(ctypes.byref(h), 32, 32, 32, 4, 5) == 1   # bad dtype
    assert lib.hyena_plan3d_create(ctypes.byref(h), 24, 32, 32, 4, 0) == 2   # A not a power of two
    assert lib.hyena_plan3d_create(ctypes.byref(h), 8, 32, 32, 4, 0) == 2    # A below 16
    assert lib.hyena_plan3d_create(ctypes.byref(h), 32, 8, 32, 4, 0) == 2    # H below 16
    assert lib.hyena_plan3d_create(ctypes.byref(h), 32, 32, 16, 4, 0) == 2   # W below 32
    assert lib.hyena_plan3d_create(ctypes.byref(h), 512, 512, 512, 4, 0) == 2  # more than 2^24 points
    assert h.value is None
    assert lib.hyena_plan3d_destroy(None) == 0
    assert lib.hyena_spectrum3d_bytes(None) == 0 and lib.hyena_workspace3d_bytes(None, 1) == 0
    assert lib.hyena_filter_spectrum3d(None, 16, 16, None) == 1
    assert lib.hyena_conv3d_forward(None, 1, 16, None, None, 16, 16, 16, 16, 1 << 20, None) == 1
    assert lib.hyena_plan2d_create_ex(ctypes.byref(h), 64, 64, 4, 0, 2) == 1       # unknown flag bit
    assert lib.hyena_plan3d_create_ex(ctypes.byref(h), 32, 32, 64, 4, 0, 2) == 1   # unknown flag bit
    assert lib.hyena_plan2d_create_ex(ctypes.byref(h), 16, 64, 4, 0, 1) == 2       # circular H below 32
    assert lib.hyena_plan2d_create_ex(ctypes.byref(h), 64, 32, 4, 0, 1) == 2       # circular W below 64
    assert lib.hyena_plan3d_create_ex(ctypes.byref(h), 16, 32, 64, 4, 0, 1) == 2   # circular A below 32
    assert h.value is None
    for nd in ("2d", "3d"):
        assert getattr(lib, f"hyena_filter_spectrum{nd}_batched")(None, 1, 16, 16, None) == 1
        assert getattr(lib, f"hyena_conv{nd}_forward_per_sample")(None, 1, 16, None, None, 16, 16, 16, 16,
                                                                   1 << 20, None) == 1


def test_valid_plan_without_gpu_reports_device_error(lib):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, _ = _create(lib, 1024, 4, 2)
    assert st == 4  # HYENA_ERR_DEVICE


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError):
        binding.load_library(str(tmp_path / "missing.so"))


def test_debug_switches_on_the_host(monkeypatch):
    """HYENA_DEBUG_SYNC leaves successful calls alone where no device is present and
    still raises for failed ones; HYENA_FORCE_PATH must name a path."""
    from fft_long_convolution_libhyena_amd import HyenaError, Plan, binding

    monkeypatch.setenv("HYENA_DEBUG_SYNC", "1")
    assert binding._env_flag("HYENA_DEBUG_SYNC")
    binding._check("hyena_forward", 0)
    with pytest.raises(HyenaError) as e:
        binding._check("hyena_forward", 3)
    assert e.value.status == 3 and "hyena_forward" in str(e.value)
    monkeypatch.setenv("HYENA_DEBUG_SYNC", "0")
    assert not binding._env_flag("HYENA_DEBUG_SYNC")
    monkeypatch.setenv("HYENA_FORCE_PATH", "no-such-path")
    with pytest.raises(ValueError):
        Plan(1024, 4, 2)


def test_plain_c_client_compiles_links_and_runs(tmp_path):
    """include/hyena.h is a C header: a C99 program includes it, links against the
    built libhyena.so and gets the documented statuses from the host-checked calls."""
    import shutil
    import subprocess

    from fft_long_convolution_libhyena_amd import binding

    if shutil.which("gcc") is None or not os.path.exists(binding.LIB_PATH):
        pytest.skip("gcc or the built library is missing")
    libdir = os.path.dirname(binding.LIB_PATH)
    exe = tmp_path / "c_client"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-isystem", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "sanitize", "c_client.c"), "-o", str(exe),
                    "-L", libdir, "-lhyena", "-Wl,-rpath," + libdir], check=True, capture_output=True,
                   text=True, timeout=120)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 unexpected" in r.stdout
