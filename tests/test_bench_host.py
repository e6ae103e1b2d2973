"""Host logic of bench.py (no GPU): the algorithmic byte and flop counts the roofline
is priced with, the one-GPU rule, and how committed counter summaries are read."""
import os
import subprocess
import sys

import pytest

import bench
from fft_long_convolution_libhyena_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_forward_bytes_by_hand():
    """long64k (B=1, D=768, L=65536, order 2, fp32): one read of the three u_proj
    channel groups, one write of y, the fp32 half-spectra (L+1 bins) of one filter
    per channel, the taps and the bias."""
    w = synth.WORKLOADS["long64k"]
    u = 4 * 3 * 768 * 65536
    y = 4 * 768 * 65536
    spec = 8 * 768 * 65537
    small = 4 * 3 * 768 * 3 + 4 * 768
    assert bench.alg_bytes_forward(w) == u + y + spec + small == 1207996416


@pytest.mark.parametrize("name,gbytes,gflops", [
    # algorithmic bytes and flops per forward, worked out from the definitions above
    # (n = 2L real transforms at 2.5 n log2 n each)
    ("tiny", 0.001576, 0.00885), ("dna_small", 0.302002, 2.936), ("lm125m", 0.453022, 8.305),
    ("long64k_o3", 1.811995, 19.08), ("long64k", 1.207996, 9.815), ("dna_1m", 6.442463, 63.08)])
def test_forward_bytes_and_flops(name, gbytes, gflops):
    w = synth.WORKLOADS[name]
    assert bench.alg_bytes_forward(w) / 1e9 == pytest.approx(gbytes, rel=1e-4)
    assert bench.alg_flops_forward(w) / 1e9 == pytest.approx(gflops, rel=1e-3)


def test_flops_of_one_step_by_hand():
    """B=1, D=1, L=16, order 2: 10*16*log2(32) + 6*17 + 2*16 for the step, 2*16 for
    the gates, 5*3*16 for the short convolution of the three channels."""
    w = synth.custom(1, 1, 16, 2)
    assert bench.alg_flops_forward(w) == 800 + 102 + 32 + 32 + 240


def test_backward_bytes_exceed_forward():
    for w in synth.WORKLOADS.values():
        assert bench.alg_bytes_backward(w) > bench.alg_bytes_forward(w)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_is_read_only_for_current_sources(tmp_path, monkeypatch):
    """A counter summary counts only while its source hash matches the kernel sources."""
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    path = tmp_path / "profiles" / "pmc_k_fs_row_long64k.txt"
    good = bench.kernel_sources_hash("k_fs_row")
    path.write_text(f"# comment: ignored\nsources_sha256: {good}\nfetch_bytes_per_dispatch: 1000\n"
                    "write_bytes_per_dispatch: 24\n")
    assert bench.measured_traffic("k_fs_row", "long64k") == 1024
    path.write_text("sources_sha256: 0000000000000000\nfetch_bytes_per_dispatch: 1000\n"
                    "write_bytes_per_dispatch: 24\n")
    assert bench.measured_traffic("k_fs_row", "long64k") is None
    assert bench.measured_traffic("k_fs_row", "dna_1m") is None  # no summary at all


def test_kernel_families_cover_the_summaries():
    """Every committed counter summary names a kernel whose family lists real sources."""
    for f in os.listdir(os.path.join(ROOT, "profiles")):
        if f.startswith("pmc_"):
            kernel = next(k for k in ("k_fs_row", "k_lds_forward", "k_lds_bwd_rows", "fs_backward",
                                      "k_implicit_filter", "k_part_inv", "k_c2_conv2d", "k_c3_conv3d")
                          if f[4:].startswith(k))
            for src in bench.KERNEL_SOURCES[bench.kernel_family(kernel)]:
                assert os.path.exists(os.path.join(bench._CSRC, src)), src


def test_cpu_baseline_of_the_small_workload_times_the_direct_definition():
    """At L <= 1024 the CPU baseline also times the O(L^2) oracle over the whole input."""
    w = synth.WORKLOADS["tiny"]
    x = synth.generate(w)
    res = bench.cpu_baseline(x, w, 1.0)
    assert res["kind"] == "oracle" and res["value"] > 0 and res["cores"] >= 1
    assert res["direct"]["value"] > 0 and "direct" in res["direct"]["sample"]
