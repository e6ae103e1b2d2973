"""bench.py end to end on the GPU, every mode on a small workload: one JSON line
with the fields the measurement contract names, a roofline object, and (with
by default) the oracle comparison within the parity bound of the mode."""
import json
import os
import subprocess
import sys

import pytest

from tests._hy import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COMMON = ["--steps", "2", "--reps", "1", "--warmup", "1", "--no-cpu-baseline"]
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config", "roofline"}
ROOF = {"bound", "achieved", "peak", "unit", "frac", "traffic"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _run(args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


@pytest.mark.parametrize("mode,workload", [
    ([], "tiny"), ([], "dna_small"), (["--backward"], "tiny"), (["--backward", "--per-sample"], "tiny"),
    (["--backward", "--circular"], "tiny"), (["--per-sample"], "tiny"), (["--circular"], "tiny"),
    (["--operator"], "tiny"), (["--filter"], "tiny"),
    (["--path", "fourstep"], "tiny"), (["--conv2d"], None), (["--conv3d", "--circular"], None),
    # full workloads in the launch configuration the benchmark times, checked on sampled outputs
    (["--circular"], "long64k"), (["--circular"], "lm125m"), (["--path", "partitioned"], "long64k"),
    (["--operator"], "lm125m"), (["--per-sample"], "long64k"), (["--backward", "--per-sample"], "lm125m"),
    (["--backward", "--circular"], "lm125m"),
    ([], "long64k"), ([], "long64k_o3"), ([], "lm125m"), (["--synthesis"], "lm125m")])
def test_bench_line(mode, workload):
    args = mode + COMMON + (["--workload", workload] if workload else [])
    out = _run(args)
    say(f"[bench] {' '.join(args)}: {out['ms_per_step'] * 1e3:.1f} us, frac {out['roofline']['frac']}")
    assert KEYS <= set(out), KEYS - set(out)
    assert ROOF <= set(out["roofline"])
    assert out["n_gpus"] == 1 and out["steps"] == 2 and out["warmup"] == 1
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["higher_is_better"] is True
    assert out["roofline"]["peak"] > 0 and 0 < out["roofline"]["frac"] < 1.5
    assert (out["roofline"]["bound"], out["roofline"]["unit"]) in {("hbm", "GB/s"), ("alu", "TFLOP/s"),
                                                                   ("mfma", "TFLOP/s")}
    assert "workload" in out["config"]
    checks = {k: v for k, v in out.items() if k.startswith("check_rel_l2")}
    if "--filter" not in mode:
        assert checks, "no oracle check in the line"
    bf16 = out["config"].get("io_dtype") == "bf16"
    for k, v in checks.items():
        bound = 1e-2 if (bf16 and k != "check_rel_l2_dh") else 1e-4
        assert v <= bound, (k, v)
