"""Host-side parts of bench.py: the one-GPU rule, the CPU baseline leg, and the code hash that gates the
recorded rocprof figures."""
import os
import subprocess
import sys

import pytest

import bench
from tiled_online_softmax_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_cpu_baseline_times_the_oracle():
    """A sample of the step's workload (reduced here to H=4, N=1024): the oracle's forward of two heads on its
    own dequantised e4m3 inputs, reported with the sample and the cores."""
    import dataclasses

    w = dataclasses.replace(inputs.WORKLOADS["long_fp8_causal"], H=4, N=1024)
    rec = bench.cpu_baseline(w, inputs.make(w, with_grad=False))
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "2 of the 4" in rec["sample"] and "all 1024 query rows" in rec["sample"]


def test_code_hash_ignores_comments_and_blank_lines(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one more\n}\n")
    b.write_text("// header comment\n\nint f(int x) {\n  return x + 1;\n\n}\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    h = lambda p: bench._hash_files([p.name], root=str(tmp_path))
    assert h(a) == h(b)
    assert h(a) != h(c)
