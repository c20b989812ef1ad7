"""CPU checks of bench.py's contract that need no GPU: more than one GPU is refused with a
message and exit status 2, and the CPU baseline (the float64 oracle timed on a bounded
sample of the workload) reports the fields of its JSON object."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_fields():
    sys.path.insert(0, ROOT)
    import bench
    import workloads
    w = workloads.by_name("tiny_ring4_f32")
    inp = workloads.make_inputs(w)
    rec = bench.cpu_baseline(w, inp, target_s=0.2)
    assert set(rec) == {"value", "unit", "cores", "kind", "sample", "cpu_model"}
    assert rec["unit"] == "TFLOP/s" and rec["kind"] == "oracle"
    assert isinstance(rec["cpu_model"], str) and rec["cpu_model"]
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "passes" in rec["sample"] or "heads" in rec["sample"]


def test_default_workload_is_the_ulysses2_share():
    """The headline line is the Ulysses-2 share (the workload the >=50%-of-peak target names), with the
    32k ring-4 share's block kernel timed beside it."""
    sys.path.insert(0, ROOT)
    import bench
    assert bench.DEFAULT_WORKLOAD == "flux1024_ulysses2_bf16"
    assert "video32k_ring4_bf16" in bench.EXTRA_ROOFLINES


@pytest.mark.parametrize("name", ["flux1024_ring2_bf16", "video32k_ring4_bf16"])
def test_workload_flops(name):
    """The TFLOP/s numerator is 4*B*H*Sq*Skv*D over every block."""
    sys.path.insert(0, ROOT)
    import workloads
    w = workloads.by_name(name)
    assert w.flops == 4 * w.B * w.attn_H * w.Sq * sum(w.block_lens) * w.D
