"""Host checks of bench.py's bookkeeping: the kernel it names for the roofline
record is the kernel the library launches (as a committed kernel trace of the
530B-like shard shows), and the workload flop counts."""
import os
import re

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_STEPS = tuple(bench.KERNEL_OF_STEP)


def traced_gemm_kernels(path):
    names = set()
    for line in open(path):
        m = re.match(r"\|\s*(gemm_\w+)\s*\|", line)
        if m and not m.group(1).endswith("_fixup") and not m.group(1).startswith("gemm_logits"):
            names.add(m.group(1))
    return names


def test_kernel_of_matches_the_committed_trace_of_the_530b_shard():
    path = os.path.join(ROOT, "profiles", "layer_step_mtnlg_530b_tp8_kernel_stats.md")
    if not os.path.exists(path):
        pytest.skip("no committed kernel trace")
    w = synth.WORKLOADS["mtnlg_530b_tp8"]
    named = {bench.kernel_of(s, w, 256) for s in GEMM_STEPS}
    assert named == traced_gemm_kernels(path)


def test_layer_flops_of_the_named_workloads():
    # 3 [2 T h (4 h_l + 2 f_l) + 2 b n_l d s (s + 1)], the algorithmic count
    assert bench.layer_flops(synth.WORKLOADS["mtnlg_530b_tp8"]) == pytest.approx(7.7954e12, rel=1e-4)
    assert bench.layer_flops(synth.WORKLOADS["gpt2_1p2b_tp1"]) == pytest.approx(1.4690e12, rel=1e-4)
    assert bench.layer_flops(synth.WORKLOADS["gpt_8p3b_tp8"]) == pytest.approx(1.4303e12, rel=1e-4)
    assert bench.layer_flops(synth.WORKLOADS["bloom_176b_tp8"]) == pytest.approx(7.6666e12, rel=1e-4)
    sf = bench.step_flops(synth.WORKLOADS["mtnlg_530b_tp8"])
    assert sum(sf.values()) == pytest.approx(bench.layer_flops(synth.WORKLOADS["mtnlg_530b_tp8"]), rel=1e-12)
