"""Host checks of bench.py's bookkeeping: the kernel it names for the roofline
record is the kernel the library launches (the library's tp_step_kernel, as
a committed kernel trace of the 530B-like shard shows), and the workload
flop counts."""
import os
import re

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_STEPS = bench.GEMM_STEPS
tp = pytest.importorskip("tensor_transformer_layer_tp_amd")


def shape_of(w, rank=0):
    return tp.TpShape.make(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn=w.ffn, n_heads=w.n_heads,
                           head_dim=w.head_dim, tp_rank=rank, tp_size=w.tp_size, dtype=w.dtype, alibi=int(w.alibi))


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(tp.library_path()):
        pytest.skip("library not built")
    tp.load_library()


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
    # without a device the library plans for 256 compute units (MI355X)
    w = synth.WORKLOADS["mtnlg_530b_tp8"]
    named = {bench.kernel_of(s, shape_of(w)) for s in GEMM_STEPS}
    assert named == traced_gemm_kernels(path)


def test_planner_takes_192_wide_tiles_where_they_fill_the_cus():
    # GPT-2-like (T 8192, h 1536): the input gradients with N = 1536 run
    # 32 x 8 = 256 tiles of 256x192 (one whole round) instead of 192 tiles of
    # 256x256 in a stream-K tail; GEMM2's input gradient (N = 6144: 768
    # tiles, three whole rounds) keeps the 256-wide tile
    s = shape_of(synth.WORKLOADS["gpt2_1p2b_tp1"])
    assert tp.tp_step_kernel(s, "fc1_dgrad") == "gemm_fc1_dgrad_n192"
    assert tp.tp_step_kernel(s, "out_dgrad") == "gemm_out_dgrad_n192"
    assert tp.tp_step_kernel(s, "qkv_dgrad") == "gemm_qkv_dgrad_n192"
    assert tp.tp_step_kernel(s, "fc2_dgrad") == "gemm_fc2_dgrad_gelu"
    # 8.3B-like (T 16384, f_l 1536, h_l 384): GEMM2's input gradient in two
    # whole rounds; the output-projection input gradient (N = 384) as 128
    # tiles of 256x192 split in two over K instead of 128 half-empty 256-wide
    s = shape_of(synth.WORKLOADS["gpt_8p3b_tp8"])
    assert tp.tp_step_kernel(s, "fc2_dgrad") == "gemm_fc2_dgrad_gelu_n192"
    assert tp.tp_step_kernel(s, "out_dgrad") == "gemm_out_dgrad_n192"
    assert tp.tp_step_kernel(s, "fc1_dgrad") == "gemm_fc1_dgrad"


def test_step_kernel_query_rejects_what_launches_nothing():
    w = synth.WORKLOADS["gpt2_1p2b_tp1"]
    assert tp.tp_step_kernel(shape_of(w), "attn_fwd") is None      # not a product
    assert tp.tp_step_kernel(shape_of(w), 99) is None              # no such step
    bad = shape_of(w)
    bad.hidden = 1535                                              # invalid shape
    assert tp.tp_step_kernel(bad, "fc1") is None
    empty = tp.TpShape.make(batch=0, seq=w.seq, hidden=w.hidden, ffn=w.ffn, n_heads=w.n_heads,
                            head_dim=w.head_dim, dtype="bf16")
    assert tp.tp_step_kernel(empty, "fc1") is None                 # empty product: no launch
    fp32 = shape_of(synth.WORKLOADS["tiny_fp32_tp2"])
    assert tp.tp_step_kernel(fp32, "fc1") == "gemm_f32_kernel"


def test_layer_flops_of_the_named_workloads():
    # 3 [2 T h (4 h_l + 2 f_l) + 2 b n_l d s (s + 1)], the algorithmic count
    assert bench.layer_flops(synth.WORKLOADS["mtnlg_530b_tp8"]) == pytest.approx(7.7954e12, rel=1e-4)
    assert bench.layer_flops(synth.WORKLOADS["gpt2_1p2b_tp1"]) == pytest.approx(1.4690e12, rel=1e-4)
    assert bench.layer_flops(synth.WORKLOADS["gpt_8p3b_tp8"]) == pytest.approx(1.4303e12, rel=1e-4)
    assert bench.layer_flops(synth.WORKLOADS["bloom_176b_tp8"]) == pytest.approx(7.6666e12, rel=1e-4)
    sf = bench.step_flops(synth.WORKLOADS["mtnlg_530b_tp8"])
    assert sum(sf.values()) == pytest.approx(bench.layer_flops(synth.WORKLOADS["mtnlg_530b_tp8"]), rel=1e-12)
