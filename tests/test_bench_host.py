"""Host-side logic of bench.py (no GPU): the algorithmic byte and FLOP counts
behind the reported roofline, the kernel the roofline names, and the refusal
of more than one GPU.

Expert weight bytes follow "Expert Parallelism for MoE Models" (apxml),
section "Memory Sizing Equations for MoE Models": experts x parameters per
expert x bytes per parameter, three d x F matrices per SwiGLU expert.
"""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from mixture_experts_layer_15_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_expert_bytes_follow_the_memory_equation():
    d, F = 2048, 768
    # bf16: 2 bytes per parameter, 3 d F parameters per expert
    assert bench.expert_bytes(d, F, "bf16", 128) == 128 * 3 * d * F * 2
    # FP8: 1 byte per parameter plus a float32 per 128 x 128 block
    assert bench.expert_bytes(d, F, "fp8", 32) == 32 * 3 * (d * F + (d // 128) * (F // 128) * 4)
    assert bench.expert_bytes(d, F, "fp8", 32, with_scales=False) == 32 * 3 * d * F
    # MXFP4: half a byte per parameter plus one E8M0 byte per 32 parameters
    assert bench.expert_bytes(d, F, "mxfp4", 8) == 8 * 3 * (d * F // 2 + d * F // 32)
    # the DeepSeek-V3 shape's 256 experts in FP8: 3 d F bytes each
    assert bench.expert_bytes(7168, 2048, "fp8", 256, with_scales=False) == 256 * 3 * 7168 * 2048


def test_expert_bytes_reproduce_the_pages_memory_example():
    """The apxml page's worked sizing ("Memory Sizing Equations for MoE
    Models"): 8 experts of 6e9 parameters at 2 bytes are 96 GB, 12 GB per GPU
    over 8 GPUs, and 6 GB per GPU at 1 byte.  A SwiGLU expert holds 3 d F
    parameters; d = 50000, F = 40000 gives the page's 6e9."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_figures.json")))["expert_memory"]
    d, F = 50000, 40000
    assert 3 * d * F == g["params_per_expert"]
    n = g["n_experts"]
    assert bench.expert_bytes(d, F, "bf16", n) == g["expert_memory_GB_16bit"] * 1e9
    assert bench.expert_bytes(d, F, "bf16", n) / g["gpus"] == g["per_gpu_GB_16bit"] * 1e9
    assert bench.expert_bytes(d, F, "fp8", n, with_scales=False) / g["gpus"] == \
        g["per_gpu_GB_8bit"] * 1e9


def test_algorithmic_counts_on_a_hand_example():
    wl = synth.WORKLOADS["decode"].replace(name="hand", T=4, d=256, E=8, num_local=8, k=2, F=128)
    counts = np.array([3, 0, 2, 0, 0, 1, 2, 0])           # N = 8 slots, 4 experts touched
    a = bench.algorithmic(wl, counts, tokens_read=4)
    d, F, E, T = 256, 128, 8, 4
    assert a["N"] == 8 and a["touched"] == 4
    assert a["layer_flop"] == 2 * T * d * E + 6 * 8 * d * F
    assert a["expert_bytes"] == 4 * 3 * d * F * 2 + 4 * d * 2 + T * d * 2
    assert a["layer_bytes"] == a["expert_bytes"] + d * E * 2
    assert a["gu_flop"] == 4 * 8 * d * F
    # gate/up: the touched experts' gate and up matrices and the token rows
    # (the materialised h is reported beside it, not counted)
    assert a["gu_bytes"] == 4 * 2 * d * F * 2 + 4 * d * 2
    assert a["gu_bytes_with_h"] == a["gu_bytes"] + 8 * F * 2
    # down: the touched experts' down matrices
    assert a["dn_flop"] == 2 * 8 * F * d and a["dn_bytes"] == 4 * d * F * 2
    assert a["gu_unit_bytes"] == 2 * d * F * 2


def test_roofline_kernel_names_follow_the_tile_plans():
    w = synth.WORKLOADS
    assert bench.gate_up_kernel_name(w["decode"], True) == \
        "grouped_gemm_kernel<1, 1, 2, 4, true, 16, 64, 4, 1, false, true>"
    assert bench.gate_up_kernel_name(w["decode"], False).endswith(", false, false>")
    assert bench.gate_up_kernel_name(w["prefill"], True).startswith("grouped_gemm_kernel<2, 4, 4, 2,")
    assert bench.gate_up_kernel_name(w["mixtral"], True).startswith("grouped_gemm_kernel<2, 4, 4, 2,")
    assert bench.gate_up_kernel_name(w["dsv3_rank"], True).startswith("grouped_gemm_kernel<4, 1, 2, 8, true, 8,")
    assert bench.gate_up_kernel_name(w["decode_mxfp4"], True) == "stream_gemm_kernel<true, 4, 4, 2, 2>"
    assert bench.gate_up_kernel_name(w["decode_mxfp4"], False).startswith(
        "grouped_gemm_kernel<1, 1, 2, 4, true, 4, 128, 2, 3,")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "only --gpus 1" in r.stderr
    assert r.stdout == ""
