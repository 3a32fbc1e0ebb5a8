"""Host-side checks of bench.py's contract (no GPU needed): the one-GPU
guard, the matmul units behind the roofline, and the profile lookup."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_units_add_up_to_the_metric():
    # the metric counts 14 N^2 d (x 1/2 when causal) per head: 7 matmul units
    # of 2 N^2 d; forward QK^T + P~V, dK/dV kernel QK^T + P^T dO + dO V^T +
    # dS^T Q, dQ kernel dS K
    assert sum(bench.KERNEL_UNITS.values()) == 7
    assert bench.KERNEL_UNITS == {"FWD_ATTN": 2, "BWD_DKDV": 4, "BWD_DQ": 1}


def test_valu_issue_ceiling():
    # 256 CUs x 4 SIMDs, one wave64 VALU instruction per SIMD every 4 cycles at 2.4 GHz
    assert bench.VALU_PEAK_INSTR_PER_S == 256 * 4 * 2.4e9 / 4


def test_profile_lookup_is_tied_to_the_kernel_source():
    assert bench.load_profile("BWD_DKDV", "no_such_workload") is None
    p = bench.load_profile("BWD_DKDV", "llama16k")
    if p is not None:                      # present only when taken on the current kernel source
        assert p["source_sha"] == bench.source_sha("BWD_DKDV")
        assert p["hbm_bytes_per_launch"] > 0 and p["avg_ms_profile"] > 0
    assert len(bench.source_sha("BWD_DKDV")) == 16
