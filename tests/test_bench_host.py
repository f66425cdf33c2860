"""Host checks of bench.py that need no GPU: the one-GPU guard and the FLOP convention."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_flop_convention_of_the_bench_workload():
    """14 d FLOPs per (query, key) pair per query head: forward 4 d, key pass 8 d, dQ pass
    2 d, causal pairs counted as T^2 / 2 (the usual causal convention, which the quoted
    68.72 / 240.52 GFLOP of T = 4096 with 32 heads follow)."""
    import bench
    from causal_streaming_attention_amd.workloads import WORKLOADS
    w = WORKLOADS["causal_gqa_t4096"]
    fl = bench.kernel_flops(w, None)
    pairs = 4096 * 4096 / 2 * 32
    assert fl["forward"] == 4 * 64 * pairs
    assert fl["key_pass"] == 8 * 64 * pairs
    assert fl["dq_pass"] == 2 * 64 * pairs
    assert abs(fl["forward"] / 1e9 - 68.72) < 0.01
    assert abs(fl["total"] / 1e9 - 240.52) < 0.01
