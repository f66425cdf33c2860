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


def test_all_kernels_summary_names_instantiations(tmp_path, monkeypatch):
    """The all-paths summary turns mangled instantiation names into name<arguments> and keeps only the
    library's kernels."""
    import bench
    d = tmp_path / "prof"
    d.mkdir()
    (d / "run_kernel_stats.csv").write_text(
        "Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs,StdDev\n"
        '"_ZN2sa12_GLOBAL__N_112sa_dq_kernelILb1ELb0ELi2EEEvPKDF16_S3_PfPKifiiiiiixNS_10DqEpilogueE",'
        "4,400000,100000,50,99000,101000,1\n"
        '"_ZN2sa12_GLOBAL__N_113sa_key_kernelILb0ELb1ELi4EEEvPKDF16_",2,380000,190000,40,189000,191000,1\n'
        '"at::native::vectorized_elementwise_kernel<4>",1,1000,1000,1,1000,1000,0\n')
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    bench.summarize_all_kernels(str(d), "w", "cmd")
    text = (tmp_path / "profiles" / "kernel_trace_all_paths_w.txt").read_text()
    assert "sa_dq_kernel<true, false, 2>" in text and "sa_key_kernel<false, true, 4>" in text
    assert "at::native" not in text


def test_trace_summary_averages_the_timed_launches(tmp_path, monkeypatch):
    """The kernel-trace summary adds each kernel's average over its last K launches (K from the recorded
    bench command), the launches the bench's own per-kernel figures cover, beside the all-launch average."""
    import bench
    d = tmp_path / "prof"
    d.mkdir()
    name = "_ZN2sa12_GLOBAL__N_117sa_forward_kernelILb1ELb0ELb0EEEv"
    durs = [300.0, 200.0, 100.0, 110.0]  # microseconds: two warm-up launches, then two timed ones
    (d / "run_kernel_stats.csv").write_text(
        "Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs,StdDev\n"
        f'"{name}",4,710000,177500,100,100000,300000,1\n')
    rows = ["Kind,Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 1000
    for i, us in enumerate(durs):
        rows.append(f'KERNEL_DISPATCH,{i + 1},"{name}",{t},{t + int(us * 1000)}')
        t += 10 ** 7
    (d / "run_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    bench.summarize_profile([str(d)], "w", "rocprofv3 --kernel-trace -- python3 bench.py --steps 2 --headline-only")
    text = (tmp_path / "profiles" / "kernel_trace_w.txt").read_text()
    line = [l for l in text.splitlines() if l.startswith("forward")][0].split()
    assert float(line[2]) == 177.5 and float(line[5]) == 105.0
