"""bench.py's contract on the host: the refusals, the algorithmic work the
roofline divides by, the traffic lookup's source check and the CPU-baseline
object.  Nothing here touches a GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run_bench(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, env=e, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_multi_rank_launch_is_refused():
    r = _run_bench(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_without_a_gpu_it_says_so():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run_bench("--no-cpu-baseline")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr and r.stdout == ""


def test_algorithmic_work_of_the_training_workload():
    """The counts the roofline uses, from the shapes: multiply-adds of the
    contractions as 2 FLOPs; every input read once and every output written
    once, in float32."""
    B, K, n_in, H = 256, 64, 128, 128
    N = H * (n_in + H + 2)
    w = bench.algorithmic_work(B, K, n_in, H)
    # forward: a = W_in x + W_rec h per row-step
    assert w["fwd_flops"] == B * K * 2 * H * (n_in + H) == 1_073_741_824
    # one-call path: the forward, then W_rec^T dL/da and the two weight-gradient
    # outer products per row-step (no recomputation of a)
    assert w["fb_flops"] == B * K * (2 * H * (n_in + H) + 2 * H * H + 2 * H * (n_in + H)) == 2_684_354_560
    # separate backward recomputes a: one more forward product
    assert w["bwd_flops"] == w["fb_flops"] - w["fwd_flops"] + B * K * 2 * H * (n_in + H)
    weights = H * (n_in + H + 2)
    assert w["fb_bytes"] == 4 * (B * K * n_in + B * H + B * K * H + B * H + B * N + B + weights) == 50_989_056
    assert w["reduce_bytes"] == 4 * (B * N + N) == 33_948_672


def test_algorithmic_work_of_the_large_workload():
    B, K, n, H = 8192, 8, 256, 256
    N = H * (n + H + 2)
    assert N == 131_584
    w = bench.algorithmic_work(B, K, n, H)
    assert w["fb_flops"] == 42_949_672_960
    assert w["reduce_bytes"] == 4 * (B * N + N)
    # the scratch dominates the one-call bytes (4.31 GB of 4.46 GB)
    assert 4 * B * N == 4_311_744_512 and w["fb_bytes"] == 4_463_298_560


def test_traffic_is_used_only_for_the_current_source(tmp_path, monkeypatch):
    src_hash = bench.source_hash()
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"source_sha256_16": src_hash, "kernels": {"cfc_fb_kernel": {"bytes_per_launch": 123.0}}}
    (prof / "traffic_wl.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    assert bench.measured_traffic("wl", "cfc_fb_kernel") == 123.0
    assert bench.measured_traffic("wl", "other_kernel") is None
    assert bench.measured_traffic("missing", "cfc_fb_kernel") is None
    rec["source_sha256_16"] = "0" * 16
    (prof / "traffic_wl.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("wl", "cfc_fb_kernel") is None


def test_profiled_kernel_duration_only_for_the_current_source(tmp_path, monkeypatch):
    """bench.py reads a kernel's rocprofv3 average from a committed trace
    summary only when the summary names the current kernel source; rows of a
    kernel split by grid size are selected by grid."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rows = ("kernel                      calls     avg_us     min_us     max_us  share%\n"
            "cfc_fb_small_kernel<true>       46      97.75      95.67     103.47   18.46\n"
            "reduce_axis0_kernel<4,16> grid=163840    21       3.70       3.52       5.12    0.32\n"
            "reduce_axis0_kernel<4,16> grid=526336    21     710.49     695.88     852.46   61.26\n")
    (tmp_path / "kernels_x.txt").write_text("t\ncommand: rocprofv3 ...\nkernel source sha256[:16]: "
                                            + bench.source_hash() + "\n\n" + rows)
    assert bench.profiled_kernel_us("kernels_x", "cfc_fb_small_kernel<true>") == 97.75
    assert bench.profiled_kernel_us("kernels_x", "reduce_axis0_kernel<4,16>", 526336) == 710.49
    assert bench.profiled_kernel_us("kernels_x", "reduce_axis0_kernel<4,16>", 163840) == 3.70
    assert bench.profiled_kernel_us("kernels_x", "reduce_axis0_kernel<4,16>", 1) is None
    # the instance and grid the library launches: 64 columns per workgroup,
    # 128 above 256 MB of input
    assert bench.reduce_kernel(32, 40960) == ("reduce_axis0_kernel<4,16>", 163840)
    assert bench.reduce_kernel(256, 33024) == ("reduce_axis0_kernel<4,16>", 132096)
    assert bench.reduce_kernel(8192, 131584) == ("reduce_axis0_kernel<4,32>", 263168)
    (tmp_path / "kernels_y.txt").write_text("t\ncommand: rocprofv3\nkernel source sha256[:16]: 0123456789abcdef\n"
                                            + rows)
    assert bench.profiled_kernel_us("kernels_y", "cfc_fb_small_kernel<true>") is None


def test_committed_profiles_name_their_source_and_command():
    """Every committed traffic summary carries the kernel-source hash it was
    taken on, and every summary the command that made it."""
    prof = os.path.join(ROOT, "profiles")
    names = sorted(os.listdir(prof))
    assert any(n.startswith("traffic_") and n.endswith(".json") for n in names)
    for n in names:
        text = open(os.path.join(prof, n)).read()
        if n.endswith(".json"):
            assert len(json.loads(text)["source_sha256_16"]) == 16
        else:
            assert "command" in text and "rocprofv3" in text or n.startswith("reduce_axis0_sweep")


def test_cpu_baseline_object():
    """The oracle timed on the host over a bounded sample: the fields the
    bench line carries, with the thread count it used."""
    from cfc_recurrent_cell_amd import workloads as W
    inp = W.make_cfc_inputs(W.TINY)
    cb = bench.cpu_baseline(inp, budget_s=0.4)
    assert cb["kind"] == "oracle" and cb["unit"] == "batch-steps/s"
    assert cb["value"] > 0 and 1 <= cb["cores"] <= 16
    assert cb["single_thread"]["cores"] == 1 and cb["single_thread"]["value"] > 0
    assert "K=8" in cb["sample"]
