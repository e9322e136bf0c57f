"""Host logic of bench.py (no GPU): the algorithmic work formula against the
numbers worked out independently for the workload table, the counter
scaling of the traffic summary on synthetic counter files, and the one-GPU
guard."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from expert_dispatch_router_amd import synth  # noqa: E402


@pytest.mark.parametrize("name,gbytes,gflop", [("mixtral_512", 2.886, 360.8),
                                               ("mixtral_128", 2.835, 90.2),
                                               ("dsv3_512", 22.597, 360.8),
                                               ("dsv3_4096", 22.939, 2886.2),
                                               ("qwen2_512", 3.573, 225.5)])
def test_algorithmic_work_matches_the_workload_table(name, gbytes, gflop):
    cfg = synth.CONFIGS[name]
    counts = np.ones(cfg.E, dtype=np.int64)  # every expert active
    alg = bench.algorithmic(cfg, counts)
    assert alg["e_act"] == cfg.E
    assert abs(alg["bytes"] / 1e9 - gbytes) < 0.0015
    assert abs(alg["flop"] / 1e9 - gflop) < 0.15
    # the fused kernel's share: gate+up weights + activation rows + h written
    assert alg["bytes_k4"] == cfg.E * 4 * cfg.ffn * cfg.d + 2 * alg["A"] * cfg.d + 2 * alg["A"] * cfg.ffn


def test_algorithmic_counts_only_active_experts():
    cfg = synth.CONFIGS["skewed_512"]
    counts = np.zeros(cfg.E, dtype=np.int64)
    counts[[0, 5, 9]] = [1000, 1000, 48]
    alg = bench.algorithmic(cfg, counts)
    assert alg["e_act"] == 3
    assert alg["bytes_k4"] == 3 * 4 * cfg.ffn * cfg.d + 2 * alg["A"] * (cfg.d + cfg.ffn)


def _counter_csv(path, counter, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


K4 = "void moe::(anonymous namespace)::grouped_gemm_kernel<192, 1, 7, 3, 0>(unsigned short const*)"
K5 = "void moe::(anonymous namespace)::grouped_gemm_kernel<192, 2, 8, 3, 1>(unsigned short const*)"
# LDS-staged tiles carry a sixth template argument (the weight cache policy):
# the output mode is still the fifth
K4L = "void moe::(anonymous namespace)::gemm_lds_kernel<192, 7, 64, 2, 0, 2>(unsigned short const*)"
K5L = "void moe::(anonymous namespace)::gemm_lds_kernel<192, 8, 64, 2, 1, 2>(unsigned short const*)"
K5W = "void moe::(anonymous namespace)::gemm_lds_kernel<128, 8, 64, 2, 4, 0>(unsigned short const*)"
K4V = "void moe::(anonymous namespace)::gemm_lds_var_kernel<128, 64, 3, 2, 2>(unsigned short const*)"
COPY = "__amd_rocclr_copyBuffer"


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path):
    gib = 1 << 30
    # the copy of 1 GiB reads half its bytes by FETCH_SIZE and all by WRITE_SIZE
    _counter_csv(str(tmp_path / "f" / "a" / "run_counter_collection.csv"), "FETCH_SIZE",
                 [(COPY, 524288.0), (COPY, 524288.0), (COPY, 4.0), (K4, 1000.0), (K4, 1100.0),
                  (K5, 7.0)])
    _counter_csv(str(tmp_path / "w" / "run_counter_collection.csv"), "WRITE_SIZE",
                 [(COPY, 1048576.0), (K4, 100.0), (K4, 100.0), (K5, 3.0)])
    out = bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "test", gib,
                                  out_dir=str(tmp_path))
    assert out["fetch_scale"] == pytest.approx(2.0)
    assert out["write_scale"] == pytest.approx(1.0)
    k4 = out["kernels"]["gate_up_swiglu"]
    assert k4["launches"] == [2, 2]
    assert out["bytes_per_launch"] == pytest.approx(1050.0 * 1024 * 2 + 100.0 * 1024)
    assert out["kernels"]["down"]["bytes_per_launch"] == pytest.approx(7.0 * 2048 + 3.0 * 1024)
    saved = json.load(open(tmp_path / "traffic_gate_up_swiglu_test.json"))
    assert saved["source_sha256_16"] == bench.source_sha()


def test_traffic_summary_classifies_lds_staged_tiles_by_their_mode(tmp_path):
    gib = 1 << 30
    _counter_csv(str(tmp_path / "f" / "run_counter_collection.csv"), "FETCH_SIZE",
                 [(COPY, 524288.0), (K4L, 500.0), (K5L, 9.0), (K5W, 9.0)])
    _counter_csv(str(tmp_path / "w" / "run_counter_collection.csv"), "WRITE_SIZE",
                 [(COPY, 1048576.0), (K4L, 50.0), (K5L, 2.0), (K5W, 2.0)])
    out = bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "lds", gib,
                                  out_dir=str(tmp_path))
    assert set(out["kernels"]) == {"gate_up_swiglu", "down"}
    assert out["bytes_per_launch"] == pytest.approx(500.0 * 2048 + 50.0 * 1024)
    assert out["kernels"]["down"]["bytes_per_launch"] == pytest.approx(9.0 * 2048 + 2.0 * 1024)
    assert out["kernels"]["down"]["launches"] == [2, 2]


def test_traffic_summary_counts_the_variable_rows_kernel_as_gate_up(tmp_path):
    """The gate/up GEMM over the variable-size block table is the gate/up
    stage, although its template arguments carry no output mode."""
    gib = 1 << 30
    _counter_csv(str(tmp_path / "f" / "run_counter_collection.csv"), "FETCH_SIZE",
                 [(COPY, 524288.0), (K4V, 300.0), (K4V, 310.0), (K5L, 9.0)])
    _counter_csv(str(tmp_path / "w" / "run_counter_collection.csv"), "WRITE_SIZE",
                 [(COPY, 1048576.0), (K4V, 20.0), (K4V, 20.0), (K5L, 2.0)])
    out = bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "var", gib,
                                  out_dir=str(tmp_path))
    assert out["kernels"]["gate_up_swiglu"]["launches"] == [2, 2]
    assert out["bytes_per_launch"] == pytest.approx(305.0 * 2048 + 20.0 * 1024)
    assert out["kernels"]["down"]["launches"] == [1, 1]


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]



def test_single_core_tiny_cpu_baseline(monkeypatch):
    """The tiny oracle figure runs in a child process pinned to one CPU with
    one OpenMP thread, also where the environment asks torch and OpenMP for
    16 threads (MKL_NUM_THREADS takes precedence in torch's own pool)."""
    monkeypatch.setenv("OMP_NUM_THREADS", "16")
    monkeypatch.setenv("MKL_NUM_THREADS", "16")
    r = bench.cpu_single_core_tiny()
    assert r["cores"] == 1 and r["omp_threads"] == 1, r
    assert r["value"] > 0 and r["kind"] == "oracle", r


def _plan(rl=1, gather=0, fused_down=0, unfused=0, fold=0):
    return {"routing_launches": rl, "gather_launch": gather, "fused_down": fused_down,
            "unfused_swiglu": unfused, "fold_combine": fold}


def test_stage_names_follow_the_launch_plan():
    """An interval between two stage events with no kernel in it is named
    None (it measures only the event records)."""
    assert bench.stage_names(_plan(1)) == ["route_histogram_scan_schedule_reorder", None, None,
                                           "gate_up_swiglu", "down", "combine"]
    assert bench.stage_names(_plan(2)) == ["route", "histogram_scan_schedule_reorder", None,
                                           "gate_up_swiglu", "down", "combine"]
    assert bench.stage_names(_plan(3, gather=1)) == ["route", "histogram_scan_schedule",
                                                     "reorder_gather", "gate_up_swiglu", "down",
                                                     "combine"]
    assert bench.stage_names(_plan(1, fused_down=1))[3:] == ["gate_up_swiglu_down", None,
                                                             "combine"]
    assert bench.stage_names(_plan(2, unfused=1, fold=1))[3:] == ["gate_up_unfused", "down", None]


def test_cpu_model_is_reported():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
