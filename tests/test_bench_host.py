"""Host-side checks of bench.py that need no GPU.

* the algorithmic byte counts per launch equal their closed forms on the
  Llama-3.1-70B-shaped layer (every dim 0 divides by 8, so no padding:
  TIDE-RS moves 2*N*Psi/N + 4*S bytes, TIDE-AG 2*Psi + 2*Psi);
* the committed counter traffic is used only for the workload, launch mode
  and library it was taken on;
* a request for more than one GPU exits with a message.
"""
import os
import subprocess
import sys

import parameter_layout_collectives_amd as tide
import workloads

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_70b_layer():
    w = workloads.WORKLOADS["llama31_70b_layer"]
    plan = tide.Plan(w.shapes, w.world)
    psi = w.psi
    assert psi == 855_654_400
    assert plan.S * w.world == psi
    assert bench.rs_bytes(plan, 0) == 2 * psi + 4 * plan.S == 2_139_136_000
    assert bench.rs_bytes_mean(plan) == 2_139_136_000
    assert bench.ag_bytes(plan) == 4 * psi == 3_422_617_600


def test_rs_bytes_count_only_real_rows():
    # [5,7] over 4 ranks: c = 2 rows, rank 2 holds 1 real row, rank 3 none.
    plan = tide.Plan([(5, 7)], 4)
    assert plan.S == 14
    assert [bench.rs_bytes(plan, r) for r in range(4)] == \
        [2 * 4 * 14 + 4 * 14, 2 * 4 * 14 + 4 * 14, 2 * 4 * 7 + 4 * 14, 4 * 14]
    # a chain with R rotating moves the mean: 2*4*(14+14+7+0)/4 + 4*14
    assert bench.rs_bytes_mean(plan) == 2 * 4 * 35 / 4 + 4 * 14


def test_counter_traffic_matches_its_run_only():
    got = bench.counter_traffic("tide_ag", "llama31_70b_layer", False, False)
    if got is None:   # profile taken on another kernel source
        assert bench.kernel_source_hash() != _profile_hash()
        return
    assert 3.42e9 < got < 3.46e9
    assert bench.counter_traffic("tide_ag", "llama3_8b_layer", False, False) is None
    assert bench.counter_traffic("tide_ag", "llama31_70b_layer_n64", False, False) is None
    assert bench.counter_traffic("tide_ag", "llama31_70b_layer", True, False) is None
    assert bench.counter_traffic("tide_ag", "llama31_70b_layer", False, True) is None


def _profile_hash():
    import json
    with open(bench.PMC_SUMMARY) as f:
        return json.load(f)["kernel_source_sha256_16"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_bytes_in_window_prorates_straddling_calls():
    calls = [(0.0, 1.0), (1.0, 3.0), (3.0, 4.0)]
    # window [0.5, 3.5] ms: half of the first call, all of the second, half
    # of the third
    assert bench.bytes_in_window(calls, 100, 0.5, 3.5) == 50 + 100 + 50
    assert bench.bytes_in_window(calls, 100, 1.0, 3.0) == 100
    assert bench.bytes_in_window(calls, 100, 5.0, 6.0) == 0
    assert bench.bytes_in_window([(2.0, 2.0)], 100, 0.0, 5.0) == 0


def test_corun_summary_rows():
    leg = {"partner_slowdown_pct": 5.0, "during_partner_GBps": 1000.0, "alone_GBps": 5000.0,
           "progress_share_of_alone": 0.2, "serial_ms": 10.0, "makespan_ms": 8.0,
           "exposed_ms": 2.0, "hidden_pct": 40.0}
    res = {"workload": "w", "partner": "p", "default": leg, "small_footprint": leg}
    rows = bench.corun_summary([("tide_rs", res), ("tide_ag", None)])
    assert [r["mode"] for r in rows] == ["default", "small_footprint"]
    assert rows[0]["exposed_ms"] == 2.0 and rows[0]["collective"] == "tide_rs"


def test_unknown_leg_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--legs", "bogus"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "unknown" in r.stderr


def test_compact_line_drops_per_repeat_lists_only():
    line = {"value": 1.0, "corun": {"default": {"exposed_ms": 2.0, "progress_runs": [{"a": 1}],
                                                "makespan": {"serial_ms": 3.0, "runs": [{}]}}},
            "corun_summary": [{"mode": "default", "exposed_ms": 2.0}]}
    got = bench.compact(line)
    assert got == {"value": 1.0, "corun": {"default": {"exposed_ms": 2.0,
                                                       "makespan": {"serial_ms": 3.0}}},
                   "corun_summary": [{"mode": "default", "exposed_ms": 2.0}]}


def test_fixed_cost_fit():
    # 10 us fixed plus 1 GB per 160 us (6.25 TB/s): two calls of 1 and 4 GB
    t0, r = bench.fit_fixed_cost((1e9, 170.0), (4e9, 650.0))
    assert abs(t0 - 10.0) < 1e-9 and abs(r - 6250.0) < 1e-6
    # three points on that line, and three off it by +2, -4 and +2 us: zero
    # mean and no correlation with the bytes, so the least-squares line is
    # the same
    t0, r = bench.fit_fixed_cost((1e9, 170.0), (2e9, 330.0), (4e9, 650.0))
    assert abs(t0 - 10.0) < 1e-9 and abs(r - 6250.0) < 1e-6
    t0, r = bench.fit_fixed_cost((1e9, 172.0), (2.5e9, 406.0), (4e9, 652.0))
    assert abs(r - 6250.0) < 1e-6 and abs(t0 - (10.0 + 0.0)) < 1e-9


def test_pages_figures_are_context_only():
    # quoted beside the measurements, never used as a target or in vs_baseline
    ctx = bench.PAGES_CONTEXT
    assert ctx["layout_conversion_pct_of_step_llama31_70b_8k_tokens"] == 6.4
    assert ctx["nccl_reduce_scatter_single_wave_gemm_slowdown_pct_max"] == 69.0
    assert ctx["step_time_reduction_vs_stock_fsdp2_pct_max"] == 27.1
    assert "context, not targets" in ctx["source"]
