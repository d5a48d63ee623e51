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
    assert bench.ag_bytes(plan) == 4 * psi == 3_422_617_600


def test_rs_bytes_count_only_real_rows():
    # [5,7] over 4 ranks: c = 2 rows, rank 2 holds 1 real row, rank 3 none.
    plan = tide.Plan([(5, 7)], 4)
    assert plan.S == 14
    assert [bench.rs_bytes(plan, r) for r in range(4)] == \
        [2 * 4 * 14 + 4 * 14, 2 * 4 * 14 + 4 * 14, 2 * 4 * 7 + 4 * 14, 4 * 14]


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
