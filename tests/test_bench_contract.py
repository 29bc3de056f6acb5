"""The benchmark's contract on the host (no GPU): one GPU only, the oracle baseline record, and that the committed
HBM-traffic summary of the distance kernel still describes the kernel source in the tree."""

import json
import os
import subprocess
import sys

import bench
from laplacian_nystr_vit_amd import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr


def test_cpu_baseline_record():
    """The oracle runs in one single-threaded process per usable host core (at most 16), three timed runs, the
    median reported with the CPU model."""
    wl = WL.TINY
    rec = bench.cpu_baseline(wl, budget_s=0.3)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert rec["cores"] == bench.oracle_workers() == min(len(os.sched_getaffinity(0)), 16,
                                                         int(os.environ.get("OMP_NUM_THREADS", 10 ** 6)))
    assert len(rec["runs_tokens_per_s"]) == 3 and rec["value"] == sorted(rec["runs_tokens_per_s"])[1]
    assert rec["value"] > 0 and wl.name in rec["sample"]
    assert rec["cpu_model"] == bench.cpu_model()


def test_cpu_baseline_runs_the_training_and_gaussian_oracles():
    for wl in (WL.GAUSS_S1.replace(B=1, H=16, W=16, r=4), WL.TRAIN_S1.replace(B=1, H=16, W=16, r=4)):
        rec = bench.cpu_baseline(wl, budget_s=0.15)
        assert rec["value"] > 0
    assert "backward" in rec["sample"]


def test_committed_traffic_summary_matches_the_kernel_source():
    """bench.py reports the distance kernel's HBM traffic only while the committed counter summary carries the hash
    of the kernel source in the tree; a kernel change without a new counter pass would silently drop it."""
    rec = json.load(open(bench.TRAFFIC_FILE))
    assert rec["source_hash"] == bench.laplace_source_hash()
    traffic = bench.load_traffic()
    assert traffic is not None
    # the algorithmic bytes of one launch on the stage-1 shape: Q and K read, C_Q, C_K and W_eps written (fp32)
    wl = WL.PVT_S1
    alg = 4 * wl.G * (2 * wl.N * wl.d + 2 * wl.N * wl.m + wl.m * wl.m) + 4 * wl.G * wl.m * wl.d
    assert 0.9 * alg <= traffic <= 1.2 * alg
