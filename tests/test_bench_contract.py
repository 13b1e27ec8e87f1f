"""bench.py contract checks that need no GPU: one GPU only, the labels of the
workloads, and the committed HBM-traffic record the roofline object reports."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(REPO, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    # The check runs before torch is imported or any device is touched.
    p = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU only" in p.stderr
    assert p.stdout == ""


def test_workload_labels_name_sizes():
    from sparse_attention_amd import workloads as wl
    b = load_bench()
    labels = {c: b.workload_label(wl.config(c)) for c in ("c1", "c3", "c4")}
    assert "64 sequences x 32,768 positions" in labels["c3"]
    assert "16 sequences x 202,752 positions" in labels["c4"]
    assert "4,096 positions" in labels["c1"]
    assert b.K_TOP == 2048 and b.HBM_PEAK_GBS == 8000.0 and b.MFMA_BF16_PEAK_TFS == 2500.0


def test_committed_traffic_record():
    """The decode indexer's HBM bytes per launch, from rocprofv3 counters,
    are reported only while the kernel source is the one they were taken on.
    The record must be well formed and close to the algorithmic bytes of the
    c3 indexer launch (537,403,392 B); when the source has changed since, the
    counters are due to be taken again."""
    b = load_bench()
    path = os.path.join(REPO, "profiles", "indexer_c3_traffic.json")
    with open(path) as f:
        rec = json.load(f)
    alg = 64 * (256 * 32768 + 8192 + 128)
    assert rec["kernel"] == "indexer_rows_kernel<false>" and rec["workload"] == "c3"
    assert rec["hbm_bytes_per_launch"] == rec["hbm_read_bytes"] + rec["hbm_write_bytes"]
    assert 0.98 * alg <= rec["hbm_bytes_per_launch"] <= 1.10 * alg
    assert os.path.exists(os.path.join(REPO, rec["summary"]))
    current = b.src_hash(["indexer.hip", "dsa_device.h"])
    if rec["source_hash"] != current:
        pytest.skip("the indexer source changed since its HBM counters were taken")
    assert b.traffic_from_profiles("indexer", "c3", current) == rec["hbm_bytes_per_launch"]
    assert b.traffic_from_profiles("indexer", "c3", "0" * 16) is None
