"""Host-side checks of bench.py: the one-GPU contract and the traffic record."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_is_reported_only_for_the_profiled_sources():
    import bench
    from selective_state_space_29_amd import workloads

    w3 = workloads.WORKLOADS[3]
    for kernel, (path, _) in bench.TRAFFIC_RECORDS.items():
        rec = json.load(open(path))
        expect = rec["traffic_bytes_per_launch"] if rec["source_sha256"] == bench.kernel_source_hash(kernel) else None
        assert bench.measured_traffic(w3, kernel) == expect, kernel
    # the default at 16 states is the lane-per-state kernel
    assert bench.measured_traffic(w3, "auto") == bench.measured_traffic(w3, "lanes")
    assert bench.resolved_kernel(w3, "auto") == "lanes"
    assert bench.resolved_kernel(w3, "auto", zoh=True) == "tiled"
    assert bench.resolved_kernel(workloads.WORKLOADS[5], "auto") == "lanes"
    assert bench.measured_traffic(w3, "generic") is None
    assert bench.measured_traffic(w3, "auto", zoh=True) is None
    assert bench.measured_traffic(workloads.WORKLOADS[4], "auto") is None


def test_backward_traffic_records_match_the_sources():
    """The backward's rocprofv3 traffic records (recomputing / from saved states) were taken on
    the current scan_bwd sources and are reported for the Mamba-130m workload only."""
    import json

    import bench
    from selective_state_space_29_amd import workloads

    w3 = workloads.WORKLOADS[3]
    for ck in (False, True):
        with open(bench.BWD_TRAFFIC_RECORDS[ck][0]) as f:
            rec = json.load(f)
        assert rec["source_sha256"] == bench.kernel_source_hash(ck, bench.BWD_TRAFFIC_RECORDS)
        assert bench.measured_bwd_traffic(w3, ck) == rec["traffic_bytes_per_launch"] > 0
        assert bench.measured_bwd_traffic(workloads.WORKLOADS[5], ck) is None
    # starting from the saved states neither writes nor re-reads them
    assert bench.measured_bwd_traffic(w3, True) < bench.measured_bwd_traffic(w3, False)


def test_sampled_indices_exist_for_every_workload():
    """The rows / channels the bench reads back from the device exist in every workload (a
    device-side index_select does not check its indices)."""
    import bench
    from selective_state_space_29_amd import workloads

    for w in workloads.WORKLOADS.values():
        rows = bench.forward_check_rows(w)
        assert rows and all(0 <= r < w.rows for r in rows), w.name
        chans = bench.sampled_channels(w)
        assert chans and all(0 <= c < w.dim for c in chans), w.name
