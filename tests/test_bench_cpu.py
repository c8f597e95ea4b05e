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
    by_name = {w.name: w for w in workloads.WORKLOADS.values()}
    for kernel, (path, _) in bench.TRAFFIC_RECORDS.items():
        rec = json.load(open(path))
        w = by_name[rec["workload"].split(":")[0]]
        expect = rec["traffic_bytes_per_launch"] if rec["source_sha256"] == bench.kernel_source_hash(kernel) else None
        assert bench.measured_traffic(w, kernel) == expect, kernel
        # a record applies to its own workload only
        other = workloads.WORKLOADS[1]
        assert bench.measured_traffic(other, kernel) is None, kernel
    # the default at 16 states is the lane-per-state kernel
    assert bench.measured_traffic(w3, "auto") == bench.measured_traffic(w3, "lanes")
    assert bench.resolved_kernel(w3, "auto") == "lanes"
    assert bench.resolved_kernel(w3, "auto", zoh=True) == "lanes"
    assert bench.resolved_kernel(workloads.WORKLOADS[4], "auto", zoh=True) == "chunked"
    assert bench.resolved_kernel(workloads.WORKLOADS[1], "auto", zoh=True) == "lanes"
    assert bench.resolved_kernel(workloads.WORKLOADS[5], "auto") == "lanes"
    # few long rows: the chunked kernel (4 x 1024 channels of 100 000 steps)
    assert bench.resolved_kernel(workloads.WORKLOADS[4], "auto") == "chunked"
    assert bench.measured_traffic(w3, "generic") is None
    assert bench.measured_traffic(w3, "auto", zoh=True) is None
    # the genomic workload runs the chunked kernel, whose record is taken there
    assert bench.measured_traffic(workloads.WORKLOADS[4], "auto") == bench.measured_traffic(
        workloads.WORKLOADS[4], "chunked")


def test_backward_traffic_records_match_the_sources():
    """The backward's rocprofv3 traffic records (per kernel; the segment-tiled one recomputing /
    from saved states) are reported only while the sources they were taken on are unchanged, and
    for the Mamba-130m workload only."""
    import json

    import bench
    from selective_state_space_29_amd import workloads

    w3 = workloads.WORKLOADS[3]
    recs = {}
    for key, (path, _) in bench.BWD_TRAFFIC_RECORDS.items():
        kernel, ck = key
        if not os.path.exists(path):
            assert bench.measured_bwd_traffic(w3, ck, kernel) is None
            continue
        with open(path) as f:
            rec = json.load(f)
        current = rec["source_sha256"] == bench.kernel_source_hash(key, bench.BWD_TRAFFIC_RECORDS)
        expect = rec["traffic_bytes_per_launch"] * rec.get("launches_per_call", 1) if current else None
        assert bench.measured_bwd_traffic(w3, ck, kernel) == expect
        assert bench.measured_bwd_traffic(workloads.WORKLOADS[5], ck, kernel) is None
        recs[key] = rec["traffic_bytes_per_launch"]
    # the segment-tiled kernel starting from the saved states neither writes nor re-reads them
    if ("tiled", True) in recs and ("tiled", False) in recs:
        assert 0 < recs[("tiled", True)] < recs[("tiled", False)]


def test_issue_floor_arithmetic():
    """The issue floor: element work at the 4 FMA : 1 exp mix rate, row-step work additively;
    co_issue compares the additive time of a unit with the mix's measured time."""
    import bench
    from selective_state_space_29_amd import workloads

    w3 = workloads.WORKLOADS[3]
    rates = {"fma_T_lane_ops_per_s": 50.0, "exp_T_lane_ops_per_s": 20.0,
             "dpp_mul_T_lane_ops_per_s": 35.0, "mix_4fma_1exp_T_units_per_s": 8.0}
    f = bench.issue_floor(w3, rates, 100.0)
    rows = w3.rows * w3.seqlen
    trans = bench.transcendentals_per_launch(w3)
    assert trans == w3.elements + rows * 4  # softplus (exp, log) and gate (exp, rcp) per row-step
    expect = (w3.elements / 8e12 + (trans - w3.elements) / 20e12
              + rows * bench.VALU_OPS_PER_ROW_STEP / 50e12) * 1e6
    assert abs(f["floor_us"] - round(expect, 2)) < 0.011
    assert abs(f["co_issue_4fma_1exp"] - round((4 / 50 + 1 / 20) * 8, 3)) < 1e-9
    assert abs(f["frac"] - round(expect / 100.0, 4)) < 1e-4
    assert bench.issue_floor(w3, None, 100.0) is None


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


def test_cpu_baseline_repeats_the_whole_workload_until_the_wall_time():
    import bench
    from selective_state_space_29_amd import workloads

    w = workloads.WORKLOADS[1]
    x = workloads.make_inputs(w)
    r = bench.cpu_baseline(w, x, min_wall_s=0.05)
    assert r["kind"] == "oracle" and r["unit"] == "Gelem/s" and r["value"] > 0 and r["cores"] >= 1
    passes = int(r["sample"].split(", ")[1].split()[0])
    assert 1 <= passes <= 64
    # the rate is over every pass: passes x elements / wall time
    wall = float(r["sample"].split(" s wall")[0].split()[-1])
    assert abs(r["value"] - passes * w.elements / max(wall, 1e-9) / 1e9) <= 0.5 * r["value"]
