"""bench.py's command-line contract that can be checked without a GPU: it
measures one GPU and refuses more before touching any device, and its
traffic records name the hash of the kernel source they were taken with
(bench.py reports a record only while that hash matches)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_records_name_their_kernel_source():
    import bench
    with open(bench.PROFILE_TRAFFIC) as f:
        records = json.load(f)
    assert "vim_s_1024_bf16" in records
    for name, rec in records.items():
        assert rec["bytes_per_launch"] > 0, name
        assert len(rec["kernel_sha"]) == 16, name
        assert rec["fetch_scale"] > 0 and rec["write_scale"] > 0, name



def test_roofline_peaks_follow_from_unit_counts():
    """The published fp32 vector peak is the non-packed issue rate times 2
    (FMA) times 2 (packed); the issue-slot ceiling divides that issue rate by
    the slots of one state update."""
    import bench
    assert abs(bench.LANE_SLOTS * 2 * 2 / 1e12 - bench.FP32_PEAK_TFLOPS) < 0.1
    assert abs(bench.UPDATE_PEAK - bench.LANE_SLOTS / bench.SLOTS_PER_UPDATE) < 1.0
    assert 6.9 < bench.SLOTS_PER_UPDATE < 7.0
