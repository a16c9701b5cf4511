"""Host-side logic of bench.py (no GPU): the single-GPU guard, the stored
traffic lookup, its source-hash check and the workload names it keys on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_stored_traffic_follows_the_attend_sources(tmp_path, monkeypatch):
    sha = bench.attend_sources_sha256()
    prof = tmp_path / "x_traffic.md"
    prof.write_text("- workload_key: `w@0.38`\n- traffic_bytes_per_launch: `123`\n"
                    f"- attend_sources_sha256: `{sha}`\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.stored_traffic("w@0.38") == 123
    assert bench.stored_traffic("other@0.38") is None
    prof.write_text("- workload_key: `w@0.38`\n- traffic_bytes_per_launch: `123`\n"
                    "- attend_sources_sha256: `0000`\n")
    assert bench.stored_traffic("w@0.38") is None  # the kernel changed since the counters were taken



def test_committed_traffic_summary_names_the_default_workload():
    import re
    import workloads as W

    keys = []
    for name in os.listdir(bench.PROFILES):
        if "traffic" in name:
            with open(os.path.join(bench.PROFILES, name)) as f:
                keys += re.findall(r"^- workload_key: `([^`]*)`", f.read(), flags=re.M)
    density = float(W.recipe("seq_512k")["density"])  # one target for every head
    default = bench.traffic_key("seq_512k", density)
    assert default in keys
    assert len(set(keys)) == len(keys)  # one summary per workload
    # other lengths or screens never pick up the default workload's figure
    assert bench.traffic_key("seq_512k", density, seq_len=4194304) != default
    assert bench.traffic_key("seq_512k", density, bound="dual") != default
