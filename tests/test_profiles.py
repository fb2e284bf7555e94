"""The committed rocprofv3 summaries name the command that made them, and the
gate/up traffic figures belong to the current kernel sources (CPU only)."""
import glob
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def test_every_summary_names_its_command():
    paths = sorted(glob.glob(os.path.join(PROFILES, "*.md")))
    assert paths, "no profile summaries"
    for p in paths:
        text = open(p).read()
        m = re.search(r"Commands? \(from the repository root\):\s*```\n(.*?)```", text, re.S)
        assert m, f"{os.path.basename(p)}: no command block"
        cmd = m.group(1).strip()
        assert "rocprofv3" in cmd, f"{os.path.basename(p)}: the command block holds no rocprofv3 command"


def test_traffic_file_names_its_commands_and_kernel_sources():
    import bench
    with open(os.path.join(PROFILES, "traffic_gate_up_int4_T16.json")) as f:
        t = json.load(f)
    assert "rocprofv3 --pmc FETCH_SIZE" in t["commands"] and "WRITE_SIZE" in t["commands"]
    assert t["bytes_per_launch"] == round(t["fetch"]["bytes_per_launch"] + t["write"]["bytes_per_launch"])
    # bench.py reports these bytes as roofline.traffic only while the kernel
    # sources match the ones the counters were taken on
    assert t["kernel_hash"] == bench.kernel_source_hash(), "gate/up sources changed since the counters were taken"
