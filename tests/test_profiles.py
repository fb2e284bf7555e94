"""The committed rocprofv3 summaries name the command that made them, the
gate/up traffic figures belong to the current kernel sources, and bench.py's
host-side refusals (more than one GPU, a summary without its command) hold
(CPU only)."""
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


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    for argv, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                           timeout=120, cwd=ROOT, env={**os.environ, **env})
        assert r.returncode == 2 and "one GPU only" in r.stderr, (argv, r.returncode, r.stderr[-300:])


def test_bench_summarizers_require_the_command():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-trace", "/nonexistent", "/dev/null"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0 and "--command" in r.stderr
