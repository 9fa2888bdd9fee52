"""bench.py end to end on the GPU (short runs): every option prints one JSON line with the
contract's keys, a roofline object and, when asked, the CPU baseline."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config", "roofline"}


def _bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1", *args],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.parametrize("args", [
    ("--workload", "decode", "--sets", "1", "--cpu-seconds", "1"),
    ("--workload", "decode", "--sets", "1", "--no-cpu-baseline", "--paged", "16"),
    ("--workload", "decode", "--sets", "1", "--no-cpu-baseline", "--graph"),
    ("--workload", "decode", "--sets", "1", "--no-cpu-baseline", "--batch", "16"),
    ("--workload", "writer", "--no-cpu-baseline"),
    ("--no-cpu-baseline",),
], ids=["decode+cpu", "paged", "graph", "batch16", "writer", "default"])
def test_bench_line(args):
    d = _bench(*args)
    assert KEYS <= set(d)
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma") and rf["peak"] > 0 and 0 < rf["frac"] < 1
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    if "--cpu-seconds" in args:
        cb = d["cpu_baseline"]
        assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    if "--paged" in args:
        assert d["config"]["caches"].startswith("paged") and rf["traffic"] is None
    if "--batch" in args:
        assert d["config"]["batch"] == 16 and rf["traffic"] is None
    if "--graph" in args:
        assert d["config"]["launch"] == "hip graph replay"
    if args == ("--no-cpu-baseline",):  # the headline: IndexShare decode, plus the other decode workloads
        assert d["config"]["workload"] == "indexshare_b32_ctx131072_l4" and d["config"]["layers"] == 4
        sp = d["step_ms_events"]
        assert sp["min"] <= sp["median"] <= sp["max"]
        assert set(d["other_workloads"]) == {"glm52_decode_b8_ctx8192", "ragged_decode_b64_ctx4k_64k"}
