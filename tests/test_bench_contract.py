"""bench.py keeps its output contract: one JSON line with the fields the
benchmark driver reads (run on the GPU with the tiny workload), and a
refusal, before touching any GPU, of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2" in r.stderr and r.stdout == ""


@pytest.mark.gpu
def test_bench_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny", "--steps", "3",
                        "--warmup", "2", "--trace"], capture_output=True, text=True, timeout=170)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(d[key], typ), key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2 and d["value"] > 0
    assert d["vs_baseline"] is None and d["config"]["workload"] == "tiny"
    assert d["config"]["sched"] == "auto" and d["config"]["sched_run"] == "separate"
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma") and rf["unit"] in ("GB/s", "TFLOP/s")
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-4)   # both rounded in the line
    assert rf["traffic"] is None                     # no counter record for this workload
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert set(d["schedules_TFLOPs"]) == {"separate", "interleaved", "expert_wave"}
    tt = d["tile_trace"]
    assert tt["tiles"] > 0 and 0 < tt["busy_frac"] <= 1.0
