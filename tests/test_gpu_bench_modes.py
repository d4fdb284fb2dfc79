"""The benchmark's optional modes end to end on the GPU, each as its own
short run on a small workload: every mode prints its JSON line, decodes
every scalar back and reports what it measured.  (The bench line itself is
run by the harness; these runs guard the modes it does not take.)"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=240):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1", "--no-cpu-baseline",
           *args]
    print("bench", " ".join(args), file=sys.stderr, flush=True)
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, r.stderr[-3000:]
    return [json.loads(line) for line in r.stdout.splitlines() if line.startswith("{")]


@pytest.mark.parametrize("args", [
    ("--channel-split",),
    ("--channel-split", "--sigma-fit", "rate", "--narrow-dof", "3"),
    ("--sigma-block", "256"),
    ("--paged", "64"),
])
def test_one_call_modes(args):
    (line,) = run_bench("--workload", "1", *args)
    assert line["roundtrip_exact"] is True
    assert line["value"] > 0 and line["encode_ms"] > 0 and line["decode_ms"] > 0
    b = line["bits_per_scalar"]
    assert b["coded"] > b["integer_model"] > 0
    if "--channel-split" in args:
        assert line["config"]["mixture_weights"].startswith("per (plane, channel)")


def test_per_layer_pipeline_and_host_offload():
    lines = run_bench("--workload", "4", "--offload", "--steps", "1", "--warmup", "0", timeout=600)
    assert len(lines) == 2
    assert lines[0]["roundtrip_exact"] is True and lines[0]["config"]["calls_per_step"] == 64
    off = lines[1]
    assert off["value"] > 0 and off["stream_bytes"] < off["raw_bytes"]
