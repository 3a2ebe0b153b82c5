"""Host-side checks of bench.py (no GPU): the one-GPU refusal and the stored
traffic record's bookkeeping."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_record_fields():
    """The stored counter record names its workload, the source hash it was
    taken on and bytes per launch that are at least the algorithmic bytes."""
    path = os.path.join(ROOT, "profiles", "palu_decode_mha_kernel_llama2_7b_traffic.json")
    with open(path) as f:
        t = json.load(f)
    assert t["workload"] == "llama2_7b"
    assert len(t["source_sha256"]) == 64
    assert t["read_bytes_per_launch"] + t["write_bytes_per_launch"] >= 536870912
    assert t["fetch_scale"] > 0 and t["write_scale"] > 0
