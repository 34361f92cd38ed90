"""Host-side checks of bench.py (no GPU): the one-GPU refusal and the rule that the
committed counter traffic is reported only for the kernel source and workload it was
measured on."""
import json
import os
import subprocess
import sys

import bench
from mixture_experts_layer_gemm_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_only_for_its_workload_and_kernel_source(tmp_path, monkeypatch):
    c1 = "olmo-64e-top4: T=4096 d_model=2048 N=64 K=4 d_r=2560 d_s=1280"
    rec = {"kernel_source_sha": bench.gemm_source_sha(), "workload": f"{c1}, 16384 kept routes",
           "hbm_bytes_per_launch": 123}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(c1) == 123
    assert bench.measured_traffic(c1.replace("T=4096", "T=8192")) is None
    assert bench.measured_traffic(c1.replace("olmo-64e-top4", "skewed-capacity-qwen-gate")) is None
    f.write_text(json.dumps(dict(rec, kernel_source_sha="0" * 16)))
    assert bench.measured_traffic(c1) is None
    f.write_text("not json")
    assert bench.measured_traffic(c1) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.measured_traffic(c1) is None


def test_committed_traffic_record_names_its_kernel_source_and_workload():
    """The committed counter summary names the gate/up kernel source and the workload it
    was taken on (the bench reports it only while both match)."""
    with open(bench.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    assert len(rec["kernel_source_sha"]) == 16
    assert rec["workload"].split(":")[0] == synth.get_config("C1").name
    assert rec["hbm_bytes_per_launch"] > rec["algorithmic_bytes_per_launch"] > 0
    assert rec["fetch_scale"] > 0 and rec["write_scale"] > 0
