"""bench.py's contract, checked on the host (no GPU): one GPU only, the
roofline object's fields and arithmetic, the algorithmic bytes per
head-token of the chunked gated-delta path, and counter figures taken only
from runs of the current kernel source."""

import hashlib
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_roofline_fields_and_fraction():
    roof = bench.hbm_roofline("some_kernel", 8e9, 2.0)   # 8 GB in 2 ms
    for key in ("kernel", "bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s"
    assert roof["peak"] == 8000.0                          # MI355X HBM3E
    assert roof["achieved"] == pytest.approx(4000.0)
    assert roof["frac"] == pytest.approx(0.5)
    assert roof["traffic"] is None                         # no counter kernels named


def test_path_bytes_per_head_token():
    # q, k, v, o in bf16 (4 x 128 x 2 bytes) and the two fp32 gates
    assert bench.path_bytes_per_head_token(128) == 1032


def test_counter_figures_follow_the_source(tmp_path, monkeypatch):
    src = "gated_delta_rule_causal_amd/csrc/gdn_mfma.hip"
    sha = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
    rec = {"kernels": {"k_now": {"bytes_per_dispatch": 100.0, "source": src, "source_sha256": sha},
                       "k_old": {"bytes_per_dispatch": 50.0, "source": src, "source_sha256": "0" * 64}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic(["k_now"]) == 100.0
    assert bench.measured_traffic(["k_now", "k_old"]) is None    # any stale kernel voids the sum
    assert bench.measured_traffic(["k_missing"]) is None
