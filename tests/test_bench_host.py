"""Host-side logic of bench.py (CPU only): the one-GPU guard, the hash check
that decides whether the committed HBM-traffic record still describes the
kernel source, and the host description that goes into cpu_baseline."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

SRC = "grouped_gemm_glu_amd/csrc/group_gemm.hpp"


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def _record(tmp_path, sha):
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps({"kernel_source": SRC, "source_sha256_16": sha,
                             "fc1_hbm_bytes_per_launch": 123.0}))
    return str(p)


def test_traffic_record_used_only_while_the_source_matches(tmp_path):
    with open(os.path.join(ROOT, SRC), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    assert bench.read_traffic(_record(tmp_path, sha)) == 123.0
    stale = ("0" if sha[0] != "0" else "1") + sha[1:]
    assert bench.read_traffic(_record(tmp_path, stale)) is None
    assert bench.read_traffic(str(tmp_path / "missing.json")) is None
    assert bench.read_traffic(None) is None


def test_committed_traffic_record_is_well_formed():
    rec = json.load(open(os.path.join(ROOT, "profiles", "fc1_glu_dsv3_traffic.json")))
    assert rec["kernel_source"] == SRC
    assert len(rec["source_sha256_16"]) == 16
    # FC1's algorithmic bytes are 2.315 GB; measured traffic can only exceed them
    assert 2.3e9 < rec["fc1_hbm_bytes_per_launch"] < 1e10


def test_host_info_names_cpu_and_blas():
    model, blas = bench._host_info()
    if os.path.exists("/proc/cpuinfo"):
        assert model
    assert blas is None or isinstance(blas, str)


@pytest.mark.parametrize("argv", [["--steps", "3", "--warmup", "1"], []])
def test_parse_defaults(monkeypatch, argv):
    monkeypatch.setattr(sys, "argv", ["bench.py"] + argv)
    a = bench.parse()
    assert a.gpus == 1
    assert a.steps == (3 if argv else 20) and a.warmup == (1 if argv else 5)
