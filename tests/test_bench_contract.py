"""bench.py's contract pieces that run without a GPU: the one-GPU guard, the
roofline object, the algorithmic byte counts of the workloads and the
profile-backed traffic lookup."""
import hashlib
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from segment_wise_compressive_amd import inputs as inp  # noqa: E402

WORKLOAD_NAMES = [inp.HEADLINE, inp.SEGMENTED, inp.DECODE, inp.NONCAUSAL]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_roofline_object():
    r = bench.roofline(83_886_080, 0.0419430, 100)
    assert set(r) == {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(2000.0, rel=1e-4)
    assert r["frac"] == pytest.approx(0.25, abs=1e-4)
    assert r["traffic"] == 100


def test_algorithmic_bytes_of_the_workloads():
    # 3 bf16 inputs + fp32 output per head-token: 640 B at d = 64
    assert bench.alg_bytes_causal(inp.WORKLOADS[inp.HEADLINE]) == 4 * 8 * 4096 * 640
    # one 2048-token segment at d = 128 plus fp32 state in and out
    seg = inp.WORKLOADS[inp.SEGMENTED]
    one = inp.Workload("segment", "causal", seg.dtype, seg.B, seg.H, seg.segment, seg.d, 0, 1.0)
    assert bench.alg_bytes_causal(one, with_state_io=True) == 16 * 2048 * (3 * 128 * 2 + 4 * 128) + \
        2 * 16 * (128 * 128 + 128) * 4
    assert bench.alg_bytes_causal(inp.WORKLOADS[inp.NONCAUSAL]) == 8 * 16 * 16384 * 640


@pytest.mark.parametrize("name", WORKLOAD_NAMES)
def test_every_workload_has_its_hbm_profile(name):
    path = os.path.join(ROOT, "profiles", f"{name}_hbm_bytes.txt")
    text = open(path).read()
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text
    assert "traffic_bytes_per_call:" in text and "source_sha256:" in text


@pytest.mark.parametrize("name", WORKLOAD_NAMES)
def test_traffic_follows_the_source_hash(name, tmp_path, monkeypatch):
    # a copy of the tree's profile and source: the traffic is reported while
    # the hash matches and withheld once the source differs
    (tmp_path / "profiles").mkdir()
    src_dir = tmp_path / "segment_wise_compressive_amd" / "csrc"
    src_dir.mkdir(parents=True)
    shutil.copy(os.path.join(ROOT, "profiles", f"{name}_hbm_bytes.txt"), tmp_path / "profiles")
    src = open(os.path.join(ROOT, "segment_wise_compressive_amd", "csrc", "linattn.hip"), "rb").read()
    (src_dir / "linattn.hip").write_bytes(src)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    text = open(tmp_path / "profiles" / f"{name}_hbm_bytes.txt").read()
    recorded = [l.split(": ", 1)[1].strip() for l in text.splitlines() if l.startswith("source_sha256:")][0]
    got = bench.measured_traffic(name)
    if recorded == hashlib.sha256(src).hexdigest():
        assert isinstance(got, int) and got > 0
    else:
        assert got is None
    (src_dir / "linattn.hip").write_bytes(src + b"\n// changed\n")
    assert bench.measured_traffic(name) is None
