"""CPU tests of bench.py's host side: the one-GPU refusal, and that the HBM
traffic it reports comes from the committed profile only while the kernel
sources are the ones the counters were taken on."""

import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_recorded_traffic_follows_the_source_digest(tmp_path, monkeypatch):
    # a copy of the repository's profile and sources, so that the sources can be changed
    (tmp_path / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, "profiles", "hbm_traffic_qwen3_8b_1m_shard.md"), tmp_path / "profiles")
    shutil.copytree(os.path.join(ROOT, "lm_head_chunked_amd", "csrc"), tmp_path / "lm_head_chunked_amd" / "csrc")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    text = (tmp_path / "profiles" / "hbm_traffic_qwen3_8b_1m_shard.md").read_text()
    fresh = f"kernel_source_sha256: {bench.kernel_source_digest()}" in text
    got = bench.recorded_traffic("qwen3_8b_1m_shard", "k_fwd_dh")
    if fresh:
        # bytes per launch of the fused forward: at least its operands (h and W, 2.2 GB, read once)
        assert got is not None and got > 2.2e9
    else:
        assert got is None
    # any change to a kernel source makes the recorded figure stale
    with open(tmp_path / "lm_head_chunked_amd" / "csrc" / "lmce_bwd.hip", "a") as f:
        f.write("\n")
    assert bench.recorded_traffic("qwen3_8b_1m_shard", "k_fwd_dh") is None
    # no profile for a workload: no figure
    assert bench.recorded_traffic("qwen3_32b", "k_fwd_dh") is None
