"""Host logic of bench.py (no GPU): the one-GPU guard, and the lookup that attaches
the counter-measured bytes of the dominant kernel to the JSON line only while the
kernel sources still match the digest recorded with the counters."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def write_summary(path, digest, nbytes):
    path.write_text("# summary\n\n"
                    f"- hbm_bytes_per_launch k_nvfp4_quant: {nbytes}\n"
                    f"- kernel_source_sha256: {digest}\n")


def test_traffic_used_only_for_matching_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.md"
    monkeypatch.setitem(bench.TRAFFIC_SUMMARIES, "grouped_nvfp4_rht", str(f))
    write_summary(f, bench.kernel_source_digest(), 226627481)
    assert bench.measured_traffic("grouped_nvfp4_rht", "k_nvfp4_quant") == 226627481
    assert bench.measured_traffic("grouped_nvfp4_rht", "k_nvfp4_amax") is None      # no figure for it
    write_summary(f, "0" * 64, 226627481)                                            # sources changed since
    assert bench.measured_traffic("grouped_nvfp4_rht", "k_nvfp4_quant") is None
    f.unlink()
    assert bench.measured_traffic("grouped_nvfp4_rht", "k_nvfp4_quant") is None
    assert bench.measured_traffic("dsa_rotate_fp8", "k_nvfp4_quant") is None         # no summary at all


def test_digest_covers_the_kernel_sources():
    for f in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, f)), f
    assert len(bench.kernel_source_digest()) == 64


def test_host_threads_is_a_one_gpu_share():
    assert 1 <= bench.host_threads() <= 16
