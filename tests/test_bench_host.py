"""Host logic of bench.py (no GPU): the one-GPU guard, and the lookup that attaches
the counter-measured bytes of a call to the JSON line only while the kernel sources
still match the digest recorded with the counters, and the host facts it reports."""
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
                    f"- hbm_bytes_per_call[grouped_nvfp4_rht]: {nbytes}\n"
                    f"- kernel_source_sha256: {digest}\n")


def test_traffic_used_only_for_matching_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.md"
    monkeypatch.setitem(bench.TRAFFIC_SUMMARIES, "grouped_nvfp4_rht", str(f))
    write_summary(f, bench.kernel_source_digest(), 361316864)
    assert bench.measured_traffic("grouped_nvfp4_rht") == 361316864
    write_summary(f, "0" * 64, 361316864)                                            # sources changed since
    assert bench.measured_traffic("grouped_nvfp4_rht") is None
    f.unlink()
    assert bench.measured_traffic("grouped_nvfp4_rht") is None
    monkeypatch.delitem(bench.TRAFFIC_SUMMARIES, "dsa_rotate_fp8")
    assert bench.measured_traffic("dsa_rotate_fp8") is None                          # no summary at all


def test_digest_covers_the_kernel_sources(tmp_path, monkeypatch):
    """Every .hip / .hpp / .cpp of the library's sources enters the digest: a change to
    any of them (here in a copy of the folder) changes it."""
    import shutil
    src = os.path.join(ROOT, bench.KERNEL_SOURCE_DIR)
    names = [n for n in os.listdir(src) if n.endswith((".hip", ".hpp", ".cpp"))]
    assert any(n.endswith(".hip") for n in names) and any(n.endswith(".hpp") for n in names)
    d0 = bench.kernel_source_digest()
    assert len(d0) == 64
    copy = tmp_path / "csrc"
    shutil.copytree(src, copy)
    monkeypatch.setattr(bench, "KERNEL_SOURCE_DIR", str(copy))          # absolute: os.path.join keeps it
    assert bench.kernel_source_digest() == d0
    for n in names:
        with open(copy / n, "ab") as fh:
            fh.write(b"\n")
        assert bench.kernel_source_digest() != d0, n
        with open(copy / n, "rb+") as fh:
            data = fh.read()[:-1]
            fh.seek(0)
            fh.write(data)
            fh.truncate()
        assert bench.kernel_source_digest() == d0


def test_host_threads_is_a_one_gpu_share():
    assert 1 <= bench.host_threads() <= 16


def test_cpu_model_is_named():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
