"""Host-side checks of the benchmark harness (no GPU): the one-GPU guard and the
rule that a committed HBM-counter summary is reported only while the kernel
sources it was taken on are unchanged."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    csrc = tmp_path / "selective_scan_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES["scan"]:
        shutil.copy(os.path.join(ROOT, "selective_scan_amd", "csrc", f), csrc / f)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def _summary(root, sha, nbytes=12345):
    (root / "profiles" / "traffic_x.md").write_text(
        f"# test\n\ntraffic_bytes_per_launch: {nbytes}\nsources_sha256: {sha}\n")


def test_traffic_reported_while_sources_match(fake_root):
    _summary(fake_root, bench.sources_sha256("scan"))
    assert bench.committed_traffic("scan", "traffic_x.md") == 12345


def test_comment_edit_keeps_and_code_edit_voids_the_measurement(fake_root):
    _summary(fake_root, bench.sources_sha256("scan"))
    src = fake_root / "selective_scan_amd" / "csrc" / bench.KERNEL_SOURCES["scan"][0]
    text = src.read_text()
    src.write_text(text + "\n// a comment only\n")
    assert bench.committed_traffic("scan", "traffic_x.md") == 12345
    src.write_text(text + "\nstatic int unused_probe_value = 1;\n")
    assert bench.committed_traffic("scan", "traffic_x.md") is None


def test_missing_or_malformed_summary_gives_none(fake_root):
    assert bench.committed_traffic("scan", "traffic_absent.md") is None
    (fake_root / "profiles" / "traffic_x.md").write_text("traffic_bytes_per_launch: 5\n")
    assert bench.committed_traffic("scan", "traffic_x.md") is None


def test_committed_summaries_are_well_formed():
    """Every counter summary under profiles/ carries a byte count, a 64-hex source
    hash and the full commands that produced it."""
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.startswith(("traffic_", "ssd_kernels_"))]
    assert names
    for n in names:
        text = open(os.path.join(prof, n)).read()
        assert re.search(r"traffic_bytes_per_launch:\s*\d+", text), n
        assert re.search(r"sources_sha256:\s*[0-9a-f]{64}", text), n
        assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text, n
