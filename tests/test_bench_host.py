"""Host-side logic of bench.py, on the CPU: the single-GPU guard, the
algorithmic byte count the roofline divides by, the rotation that keeps
weights out of the Infinity Cache, and the gate that drops the measured
traffic once the decode kernel's sources change."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_decode_algorithmic_bytes():
    # packed int4 weights N*K/2, fp16 group scales N*(K/128)*2, fp16
    # activations M*K*2, fp16 output M*N*2
    M, K, N = 64, 5120, 5120
    assert bench.gemm_bytes(M, K, N) == 13_107_200 + 409_600 + 655_360 + 655_360 == 14_827_520


def test_weight_rotation_passes_the_infinity_cache():
    for nbytes in (1 << 20, 13_516_800, 92_000_000, 700_000_000):
        n = bench.copies_for(nbytes)
        assert n >= 2
        # every call reads a copy last touched more than twice the cache's size of traffic ago
        assert (n - 1) * nbytes >= 2 * bench.MALL_BYTES or n == 2 and nbytes >= 2 * bench.MALL_BYTES


def test_traffic_is_reported_only_for_the_measured_sources(monkeypatch, tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("// a kernel\n")
    import hashlib
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "traffic.md"
    prof.write_text(f"traffic_bytes_per_launch: 1234\nkernel_sources_sha256: {digest} (kernel.hip)\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(prof))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["kernel.hip"])
    assert bench.measured_traffic() == 1234
    src.write_text("// a kernel, changed\n")
    assert bench.measured_traffic() is None
    prof.write_text("no fields here\n")
    assert bench.measured_traffic() is None


@pytest.mark.parametrize("flag", ["--extras", "--no-clocks", "--no-extra", "--copy-calibration"])
def test_cli_lists_its_options(flag):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 0 and flag in r.stdout
    assert set(bench.EXTRA_SECTIONS) == {"gemm", "norm", "attention", "vocab", "heads", "sampler"}
