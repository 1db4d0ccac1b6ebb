"""Host-side logic of bench.py that needs no GPU: the one-GPU guard and the
gating of the recorded HBM traffic on the kernel source it was measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (stdlib-only at import time)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=60, env={**os.environ, "WORLD_SIZE": "1"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _traffic_file_values():
    vals = {}
    with open(bench.TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                vals[parts[0]] = parts[1]
    return vals


def test_recorded_traffic_follows_the_summary_digest():
    # the summary's figure is reported exactly while it was taken on the kernel
    # source in the tree, and not at all once that source has changed
    vals = _traffic_file_values()
    if vals["kernel_source_digest"] == bench.kernel_source_digest():
        assert bench.recorded_traffic("verify512") == int(vals["hbm_bytes_per_launch"])
    else:
        assert bench.recorded_traffic("verify512") is None


def test_recorded_traffic_only_for_the_workload_it_was_measured_on():
    for w in ("decode8", "prefill8192", "hash2048", "draft448"):
        assert bench.recorded_traffic(w) is None


def test_recorded_traffic_is_dropped_when_the_kernel_source_changes(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
    assert bench.recorded_traffic("verify512") is None


def test_recorded_traffic_is_dropped_without_a_summary(monkeypatch, tmp_path):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert bench.recorded_traffic("verify512") is None


@pytest.mark.parametrize("content", ["kernel_source_digest {d}\n", "kernel_source_digest {d}\nhbm_bytes_per_launch many\n"])
def test_a_malformed_summary_gives_no_traffic(monkeypatch, tmp_path, content):
    p = tmp_path / "t.txt"
    p.write_text(content.format(d=bench.kernel_source_digest()))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.recorded_traffic("verify512") is None


def test_probe_options_parse_and_the_probe_library_is_required(monkeypatch):
    # the streaming-read probe runs by default; --no-hbm-probe leaves it out of profiling runs
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    args = bench.parse()
    assert not args.no_hbm_probe and not args.hbm_probe_only
    monkeypatch.setattr(sys, "argv", ["bench.py", "--no-hbm-probe", "--only"])
    assert bench.parse().no_hbm_probe
    # the probe's bytes are 8x the 256 MB memory-side cache and whole 16-byte pieces
    assert bench.HBM_PROBE_BYTES >= 8 * 256 * 2 ** 20 and bench.HBM_PROBE_BYTES % 16 == 0
    # without its library the probe stops with a message instead of reporting a figure
    monkeypatch.setattr(bench, "HBM_PROBE_LIB", os.path.join(ROOT, "no_such_dir", "libmoe_hbm.so"))
    with pytest.raises(SystemExit, match="libmoe_hbm.so is missing"):
        bench.hbm_read_peak(None, None, None)
