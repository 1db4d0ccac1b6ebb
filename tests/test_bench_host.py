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


def test_algorithmic_bytes_and_flops_follow_the_expert_size():
    # one MXFP4 expert (gate, up, down at d 4096, I 2048) is 3 x 4096 x 2048 values at 4 bits plus one
    # E8M0 byte per 32 values: 13,369,344 bytes, the 13.4 MB per expert the pages give for V4 Flash
    # (FaStar README, "Expert virtual memory"); the verify512 layer touches all 256 routed experts + shared
    from mxfp4_routed_expert_sqrt_amd.configs import SHAPES
    sh = SHAPES["verify512"]
    a = bench.algorithmic(sh, 256)
    per_expert = 3 * (4096 * 2048 // 2 + 4096 * 2048 // 32)
    assert per_expert == 13_369_344
    x = out = 512 * 4096 * 2
    assert a["layer_bytes"] == 257 * per_expert + 256 * 4096 * 4 + x + out == 3_448_504_320
    assert a["gateup_bytes"] == 257 * per_expert * 2 // 3 + x == 2_294_808_576
    assert a["down_bytes"] == 257 * per_expert // 3
    # FP4-equivalent flops: 2 per multiply-add, 3 matrices of d x I per (row, expert), k + 1 experts per row
    assert a["layer_flops"] == 6 * 4096 * 2048 * 512 * 7 == 180_388_626_432
    assert a["gateup_flops"] + a["down_flops"] == a["layer_flops"]
    # an expert with no rows reads no weights: fewer touched experts, fewer bytes
    assert bench.algorithmic(sh, 100)["layer_bytes"] == a["layer_bytes"] - 156 * per_expert
