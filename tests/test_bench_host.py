"""Host-side logic of bench.py that needs no GPU: the one-GPU guard, the
kernel-source hash that keys the stored counter data, and the lookup of
that data."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_sha_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    hdr = tmp_path / "h.h"
    src.write_text("int a = 1;  // one\n\n// a comment line\nint b = 2;\n")
    hdr.write_text("int c = 3;\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    monkeypatch.setattr(bench, "KERNEL_HEADERS", [str(hdr)])
    h1 = bench.kernel_sha()
    src.write_text("int a = 1;   \n// another comment\nint b = 2;  // two\n\n")
    assert bench.kernel_sha() == h1
    src.write_text("int a = 1;\nint b = 3;\n")
    assert bench.kernel_sha() != h1


def test_kernel_sha_covers_the_device_header_and_flags(tmp_path, monkeypatch):
    from exact_tiled_attention_attn_amd import build
    src = tmp_path / "k.hip"
    hdr = tmp_path / "h.h"
    src.write_text("int a = 1;\n")
    hdr.write_text("int c = 3;\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    monkeypatch.setattr(bench, "KERNEL_HEADERS", [str(hdr)])
    h1 = bench.kernel_sha()
    hdr.write_text("int c = 4;\n")
    h2 = bench.kernel_sha()
    assert h2 != h1
    monkeypatch.setattr(build, "DEVICE_ONLY", build.DEVICE_ONLY + ["-DX"])
    assert bench.kernel_sha() != h2


def test_traffic_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"kernel_source_sha": "abc",
                             "workloads": {"w": {"hbm_bytes_per_launch": 123}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for("w", "abc") == 123
    assert bench.traffic_for("w", "abd") is None
    assert bench.traffic_for("other", "abc") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for("w", "abc") is None


def test_committed_traffic_matches_the_current_kernel_source():
    """The stored HBM counters are those of the kernel as it stands, so the
    bench line's roofline.traffic is not null."""
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    assert t["kernel_source_sha"] == bench.kernel_sha()
    e = t["workloads"]["c2_causal_mha"]
    scaled = e["fetch_kib"] * 1024 * t["fetch_scale"] + e["write_kib"] * 1024 * t["write_scale"]
    assert abs(scaled - e["hbm_bytes_per_launch"]) <= 1
