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
    f.write_text(json.dumps({"workloads": {"w": {"kernel_source_sha": "abc",
                                                 "hbm_bytes_per_call": 123},
                                           "bwd:w": {"kernel_source_sha": "def",
                                                     "hbm_bytes_per_call": 456}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for("w", "abc") == 123
    assert bench.traffic_for("w", "abd") is None
    assert bench.traffic_for("bwd:w", "def") == 456
    assert bench.traffic_for("bwd:w", "abc") is None
    assert bench.traffic_for("other", "abc") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for("w", "abc") is None


def test_forward_traffic_keys_name_the_variant():
    assert bench.fwd_key("c2", 0) == "c2"
    assert bench.fwd_key("c2", 2) == "c2@v2"


def test_roofline_names_the_kernel_the_variant_runs():
    """The line's roofline.kernel follows the library's dispatch: the
    ping-pong variants (and the d = 128 default) run attn_fwd_pp_kernel,
    whose trace is the committed forward profile."""
    from exact_tiled_attention_attn_amd import attn
    for v in (1, 2, 3, 4):
        pp = "pingpong" in attn.attn_variant_name(v)
        assert (bench.fwd_kernel_name(128, v) == "attn_fwd_pp_kernel") == pp, v
    assert bench.fwd_kernel_name(128, 0) == "attn_fwd_pp_kernel"
    assert bench.fwd_kernel_name(64, 0) == "attn_fwd_kernel"
    assert os.path.exists(os.path.join(ROOT, "profiles",
                                       "attn_fwd_pp_kernel_c2_c2sharp_c3_c4_c5_c5w.md"))


def test_kernel_kinds_hash_their_own_source():
    shas = {k: bench.kernel_sha(k) for k in bench.KERNEL_SOURCES}
    assert shas["fwd"] == shas["varlen"] == bench.kernel_sha()
    assert len({shas["fwd"], shas["bwd"], shas["fp8"], shas["decode"]}) == 4


def test_committed_traffic_is_consistent():
    """Each stored entry's bytes are its scaled counters; the main workload's
    entry is that of the forward kernel as it stands, so the bench line's
    roofline.traffic is not null."""
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    for key, e in t["workloads"].items():
        scaled = (e["fetch_kib"] * 1024 * t["fetch_scale"]
                  + e["write_kib"] * 1024 * t["write_scale"])
        assert abs(scaled - e["hbm_bytes_per_call"]) <= 1, key
        kind = key.split(":", 1)[0] if ":" in key else "fwd"
        assert kind in bench.KERNEL_SOURCES, key
    assert t["workloads"][bench.MAIN]["kernel_source_sha"] == bench.kernel_sha()


def test_peaks_from_device_properties():
    p = bench.derive_peaks((256, 2400000, 2000000, 8192), 2516.6, 5033.2)
    assert p["bf16_tflops"] == 2516.6 and p["fp8_tflops"] == 5033.2
    assert p["bf16_flop_per_cu_clock"] == 4096 and p["max_clock_mhz"] == 2400.0
    assert bench.derive_peaks((128, 2100000, 0, 0), 0, 0)["bf16_tflops"] == 1101.0
    import pytest
    with pytest.raises(RuntimeError):
        bench.derive_peaks((0, 2400000, 0, 0), 0, 0)


def test_kernel_sha_does_not_depend_on_where_the_repository_sits(monkeypatch):
    from exact_tiled_attention_attn_amd import build
    h1 = bench.kernel_sha()
    moved = [f.replace(build.ROOT, "/elsewhere/repo") for f in build.COMMON]
    assert moved != build.COMMON
    monkeypatch.setattr(build, "COMMON", moved)
    assert bench.kernel_sha() == h1
