"""Host logic of bench.py that needs no GPU: the byte and FLOP counts the
roofline uses, the issue-slot floor, and how a committed counter summary is
tied to the kernel sources it was taken on."""
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_and_flops_at_the_1p4b_shape():
    b, d, n, L = 8, 4096, 16, 2048
    # u, delta, z read and y written (bf16), B and C read (bf16), A fp32
    # [d, n], D and delta_bias fp32 [d], last_state fp32 [b, d, n]
    expect = 4 * b * d * L * 2 + 2 * b * n * L * 2 + 4 * d * n + 8 * d + 4 * b * d * n
    assert bench.mamba1_bytes(b, d, n, L, 2) == expect == 540_311_552


def test_ssd_work_and_bytes_at_the_ssd_shape():
    b, L, h, p, n, g, Q = 4, 4096, 24, 64, 128, 1, 256
    nc = L // Q
    # C B^T per (b, chunk, group), masked product, chunk states and
    # state-to-output per (b, chunk, head)
    flops = 2 * Q * Q * n * b * nc * g + 2 * Q * Q * p * b * nc * h + 2 * (2 * Q * n * p) * b * nc * h
    assert bench.ssd_flops(b, L, h, p, n, g, Q) == flops == 26_843_545_600
    # x, y (bf16), dt (bf16), B, C (bf16), A/D/dt_bias fp32, final_state fp32
    nbytes = 2 * b * L * h * p * 2 + b * L * h * 2 + 2 * b * L * g * n * 2 + 12 * h + 4 * b * h * p * n
    assert bench.ssd_bytes(b, L, h, p, n, g) == nbytes
    assert abs(nbytes - 113.0e6) < 0.1e6


def test_alu_floor():
    updates = 8 * 4096 * 2048 * 16
    f = bench.alu_floor(updates, 272.0)
    # 6 lane-slots per update at 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
    floor_us = updates * 6 / (256 * 4 * 16 * 2.4e9) * 1e6
    assert f["slots_per_update"] == 6
    assert f["floor_us"] == pytest.approx(floor_us, abs=0.05)
    assert f["frac"] == pytest.approx(floor_us / 272.0, abs=1e-4)


def test_sources_sha256_covers_every_file_in_order(tmp_path):
    a, b = tmp_path / "a.hip", tmp_path / "b.h"
    a.write_bytes(b"kernel")
    b.write_bytes(b"header")
    h1 = bench.sources_sha256([str(a), str(b)])
    b.write_bytes(b"header changed")
    assert bench.sources_sha256([str(a), str(b)]) != h1   # a header change counts
    b.write_bytes(b"header")
    assert bench.sources_sha256([str(a), str(b)]) == h1
    assert bench.sources_sha256([str(b), str(a)]) != h1   # order is part of the key


def test_measured_traffic_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_bytes(b"v1")
    prof = tmp_path / "profiles"
    prof.mkdir()
    sha = bench.sources_sha256([str(src)])
    (prof / "kern_work_hbm_traffic.md").write_text(
        "# summary\n\n| a | b |\n|---|---|\n\n"
        f"kernel_sources_sha256: {sha}\n"
        "traffic_bytes_per_launch: 12345\n"
        "traffic_bytes_per_call: 678\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("kern_work", [str(src)]) == 12345
    assert bench.measured_traffic("kern_work", [str(src)], per="call") == 678
    assert bench.measured_traffic("missing", [str(src)]) is None
    src.write_bytes(b"v2")  # the kernel changed since the counters were taken
    assert bench.measured_traffic("kern_work", [str(src)]) is None


def test_committed_summaries_name_existing_sources():
    for name in ("selective_scan_fwd_kernel_m1p4b_hbm_traffic.md",
                 "ssd_chunk_scan_ssd_hbm_traffic.md"):
        text = open(os.path.join(ROOT, "profiles", name)).read()
        line = [l for l in text.splitlines() if l.startswith("kernel_sources:")][0]
        for rel in line.split(":", 1)[1].split(","):
            assert os.path.exists(os.path.join(ROOT, rel.strip())), rel


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def _profile(name):
    return open(os.path.join(ROOT, "profiles", name)).read()


def test_committed_trace_agrees_with_bench_event_time():
    """The kernel trace's average duration of the headline kernel agrees with
    the HIP-event average bench.py measured in the same traced run (the trace
    also counts the warm-up launches, so a few percent apart)."""
    import re
    text = _profile("selective_scan_fwd_kernel_m1p4b_kernel_trace.md")
    row = [l for l in text.splitlines() if l.startswith("| `selective_scan_fwd_kernel<")][0]
    trace_us = float(row.split("|")[3]) / 1000.0
    event_us = float(re.search(r"selective_scan_fwd_kernel ([0-9.]+) us", text).group(1))
    assert abs(trace_us - event_us) / event_us < 0.05, (trace_us, event_us)


def test_committed_traffic_is_close_to_the_algorithmic_bytes():
    """HBM bytes measured by FETCH_SIZE/WRITE_SIZE for the headline kernel
    stay within 5% of the bytes the method must move (no wasted re-reads)."""
    text = _profile("selective_scan_fwd_kernel_m1p4b_hbm_traffic.md")
    measured = int([l for l in text.splitlines()
                    if l.startswith("traffic_bytes_per_launch:")][0].split(":")[1])
    algorithmic = bench.mamba1_bytes(8, 4096, 16, 2048, 2)
    assert 0.98 <= measured / algorithmic <= 1.05, measured / algorithmic
