"""Host-side logic of bench.py (no GPU): the one-GPU guard, the byte counts
behind the roofline figures, the source hash that ties committed rocprofv3
summaries to the kernel code they were taken on, and the parsing of those
summaries."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    # The guard runs before torch is imported, so this needs no GPU.
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_byte_counts():
    # [8192, 28672] fused: packed weights + bf16 row + int8 row + scale + fp32 y
    assert bench.algo_bytes_fused(8192, 28672) == 58_720_256 + 57_344 + 28_672 + 4 + 32_768
    assert bench.algo_bytes_fused(8192, 28672) == 58_839_044
    # int8 form at M rows: weights + M*K int8 + M scales + M*N fp32
    assert bench.algo_bytes(2560, 6912, M=4) == 4_423_680 + 4 * 6912 + 16 + 4 * 4 * 2560
    assert bench.weight_bytes(28672, 8192) == 58_720_256
    step = sum(bench.weight_bytes(N, K) for N, K in bench.SHAPES.values())
    assert step == 121_864_192


def test_graph_sizes_cover_every_step_evenly():
    # every timed step is in a multi-step graph of at most 12 steps; sizes
    # differ by at most one (no one-step remainder graphs)
    assert bench.graph_sizes(20) == [10, 10]
    assert bench.graph_sizes(12) == [12]
    assert bench.graph_sizes(5) == [5]
    assert bench.graph_sizes(1) == [1]
    for k in (13, 50, 199, 200, 1000):
        g = bench.graph_sizes(k)
        assert sum(g) == k and max(g) <= bench.STEP_COPIES
        assert max(g) - min(g) <= 1 and len(g) == -(-k // bench.STEP_COPIES)


def test_code_only_ignores_comments_and_blank_lines():
    a = "int x = 1;  // one\n\n// a comment line\nint y = 2;\n"
    b = "int x = 1;\nint y = 2;   // two\n\n\n"
    assert bench.code_only(a) == bench.code_only(b) == "int x = 1;\nint y = 2;"
    assert bench.code_only("int x = 1;") != bench.code_only("int x = 2;")


def test_source_hash_tracks_code_not_comments():
    base = {rel: open(os.path.join(ROOT, rel), encoding="utf-8").read()
            for rel in bench.KERNEL_SOURCES}
    h0 = bench.kernel_source_hash(lambda rel: base[rel])
    assert h0 == bench.kernel_source_hash()
    first = bench.KERNEL_SOURCES[0]
    commented = dict(base)
    commented[first] = base[first] + "\n// a new comment\n\n"
    assert bench.kernel_source_hash(lambda rel: commented[rel]) == h0
    changed = dict(base)
    changed[first] = base[first] + "\nstatic int unused_marker;\n"
    assert bench.kernel_source_hash(lambda rel: changed[rel]) != h0


def test_read_profile_needs_the_current_source(tmp_path):
    good = tmp_path / "good.txt"
    good.write_text("# a comment: with a colon\n"
                    f"kernel_source_sha256_16: {bench.kernel_source_hash()}\n"
                    "dominant_trace_avg_us: 13.5\n"
                    "dominant_trace_median_us: 13.25\n")
    f = bench.read_profile(str(good))
    assert f["dominant_trace_avg_us"] == "13.5"
    assert "# a comment" not in f
    stale = tmp_path / "stale.txt"
    stale.write_text("kernel_source_sha256_16: 0000000000000000\n"
                     "dominant_trace_avg_us: 13.5\n")
    assert bench.read_profile(str(stale)) is None
    assert bench.read_profile(str(tmp_path / "missing.txt")) is None


def test_trace_fields_arithmetic():
    t = bench.trace_fields((13.5, 13.25), 58_839_044)
    assert t["frac_from_avg"] == pytest.approx(58_839_044 / 13.5e-6 / 8e12, abs=1e-4)
    assert t["frac_from_median"] == pytest.approx(58_839_044 / 13.25e-6 / 8e12, abs=1e-4)
    assert bench.trace_fields(None, 1) is None


@pytest.mark.parametrize("path,keys", [
    (bench.TRACE_FILE, ("kernel_source_sha256_16", "dominant_trace_avg_us",
                        "dominant_trace_median_us", "dominant_trace_dispatches")),
    (bench.COUNTER_FILE, ("kernel_source_sha256_16", "fetch_kib_per_dispatch",
                          "write_kib_per_dispatch", "fetch_factor", "write_factor",
                          "hbm_bytes_per_launch")),
])
def test_committed_profiles_carry_their_fields(path, keys):
    assert os.path.exists(path), path
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    for k in keys:
        assert k in fields, (path, k)
    if "hbm_bytes_per_launch" in fields:
        # traffic = fetch KiB x factor + write KiB x factor, in bytes
        f = fields
        t = (float(f["fetch_kib_per_dispatch"]) * float(f["fetch_factor"]) +
             float(f["write_kib_per_dispatch"]) * float(f["write_factor"])) * 1024
        assert float(f["hbm_bytes_per_launch"]) == pytest.approx(t, rel=2e-3)
