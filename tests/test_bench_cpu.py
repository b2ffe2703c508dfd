"""Host-side checks of bench.py that need no GPU: the one-GPU guard, the
argument checks that run before any device work, and the lookup of counter
traffic in the committed rocprofv3 summaries (keyed on the kernel's sources)."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_receive_without_dedup_is_refused():
    r = _run("--receive")
    assert r.returncode == 2
    assert "--receive needs --dedup" in r.stderr


def _digest(bench, kernel, pkg):
    return bench.sources_digest(kernel, pkg)


def test_counter_traffic_follows_the_sources(tmp_path, monkeypatch):
    """A traffic line counts only while the SHA-256 of the kernel's sources
    matches the one recorded with it; other workloads and modes are not
    confused with it."""
    bench = _bench_module()
    prof = tmp_path / "profiles"
    prof.mkdir()
    kernel = "moe_dispatch_permute"
    good = _digest(bench, kernel, bench.PKG)
    (prof / "hbm_traffic_x.md").write_text(
        "# summary\n\n```\n"
        f"traffic kernel={kernel} workload=wl_a dispatch=nondedup sources_sha256={good} "
        "fetch_kib=1.0 fetch_factor=2.0 write_kib=1.0 write_factor=1.0 bytes=123456\n"
        f"traffic kernel={kernel} workload=wl_b dispatch=nondedup sources_sha256=0000000000000000 "
        "fetch_kib=1.0 fetch_factor=2.0 write_kib=1.0 write_factor=1.0 bytes=654321\n"
        "```\n")
    # a second file: fp8 rows of the same workload
    (prof / "hbm_traffic_y.md").write_text(
        f"traffic kernel={kernel} workload=wl_a dispatch=nondedup dtype=fp8 sources_sha256={good} "
        "fetch_kib=1.0 fetch_factor=2.0 write_kib=1.0 write_factor=1.0 bytes=777\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic(kernel, "wl_a", "nondedup") == 123456
    assert bench.counter_traffic(kernel, "wl_a", "nondedup", "bf16") == 123456
    assert bench.counter_traffic(kernel, "wl_a", "nondedup", "fp8") == 777
    assert bench.counter_traffic(kernel, "wl_b", "nondedup", "fp8") is None
    assert bench.counter_traffic(kernel, "wl_b", "nondedup") is None   # stale sources
    assert bench.counter_traffic(kernel, "wl_a", "dedup") is None      # other mode
    assert bench.counter_traffic(kernel, "wl_c", "nondedup") is None   # no line


def test_digest_covers_every_source_of_a_kernel(tmp_path):
    """Changing any file that holds an entry point's kernel code - its .hip
    file, the headers with its device routines, common.hpp, build.py - changes
    the digest that gates its counter records."""
    import shutil
    bench = _bench_module()
    pkg = tmp_path / "pkg"
    shutil.copytree(os.path.join(bench.PKG, "csrc"), pkg / "csrc")
    shutil.copy(os.path.join(bench.PKG, "build.py"), pkg / "build.py")
    for kernel, files in bench.KERNEL_SOURCES.items():
        base = bench.sources_digest(kernel, str(pkg))
        assert base == bench.sources_digest(kernel)
        for f in files + bench.COMMON_SOURCES:
            path = pkg / f
            text = path.read_bytes()
            path.write_bytes(text + b"\n")
            assert bench.sources_digest(kernel, str(pkg)) != base, (kernel, f)
            path.write_bytes(text)
    # the combine's routines are in the header the combine kernels share
    assert "csrc/combine_rows.hpp" in bench.KERNEL_SOURCES["moe_combine"]


@pytest.mark.parametrize("path", sorted(
    os.path.join(ROOT, "profiles", f) for f in os.listdir(os.path.join(ROOT, "profiles"))
    if f.startswith("hbm_traffic_")))
def test_committed_traffic_lines_are_well_formed(path):
    bench = _bench_module()
    lines = [ln for ln in open(path) if ln.startswith("traffic ")]
    assert lines, f"{path} has no traffic line"
    for ln in lines:
        kv = dict(t.split("=", 1) for t in ln.split()[1:])
        assert kv["kernel"] in bench.KERNEL_SOURCES
        assert kv.get("dtype", "bf16") in ("bf16", "fp8")
        assert len(kv["sources_sha256"]) == 16
        fetch = float(kv["fetch_kib"]) * float(kv["fetch_factor"]) * 1024
        write = float(kv["write_kib"]) * float(kv["write_factor"]) * 1024
        # the factors are printed to 4 decimals, the bytes at full precision
        assert abs(int(kv["bytes"]) - (fetch + write)) <= 1e-4 * (fetch + write)


def test_algorithmic_bytes_c2():
    """The 4096-token, top-6 of 64 experts, hidden-2048 workload: 4096-byte rows,
    24576 sent rows - the per-launch figures the roofline divides by."""
    bench = _bench_module()
    ab = bench.algorithmic_bytes(4096, 2048, 64, 6, 2, 24576, False)
    assert ab["dispatch"] == 4096 * (4096 + 24576) == 117_440_512
    assert ab["combine"] == 4096 * 24576 + 4096 * 4096 == 117_440_512
    assert ab["metadata"] == 24576 * 12 + 4096 * 6 * 4 == 393_216
    assert ab["route"] == 4096 * 64 * 4 + 4096 * 6 * 8 == 1_245_184
    assert ab["job"] == ab["dispatch"] + ab["combine"] + ab["metadata"] + ab["route"]
    assert "expand" not in ab


def test_algorithmic_bytes_receive_side():
    """Dedup with the receive side: 21744 received rows expanded into 24576.
    With fp8 rows the step's combine reads the reduced rows, which are bf16."""
    bench = _bench_module()
    ab = bench.algorithmic_bytes(4096, 2048, 64, 6, 2, 21744, True, 24576)
    assert ab["expand"] == ab["reduce"] == 4096 * (21744 + 24576) == 189_726_720
    assert ab["metadata"] == 21744 * (8 + 8 * 6) + 4096 * 6 * 4
    assert ab["job"] == (ab["dispatch"] + ab["combine"] + ab["metadata"] + ab["route"] +
                         ab["expand"] + ab["reduce"])  # bf16: reduced rows = sent rows in size
    f8 = bench.algorithmic_bytes(4096, 2048, 64, 6, 1, 21744, True, 24576)
    assert f8["dispatch"] == 2048 * (4096 + 21744)
    assert f8["combine"] == 2048 * 21744 + 4096 * 4096          # the send-side combine kernel
    assert f8["expand"] == 2048 * (21744 + 24576)
    assert f8["reduce"] == 2048 * 24576 + 4096 * 21744
    step_combine = 4096 * 21744 + 4096 * 4096                   # reads the bf16 reduced rows
    assert f8["job"] == (f8["dispatch"] + step_combine + f8["metadata"] + f8["route"] +
                         f8["expand"] + f8["reduce"])
