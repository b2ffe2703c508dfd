"""The oracle and the library's host placement search, built for the host
with AddressSanitizer and UndefinedBehaviorSanitizer (gcc/g++), run on small
and edge-case shapes by tests/sanitize_driver.cpp (no GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def test_oracle_and_search_under_sanitizers(tmp_path):
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("no host compiler")
    search_src = tmp_path / "placement_search.cpp"      # the library's host search, as C++
    shutil.copy(os.path.join(ROOT, "combine_top_router_select_amd", "csrc", "placement.hip"),
                search_src)
    objs = []
    for src, comp, std in ((os.path.join(ROOT, "oracle", "oracle.c"), "gcc", "-std=c11"),
                           (str(search_src), "g++", "-std=c++17"),
                           (os.path.join(ROOT, "tests", "sanitize_driver.cpp"), "g++", "-std=c++17")):
        obj = tmp_path / (os.path.basename(src) + ".o")
        r = subprocess.run([comp, std, *SAN, "-ffp-contract=off", "-c", src, "-o", str(obj)],
                           capture_output=True, text=True)
        if r.returncode != 0 and "asan" in r.stderr.lower():
            pytest.skip("sanitizer runtime not available")
        assert r.returncode == 0, r.stderr
        objs.append(str(obj))
    exe = tmp_path / "driver"
    r = subprocess.run(["g++", *SAN, *objs, "-o", str(exe), "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr
