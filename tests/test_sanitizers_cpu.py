"""The host code of libslide that runs threads of its own (the CPU AdamW's worker threads, the
disk tier's I/O pool and streamed update) built with AddressSanitizer + UndefinedBehaviorSanitizer
and, separately, with ThreadSanitizer, and driven by tests/sanitize/host_driver.cpp: any memory
error, undefined behaviour or data race fails the run. CPU only (g++)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "layer_sliding_offloaded_fwd_amd", "csrc")
SOURCES = [os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
           os.path.join(CSRC, "adamw.cpp"), os.path.join(CSRC, "tier.cpp")]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_host_code_under_sanitizer(tmp_path, san):
    exe = tmp_path / "driver"
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-ffp-contract=off", "-pthread",
           f"-fsanitize={san}", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
           *SOURCES, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe), str(tmp_path)], capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0 and "host driver: ok" in r.stdout, (r.stdout + r.stderr)[-4000:]
    assert "WARNING: ThreadSanitizer" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
