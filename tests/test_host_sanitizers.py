"""The library's host functions (quantisation, selection, packing, layouts,
pool files) built with AddressSanitizer and UndefinedBehaviorSanitizer and
run on ragged and degenerate shapes with exact-size buffers
(tests/sanitize/host_checks.cpp), on the default thread count and on one
thread.  Host code only: no GPU code is compiled here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_quantized_quantize_amd", "csrc")


def _clang():
    for cand in ("/opt/rocm/lib/llvm/bin/clang++", "/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_host_functions_under_asan_and_ubsan(tmp_path):
    cxx = _clang()
    if cxx is None:
        pytest.skip("no clang++ with the sanitizer runtimes")
    exe = str(tmp_path / "host_checks")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"),
           os.path.join(CSRC, "woq_host.cpp"), os.path.join(CSRC, "woq_pool.cpp"), "-lpthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr + r.stdout).lower() and "cannot find" in (r.stderr + r.stdout):
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stdout + r.stderr
    for threads in (None, "1"):
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
        if threads:
            env["WOQ_NUM_THREADS"] = threads
        r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0 and "host checks ok" in r.stdout, (threads, r.stdout[-4000:], r.stderr[-4000:])
