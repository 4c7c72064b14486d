"""The host-side W_KV solver (threaded blocked LU) and the float64 -> bf16
rounding under AddressSanitizer + UndefinedBehaviorSanitizer and under
ThreadSanitizer: tests/host_sanitize/wkv_check.cpp is compiled with g++
together with the library's wkv_host.cpp and run with four solver threads."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = [os.path.join(HERE, "host_sanitize", "wkv_check.cpp"),
       os.path.join(ROOT, "kv_cache_reduction_amd", "csrc", "wkv_host.cpp")]


def _build_and_run(tmp_path, flags, name):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / name)
    r = subprocess.run([gxx, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", *flags, *SRC, "-o", exe,
                        "-lpthread"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, SLIM_HOST_THREADS="4", ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok"), r.stdout


def test_wkv_host_address_and_undefined_behaviour(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"], "wkv_asan")


def test_wkv_host_threads(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=thread"], "wkv_tsan")
