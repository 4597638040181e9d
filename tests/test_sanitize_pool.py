"""The host block pool (fork, copy on write, growth, release, error paths)
built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
driven against a reference-count model, and under ThreadSanitizer with eight
threads that keep the pool's rule (one pool, one caller at a time): private
pools per thread and a shared pool behind a mutex (host code only, no
GPU)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_pool_under_sanitizers(tmp_path):
    exe = str(tmp_path / "pool_driver")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", f"-I{ROOT}/include", f"-I{ROOT}/transformer_attention_05_amd/csrc",
           f"{ROOT}/transformer_attention_05_amd/csrc/pool.cpp", f"{ROOT}/tests/sanitize/pool_driver.cpp", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr + r.stdout).lower():
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-3000:]
    assert "pool driver: ok" in run.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_pool_threads_under_tsan(tmp_path):
    exe = str(tmp_path / "pool_threads")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=thread", "-pthread",
           f"-I{ROOT}/include", f"-I{ROOT}/transformer_attention_05_amd/csrc",
           f"{ROOT}/transformer_attention_05_amd/csrc/pool.cpp", f"{ROOT}/tests/sanitize/pool_threads.cpp", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "tsan" in (r.stderr + r.stdout).lower():
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:exitcode=66")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    if run.returncode != 0 and "unexpected memory mapping" in run.stderr:
        pytest.skip("ThreadSanitizer cannot map its shadow memory here")
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-3000:]
    assert "WARNING: ThreadSanitizer" not in run.stderr
    assert "pool threads: ok" in run.stdout
