"""The library's host threads under ThreadSanitizer, on the CPU.

The DMA copy engine's packing pool (csrc/worker_pool.h) and the layer
pipeline's copy worker (csrc/copy_queue.h) are plain C++ headers, the same
ones liboasis.so is built from.  tests/tsan_host_threads.cpp drives both from
several threads; here it is built with g++ -fsanitize=thread and run.  A data
race, a lock-order inversion or a failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefetch_block_scoring_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "tsan_host_threads.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_host_threads_are_race_free(tmp_path):
    exe = str(tmp_path / "tsan_host_threads")
    build = ["g++", "-std=c++17", "-O1", "-g", "-pthread", "-fsanitize=thread", "-I", CSRC, SRC, "-o", exe]
    subprocess.run(build, check=True)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 second_deadlock_stack=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    assert "all checks passed" in r.stdout
