"""libecf's host C++ (the shared LRU cache and its resize, the q* split, the host
expert FFN on its thread pool, the C entry points around them) built with g++
under AddressSanitizer + UndefinedBehaviorSanitizer and, separately,
ThreadSanitizer, running the checks in tests/sanitize/host_checks.cpp.  CPU only:
the GPU kernel launchers are stubbed out and never called."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("make") is None, reason="needs g++ and make")
@pytest.mark.parametrize("target", ["asan", "tsan"])
def test_host_code_under_sanitizers(target, tmp_path):
    env = dict(os.environ, OUT=str(tmp_path))
    p = subprocess.run(["make", "-C", os.path.join(HERE, "sanitize"), target], env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=900)
    assert p.returncode == 0, p.stdout[-4000:]
    assert "host checks passed" in p.stdout
    for bad in ("ERROR: AddressSanitizer", "ERROR: LeakSanitizer", "runtime error:", "WARNING: ThreadSanitizer"):
        assert bad not in p.stdout, p.stdout[-4000:]
