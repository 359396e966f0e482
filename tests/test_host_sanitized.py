"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the host library with g++ -fsanitize=address,undefined, with the
kernel launchers replaced by a launch-plan checker, then runs the host/ABI
tests (test_library_host.py) and the launch-extent checks
(extents_under_sanitizer.py) against it in a child process that preloads the
sanitizer runtimes. Any out-of-bounds access, use after free or undefined
behaviour in the host code aborts that process and fails this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    gcc = shutil.which("gcc")
    if gcc is None:
        return None
    path = subprocess.run([gcc, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_library_under_asan_and_ubsan(tmp_path):
    from skip_softmax_video_amd.build import build_host_check
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if shutil.which("g++") is None or asan is None or ubsan is None:
        pytest.skip("g++ with the ASan/UBSan runtimes is needed")
    lib = build_host_check(str(tmp_path / "libssa_hostcheck.so"))
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", SSA_LIBRARY=lib)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_library_host.py"),
           os.path.join(ROOT, "tests", "extents_under_sanitizer.py")]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in res.stdout and "skipped" not in res.stdout.splitlines()[-1], tail
