"""The benchmark's contract on the CPU: it refuses more than one GPU before
touching one, and the recorded counter figures it reports (HBM traffic) and
the committed profile summaries describe the kernel source as it stands."""
import importlib.util
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_recorded_traffic_and_profiles_match_the_kernel_source():
    bench = _bench_module()
    digest = bench.kernel_digest()
    assert bench.TRAFFIC is not None and bench.TRAFFIC["kernel_sha256"] == digest, \
        "the recorded FETCH_SIZE/WRITE_SIZE figures were taken on another kernel build"
    assert bench.traffic_bytes() == bench.TRAFFIC["fetch_bytes"] + bench.TRAFFIC["write_bytes"]
    pdir = os.path.join(ROOT, "profiles")
    seen = 0
    for name in sorted(os.listdir(pdir)):
        text = open(os.path.join(pdir, name)).read()
        m = re.search(r"Kernel code sha256: `([0-9a-f]{64})`", text)
        if m:
            seen += 1
            assert m.group(1) == digest, f"{name} profiles another kernel build"
    assert seen >= 3

