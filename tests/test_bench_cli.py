"""bench.py's contract on a machine without a GPU: one GPU only, a clear exit
without a device, and the profile-backed traffic figure only while the kernel
sources match the profile."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_no_device_is_an_error():
    env_run = subprocess.run([sys.executable, "-c",
                              "import sys, torch; sys.exit(0 if torch.cuda.is_available() else 3)"],
                             timeout=300)
    if env_run.returncode == 0:
        return  # a GPU is present: nothing to check here
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 1 and "HIP device" in r.stderr


def test_traffic_comes_from_a_matching_profile():
    sys.path.insert(0, ROOT)
    import bench

    with open(bench.TRAFFIC_PROFILE) as f:
        text = f.read()
    assert "source_sha256:" in text
    recorded = text.split("source_sha256:")[1].split()[0]
    t = bench.traffic_from_profile()
    if recorded == bench.kernel_source_hash():
        assert isinstance(t, int) and t > 60_000_000  # at least the algorithmic bytes
    else:
        assert t is None


def test_help_lists_the_modes():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--all-configs", "--collectives", "--activation-quant", "--stream-sweep",
                 "--tile-sweep", "--skip-warm", "--steps"):
        assert flag in r.stdout
