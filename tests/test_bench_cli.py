"""bench.py's command line without a GPU: the one-GPU rule and the help text."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_probe_modes():
    r = _bench("--help")
    assert r.returncode == 0
    for flag in ("--copy-probe", "--vendor-pair", "--workload", "--only-headline"):
        assert flag in r.stdout
