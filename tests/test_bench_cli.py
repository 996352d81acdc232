"""bench.py's command line, checked before any device work: an unknown
extra workload and more than one GPU are rejected with exit status 2."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True, timeout=120)


def test_unknown_extra_is_rejected():
    r = run("--extras", "llama3_70b_batch,nonsense")
    assert r.returncode == 2 and "nonsense" in r.stdout


def test_more_than_one_gpu_is_rejected():
    r = run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stdout
