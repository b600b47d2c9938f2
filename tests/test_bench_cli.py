"""bench.py's command line on the CPU: more than one GPU is refused before any
device work (the library has no collectives), and --help lists the options."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--config", "--rank", "--layout", "--kv-rings", "--merge",
                "--no-cpu-baseline", "--no-gemm-ref", "--gemm-ref-only", "--copy-probe"):
        assert opt in r.stdout
