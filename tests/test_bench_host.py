"""bench.py's command line, on the host: it runs on exactly one GPU and says so for any other
count before touching a device, and its help lists the step variants it can time."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    for n in ("2", "8"):
        r = _run("--gpus", n)
        assert r.returncode == 2
        assert "exactly one GPU" in r.stderr
        assert r.stdout == ""


def test_help_lists_the_step_variants():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--eager", "--entry", "--exit", "--tbo", "--seg-stride", "--eplb", "--workload"):
        assert opt in r.stdout, opt
