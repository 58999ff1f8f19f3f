"""bench.py's command line on the CPU: several GPUs are refused with a
message before anything touches a device, and the help text lists the
optional paths."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_several_gpus_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_help_lists_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--workload", "--kv-fp8", "--paged", "--min-p", "--eta", "--overlap", "--walk-mode", "--cpu-seconds"):
        assert opt in r.stdout, opt
