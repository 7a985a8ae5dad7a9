"""bench.py's command-line contract on the host: more than one GPU is refused with a message
and exit status 2 (this layer runs on one GPU), and --help lists the sweep options."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_modes():
    r = run("--help")
    assert r.returncode == 0
    for opt in ("--sweep", "--sweep-block-m", "--routing", "--graph", "--dense-reference",
                "--copy-calibration", "--cpu-baseline"):
        assert opt in r.stdout
