"""bench.py's command-line contract on the host: more than one GPU is refused with a
message and a non-zero status before any device work; --help lists the flags."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_help_lists_the_contract_flags():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout
