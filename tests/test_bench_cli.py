"""Host-side checks of bench.py's command line (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_help_lists_every_mode():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--sweep-small-t", "--prefill", "--backward", "--replay", "--policy", "--traffic-from"):
        assert flag in r.stdout


def test_more_than_one_gpu_is_refused_in_every_mode():
    for mode in (("--prefill",), ("--sweep-small-t",), ("--replay",), ("--backward",)):
        r = _run("--gpus", "4", *mode)
        assert r.returncode == 2, mode
        assert json.loads(r.stdout.strip().splitlines()[-1])["n_gpus"] == 4
