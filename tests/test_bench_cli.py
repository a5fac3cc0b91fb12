"""bench.py's command-line contract on the CPU: more than one GPU is refused
with a message before anything touches a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "--gpus 2" in r.stderr and r.stdout == ""


def test_incompatible_modes_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--graph", "--ring-copy"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0 and "--ring-copy" in r.stderr
