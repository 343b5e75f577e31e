"""bench.py's command line on the host: a run on more than one GPU is refused with a message and
exit status 2, before anything touches a device, and prints no result line."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""
