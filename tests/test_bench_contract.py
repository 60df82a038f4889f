"""bench.py on the host (no GPU): it measures one GPU only, so a request for
several GPUs, or a launch as one rank of several, ends at once with exit code 2
and a message saying so, before anything touches a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                          text=True, timeout=120, env=env)


def test_several_gpus_refused():
    r = _run(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_rank_of_a_multi_process_launch_refused():
    r = _run(["--steps", "1", "--warmup", "0"], {"WORLD_SIZE": "4", "RANK": "1"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
