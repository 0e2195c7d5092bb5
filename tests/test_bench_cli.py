"""bench.py's command line on the CPU: it measures one GPU only, so any other GPU count (or a
launcher's world size above one) ends it with status 2 and a message, before any GPU work."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in (r.stdout + r.stderr)


def test_a_launcher_world_above_one_is_refused():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU only" in (r.stdout + r.stderr)
