"""CPU checks of the benchmark's command-line contract: it runs on exactly
one GPU and says so (one JSON line, exit status 2) before touching a device."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["requested_gpus"] == 2


def test_a_multi_rank_launch_is_refused():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "error" in json.loads(r.stdout.strip().splitlines()[-1])
