"""Host-side behaviour of bench.py that needs no GPU: it measures one GPU and
refuses a multi-GPU run with a message, before touching any device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, env=env, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    res = _run("--gpus", "2")
    assert res.returncode == 2
    assert "one GPU" in res.stderr and "shards" in res.stderr
    assert res.stdout == ""


def test_launched_as_one_of_several_ranks_exits_too():
    res = _run(env_extra={"WORLD_SIZE": "8"})
    assert res.returncode == 2
    assert "one GPU" in res.stderr
