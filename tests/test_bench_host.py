"""bench.py's command-line contract on the host (no GPU): a request for more
than one GPU, by flag or by a launcher's WORLD_SIZE, exits with status 2 and
says why, before anything touches a device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=60)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None),
                                      (["--gpus", "8", "--steps", "1"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = _run(args, env)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_contract_flags():
    r = _run(["--help"])
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout
