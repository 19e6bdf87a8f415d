"""bench.py's argument checks, which run before anything touches a GPU: a
request for more than one GPU, and configuration names it does not know."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    e = dict(os.environ)
    e.pop("WORLD_SIZE", None)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=e,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
    r = _run(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "WORLD_SIZE 4" in r.stderr


def test_unknown_configuration_is_refused():
    r = _run("--all-configs", "--configs", "svgB,fgattn_M65")
    assert r.returncode == 2 and "fgattn_M65" in r.stderr and r.stdout == ""
    r = _run("--configs", "svgB")  # needs --all-configs
    assert r.returncode == 2 and "--all-configs" in r.stderr
