"""The require-GPU switch (``tests/gpu_env.py``): without a usable GPU a GPU
test module is skipped, unless GPU use is required, and then it errors.  The
pegainfer pull request page #1002 gives the reason for such a switch: a
missing device would otherwise read as a suite that passed having run
nothing.  Run here, on a machine where the GPU tests cannot run."""
import os
import subprocess
import sys

import pytest

from tests.gpu_env import why_no_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_gpu_module(flag):
    env = dict(os.environ)
    env["PGQA_REQUIRE_GPU"] = flag
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "gpu",
                           "tests/test_gpu_edges.py"], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=300)


@pytest.mark.skipif(why_no_gpu() is None, reason="a GPU is usable here: the GPU tests run instead")
def test_require_gpu_turns_the_skip_into_an_error():
    off = run_gpu_module("0")
    assert off.returncode in (0, 5), off.stdout + off.stderr  # skipped (or nothing collected)
    assert "skipped" in off.stdout or "no tests ran" in off.stdout
    on = run_gpu_module("1")
    assert on.returncode not in (0, 5), on.stdout + on.stderr
    assert "GPU tests required" in on.stdout + on.stderr
