"""The C ABI's fork/join on its side stream, on the host: csrc/api.hip is built
with g++ against a stand-in HIP runtime (tests/hostmock) whose kernel launchers
can be made to fail one by one.  Whatever launch fails, the call must leave the
caller's stream ordered after all side-stream work and no fork open; on the
normal path every kernel is ordered after the kernels whose outputs it reads."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MOCK = os.path.join(ROOT, "tests", "hostmock")
CSRC = os.path.join(ROOT, "parameter_efficient_fine_dora_amd", "csrc")

# every launch label of the forward and the detached backward
LABELS = ["", "down_proj_xs", "gram_AAt", "gram_finalize", "cross_gram_proj",
          "fused_fwd_gemm", "compose_bwd", "dm_finalize", "dB_gemm", "bg_scale", "t_proj",
          "dx_gemm", "dA_gemm"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    out = tmp_path_factory.mktemp("forkjoin") / "fork_join"
    cmd = [gxx, "-std=c++17", "-O0", "-g", "-I", MOCK, "-I", CSRC, "-x", "c++",
           os.path.join(CSRC, "api.hip"), "-x", "c++", os.path.join(MOCK, "mock_runtime.cpp"),
           os.path.join(MOCK, "fork_join_main.cpp"), "-o", str(out), "-lpthread"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return str(out)


@pytest.mark.parametrize("label", LABELS, ids=[l or "none" for l in LABELS])
def test_side_stream_joined_on_every_exit(driver, label):
    env = dict(os.environ, DORA_MOCK_FAIL=label)
    res = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    lines = res.stdout.strip().splitlines()
    assert len(lines) == 2 and all(l.endswith(" ok") for l in lines), lines
    rcs = [int(l.split("rc=")[1].split()[0]) for l in lines]
    if not label:
        assert rcs == [0, 0]
    else:
        assert -6 in rcs, f"the failing launch {label} is reported as DORA_ERR_HIP: {lines}"
