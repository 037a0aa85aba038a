"""Build libdora.so (HIP, gfx950) in-tree with hipcc.

    python -m parameter_efficient_fine_dora_amd.build

Each source is compiled to an object in _build/ (in parallel), then linked
into parameter_efficient_fine_dora_amd/libdora.so next to the Python binding.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdora.so")
SOURCES = ["api.hip", "gemm.hip", "gram.hip", "rowwise.hip", "small.hip", "probe.hip", "noalloc.hip"]
HEADERS = ["common.h", "kernels.h", "entry.h"]
ARCH = "gfx950"


def hipcc() -> str:
    env = os.environ.get("HIPCC")
    if env:
        return env
    found = shutil.which("hipcc")
    return found or "/opt/rocm/bin/hipcc"


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        # packed-FP32 VALU forms are kept out of the generated code on purpose
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
    ]


def _run(cmd: list[str]) -> tuple[int, str]:
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    return p.returncode, out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 2) // 2))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if verbose or rc:
            print(" ".join(cmd), file=sys.stderr)
            if out.strip():
                print(out, file=sys.stderr)
        if rc:
            raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-3]}")
    tmp = LIB + ".tmp"
    rc, out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc:
        print(out, file=sys.stderr)
        raise RuntimeError("link of libdora.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
