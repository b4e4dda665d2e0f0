"""Build libhaste.so (the HIP kernels + the C ABI) for gfx950 with hipcc.

Every source is compiled on every call (the build check must really build).
Objects go to sparse_output_layer_amd/_build/, the library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhaste.so")
SOURCES = ["abi.hip", "tail.hip", "dxs.hip", "head.hip", "f32path.hip", "topk.hip", "probe.hip", "rewire.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> subprocess.Popen:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = [(s, _compile(s)) for s in SOURCES]
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if verbose and lines:
            print(f"--- {src}\n" + "\n".join(lines))
        if p.returncode != 0:
            failed.append((src, "\n".join(lines)))
    if failed:
        msg = "\n".join(f"== {s} ==\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    objs = [os.path.join(BUILD, s + ".o") for s in SOURCES]
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
