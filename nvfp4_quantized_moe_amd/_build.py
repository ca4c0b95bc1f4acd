"""Build libnvfp4moe.so for gfx950 with hipcc (in-tree, no JIT cache)."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libnvfp4moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


PROBE_LIB = os.path.join(PKG, "libnvfp4probe.so")


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def probe_sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "probe", "*.hip")))


def _compile(srcs, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        msg = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
        if msg.strip():
            print(msg)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source of the layer into one shared library next to
    this file, and the benchmark's roofline probes into a second one."""
    _compile(sources(), LIB, verbose)
    _compile(probe_sources(), PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
