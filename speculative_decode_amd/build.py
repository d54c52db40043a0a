"""Build libgdn_spec.so (gfx950 only) in-tree with hipcc.

    python -m speculative_decode_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in
           ("gdn_kernels.hip", "conv_kernels.hip", "prefill_kernels.hip", "probe_kernels.hip",
            "gdn_host.cpp", "conv_host.cpp")]
LIB = os.path.join(HERE, "libgdn_spec.so")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


FLAGS = ["-O3", "-std=c++17", "-fPIC",
         # packed-FP32 VALU forms are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # fused multiply-adds only where the source writes fmaf: every
         # instantiation then rounds the same expression the same way
         "-ffp-contract=off",
         "-Wall", "-Wno-unused-command-line-argument"]
OBJDIR = os.path.join(HERE, "_build")


def compile_command(src: str, obj: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}"] + FLAGS + ["-c", src, "-o", obj]


def link_command(objs: list, out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out] + objs


def _run(cmd: list, verbose: bool):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature;
    # that is expected and not shown.
    msgs = [l for l in (res.stderr or "").splitlines()
            if l.strip() and "packed-fp32-ops" not in l and "target-feature" not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel, one hipcc per file) and link the
    shared library; always recompiles."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.basename(src) + ".o") for src in SOURCES]
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        list(ex.map(lambda so: _run(compile_command(*so), verbose), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    _run(link_command(objs, tmp), verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
