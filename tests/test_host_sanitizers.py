"""The CPU oracle and the library's host-side checks under AddressSanitizer
and UndefinedBehaviorSanitizer (CPU only).

tests/c/host_sanitize.cpp runs every oracle entry over the edge cases of the
caller-supplied metadata (acceptance 0 .. T, empty sequences, padding,
gathers, chunk ends, rejected indices) and every host validator and argument
check over valid and invalid metadata.  It is compiled here with gcc/g++ and
-fsanitize=address,undefined -fno-sanitize-recover=all, from the oracle's C
sources and the library's host sources (no device code), so that an
out-of-bounds access or an undefined operation aborts the run.  The vLLM PR
#46090 report's one memory bug on this path (评论区精华: acc - 1 underflowing
into an out-of-bounds read at num_accepted = 0) is of exactly this kind.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def build_host_sanitize(out_dir: str) -> str:
    """Compile tests/c/host_sanitize.cpp with the sanitizers; returns the
    executable's path."""
    objs = []
    for src in ("oracle/gdn_oracle.c", "oracle/conv_oracle.c"):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        subprocess.run(["gcc", "-std=c99", "-ffp-contract=off", "-c", os.path.join(ROOT, src),
                        "-o", obj] + SAN, check=True)
        objs.append(obj)
    for src in ("speculative_decode_amd/csrc/gdn_host.cpp",
                "speculative_decode_amd/csrc/conv_host.cpp", "tests/c/host_sanitize.cpp"):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        subprocess.run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-c", os.path.join(ROOT, src), "-o", obj] + SAN, check=True)
        objs.append(obj)
    exe = os.path.join(out_dir, "host_sanitize")
    subprocess.run(["g++", "-o", exe] + objs + SAN + ["-lm"], check=True)
    return exe


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc/g++")
def test_oracle_and_host_checks_are_clean_under_asan_ubsan(tmp_path):
    exe = build_host_sanitize(str(tmp_path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "HOST_SANITIZE ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
