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


def build_host_sanitize(out_dir: str, gdn_oracle: str = None) -> str:
    """Compile tests/c/host_sanitize.cpp with the sanitizers; returns the
    executable's path.  ``gdn_oracle`` replaces oracle/gdn_oracle.c (a copy
    with a planted mistake)."""
    objs = []
    for src in (gdn_oracle or os.path.join(ROOT, "oracle/gdn_oracle.c"),
                os.path.join(ROOT, "oracle/conv_oracle.c")):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        subprocess.run(["gcc", "-std=c99", "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
                        "-c", src, "-o", obj] + SAN, check=True)
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
    r = subprocess.run([exe], capture_output=True, text=True, env=sanitizer_env(), timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "HOST_SANITIZE ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc/g++")
def test_a_planted_unclamped_rewind_is_caught(tmp_path):
    """The same driver over a copy of the oracle whose rewind index is not
    clamped (slot index acc - 1 at num_accepted = 0, the #46090 bug): its
    first spec case has acc = 0 in sequence 0, so the oracle reads the slot
    list one entry before its start, and the run must abort with an
    AddressSanitizer report.  This shows the clean run above would catch
    that bug."""
    src = open(os.path.join(ROOT, "oracle/gdn_oracle.c")).read()
    clamp = "acc - 1 > 0 ? acc - 1 : 0"
    assert src.count(clamp) == 2, "the oracle's two rewind clamps moved"
    planted = os.path.join(str(tmp_path), "gdn_oracle.c")
    open(planted, "w").write(src.replace(clamp, "acc - 1"))
    exe = build_host_sanitize(str(tmp_path), gdn_oracle=planted)
    r = subprocess.run([exe], capture_output=True, text=True, env=sanitizer_env(), timeout=300)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr and "buffer-overflow" in r.stderr, r.stderr[-4000:]


def sanitizer_env():
    # verify_asan_link_order=0: the run may start with another library
    # preloaded ahead of the ASan runtime; the preload is left as it is.
    return dict(os.environ,
                ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1:"
                             "verify_asan_link_order=0",
                UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
