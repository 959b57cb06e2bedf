"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

The library's sources are compiled as for libkla.so, with the sanitizers switched on for the
host side only (each -fsanitize= right after -Xarch_host; device code is unchanged), and linked
with tests/sanitize/kla_abi_sanitize.c (C, as the ABI's callers are: an enum argument may carry
any int) into one executable.  That driver calls every entry
point of include/kla.h with arguments its validation rejects (or that leave nothing to do) and
runs the workspace queries, including shapes near the 32-bit limits; by the header's contract
none of this reaches a HIP call.  A wrong status, an out-of-bounds access, an overflow or any
other sanitizer report fails the test.  The executable is cached under
gated_delta_rule_kla_amd/_build/asan/, keyed by the sources' hash, so only the first run after a
change pays for the build (about a minute and a half on eight cores)."""

import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from gated_delta_rule_kla_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "sanitize", "kla_abi_sanitize.c")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
       "-Xarch_host", "-g"]


def _hipcc():
    try:
        return libbuild._hipcc()
    except RuntimeError:
        return None


def _sources():
    return [os.path.join(libbuild.CSRC, s) for s in libbuild.SOURCES]


def _clang(hipcc):
    # the C compiler of the same ROCm toolchain (its sanitizer runtimes are the ones hipcc links)
    for cand in (os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin", "clang"),
                 "/opt/rocm/lib/llvm/bin/clang"):
        if os.path.exists(cand):
            return os.path.realpath(cand)
    return None


def _key(flags):
    h = hashlib.sha256(" ".join(flags).encode())
    for p in _sources() + [DRIVER, os.path.join(ROOT, "include", "kla.h")] + [
            os.path.join(libbuild.CSRC, f) for f in sorted(os.listdir(libbuild.CSRC)) if f.endswith(".h")]:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _build(hipcc):
    flags = libbuild._flags() + SAN
    out = os.path.join(libbuild.BUILD, "asan", _key(flags))
    exe = os.path.join(out, "kla_abi_sanitize")
    if os.path.exists(exe):
        return exe
    # builds for older sources are of no further use
    root = os.path.join(libbuild.BUILD, "asan")
    if os.path.isdir(root):
        for d in os.listdir(root):
            shutil.rmtree(os.path.join(root, d), ignore_errors=True)
    os.makedirs(out, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(out, os.path.splitext(os.path.basename(src))[0] + ".o")
        r = subprocess.run([hipcc, *flags, "-x", "hip", "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, f"sanitized compile of {src} failed:\n{r.stdout}{r.stderr}"
        return obj

    def compile_driver(src):
        obj = os.path.join(out, "kla_abi_sanitize_driver.o")
        cmd = [_clang(hipcc), "-x", "c", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"compile of {src} failed:\n{r.stdout}{r.stderr}"
        return obj

    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        jobs = [ex.submit(compile_one, s) for s in _sources()] + [ex.submit(compile_driver, DRIVER)]
        objs = [j.result() for j in jobs]
    r = subprocess.run([hipcc, f"--offload-arch={libbuild.ARCH}", *SAN, *objs, "-o", exe + ".tmp"],
                       capture_output=True, text=True)
    assert r.returncode == 0, f"sanitized link failed:\n{r.stdout}{r.stderr}"
    os.replace(exe + ".tmp", exe)
    return exe


@pytest.mark.timeout(900)
def test_abi_host_code_under_asan_and_ubsan():
    hipcc = _hipcc()
    if hipcc is None or _clang(hipcc) is None:
        pytest.skip("hipcc or its clang not available")
    exe = _build(hipcc)
    env = dict(os.environ)
    # the HIP runtime keeps allocations until exit by design: leak checking is off
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    log = r.stdout + r.stderr
    assert "AddressSanitizer" not in log and "runtime error" not in log, log
    assert r.returncode == 0, log
    assert "ok: 0 failure(s)" in r.stdout, log
