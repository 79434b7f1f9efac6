"""The CPU suite under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds, into a temporary directory, the oracle and the C-ABI library with
the sanitizers on their host code (the library's device code is built as
usual; nothing here runs a kernel), then runs every other CPU test against
those builds in a child process with clang's ASan runtime preloaded.  Any
sanitizer report aborts the child, so the test fails on the first one.
The oracle is built with clang here so that one sanitizer runtime serves
both libraries.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "mla_latent_kv_08_amd", "csrc")
SANITIZE = ["address", "undefined"]


def _host_sanitizer_flags():
    # every -fsanitize= on the hipcc line applies to the host compilation only
    flags = []
    for f in [f"-fsanitize={s}" for s in SANITIZE] + ["-fno-sanitize-recover=undefined",
                                                      "-fno-omit-frame-pointer"]:
        flags += ["-Xarch_host", f]
    return flags


@pytest.mark.skipif(not (os.path.exists(CLANG) and os.path.exists(HIPCC)), reason="ROCm clang/hipcc missing")
def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    oracle_so = str(tmp_path / "liboracle_san.so")
    lib_so = str(tmp_path / "libmla_san.so")
    subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fsanitize=" + ",".join(SANITIZE), "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-o", oracle_so,
                    os.path.join(ROOT, "oracle", "mla_oracle.c"), "-lm"], check=True)
    from mla_latent_kv_08_amd import build as libbuild
    sources = [os.path.join(CSRC, s) for s in libbuild.SOURCES]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *_host_sanitizer_flags(),
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, *sources, "-o", lib_so],
                   check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    runtime = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                             capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=runtime, MLA_LIB=lib_so, ORACLE_LIB=oracle_so,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-s",
                        "-m", "not gpu", "-p", "no:cacheprovider", "--deselect",
                        "tests/test_sanitizers.py::test_cpu_suite_under_asan_and_ubsan"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stdout + r.stderr and "AddressSanitizer" not in r.stdout + r.stderr, tail
    assert " passed" in r.stdout, tail
