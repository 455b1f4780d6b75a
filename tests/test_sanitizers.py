"""The CPU suite under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host code (argument checks, table checks, the work-list
planner, the heuristics: pointer arithmetic over caller arrays) is built with
hipcc with the sanitizers on its host pass only (-Xarch_host; the device code
is unchanged), the oracle with clang and the same sanitizers, and every
`-m "not gpu"` test then runs in a child process against those builds with
the sanitizer runtime preloaded.  Any sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _hipcc():
    from mla_latent_kv_13_amd import build
    return build.hipcc()


@pytest.fixture(scope="module")
def sanitized_libs(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang not found")
    d = tmp_path_factory.mktemp("sanitized")
    from mla_latent_kv_13_amd import build
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libsan"]
    lib = str(d / "libmla_decode_san.so")
    flags = [f for f in build.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    subprocess.run([_hipcc(), *flags, *san, "-I", build.INCLUDE, *build.SOURCES, "-o", lib], check=True,
                   capture_output=True)
    orc = str(d / "liboracle_san.so")
    subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                    "-ffp-contract=off", "-fsanitize=address,undefined", "-shared-libsan", "-fno-omit-frame-pointer",
                    os.path.join(REPO, "oracle", "oracle.c"), "-o", orc, "-lm"], check=True, capture_output=True)
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], check=True, capture_output=True,
                        text=True).stdout.strip()
    return lib, orc, rt


def test_cpu_suite_under_asan_and_ubsan(sanitized_libs):
    lib, orc, rt = sanitized_libs
    env = dict(os.environ)
    env.update(MLA_TEST_LIB=lib, ORACLE_TEST_LIB=orc, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "tests", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                          "--ignore", os.path.join("tests", "test_sanitizers.py")],
                         cwd=REPO, env=env, capture_output=True, text=True, timeout=1200)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert res.returncode == 0, out[-6000:]
    assert " passed" in out and " failed" not in out, out[-3000:]
