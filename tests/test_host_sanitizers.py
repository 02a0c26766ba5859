"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A second build of the library compiles its host code with
-fsanitize=address,undefined (no recovery: the first report ends the run); the
ABI tests and the planner tests then run against it in a child process with
the sanitizer runtime preloaded.  Every host path they reach -- the argument
checks of each entry point, the host planner, the workspace sizing, the status
strings -- runs with out-of-bounds accesses, uses after free and undefined
operations reported.  None of these tests touches a GPU.
"""

import os
import subprocess
import sys

import pytest

from paged_mla_decode_04_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized():
    try:
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    return build.build_sanitized(), runtime


@pytest.mark.parametrize("tests", ["tests/test_abi.py", "tests/test_plan.py"])
def test_host_code_is_clean_under_sanitizers(sanitized, tests):
    lib, runtime = sanitized
    env = dict(os.environ)
    env.update(MLA_DECODE_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", tests, "-q", "-s", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=600)
    out = r.stdout.decode(errors="replace")
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and " failed" not in out, out[-2000:]


def test_a_planted_fault_is_reported(sanitized, tmp_path):
    """The preloaded runtime does catch faults in this setting: an
    out-of-range enum read, the mistake the status strings once had."""
    lib, runtime = sanitized
    prog = tmp_path / "probe.cpp"
    prog.write_text("enum e { A, B };\n"
                    "static int f(enum e v) { switch (v) { case A: return 1; case B: return 2; } return 0; }\n"
                    "extern \"C\" int planted(int x) { enum e v; __builtin_memcpy(&v, &x, sizeof v); return f(v); }\n")
    so = tmp_path / "libprobe.so"
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang++")
    san = "-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-sanitize-recover=undefined".split()
    r = subprocess.run([clang, "-x", "c++", "-shared", "-fPIC", "-O0", *san, str(prog), "-o", str(so)],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    assert r.returncode == 0, r.stdout.decode()
    code = ("import ctypes, sys\n"
            "lib = ctypes.CDLL(sys.argv[1])\n"
            "lib.planted.argtypes = [ctypes.c_int]\n"
            "print(lib.planted(99))\n")
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code, str(so)], env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=120)
    assert r.returncode != 0 and "runtime error:" in r.stdout.decode(errors="replace")
