"""CPU sanitizer runs: the oracle, and the host side of the HIP library (CPU only).

1. The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

spec_oracle.c is built with -fsanitize=address,undefined (no recovery) into a
temporary directory and the fast pins of tests/oracle_pins.py run against it
in a child Python process with the sanitizer runtime preloaded: an
out-of-bounds access, a use after free or an undefined operation (signed
overflow, a shift out of range, a misaligned load) anywhere those pins reach
stops the child with a report.  Two planted mistakes show that the harness
does catch such errors: a row scan one element past the end of its row, and a
signed overflow in the commit step's capacity check.

2. The HIP library rebuilt with its host code (not its device code) under the
same sanitizers (hipcc -Xarch_host -fsanitize=...), with the host ABI tests
(tests/test_abi_host.py: workspace sizing, argument validation, status
strings, the refusals that happen before any HIP call) run against it in a
child process with clang's sanitizer runtime preloaded.
"""
import os
import subprocess
import sys
import tempfile

import glob

import pytest

import oracle
from rejection_sampling_verify_scaled_amd import build as hip_build

HERE = os.path.dirname(os.path.abspath(__file__))
SAN_FLAGS = ("-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer")
FAST_PINS = ["pin_philox_kat", "pin_u01", "pin_softmax_vs_scipy", "pin_greedy_vs_numpy",
             "pin_faults", "pin_accept_near_tie_flag", "pin_bonus_race_near_tie_flag",
             "pin_residual_race_near_tie_flag", "pin_residual_empty_fallback",
             "pin_temperature_invariance", "pin_identical_draft_accepts", "pin_draft_greedy",
             "pin_draft_faults", "pin_draft_race_near_tie_flag", "pin_commit_example",
             "pin_commit_after_verify", "pin_tree_page_example", "pin_tree_faults",
             "pin_tree_chain_is_linear", "pin_tree_brute_force"]

CHILD = """
import sys
sys.path.insert(0, {tests!r})
import oracle, oracle_pins as P
lib = oracle.load({so!r})
for name in {pins!r}:
    getattr(P, name)(lib)
    print(name, "ok", flush=True)
"""


def asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def build_and_run(src_text, pins, tmp):
    rt = asan_runtime()
    if rt is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    c_path = os.path.join(tmp, "oracle_san.c")
    so_path = os.path.join(tmp, "oracle_san.so")
    with open(c_path, "w") as f:
        f.write(src_text)
    oracle.build(force=True, out=so_path, src=c_path, extra_flags=SAN_FLAGS)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", ORACLE_THREADS="4")
    code = CHILD.format(tests=HERE, so=so_path, pins=list(pins))
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          env=env, timeout=600)


def oracle_source():
    with open(oracle.SRC) as f:
        return f.read()


def test_pins_clean_under_sanitizers():
    with tempfile.TemporaryDirectory(prefix="oracle_san_") as tmp:
        r = build_and_run(oracle_source(), FAST_PINS, tmp)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.count(" ok") == len(FAST_PINS), r.stdout


@pytest.mark.parametrize("name,old,new,pin,report", [
    ("row scan past the end", "static double row_max(const void* base, int dtype, int64_t row, "
     "int32_t V) {\n  double m = -INFINITY;\n  for (int32_t v = 0; v < V; ++v) {",
     "static double row_max(const void* base, int dtype, int64_t row, int32_t V) {\n"
     "  double m = -INFINITY;\n  for (int32_t v = 0; v <= V; ++v) {",
     "pin_softmax_vs_scipy", "AddressSanitizer"),
    ("signed overflow", "if (L < 0 || (int64_t)L + n + 1 > capacity) {",
     "if (L < 0 || L + n + 1 + 2147483647 > capacity) {", "pin_commit_example",
     "runtime error"),
])
def test_planted_errors_are_reported(name, old, new, pin, report):
    src = oracle_source()
    assert src.count(old) == 1, name
    with tempfile.TemporaryDirectory(prefix="oracle_san_") as tmp:
        r = build_and_run(src.replace(old, new), [pin], tmp)
    assert r.returncode != 0, name
    assert report in r.stderr, r.stderr[-2000:]


def clang_asan_runtime():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    found = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    return found[-1] if found else None


def test_host_code_under_sanitizers():
    rt = clang_asan_runtime()
    if rt is None or not os.path.exists(hip_build.hipcc()):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is missing")
    with tempfile.TemporaryDirectory(prefix="hostasan_") as tmp:
        so = os.path.join(tmp, "libspecverify_hostasan.so")
        flags = []
        for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer"):
            flags += ["-Xarch_host", f]
        hip_build.build(out=so, extra=flags)
        syms = subprocess.run(["nm", "-D", "--undefined-only", so], capture_output=True,
                              text=True).stdout
        assert "__asan_" in syms and "__ubsan_" in syms  # the host code is instrumented
        env = dict(os.environ, LD_PRELOAD=rt, SPECVERIFY_HOST_TEST_LIB=so,
                   ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                            os.path.join(HERE, "test_abi_host.py")], capture_output=True,
                           text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
    assert " passed" in r.stdout and "failed" not in r.stdout
