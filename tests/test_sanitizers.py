"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only):
the C oracle running every pin, and the library's host side (argument
validation of every entry point, the verify-budget scheduler) running the
host tests.  Sanitizers instrument host code only: the HIP translation units
are compiled with the sanitizer flags behind -Xarch_host, so no GPU code is
built with them, and nothing here launches a kernel."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_verification_attn_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for v in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def _env(preload):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    env["PYTHONPATH"] = os.pathsep.join([ROOT, os.path.join(ROOT, "tests")])
    return env


def _build_oracle(src, out):
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", src, "-o", out, "-lm"])


PINS_SCRIPT = """
import sys
import oracle, pins
with oracle.use_library(sys.argv[1]):
    for check in pins.ALL_CHECKS:
        check()
print("all pins passed")
"""

needs_gcc_san = pytest.mark.skipif(_gcc_runtime("libasan.so") is None or _gcc_runtime("libubsan.so") is None,
                                   reason="gcc sanitizer runtimes not installed")


@needs_gcc_san
def test_oracle_pins_under_asan_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    _build_oracle(os.path.join(ROOT, "oracle", "oracle.c"), so)
    env = _env(_gcc_runtime("libasan.so") + ":" + _gcc_runtime("libubsan.so"))
    r = subprocess.run([sys.executable, "-c", PINS_SCRIPT, so], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0 and "all pins passed" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]


@needs_gcc_san
def test_oracle_sanitizer_is_live(tmp_path):
    """A copy of the oracle with a planted one-element heap overflow (the score
    buffer one short) must be stopped by AddressSanitizer, so the run above is
    really instrumented."""
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    old = "double *s = (double *)malloc(sizeof(double) * (size_t)nk);\n    if (!mask || !s)"
    assert src.count(old) == 1
    c = tmp_path / "oracle_overflow.c"
    c.write_text(src.replace(old, "double *s = (double *)malloc(sizeof(double) * (size_t)(nk - 1));\n"
                                  "    if (!mask || !s)"))
    so = str(tmp_path / "liboracle_overflow.so")
    _build_oracle(str(c), so)
    env = _env(_gcc_runtime("libasan.so") + ":" + _gcc_runtime("libubsan.so"))
    r = subprocess.run([sys.executable, "-c", PINS_SCRIPT, so], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]


HOST_TESTS_SCRIPT = """
import sys
from speculative_decoding_verification_attn_amd import ops
ops.LIB_PATH = sys.argv[1]
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu", "-k", "not catch_planted",
                      "tests/test_capi.py", "tests/test_budget.py"]))
"""


@pytest.mark.skipif(_clang_asan_runtime() is None or not os.path.exists(HIPCC), reason="no hipcc / clang asan")
def test_library_host_code_under_asan_ubsan(tmp_path):
    """The library with its host translation units (C ABI validation, the
    verify-budget scheduler) built with ASan + UBSan on the host side only,
    linked with the regular kernel objects, runs the host tests."""
    from speculative_decoding_verification_attn_amd import build as B
    objs = {s: os.path.join(B.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES}
    if not all(os.path.exists(o) for o in objs.values()):
        B.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    host_tus = ["capi.hip", "verify_budget.hip"]
    for s in host_tus:
        out = str(tmp_path / (os.path.splitext(s)[0] + "_san.o"))
        subprocess.check_call([B.HIPCC, *[f for f in B.CFLAGS if f != "-O3"], "-O1", "-g", *san, "-c",
                               os.path.join(CSRC, s), "-o", out])
        objs[s] = out
    so = str(tmp_path / "libspecverify_san.so")
    subprocess.check_call([B.HIPCC, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *objs.values(), "-o", so,
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                           "-shared-libsan"])
    needed = subprocess.run(["readelf", "-d", so], capture_output=True, text=True).stdout
    assert "libclang_rt.asan" in needed  # the host code really is instrumented
    env = _env(_clang_asan_runtime())
    r = subprocess.run([sys.executable, "-c", HOST_TESTS_SCRIPT, so], env=env, capture_output=True, text=True,
                       cwd=ROOT, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
