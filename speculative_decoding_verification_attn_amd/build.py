"""Build libspecverify.so (HIP, gfx950) in-tree with hipcc.

Every HIP source under csrc/ is compiled for gfx950 only and linked into a
shared library next to this file.  Packed-fp32 VALU instructions are
disabled (see -packed-fp32-ops below): the compiler would otherwise emit
them from ordinary float code.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libspecverify.so")
TRACE_LIB = os.path.join(PKG, "libspecverify_trace.so")
SOURCES = ["capi.hip", "verify_attn.hip", "accept.hip", "kv_compact.hip", "verify_budget.hip", "stochastic.hip",
           "read_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMA accumulators in VGPRs: the AGPR form made the allocator copy every
          # accumulator between the two register files each round
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-Wall", "-Wno-unused-function"]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every HIP source for gfx950 and link libspecverify.so; returns its path."""
    extra = list(extra or [])
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    _link(objs, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build_trace(verbose: bool = False) -> str:
    """The diagnostic library libspecverify_trace.so: the attention kernel
    compiled with SV_PHASE_TRACE (phase timeline, see
    spec_verify_attn_phase_trace), the other sources as in the production
    build (which must exist: build() first)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    src = "verify_attn.hip"
    obj = os.path.join(BUILD_DIR, "verify_attn_trace.o")
    cmd = [HIPCC, *CFLAGS, "-DSV_PHASE_TRACE", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src} (trace):\n{r.stderr}")
    others = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != src]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build() first: missing {missing}")
    _link([obj] + others, TRACE_LIB)
    if verbose:
        print(f"built {TRACE_LIB}")
    return TRACE_LIB


if __name__ == "__main__":
    if sys.argv[1:] == ["--trace"]:
        build_trace(verbose=True)
    else:
        build(verbose=True, extra=sys.argv[1:])
