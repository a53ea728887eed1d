"""Build libmoegmm.so in-tree with hipcc for gfx950.

    python -m grouped_gemm_moe_amd.build          # or build() from Python

Every source is compiled to an object under ``_build/`` (in parallel), then
linked into ``grouped_gemm_moe_amd/libmoegmm.so``.  The library is replaced
atomically, so a process that already loaded the old one is not disturbed.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoegmm.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["api.cpp", "permute.hip", "gmm.hip", "gmm_stream.hip", "gmm_mx.hip", "mx_quant.hip",
           "elementwise.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libmoegmm")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source and link libmoegmm.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = COMMON_FLAGS + list(extra_flags or [])
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([hipcc] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(cmds), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Host-side checking build: the C ABI layer (api.cpp: argument validation,
# workspace sizing, dispatch) compiled by g++ with AddressSanitizer and
# UndefinedBehaviorSanitizer, linked with the release objects of the kernels
# (their host launchers and device code unchanged).  Only CPU tests load it,
# through MOEGMM_LIB, with the sanitizer runtime preloaded; see
# host_check_env().
HOST_CHECK_DIR = os.path.join(BUILD_DIR, "hostcheck")
HOST_CHECK_LIB = os.path.join(HOST_CHECK_DIR, "libmoegmm_hostcheck.so")
HOST_CHECK_FLAGS = ["-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def build_host_check(verbose: bool = False) -> str:
    """Build the sanitizer-instrumented host library (after build())."""
    gxx = shutil.which("g++")
    if gxx is None:
        raise RuntimeError("g++ not found; the host-check build needs it")
    os.makedirs(HOST_CHECK_DIR, exist_ok=True)
    api_obj = os.path.join(HOST_CHECK_DIR, "api.o")
    _run([gxx] + HOST_CHECK_FLAGS + ["-D__HIP_PLATFORM_AMD__", f"-I{_rocm()}/include", f"-I{INCLUDE}",
                                     f"-I{CSRC}", "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj],
         verbose)
    kernels = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "api.cpp"]
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        raise RuntimeError(f"build() first: {missing} missing")
    tmp = HOST_CHECK_LIB + f".tmp{os.getpid()}"
    _run([gxx, "-shared", "-fsanitize=address,undefined", "-o", tmp, api_obj] + kernels +
         [f"-L{_rocm()}/lib", "-lamdhip64", f"-Wl,-rpath,{_rocm()}/lib"], verbose)
    os.replace(tmp, HOST_CHECK_LIB)
    return HOST_CHECK_LIB


def host_check_env(base=None) -> dict:
    """Environment for a child process that loads the host-check library:
    MOEGMM_LIB points at it and g++'s AddressSanitizer runtime is preloaded
    ahead of whatever the parent preloads (it must come first).  Leak
    detection is off (the interpreter itself is not instrumented); any
    sanitizer report aborts the child."""
    env = dict(os.environ if base is None else base)
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], stdout=subprocess.PIPE,
                          text=True).stdout.strip()
    env["MOEGMM_LIB"] = HOST_CHECK_LIB
    env["LD_PRELOAD"] = ":".join(p for p in (asan, env.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
