"""Build libpa.so (HIP, gfx950) in-tree with hipcc.

Every HIP translation unit is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns
that it does not know the feature, which is harmless.  Matrix-core
accumulators are kept in ordinary VGPRs (``-mllvm -amdgpu-mfma-vgpr-form``).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpa.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["pa_api.hip", "pa_cache.hip", "pa_check.hip", "pa_decode.hip", "pa_decode_mfma.hip", "pa_prefill.hip",
           "pa_probe.hip"]
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def common_flags():
    # -amdgpu-mfma-vgpr-form: matrix-core accumulators live in ordinary VGPRs
    # (gfx950 MFMAs take either register file); without it the prefill loop
    # copied its accumulators between the two files every iteration
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines()
                    if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), out))
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source and link libpa.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj])
    jobs = min(len(cmds), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """libpa.so with its host code (argument checks, sizing, dispatch: pa_api)
    built with AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
    regular objects of the other sources (run build() first).  The sanitizer
    flags apply to the host pass only (-Xarch_host); device code is unchanged.
    Load it by setting PA_LIBPA, with clang's ASan runtime preloaded."""
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES if s != "pa_api.hip"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError("build() first: missing %s" % missing)
    san = os.path.join(os.path.dirname(out), "pa_api_san.o")
    flags = common_flags() + ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                              "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                              "-Xarch_host", "-fno-omit-frame-pointer"]
    _run([hipcc()] + flags + ["-c", os.path.join(CSRC, "pa_api.hip"), "-o", san], verbose)
    _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out, san] + objs, verbose)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
