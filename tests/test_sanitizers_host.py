"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, each in a
child process with its sanitizer runtime preloaded (any finding aborts it):

- the oracle's C source built with gcc -fsanitize=address,undefined, running
  the oracle pins (decode and prefill);
- libpa's host code (argument checks, sizing, launch decisions in pa_api)
  built with hipcc -Xarch_host -fsanitize=address / undefined, running the
  C-ABI tests.  Device code is built as usual and not run here.
"""
import os
import subprocess
import sys

import oracle
from paged_kv_cache_401_amd import build as pa_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_OPTIONS = "detect_leaks=0:halt_on_error=1:abort_on_error=1"


def _child(env_extra, args):
    env = dict(os.environ, ASAN_OPTIONS=ASAN_OPTIONS, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"] + args,
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=900)
    tail = "\n".join(r.stdout.splitlines()[-30:])
    assert r.returncode == 0, tail
    assert "passed" in tail, tail


def _gcc_runtime(name):
    return subprocess.check_output(["gcc", "-print-file-name=" + name], text=True).strip()


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    _child({"PA_ORACLE_LIB": lib,
            "LD_PRELOAD": "%s %s" % (_gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so"))},
           ["tests/test_oracle_pins.py", "tests/test_oracle_prefill_pins.py"])


def _clang_asan_runtime():
    out = subprocess.check_output([pa_build.hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                                  text=True).strip()
    if not os.path.isabs(out):
        out = subprocess.check_output([os.path.join(os.path.dirname(pa_build.hipcc()), "..", "llvm",
                                                    "bin", "clang"),
                                       "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        root = "/opt/rocm/llvm/lib/clang"
        for ver in sorted(os.listdir(root)):
            cand = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
            if os.path.exists(cand):
                out = cand
    return out


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    if not all(os.path.exists(os.path.join(pa_build.BUILD_DIR, s.replace(".hip", ".o")))
               for s in pa_build.SOURCES):
        pa_build.build()
    lib = pa_build.build_host_sanitized(str(tmp_path / "libpa_san.so"))
    _child({"PA_LIBPA": lib, "LD_PRELOAD": _clang_asan_runtime()}, ["tests/test_abi.py"])
