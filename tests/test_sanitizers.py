"""Host sanitizers: the C-ABI validation layer and the oracle under AddressSanitizer + UndefinedBehaviorSanitizer.

Builds (CPU only, into a temporary directory):
  * libdiffattn.so with diffattn_api.cpp's host code instrumented (hipcc, each -fsanitize= after -Xarch_host, so
    the gfx950 device code is built as usual) and linked with the ordinary kernel objects;
  * the oracle with clang, instrumented.
Then the host ABI tests and the oracle's own tests (its pins, mutants excluded) run against these builds in a
Python process with the sanitizer runtime preloaded, halting on the first report.  Two canaries first show that
the runtime catches a heap overflow and a signed overflow in this set-up at all.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)
from differential_attention_fwd_amd import build as dbuild  # noqa: E402

CLANG = "/opt/rocm/llvm/bin/clang"
LLVM_LIB = "/opt/rocm/llvm/lib"
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
C_SAN = ["-fsanitize=address,undefined"]
DEBUG = ["-O1", "-g", "-fno-omit-frame-pointer"]
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def asan_runtime():
    if not os.path.exists(CLANG):
        return None
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


def san_env():
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    env["PYTHONPATH"] = os.pathsep.join([ROOT, HERE] + [p for p in [env.get("PYTHONPATH")] if p])
    return env


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)} failed ({r.returncode}):\n{r.stdout[-4000:]}{r.stderr[-4000:]}")
    return r


def kernel_objects():
    """The ordinary (uninstrumented) objects of the kernel sources, compiled if missing or stale."""
    objs = []
    headers = [os.path.join(dbuild.CSRC, h) for h in dbuild.HEADERS]
    for src in dbuild.SOURCES:
        if src == "diffattn_api.cpp":
            continue
        obj = os.path.join(dbuild.BUILD, os.path.splitext(src)[0] + ".o")
        deps = [os.path.join(dbuild.CSRC, src), *headers]
        if not os.path.exists(obj) or os.path.getmtime(obj) < max(os.path.getmtime(d) for d in deps):
            os.makedirs(dbuild.BUILD, exist_ok=True)
            dbuild._compile(src)
        objs.append(obj)
    return objs


@pytest.fixture(scope="module")
def san_libs(tmp_path_factory):
    if asan_runtime() is None or shutil.which(dbuild.HIPCC) is None and not os.path.exists(dbuild.HIPCC):
        pytest.skip("clang sanitizer runtime or hipcc not available")
    d = tmp_path_factory.mktemp("sanitized")
    flags = [f for f in dbuild.FLAGS if f != "-O3"]
    api_o = str(d / "diffattn_api.o")
    run([dbuild.HIPCC, *flags, *DEBUG, *HOST_SAN, "-c", os.path.join(dbuild.CSRC, "diffattn_api.cpp"), "-o", api_o])
    lib = str(d / "libdiffattn.so")
    run([dbuild.HIPCC, f"--offload-arch={dbuild.ARCH}", "-shared", "-fPIC", "-o", lib, api_o, *kernel_objects()])
    orc = str(d / "liboracle.so")
    run([CLANG, *DEBUG, "-std=c99", "-fPIC", "-shared", "-fopenmp", "-Wall", *C_SAN, "-DORACLE_MUTANT=0",
         os.path.join(ROOT, "oracle", "diffattn_oracle.c"), "-o", orc, "-lm", f"-Wl,-rpath,{LLVM_LIB}"])
    # The host code really is instrumented.
    syms = run(["nm", "-D", "--undefined-only", lib]).stdout
    assert "__asan_" in syms and "__ubsan_handle_" in syms
    return d, lib, orc


CANARY = r"""
#include <stdlib.h>
int heap_overflow(int i) { int* p = (int*)malloc(4 * sizeof(int)); p[i] = 1; int r = p[0]; free(p); return r; }
int add(int a, int b) { return a + b; }
"""


def test_canaries_are_caught(san_libs):
    d, _, _ = san_libs
    src = d / "canary.c"
    src.write_text(CANARY)
    lib = str(d / "libcanary.so")
    run([CLANG, *DEBUG, "-fPIC", "-shared", *C_SAN, str(src), "-o", lib])
    for call, want in [("heap_overflow(4)", "heap-buffer-overflow"), ("add(2147483647, 1)", "runtime error:"),
                       ("heap_overflow(3)", None)]:
        code = f"import ctypes; L = ctypes.CDLL({lib!r}); L.{call}; print('survived')"
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=san_env(), timeout=120)
        if want is None:
            assert r.returncode == 0 and "survived" in r.stdout, r.stderr[-2000:]
        else:
            assert r.returncode != 0 and want in r.stderr, (call, r.returncode, r.stderr[-2000:])


def run_sanitized(san_libs, *pytest_args):
    _, lib, orc = san_libs
    cmd = [sys.executable, os.path.join(HERE, "sanitized_run.py"), lib, orc, "--", "-x", "-q", *pytest_args]
    r = subprocess.run(cmd, capture_output=True, text=True, env=san_env(), cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and not any(s in out for s in REPORTS), out[-6000:]
    return out


def test_abi_host_under_sanitizers(san_libs):
    out = run_sanitized(san_libs, os.path.join(HERE, "test_abi_host.py"))
    assert " passed" in out


def test_oracle_under_sanitizers(san_libs):
    out = run_sanitized(san_libs, "-k", "not planted", os.path.join(HERE, "test_oracle_pins.py"),
                        os.path.join(HERE, "test_oracle_bwd.py"), os.path.join(HERE, "test_oracle_per_head.py"))
    assert " passed" in out
