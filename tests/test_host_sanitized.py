"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every library source is compiled with the sanitizers on its host side only (each
flag behind -Xarch_host; device code is built as usual and never runs here), linked
into a separate libdflash, and the CPU-only C-ABI tests (argument validation, size
queries over extreme dims, symbol exports) run against it in a child process with
the sanitizer runtime preloaded: an out-of-bounds host access, a signed overflow in
a size computation or a misaligned host load aborts the run.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_diffusion_speculative_dflash_amd import build as pkg_build

pytestmark = pytest.mark.slow

SAN_DIR = os.path.join(pkg_build.ROOT, "_build", "host_sanitized")
SAN_LIB = os.path.join(SAN_DIR, "libdflash_host_sanitized.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _build():
    os.makedirs(SAN_DIR, exist_ok=True)
    base = [f for f in pkg_build.FLAGS if f != "-O3"] + ["-O1"]

    def one(src):
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [pkg_build.HIPCC, *base, *pkg_build.SOURCE_FLAGS.get(src, []), *HOST_SAN, "-c",
               os.path.join(pkg_build.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(one, pkg_build.LIB_SOURCES))
    # a shared library takes the sanitizer runtime from the preloaded one
    r = subprocess.run([pkg_build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", SAN_LIB, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]


def test_abi_host_code_is_clean_under_asan_and_ubsan():
    rt = _runtime()
    if rt is None or not os.path.exists(pkg_build.HIPCC):
        pytest.skip("no hipcc / clang sanitizer runtime in this environment")
    import torch
    if torch.cuda.is_available():
        pytest.skip("the fake-pointer validation tests run on CPU-only hosts")
    _build()
    env = dict(os.environ, DFLASH_LIBRARY=SAN_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    probe = ("import os; from block_diffusion_speculative_dflash_amd import binding as bd; bd.lib(); "
             "m = open('/proc/self/maps').read(); "
             "assert os.environ['DFLASH_LIBRARY'] in m and 'libclang_rt.asan' in m; print('sanitized build loaded')")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=pkg_build.ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and "sanitized build loaded" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_abi_cpu.py")],
                       env=env, cwd=pkg_build.ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
