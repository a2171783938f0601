"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every HIP source is compiled with the sanitizers on the host side only (each
-fsanitize= follows -Xarch_host; the gfx950 device code is built as usual) into
a separate library, and the host-side tests of the ABI and of the binding run
against it in a child process with the sanitizer runtime preloaded.  Any
sanitizer report, or a failing test, fails this test.
"""

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _build(cc, flags, sources):
    os.makedirs(OUT, exist_ok=True)
    sanit = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]

    def one(src):
        obj = os.path.join(OUT, os.path.basename(src)[:-4] + ".o")
        r = subprocess.run([cc, *flags, *sanit, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, sources))
    lib = os.path.join(OUT, "libhybrid_swa_kv.so")
    r = subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return lib


def test_abi_host_code_under_asan_and_ubsan():
    from hybrid_swa_kv_amd import build

    rt = _runtime()
    if rt is None or shutil.which(build.hipcc()) is None:
        pytest.skip("no ASan runtime or hipcc in this image")
    lib = _build(build.hipcc(), build.FLAGS, build.sources())
    env = dict(os.environ)
    env.update({
        "HYBRID_SWA_KV_LIB": lib,
        "LD_PRELOAD": rt,
        # the HIP runtime's own allocations are not this library's to answer for
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_binding_shapes.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
