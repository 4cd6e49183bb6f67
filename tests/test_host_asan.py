"""The library's host code under AddressSanitizer, on the CPU.

A build of librkv.so whose host pass is instrumented (the device code is
compiled as usual) runs the ABI tests and the page-accounting tests in a
child process with the sanitizer's runtime preloaded: every argument check,
workspace plan, paged plan and error path of the C ABI then executes with
its heap and stack accesses checked. A sanitizer report makes the child fail.
The tests need no GPU: no call reaches a kernel launch.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_host_asan(dst: str) -> str:
    """Compile every HIP source with the host pass sanitized; link into dst."""
    from decode_kv_cache_03_amd import build as b
    hipcc = b._hipcc()
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

    def one(src):
        obj = os.path.join(dst, os.path.basename(src) + ".o")
        r = subprocess.run([hipcc, *b.FLAGS, *host_asan, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    srcs = b.sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    lib = os.path.join(dst, "librkv_host_asan.so")
    r = subprocess.run([hipcc, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-Xarch_host",
                        "-fsanitize=address", "-o", lib, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return lib


def test_abi_host_code_under_address_sanitizer(tmp_path):
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    try:
        from decode_kv_cache_03_amd import build as b
        b._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    lib = build_host_asan(str(tmp_path))
    env = dict(os.environ, LD_PRELOAD=rt, RKV_TEST_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    # the child checks that it really runs the sanitized build under the runtime
    probe = ("import os; from decode_kv_cache_03_amd import _lib; "
             f"_lib.LIB_PATH = {lib!r}; _lib.load(); maps = open('/proc/self/maps').read(); "
             "assert 'librkv_host_asan.so' in maps and 'libclang_rt.asan' in maps, 'not sanitized'")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_page_plan.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stdout + r.stderr
