"""The ABI checks of test_abi.py once more against a build of the library
whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer
(host validation, descriptor carving and status strings run instrumented;
the device code is compiled as usual and not executed here: no GPU needed).

The build goes to dynamic_sparse_attention_index_amd/_build_asan/ and the
checks run in a child interpreter with the sanitizer runtime preloaded; any
report ends that interpreter with a failure.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

import pytest

from dynamic_sparse_attention_index_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(_build.PKG, "_build_asan")
LIB = os.path.join(OUT, "libvsattn_asan.so")


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _compile(src):
    obj = os.path.join(OUT, os.path.basename(src).replace(".hip", ".o"))
    flags = [f for f in _build.FLAGS if f != "-O3"]
    cmd = [_build.HIPCC, "-O1", "-g", *flags, "-Xarch_host", "-fsanitize=address,undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return obj


def _build_lib():
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(_build.CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    # the instrumented objects' sanitizer symbols resolve against the
    # preloaded runtime
    res = subprocess.run([_build.HIPCC, "-shared", f"--offload-arch={_build.ARCH}", *objs, "-o", LIB],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]


@pytest.mark.timeout(900)
def test_abi_under_host_sanitizers():
    rt = _runtime()
    if rt is None or not os.path.exists(_build.HIPCC):
        pytest.skip("no hipcc or sanitizer runtime")
    _build_lib()
    env = dict(os.environ)
    env.update({"LD_PRELOAD": rt, "VS_ATTN_LIB": LIB,
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail
