"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

race_api.cpp (argument checks, size queries, plans, launch set-up) is rebuilt
with host-side ASan + UBSan (device code is compiled as usual) and linked
with the kernel instance objects of the in-place build into a separate
library.  The plain C client and the Python ABI tests then run against it;
any sanitizer report fails them.  No GPU is used: every call fails its host
checks before anything is enqueued.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from linear_attention_soft_amd import build as B  # noqa: E402

CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if not (os.path.exists(CLANG) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm clang not found")
    objs = [os.path.join(B.BUILD, f"race_inst_{n}.o") for n in B.instance_names()]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        pytest.fail(f"kernel objects missing ({missing[0]}); build with python -m linear_attention_soft_amd.build")
    d = tmp_path_factory.mktemp("san")
    api = str(d / "race_api.o")
    # host-only sanitizers: every -fsanitize= on the hipcc line sits behind -Xarch_host
    _run([B.hipcc(), "-x", "hip", *B.FLAGS, "-O1", "-g",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
          "-c", os.path.join(B.CSRC, "race_api.cpp"), "-o", api])
    lib = str(d / "librace_attn.so")
    _run([CLANGXX, "-shared", "-fPIC", "-shared-libsan", "-fsanitize=address,undefined", *objs, api,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    return d, lib


def _asan_runtime():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not hits:
        pytest.skip("ASan runtime not found")
    return hits[0]


def test_c_client_under_sanitizers(sanitized_lib):
    d, lib = sanitized_lib
    exe = str(d / "c_abi_check")
    rt_dir = os.path.dirname(_asan_runtime())
    _run([CLANG, "-std=c99", "-Wall", "-Werror", "-g", "-fsanitize=address,undefined", "-shared-libsan",
          "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "c_abi_check.c"), lib, f"-Wl,-rpath,{d}", f"-Wl,-rpath,{rt_dir}", "-o", exe])
    r = _run([exe], env={**os.environ, **SAN_ENV}, timeout=120)
    assert r.stdout.strip() == "ok"


def test_python_abi_tests_under_sanitizers(sanitized_lib):
    _, lib = sanitized_lib
    env = {**os.environ, **SAN_ENV, "LD_PRELOAD": _asan_runtime(), "RACE_ATTN_LIBRARY": lib}
    _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py"),
          "-k", "not plain_c_client"], env=env, cwd=ROOT, timeout=600)
