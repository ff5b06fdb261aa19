"""Build librace_attn.so (HIP kernels + C ABI) for gfx950 in place.

    python -m linear_attention_soft_amd.build [--jobs N]

Each translation unit is compiled with hipcc in parallel, then linked into
``linear_attention_soft_amd/librace_attn.so``.  Every call rebuilds.  The
kernel instance files are exactly those the registry names
(``RACE_INSTANCE_FILES`` in ``csrc/race_registry.hpp``); a listed source that
is missing, or an instance file the registry does not name, is an error.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librace_attn.so")
ARCH = os.environ.get("RACE_OFFLOAD_ARCH", "gfx950")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 VALU forms are disabled on purpose
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def instance_names() -> list[str]:
    """Instance files named by the registry macro, in its order."""
    text = open(os.path.join(CSRC, "race_registry.hpp")).read()
    m = re.search(r"#define RACE_INSTANCE_FILES\(X\)((?:[^\n]*\\\n)*[^\n]*)", text)
    if not m:
        raise RuntimeError("RACE_INSTANCE_FILES not found in race_registry.hpp")
    return re.findall(r"X\((\w+)\)", m.group(1))


def sources() -> list[str]:
    names = instance_names()
    srcs = [f"race_inst_{n}.hip" for n in names] + ["race_api.cpp"]
    missing = [s for s in srcs if not os.path.exists(os.path.join(CSRC, s))]
    if missing:
        raise RuntimeError(f"listed sources are missing: {missing}")
    present = {os.path.basename(p) for p in glob.glob(os.path.join(CSRC, "race_inst_*.hip"))}
    extra = sorted(present - set(srcs))
    if extra:
        raise RuntimeError(f"instance files not named in RACE_INSTANCE_FILES: {extra}")
    return srcs


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, out_dir: str = BUILD, extra: tuple = ()) -> str:
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return out


def link(objs: list[str], out: str, extra: tuple = ()) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    link(objs, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
    sys.exit(0)
