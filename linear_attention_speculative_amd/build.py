"""Compiles the HIP sources of the KDA RecoverSSM library into
`libkda_recoverssm.so` inside this package, for gfx950.

Usage: python -m linear_attention_speculative_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libkda_recoverssm.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["kda_verify_d128.hip", "kda_verify_d64.hip", "kda_verify_d32.hip",
           "kda_verify_d16.hip", "kda_verify.hip", "kda_commit.hip",
           "kda_plan.hip", "kda_api.cpp"]
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU ops are disabled for all device code.
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-kernel resource usage, checked for spills after each compile.
REMARKS = ["-Rpass-analysis=kernel-resource-usage"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         text=True)
    lines = [line for line in res.stdout.splitlines()
             if "packed-fp32-ops' is not a recognized" not in line]
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): "
                           f"{' '.join(cmd)}\n" + "\n".join(lines))
    _check_no_spills(lines)
    out = "\n".join(line for line in lines if "remark:" not in line and
                    "Rpass-analysis" not in line)
    if verbose and out.strip():
        print(out)


def _check_no_spills(lines):
    """Every kernel must run without scratch (register spills): the
    resource-usage remarks of the compiler name each kernel, then its
    per-lane scratch size."""
    kernel = None
    for line in lines:
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            kernel = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            raise RuntimeError(f"kernel {kernel} spills {m.group(1)} bytes "
                               "per lane to scratch")


def build_library(verbose: bool = False) -> str:
    """Compile every source (always; no staleness check) and link the
    shared library in place.  Returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD_DIR, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        jobs.append([hipcc] + COMMON_FLAGS + lang + REMARKS +
                    ["-c", path, "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp]
         + objs, verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
