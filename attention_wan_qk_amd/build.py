"""Build libwanattn.so in-tree with hipcc for gfx950.

Usage: python -m attention_wan_qk_amd.build  (or build() from Python)

Every .hip source and the C ABI layer are compiled to objects under
``_build/`` at the repository root, in parallel, and linked into
``attention_wan_qk_amd/libwanattn.so``. The measurement aids in
``csrc/probe/`` (include/wanpeak.h) are linked into a library of their own,
``attention_wan_qk_amd/libwanpeak.so``. Always recompiles.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwanattn.so")
PROBE_SRC = os.path.join(CSRC, "probe", "peaks.hip")
PROBE_LIB = os.path.join(PKG, "libwanpeak.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    names = sorted(n for n in os.listdir(CSRC) if n.endswith((".hip", ".cpp")))
    return [os.path.join(CSRC, n) for n in names]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(lib: str, objs) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        probe = ex.submit(_compile, PROBE_SRC)
        objs = list(ex.map(_compile, srcs))
        probe_obj = probe.result()
    _link(LIB, objs)
    _link(PROBE_LIB, [probe_obj])
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
