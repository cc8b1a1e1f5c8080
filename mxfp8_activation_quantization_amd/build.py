"""Ahead-of-time build of libmxfp8.so for gfx950 with hipcc (in-tree, no JIT).

    python mxfp8_activation_quantization_amd/build.py

(Run by path: importing the package loads the library this script builds.)

Every call recompiles all sources (hipcc cross-compiles for gfx950 on a host
without a GPU).  Objects go to ``_build/`` beside this file; the shared library
lands next to the Python binding, which loads it from there.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libmxfp8.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["api.cpp", "quantize.hip", "rmsnorm_quantize.hip", "gemm_tiled.hip", "gemm_skinny.hip", "noalloc.hip"]
# Sources compiled once per instance (macro = 0 .. count - 1), one object each: the tile kernel's
# launcher instances, which are the slowest to compile, build in parallel.
INSTANCED = {"gemm_tiled_inst.hip": ("TILE_INST", 12)}
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms stay out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError(f"hipcc not found (looked for {cand})")
    return cand


def _run(cmd: list[str]) -> None:
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l]
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n" + "\n".join(lines))
    # Every kernel must fit its registers: register spills go to scratch memory,
    # cost bandwidth, and spill code inside lane-masked regions has produced wrong
    # results.  The resource remarks name each kernel and its scratch bytes.
    spilled, current = [], None
    for l in lines:
        m = re.search(r"Function Name: (\S+)", l)
        if m:
            current = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", l)
        if m and int(m.group(1)) > 0:
            spilled.append(f"{current}: {m.group(1)} bytes/lane")
    if spilled:
        raise RuntimeError("kernels spill registers to scratch:\n  " + "\n  ".join(spilled))
    out = "\n".join(l for l in lines if "remark:" not in l and "-Rpass-analysis" not in l
                    and not re.match(r"^\s*(\d+\s*)?\|", l))
    if out.strip():
        print(out, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source and link LIB_PATH; returns its path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    units = [(src, os.path.splitext(src)[0], []) for src in SOURCES]
    for src, (macro, count) in INSTANCED.items():
        units += [(src, f"{os.path.splitext(src)[0]}_{i}", [f"-D{macro}={i}"]) for i in range(count)]
    for src, stem, defs in units:
        obj = os.path.join(BUILD_DIR, stem + ".o")
        lang = ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
        cmds.append([cc, *COMMON_FLAGS, *defs, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(min(len(cmds), os.cpu_count() or 1)) as ex:
        for cmd, _ in zip(cmds, ex.map(_run, cmds)):
            if verbose:
                print(" ".join(cmd))
    tmp = LIB_PATH + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link))
    _run(link)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
