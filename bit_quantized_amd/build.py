"""Build libfourtune.so (HIP for gfx950) in-tree with hipcc.

    python -m bit_quantized_amd.build        # or bit_quantized_amd.build.build()

Objects go to _build/ at the repository root; the shared library is written
next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfourtune.so")
SOURCES = ["api.cpp", "quantize.hip", "gemm.hip", "gemm_mlp.hip", "lora.hip", "act.hip",
           "scratch.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the gfx950 feature above; that note is harmless
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libfourtune.so; return its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]

    def compile_one(i):
        src = os.path.join(CSRC, SOURCES[i])
        cmd = [hipcc, *COMMON, "-c", src, "-o", objs[i]]
        if SOURCES[i].endswith(".cpp"):
            cmd = [hipcc, *[a for a in COMMON if not a.startswith("--offload")], "-c", src,
                   "-o", objs[i]]
        return _run(cmd)

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        outs = list(ex.map(compile_one, range(len(SOURCES))))
    tmp = LIB + ".tmp"
    outs.append(_run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
