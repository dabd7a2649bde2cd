"""Build libescha.so (HIP, gfx950) in-tree with hipcc.

``python -m bit_trellis_quantized_amd.build`` compiles every source under
``csrc/`` into ``bit_trellis_quantized_amd/libescha.so``. The build always
recompiles; the binding only loads what is already built.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libescha.so"
ARCH = "gfx950"

SOURCES = ["escha_kernels.hip", "escha_grouped.hip", "escha_stack.hip", "escha_shared.hip",
           "escha_static.hip", "escha_api.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libescha.so)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-fvisibility=hidden", "-ffp-contract=off",
        # packed fp32 VALU forms are kept out of the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{ROOT / 'include'}", f"-I{CSRC}",
        "-Wall", "-Wno-unused-command-line-argument",
    ]


def build(verbose: bool = False, save_temps: Path | None = None) -> Path:
    objs = []
    tmpdir = PKG / "_build"
    tmpdir.mkdir(exist_ok=True)
    cc = hipcc()
    for src in SOURCES:
        s = CSRC / src
        if not s.exists():
            continue
        o = tmpdir / (s.stem + ".o")
        cmd = [cc, *compile_flags(), "-c", str(s), "-o", str(o)]
        if save_temps is not None:
            save_temps.mkdir(parents=True, exist_ok=True)
            cmd += ["-save-temps=obj"]
            o = save_temps / (s.stem + ".o")
            cmd[-1] = str(o)
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(str(o))
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", str(tmp)]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
