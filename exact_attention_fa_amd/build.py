"""Builds libfa.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

    python -m exact_attention_fa_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
# measurement only: the matrix-core calibration loop the benchmark runs beside the kernels
CALIB_LIB = os.path.join(PKG, "libfa_calib.so")
CALIB_SOURCES = ["fa_calib.hip"]
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_fp8.hip",
           "fa_noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def compile_flags() -> list[str]:
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # no NaN ever flows through the kernels (inputs are finite and -inf - -inf is avoided),
        # so fmaxf needs no NaN canonicalisation and maps to v_max3_f32
        "-fno-honor-nans",
        # MFMA results in VGPRs: the score tiles feed vector ALU work directly, and keeping the
        # accumulators out of AGPRs avoids register-class copies in the backward kernels
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wall", "-Wno-unused-result",
    ]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def one(src: str) -> str:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"]
        cmd = [cc, *compile_flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, SOURCES + CALIB_SOURCES))
    for out, parts in ((LIB, objs[:len(SOURCES)]), (CALIB_LIB, objs[len(SOURCES):])):
        tmp = out + ".tmp"
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *parts, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
