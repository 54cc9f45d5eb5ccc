"""Build libattnprefix.so in-tree with hipcc for gfx950.

Usage: ``python -m long_context_prefix_amd.build`` (or ``build_library()``).
The device assembly of the same compile is kept in ``_build/`` and checked
for early reads of inline MFMA results and for scratch use by the bf16
forward kernels (``isa_check``); a finding fails the build.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "attn_api.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattnprefix.so")
ASM = os.path.join(PKG, "_build", "libattnprefix.gfx950.s")
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if os.path.exists(cand):
        return cand
    found = shutil.which("hipcc")
    if not found:
        raise RuntimeError("hipcc not found (set ROCM_PATH)")
    return found


def compile_command(out: str) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep hipcc from forming packed-fp32 VALU ops (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", os.path.join(PKG, "csrc"),
        SRC, "-o", out,
    ]


def build_library(verbose: bool = False) -> str:
    from .isa_check import inline_mfma_hazards, scratch_findings

    tmp = LIB + ".tmp"
    cmd = compile_command(tmp) + ["-save-temps"]
    if verbose:
        print(" ".join(cmd), flush=True)
    with tempfile.TemporaryDirectory() as work:  # -save-temps writes into the working directory
        res = subprocess.run(cmd, capture_output=True, text=True, cwd=work)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
        asm_files = glob.glob(os.path.join(work, f"*-hip-amdgcn-amd-amdhsa-{ARCH}.s"))
        if len(asm_files) != 1:
            raise RuntimeError(f"expected one device assembly file, found {asm_files}")
        os.makedirs(os.path.dirname(ASM), exist_ok=True)
        shutil.copyfile(asm_files[0], ASM)
    with open(ASM) as f:
        text = f.read()
    hazards = inline_mfma_hazards(text)
    if hazards:
        os.remove(tmp)
        raise RuntimeError("inline MFMA result read too early:\n" + "\n".join(hazards[:10]))
    spills = scratch_findings(text)
    if spills:
        os.remove(tmp)
        raise RuntimeError("forward kernels use scratch memory:\n" + "\n".join(spills[:10]))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
