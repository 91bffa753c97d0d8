"""Compile the HIP library ``libattn.so`` (forward and backward kernels) for gfx950 in-tree,
and the instruction-rate probes ``libattn_probe.so`` that ``bench.py --probe`` runs.

Usage: ``python -m tiled_attention_16_amd.build`` (or ``build_library()``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
SRCS = [os.path.join(PKG_DIR, "csrc", "attn_fwd.hip"), os.path.join(PKG_DIR, "csrc", "attn_bwd.hip"),
        os.path.join(PKG_DIR, "csrc", "attn_fwd_fp8.hip")]
LIB = os.path.join(PKG_DIR, "libattn.so")
# instruction-rate microbenchmarks (bench.py --probe); not part of the attention C ABI
PROBE_SRC = os.path.join(PKG_DIR, "csrc", "probes.hip")
PROBE_LIB = os.path.join(PKG_DIR, "libattn_probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results and operands of the compiler-scheduled (builtin) MFMAs in
    # VGPRs: a kernel that uses no AGPRs gets the whole register budget as
    # VGPRs instead of a fixed VGPR/AGPR split, and needs no v_accvgpr moves
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
]


def build_library(verbose: bool = False) -> str:
    """Build ``libattn.so`` next to this file; return its path. Raises on failure.

    The device code is also compiled to assembly with the same flags and
    checked by ``hazards.check`` (MFMA operand written by a VALU instruction
    too close before the MFMA); a violation fails the build.
    """
    from .hazards import check

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    asm = LIB + ".s.tmp"
    inc = ["-I", os.path.join(REPO_DIR, "include")]
    cmd = [hipcc, *HIPCC_FLAGS, *inc, *SRCS, "-o", tmp]
    flags_s = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    # the forward kernel's hand-placed MFMAs are the ones the hazard check is for
    cmd_s = [hipcc, *flags_s, *inc, "--cuda-device-only", "-S", SRCS[0], "-o", asm]
    probe_tmp = PROBE_LIB + ".tmp"
    cmd_p = [hipcc, *HIPCC_FLAGS, PROBE_SRC, "-o", probe_tmp]
    cmds = (cmd, cmd_s, cmd_p)
    procs = [subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True) for c in cmds]
    outs = [p.communicate() for p in procs]
    for c, p, (out, err) in zip(cmds, procs, outs):
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed ({p.returncode}):\n{' '.join(c)}\n{out}\n{err}")
    if verbose and outs[0][1]:
        sys.stderr.write(outs[0][1])
    with open(asm) as f:
        problems = check(f.read())
    os.remove(asm)
    if problems:
        os.remove(tmp)
        raise RuntimeError("MFMA hazard in the compiled kernel:\n" + "\n".join(problems))
    os.replace(tmp, LIB)
    os.replace(probe_tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
