"""Build libpd_attn.so (host runtime + gfx950 kernels) in place with hipcc.

``python decode_attention_kv_pd_amd/build.py`` (a plain script: importing the
package itself needs the built library).
Always recompiles; the library lands next to this file, where the Python
binding loads it from.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpd_attn.so")
SOURCES = [os.path.join(HERE, "csrc", n) for n in ("api.cpp", "attention.hip", "mla.hip", "kv_ops.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpd_attn.so)")


def command(out: str):
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # matrix-product results in architectural registers: the MLA
            # kernel keeps its query operand in the accumulation registers
            # (the attention kernels' code is the same either way)
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
            *SOURCES, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
