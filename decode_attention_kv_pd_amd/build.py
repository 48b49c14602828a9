"""Build libpd_attn.so (host runtime + gfx950 kernels) in place with hipcc.

``python decode_attention_kv_pd_amd/build.py`` (a plain script: importing the
package itself needs the built library).
Always recompiles; the library lands next to this file, where the Python
binding loads it from.
"""
from __future__ import annotations

import importlib.util
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpd_attn.so")
SOURCES = [os.path.join(HERE, "csrc", n) for n in ("api.cpp", "attention.hip", "mla.hip", "mla_wide.hip", "kv_ops.hip", "noalloc.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpd_attn.so)")


EXTRA: dict = {}  # per-source extra flags (none at present)
COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
          # packed fp32 VALU forms are kept out of the generated code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # matrix-product results in architectural registers: the MLA
          # kernels keep their query operand (mla.hip) or O^T (mla_wide.hip,
          # through inline asm) in the accumulation registers; the attention
          # kernels' code is the same either way
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def compile_command(src: str, obj: str):
    return [hipcc(), *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]


def link_command(objs, out: str):
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _errors(res) -> str:
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    return "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="pd_attn_build_") as d:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(d, os.path.basename(src) + ".o")
            cmd = compile_command(src, obj)
            if verbose:
                print(" ".join(cmd), flush=True)
            objs.append(obj)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        failed = []
        for src, pr in procs:
            out, err = pr.communicate()
            res = subprocess.CompletedProcess(pr.args, pr.returncode, out, err)
            if res.returncode != 0:
                failed.append(f"{os.path.basename(src)}: hipcc failed ({res.returncode}):\n{_errors(res)}")
            elif verbose and _errors(res).strip():
                print(_errors(res), file=sys.stderr)
        if failed:
            raise RuntimeError("\n".join(failed))
        cmd = link_command(objs, tmp)
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{_errors(res)}")
    os.replace(tmp, LIB)
    # static checks of the 32-row MLA kernel's generated code (isa_check.py)
    spec = importlib.util.spec_from_file_location("_pd_isa_check", os.path.join(HERE, "isa_check.py"))
    chk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(chk)
    chk.run(hipcc(), COMMON)
    if verbose:
        print("isa check: mla_wide_kernel ok", flush=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
