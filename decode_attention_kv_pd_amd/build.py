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


# Host-code sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer) for the
# planner and the C ABI: applied to the host pass only (-Xarch_host), never to
# GPU code.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-fno-sanitize-recover=undefined"]


def compile_command(src: str, obj: str, sanitize: bool = False):
    extra = HOST_SANITIZE if sanitize and src.endswith(".cpp") else []
    return [hipcc(), *COMMON, *EXTRA.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]


def link_command(objs, out: str, sanitize: bool = False):
    extra = ["-fsanitize=address,undefined", "-shared-libasan"] if sanitize else []
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", out]


def _errors(res) -> str:
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    return "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)


def build_c_step(verbose: bool = False) -> str:
    """tests/c_step: the C program of tests/test_gpu_c_abi.py, which drives a
    step through the C ABI with the HIP runtime alone (no PyTorch); built
    with the C compiler against include/pd_attn.h and the library."""
    cc = shutil.which("gcc") or shutil.which("cc")
    src = os.path.join(ROOT, "tests", "c_step.c")
    exe = os.path.join(ROOT, "tests", "c_step")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(rocm, "include"), src, "-o", exe, "-L", HERE, "-lpd_attn", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../decode_attention_kv_pd_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"c_step build failed ({res.returncode}):\n{res.stderr}")
    return exe


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    """Compile every source and link the library at `out`.  `sanitize`
    instruments the host code (api.cpp) with ASan and UBSan; such a library
    is loaded with the sanitizer runtime preloaded (see __main__ below)."""
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory(prefix="pd_attn_build_") as d:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(d, os.path.basename(src) + ".o")
            cmd = compile_command(src, obj, sanitize)
            if verbose:
                print(" ".join(cmd), flush=True)
            objs.append(obj)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        failed = []
        for src, pr in procs:
            o, e = pr.communicate()
            res = subprocess.CompletedProcess(pr.args, pr.returncode, o, e)
            if res.returncode != 0:
                failed.append(f"{os.path.basename(src)}: hipcc failed ({res.returncode}):\n{_errors(res)}")
            elif verbose and _errors(res).strip():
                print(_errors(res), file=sys.stderr)
        if failed:
            raise RuntimeError("\n".join(failed))
        cmd = link_command(objs, tmp, sanitize)
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{_errors(res)}")
    os.replace(tmp, out)
    if out == LIB:
        build_c_step(verbose)
    # static checks of the 32-row MLA kernel's generated code (isa_check.py)
    spec = importlib.util.spec_from_file_location("_pd_isa_check", os.path.join(HERE, "isa_check.py"))
    chk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(chk)
    chk.run(hipcc(), COMMON)
    if verbose:
        print("isa check: mla_wide_kernel ok", flush=True)
    return out


if __name__ == "__main__":
    # python decode_attention_kv_pd_amd/build.py                  -> the library in place
    # python decode_attention_kv_pd_amd/build.py --host-sanitize DIR
    #   -> DIR/libpd_attn.so with ASan/UBSan host code; run the host tests
    #      against it with the runtime preloaded, e.g.
    #      LD_PRELOAD=$(hipcc --print-file-name=libclang_rt.asan-x86_64.so)
    #      ASAN_OPTIONS=detect_leaks=0 PD_ATTN_LIB=DIR/libpd_attn.so
    #      python -m pytest tests/test_host_abi.py tests/test_host_mla.py
    if len(sys.argv) == 3 and sys.argv[1] == "--host-sanitize":
        os.makedirs(sys.argv[2], exist_ok=True)
        print(build(verbose=True, out=os.path.join(sys.argv[2], "libpd_attn.so"), sanitize=True))
    else:
        print(build(verbose=True))
