"""Static checks of generated gfx950 code: the 32-row MLA kernel, and the
attention kernel's inline-asm register loads.

mla_wide.hip keeps O^T in accumulation registers that only its inline asm
names, and places by hand the wait states that the compiler's hazard
recognizer cannot see across that asm.  This module compiles the file to
assembly (device code only) and checks, in the kernel's code:

* no accumulation register (a0..a255) is referenced outside inline asm, so
  nothing of the compiler's own shares the registers that hold O^T;
* no matrix product reads a VGPR that a VALU instruction wrote fewer than
  2 wait states before it (an s_nop n counts n + 1, any other instruction
  1);
* no scratch: the kernel neither spills nor uses private memory.

The attention kernel's decode role loads its K and Q fragments from inline
asm (the compiler does not see those loads, so it cannot wait for them; the
kernel waits with explicit s_waitcnt and then pins the registers with an
empty asm).  A copy of such a register that the compiler placed between the
load and the wait would read data still in flight, so for the attention
kernels this module also checks:

* every instruction that reads a register written by an inline-asm
  global_load_dwordx4, up to the next write of that register, is a matrix
  product (the only consumer the source gives those fragments).

build.py runs it after every build; tests/test_host_isa.py runs it too.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
KERNEL = "mla_wide_kernel"
VALU_WAIT_STATES = 2

_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")
_AREG = re.compile(r"\ba\[(\d+):(\d+)\]|\ba(\d+)\b")


def _regs(text: str, pat=_VREG) -> set:
    out = set()
    for m in pat.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def kernel_lines(asm: str, kernel: str = KERNEL):
    """(text, in_inline_asm) for each instruction line of the kernel's body."""
    lines, inside, in_asm = [], False, False
    for raw in asm.splitlines():
        s = raw.strip()
        code = s.split(";")[0].strip()
        if not inside:
            inside = code.endswith(":") and kernel in code and not code.startswith(".")
            continue
        if code.startswith(".Lfunc_end"):
            break
        if s.startswith(";;#ASMSTART"):
            in_asm = True
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        elif code and not code.startswith(".") and not code.endswith(":"):
            lines.append((code, in_asm))
    return lines


def check_asm(asm: str, kernel: str = KERNEL) -> list:
    """Problems found in the kernel's code (empty when it passes)."""
    body = kernel_lines(asm, kernel)
    if not body:
        return [f"kernel {kernel} not found in the assembly"]
    problems = []
    for text, in_asm in body:
        if not in_asm and _regs(text.split(None, 1)[1] if " " in text else "", _AREG) and \
                not text.startswith("s_"):
            problems.append(f"accumulation register outside inline asm: {text}")
    for i, (text, _) in enumerate(body):
        if not text.startswith("v_mfma"):
            continue
        ops = [o.strip() for o in text.split(None, 1)[1].split(",")]
        srcs = _regs(ops[1]) | _regs(ops[2])
        waits = 0
        for prev, _ in reversed(body[max(0, i - 8):i]):
            if waits >= VALU_WAIT_STATES:
                break
            op = prev.split()[0]
            if op.startswith("v_") and not op.startswith(("v_mfma", "v_accvgpr_write")):
                dst = prev.split(None, 1)[1].split(",")[0] if " " in prev else ""
                if _regs(dst) & srcs:
                    problems.append(f"VALU write {waits} wait states before a product reads it: {prev!r} -> {text!r}")
            m = re.match(r"s_nop\s+(\d+)", prev)
            waits += int(m.group(1)) + 1 if m else 1
    m = re.search(r"\.amdhsa_kernel\s+\S*" + kernel + r"\S*\s.*?\.amdhsa_private_segment_fixed_size\s+(\d+)", asm,
                  re.S)
    if m is None or int(m.group(1)) != 0:
        problems.append(f"the kernel uses scratch (private segment size {m.group(1) if m else 'unknown'})")
    return problems


ATTN_KERNELS = ("attn_bf16_kernelILi128", "attn_bf16_kernelILi64")
_NO_DEST = ("global_store", "buffer_store", "flat_store", "scratch_store", "ds_write", "ds_add", "ds_store",
            "global_atomic", "buffer_atomic", "s_", "global_load_lds", "buffer_load_lds")
_ANY_REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def _all_regs(text: str) -> set:
    out = set()
    for m in _ANY_REG.finditer(text):
        if m.group(1):
            out.update((m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _reads_writes(text: str):
    op = text.split()[0]
    rest = text.split(None, 1)[1] if " " in text else ""
    if not rest or op.startswith(_NO_DEST):
        return _all_regs(rest), set()
    ops = rest.split(",")
    return _all_regs(",".join(ops[1:])), _all_regs(ops[0])


def check_asm_loads(asm: str, kernel: str) -> list:
    """Readers other than matrix products of registers loaded by inline asm."""
    body = kernel_lines(asm, kernel)
    if not body:
        return [f"kernel {kernel} not found in the assembly"]
    loads = [(i, _reads_writes(t)[1]) for i, (t, in_asm) in enumerate(body)
             if in_asm and t.startswith("global_load_dwordx4")]
    if not loads:
        return [f"{kernel}: no inline-asm register loads found"]
    problems = []
    for i, dst in loads:
        for text, _ in body[i + 1:]:
            rd, wr = _reads_writes(text)
            if rd & dst and not text.startswith("v_mfma"):
                problems.append(f"{kernel}: {text!r} reads a register of {body[i][0]!r} (only matrix products may)")
                break
            if wr & dst:
                break
    return problems


def compile_to_asm(hipcc: str, common_flags: list, src: str) -> str:
    with tempfile.TemporaryDirectory(prefix="pd_isa_") as d:
        out = os.path.join(d, "k.s")
        cmd = [hipcc, *[f for f in common_flags if f != "-fPIC"], "--cuda-device-only", "-S", src, "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc -S failed ({res.returncode}):\n{res.stderr}")
        return open(out).read()


def run(hipcc: str, common_flags: list) -> None:
    """Compile mla_wide.hip and attention.hip to assembly and raise if a check
    fails."""
    asm = compile_to_asm(hipcc, common_flags, os.path.join(HERE, "csrc", "mla_wide.hip"))
    problems = check_asm(asm)
    if problems:
        raise RuntimeError("mla_wide_kernel code check failed:\n  " + "\n  ".join(problems[:20]))
    asm = compile_to_asm(hipcc, common_flags, os.path.join(HERE, "csrc", "attention.hip"))
    problems = [p for k in ATTN_KERNELS for p in check_asm_loads(asm, k)]
    if problems:
        raise RuntimeError("attention kernel code check failed:\n  " + "\n  ".join(problems[:20]))
