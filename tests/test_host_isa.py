"""Static checks of the 32-row MLA kernel's generated gfx950 code (CPU only:
hipcc cross-compiles).  The kernel keeps O^T in accumulation registers named
only by its inline asm and places wait states by hand around that asm; the
checker must pass on the real code and catch each kind of planted fault."""
import importlib.util
import os
import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "decode_attention_kv_pd_amd")


def _load(name, path):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def asm_and_checker():
    build = _load("_pd_build_t", os.path.join(PKG, "build.py"))
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    chk = _load("_pd_isa_t", os.path.join(PKG, "isa_check.py"))
    return chk.compile_to_asm(hipcc, build.COMMON, os.path.join(PKG, "csrc", "mla_wide.hip")), chk


def test_generated_code_passes(asm_and_checker):
    asm, chk = asm_and_checker
    body = chk.kernel_lines(asm)
    # score + value products of a step, in its two forms (with and without
    # the next stage's loads between the score products)
    assert sum(1 for t, _ in body if t.startswith("v_mfma")) == 2 * (36 + 32)
    assert chk.check_asm(asm) == []


def test_planted_accumulation_register_use_is_caught(asm_and_checker):
    asm, chk = asm_and_checker
    bad = asm.replace("v_dot2c_f32_bf16_e32", "v_accvgpr_read_b32 v0, a3\n\tv_dot2c_f32_bf16_e32", 1)
    assert any("outside inline asm" in p for p in chk.check_asm(bad))


def test_planted_operand_hazard_is_caught(asm_and_checker):
    asm, chk = asm_and_checker
    lines = asm.splitlines()
    for i, line in enumerate(lines):
        if "v_mfma_f32_32x32x16_bf16 a[" in line:
            first = line.split(None, 1)[1].split(",")[1].strip()
            reg = first.split("[")[1].split(":")[0]
            lines.insert(i, f"\tv_mov_b32_e32 v{reg}, 0")
            break
    assert any("wait states before a product" in p for p in chk.check_asm("\n".join(lines)))


def test_planted_scratch_is_caught(asm_and_checker):
    asm, chk = asm_and_checker
    bad = asm.replace(".amdhsa_private_segment_fixed_size 0", ".amdhsa_private_segment_fixed_size 16")
    assert any("scratch" in p for p in chk.check_asm(bad))


@pytest.fixture(scope="module")
def attn_asm():
    build = _load("_pd_build_t2", os.path.join(PKG, "build.py"))
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    chk = _load("_pd_isa_t2", os.path.join(PKG, "isa_check.py"))
    return chk.compile_to_asm(hipcc, build.COMMON, os.path.join(PKG, "csrc", "attention.hip")), chk


def test_attention_asm_loads_feed_only_matrix_products(attn_asm):
    asm, chk = attn_asm
    for k in chk.ATTN_KERNELS:
        body = chk.kernel_lines(asm, k)
        # K fragments (2 x D/32 per step) and Q fragments come from inline asm
        assert sum(1 for t, a in body if a and t.startswith("global_load_dwordx4")) >= 8
        assert chk.check_asm_loads(asm, k) == []


def test_planted_copy_of_an_asm_load_is_caught(attn_asm):
    asm, chk = attn_asm
    lines = asm.splitlines()
    start = next(i for i, l in enumerate(lines) if l.startswith("_Z") and chk.ATTN_KERNELS[0] in l)
    in_asm = False
    for i in range(start, len(lines)):
        s = lines[i].strip()
        in_asm = True if s.startswith(";;#ASMSTART") else False if s.startswith(";;#ASMEND") else in_asm
        if in_asm and s.startswith("global_load_dwordx4"):
            reg = s.split()[1].split("[")[1].split(":")[0]
            break
    # a copy of the loaded register placed right after the load asm
    j = next(k for k in range(i, len(lines)) if lines[k].strip().startswith(";;#ASMEND"))
    lines.insert(j + 1, f"\tv_mov_b32_e32 v0, v{reg}")
    probs = chk.check_asm_loads("\n".join(lines), chk.ATTN_KERNELS[0])
    assert probs and "reads a register" in probs[0]
