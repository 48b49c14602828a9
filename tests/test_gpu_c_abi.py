"""GPU: one step of the path driven from C through the C ABI alone
(tests/c_step.c, built by build.py; HIP runtime for device memory, no
PyTorch): plan, upload, append, attention, pack and unpack of the tiny fp32
batch (prompts of 16 and 33 tokens and a decode over 40 cached tokens, 4/2
heads, head_dim 64, page 16).  The outputs match the oracle (1e-4 for fp32
inputs); the pool after the append and the unpack, and the packed buffer,
match the oracle's page operations bit for bit."""
import os
import subprocess

import numpy as np
import pytest

from oracle import paged_kv as OP
from tests.harness import oracle_outputs, prefix_pool, report, tolerance
from workloads import make_batch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_step")


def test_c_program_step_matches_oracle(tmp_path):
    assert os.path.exists(EXE), "tests/c_step is missing: build with __graft_entry__.build()"
    b = make_batch("tiny")
    assert b.dtype == "f32"
    pool0 = prefix_pool(b)
    ids = np.asarray(b.request_pages(1), np.int32)  # the 33-token prompt's 3 pages
    # destination ids: the spare page, then pages of other requests (the
    # unpack overwrites them after the attention has read them)
    others = [p for p in range(b.num_pool_pages) if p not in set(ids) | set(b.spare_pages)]
    dst = np.asarray(list(b.spare_pages[:1]) + others[:len(ids) - 1], np.int32)
    assert len(set(dst.tolist())) == len(ids)
    rows = int(b.qo_indptr[-1])
    hdr = np.array([b.H_q, b.H_kv, b.D, b.ps, 0, int(b.causal), b.B, b.num_pool_pages, len(b.page_indices), rows],
                   np.int32)
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        for a in (hdr, np.array([b.sm_scale], np.float32), b.qo_lens.astype(np.int32), b.kv_lens.astype(np.int32),
                  b.page_indptr.astype(np.int32), b.page_indices.astype(np.int32), pool0.astype(np.float32),
                  b.q.astype(np.float32), b.k_new.astype(np.float32), b.v_new.astype(np.float32),
                  np.array([len(ids)], np.int32), ids, dst):
            f.write(np.ascontiguousarray(a).tobytes())
    out_path = tmp_path / "out.bin"
    print("c_step: tiny fp32 batch", flush=True)
    res = subprocess.run([EXE, str(src), str(out_path)], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0
    raw = np.fromfile(out_path, np.uint8)
    n_out, n_lse, n_pool = rows * b.H_q * b.D, rows * b.H_q, pool0.size
    out = raw[:4 * n_out].view(np.float32).reshape(rows, b.H_q, b.D)
    lse = raw[4 * n_out:4 * (n_out + n_lse)].view(np.float32).reshape(rows, b.H_q)
    pool = raw[4 * (n_out + n_lse):4 * (n_out + n_lse + n_pool)].view(np.float32).reshape(pool0.shape)
    buf = raw[4 * (n_out + n_lse + n_pool):]
    O, L = oracle_outputs(b)
    assert report("c_step", out, O) <= tolerance(b)
    assert np.abs(lse - L).max() <= 1e-4
    ref_pool = pool0.copy()
    OP.kv_append(ref_pool, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.k_new, b.v_new)
    ref_buf = OP.kv_pack(ref_pool, ids)
    assert buf.tobytes() == ref_buf.tobytes()
    ref_pool = OP.kv_unpack(ref_pool, dst, ref_buf)
    assert pool.tobytes() == ref_pool.tobytes()
