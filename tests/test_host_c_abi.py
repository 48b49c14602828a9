"""Host: the C ABI from plain C.  A C99 program, compiled with gcc against
include/pd_attn.h (no C++ in the header's C view) and linked with
libpd_attn.so, plans the tiny mixed batch (3 requests: prompts of 16 and 33
tokens and one decode over 40 cached tokens, 4/2 heads, head_dim 64, page 16,
fp32), reads the plan's statistics and work lists, asks for the transfer
sizes and the sharded-transfer table, and takes two error paths.  No GPU
call is made.  The printed figures are checked against the arithmetic of the
layout and against the Python binding's view of the same plan."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from tests.harness import pd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "decode_attention_kv_pd_amd")

C_SOURCE = r"""
#include <stdio.h>
#include <string.h>
#include "pd_attn.h"

int main(void) {
  pd_attn_desc d;
  d.num_qo_heads = 4; d.num_kv_heads = 2; d.head_dim = 64; d.page_size = 16;
  d.dtype = PD_F32; d.causal = 1; d.sm_scale = 0.125f;
  const int32_t qo[3] = {16, 33, 1}, kv[3] = {16, 33, 40};
  const int32_t indptr[4] = {0, 1, 4, 7};
  const int32_t pages[7] = {5, 0, 7, 2, 6, 1, 3};
  pd_plan_t plan = NULL;
  pd_status s = pd_plan(&d, 3, qo, kv, indptr, pages, 8, NULL, &plan);
  printf("plan_status=%d\n", (int)s);
  if (s != PD_OK) return 1;
  pd_plan_stats st;
  memset(&st, 0, sizeof st);
  printf("stats_status=%d\n", (int)pd_plan_get_stats(plan, &st));
  printf("batch=%d\ntotal_q_rows=%d\nprefill_tiles=%d\ndecode_units=%d\n", st.batch, st.total_q_rows,
         st.prefill_tiles, st.decode_units);
  printf("prefill_flops=%lld\ndecode_kv_bytes=%lld\nworkspace_bytes=%lld\n", (long long)st.prefill_flops,
         (long long)st.decode_kv_bytes, (long long)st.workspace_bytes);
  printf("workspace_call=%zu\n", pd_plan_workspace_bytes(plan));
  printf("n_tiles=%d\nn_units=%d\nn_groups=%d\n", pd_plan_work_items(plan, 0, NULL, 0),
         pd_plan_work_items(plan, 1, NULL, 0), pd_plan_work_items(plan, 2, NULL, 0));
  printf("bad_kind=%d\n", pd_plan_work_items(plan, 9, NULL, 0));
  pd_plan_free(plan);
  pd_plan_free(NULL);
  printf("pack_bytes=%zu\npack_heads_bytes=%zu\n", pd_kv_pack_bytes(&d, 7), pd_kv_pack_heads_bytes(&d, 7, 0, 1));
  pd_head_transfer t[8];
  int32_t n = 0;
  s = pd_kv_shard_transfers(8, 2, 4, t, 8, &n);
  printf("shard_status=%d\nshard_n=%d\n", (int)s, n);
  for (int i = 0; i < n; ++i)
    printf("shard%d=%d %d %d %d %d %d\n", i, t[i].src_rank, t[i].dst_rank, t[i].src_h0, t[i].src_h1, t[i].dst_h0,
           t[i].dst_h1);
  const int32_t bad_qo[3] = {16, 34, 1};  /* qo > kv */
  pd_plan_t p2 = NULL;
  s = pd_plan(&d, 3, bad_qo, kv, indptr, pages, 8, NULL, &p2);
  printf("bad_plan_status=%d\nbad_plan_null=%d\nerror_set=%d\n", (int)s, p2 == NULL,
         pd_last_error() != NULL && strlen(pd_last_error()) > 0);
  d.head_dim = 96;
  s = pd_plan(&d, 3, qo, kv, indptr, pages, 8, NULL, &p2);
  printf("unsupported_status=%d\n", (int)s);
  printf("status_string=%s\nversion_set=%d\n", pd_status_string(PD_ERR_WORKSPACE),
         pd_version() != NULL && strlen(pd_version()) > 0);
  return 0;
}
"""


def run_c_program(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    exe = tmp_path / "abi"
    src.write_text(C_SOURCE)
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), os.path.join(LIB_DIR, "libpd_attn.so"), f"-Wl,-rpath,{LIB_DIR}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    return dict(line.split("=", 1) for line in run.stdout.splitlines())


def test_c_program_plans_and_sizes(tmp_path):
    m = pd()
    out = run_c_program(tmp_path)
    assert out["plan_status"] == "0" and out["stats_status"] == "0"
    assert out["batch"] == "3" and out["total_q_rows"] == "50"
    # the same plan through the Python binding
    d = m.make_desc(4, 2, 64, 16, "f32", True, 0.125)
    plan = m.pd_plan(d, np.array([16, 33, 1], np.int32), np.array([16, 33, 40], np.int32),
                     np.array([0, 1, 4, 7], np.int32), np.array([5, 0, 7, 2, 6, 1, 3], np.int32), 8)
    st = plan.stats()
    assert int(out["prefill_tiles"]) == st.prefill_tiles == int(out["n_tiles"])
    assert int(out["decode_units"]) == st.decode_units == int(out["n_units"])
    assert int(out["prefill_flops"]) == st.prefill_flops
    assert int(out["decode_kv_bytes"]) == st.decode_kv_bytes
    assert int(out["workspace_bytes"]) == int(out["workspace_call"]) == plan.workspace_bytes
    # decode-routed rows (qo * g <= 64): the 16-token prompt and the decode,
    # 2 KV heads each; the 33-token prompt (66 rows) is one prefill tile per
    # KV head, 4 * D * H_q * its 33 * 34 / 2 causal pairs
    assert int(out["n_groups"]) == 4 and st.prefill_tiles == 2
    assert st.prefill_flops == 4 * 64 * 4 * (33 * 34 // 2)
    assert st.decode_kv_bytes == 2 * (16 + 40) * 2 * 64 * 4
    assert int(out["bad_kind"]) < 0
    # page images: n * 2 * H_kv * ps * D * 4 bytes (the tiny batch's 7 pages)
    assert int(out["pack_bytes"]) == 7 * 2 * 2 * 16 * 64 * 4 == 114688
    assert int(out["pack_heads_bytes"]) == 114688 // 2


def test_c_program_transfer_table_and_errors(tmp_path):
    out = run_c_program(tmp_path)
    assert out["shard_status"] == "0" and out["shard_n"] == "4"
    # 8 heads from 2 ranks (4 each) to 4 ranks (2 each): each destination
    # rank takes its two heads from one source rank
    got = [tuple(int(v) for v in out[f"shard{i}"].split()) for i in range(4)]
    assert got == [(0, 0, 0, 2, 0, 2), (0, 1, 2, 4, 0, 2), (1, 2, 0, 2, 0, 2), (1, 3, 2, 4, 0, 2)]
    assert int(out["bad_plan_status"]) == -1 and out["bad_plan_null"] == "1" and out["error_set"] == "1"
    assert int(out["unsupported_status"]) == -2
    assert out["status_string"] and out["version_set"] == "1"
