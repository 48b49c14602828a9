"""pd_attention_run_noalloc, the call for callers that cannot allocate: its
output, LSE and appended pool match pd_kv_append + pd_attention_run over a
caller workspace bit for bit (same plan, same kernels), and the oracle within
the usual bars, on two calls in a row, the second one smaller, so the second
call runs over the first call's leftovers in the static scratch."""
import numpy as np
import pytest
import torch

from tests.harness import DeviceRun, dev_array, host_array, oracle_outputs, pd, report, tolerance
from workloads import make_batch

CASES = [
    # larger call first: split decode rows (several key chunks each), a
    # prefill request, a multi-token decode step and an empty request
    ("mixed", dict(lengths=([300, 1, 1, 3, 0, 1], [700, 1500, 2000, 40, 9, 4096])), 256),
    # then a smaller one
    ("mixed", dict(lengths=([1, 17], [900, 60])), 128),
]


def run_noalloc(run, b, with_append):
    m = pd()
    n = max(int(b.qo_indptr[-1]), 1)
    pool = dev_array(run.pool_host, run.pool.device)
    if not with_append:   # attention only, over a pool that already holds the new rows
        m.pd_kv_append(run.plan, run.ws, pool, run.k_new, run.v_new)
    out = torch.full((n, b.H_q, b.D), float("nan"), dtype=torch.float32, device=pool.device)
    lse = torch.full((n, b.H_q), float("nan"), dtype=torch.float32, device=pool.device)
    if with_append:
        m.pd_attention_run_noalloc(run.plan, run.q, pool, out, lse, k_new=run.k_new, v_new=run.v_new)
    else:
        m.pd_attention_run_noalloc(run.plan, run.q, pool, out, lse)
    torch.cuda.synchronize()
    return pool, out, lse


@pytest.mark.gpu
@pytest.mark.parametrize("with_append", [True, False])
def test_noalloc_matches_workspace_call_on_two_calls(with_append):
    for wid, kw, chunk in CASES:
        b = make_batch(wid, **kw)
        print(f"[noalloc] {wid} {kw} chunk {chunk} append={with_append}", flush=True)
        run = DeviceRun(b, decode_chunk_keys=chunk)
        assert run.plan.workspace_bytes <= pd().NOALLOC_SCRATCH_BYTES
        ref_out, ref_lse = run.step()
        pool, out, lse = run_noalloc(run, b, with_append)
        n = int(b.qo_indptr[-1])
        got_out, got_lse = out[:n].cpu().numpy(), lse[:n].cpu().numpy()
        assert np.array_equal(got_out.view(np.uint32), ref_out.view(np.uint32))
        assert np.array_equal(got_lse.view(np.uint32), ref_lse.view(np.uint32))
        assert host_array(pool, b.np_dtype).tobytes() == host_array(run.pool, b.np_dtype).tobytes()
        O, L = oracle_outputs(b)
        assert report(f"noalloc {wid}", got_out, O) <= tolerance(b)
        assert float(np.abs(got_lse - L).max()) <= 5e-3


@pytest.mark.gpu
def test_noalloc_fp32_tiny_then_larger_bf16():
    """fp32 kernels through the static scratch, then the bf16 path again."""
    for b in (make_batch("tiny"), make_batch("mixed", lengths=([1, 1, 64], [3000, 33, 64]))):
        run = DeviceRun(b, decode_chunk_keys=64)
        ref_out, ref_lse = run.step()
        pool, out, lse = run_noalloc(run, b, True)
        n = int(b.qo_indptr[-1])
        assert np.array_equal(out[:n].cpu().numpy().view(np.uint32), ref_out.view(np.uint32))
        assert np.array_equal(lse[:n].cpu().numpy().view(np.uint32), ref_lse.view(np.uint32))
        O, _ = oracle_outputs(b)
        assert report(f"noalloc {b.name}", out[:n].cpu().numpy(), O) <= tolerance(b)
