"""GPU: the long-context workload at full size (an 8192-token chunk over 24576
cached tokens plus 256 single-token decodes over 32768 cached tokens; 64/8
heads, head_dim 128, bf16, page size 64), in the launch configuration the
benchmark times (default plan).  The pool (about 36 GB) is drawn on the
device; sampled output rows (33 decode requests, about 75 chunk tokens at
32-token tile edges) are checked one by one against the oracle, the sampled
requests' pages are checked bit-exactly after the append, and the chunk
request's 512 pages go through pack and unpack."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import paged_kv as OP
from tests.harness import desc_of, pd
from workloads import device_normal_, device_seed, make_batch

pytestmark = pytest.mark.gpu

# the chunk request and 33 of the 256 decode requests, spread over the launch
# (their units land in blocks of every XCD and both key chunks)
SAMPLE_REQUESTS = (0,) + tuple(range(1, 257, 8)) + (256,)
# chunk tokens at the edges of its 32-token tiles (every eighth tile), at the
# start, the middle and the end
PREFILL_TOKENS = tuple(sorted({0, 1, 2, 63, 64, 127, 4095, 4096, 8190, 8191} |
                              {e for k in range(1, 256, 8) for e in (32 * k - 1, 32 * k)}))


def pages_host(pool, ids):
    """Copy of the listed pages as raw bf16 bits [n, 2, H_kv, ps, D]."""
    idx = torch.as_tensor(np.asarray(ids, np.int64), device=pool.device)
    return pool.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_long_context_full_size():
    b = make_batch("long", materialize=False)
    m = pd()
    desc = desc_of(b)
    plan = m.pd_plan(desc, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages)
    print("plan", plan.stats(), flush=True)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    m.pd_plan_upload(plan, ws)
    pool = torch.empty(b.pool_shape, dtype=torch.bfloat16, device="cuda")
    device_normal_(pool, device_seed(5, 0, 0))
    n = int(b.qo_indptr[-1])
    q = device_normal_(torch.empty((n, b.H_q, b.D), dtype=torch.bfloat16, device="cuda"), device_seed(5, 0, 1))
    k_new = device_normal_(torch.empty((n, b.H_kv, b.D), dtype=torch.bfloat16, device="cuda"), device_seed(5, 0, 2))
    v_new = device_normal_(torch.empty((n, b.H_kv, b.D), dtype=torch.bfloat16, device="cuda"), device_seed(5, 0, 3))
    before = {r: pages_host(pool, b.request_pages(r)) for r in SAMPLE_REQUESTS}
    out = torch.full((n, b.H_q, b.D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((n, b.H_q), float("nan"), dtype=torch.float32, device="cuda")
    m.pd_kv_append(plan, ws, pool, k_new, v_new)
    m.pd_attention_run(plan, ws, q, pool, out, lse)
    torch.cuda.synchronize()
    print("ran append + attention", flush=True)

    kn = k_new.view(torch.int16).cpu().numpy().view(np.uint16)
    vn = v_new.view(torch.int16).cpu().numpy().view(np.uint16)
    qh = q.view(torch.int16).cpu().numpy().view(np.uint16)
    g = b.H_q // b.H_kv
    worst = 0.0
    for r in SAMPLE_REQUESTS:
        qo, kv = int(b.qo_lens[r]), int(b.kv_lens[r])
        q0 = int(b.qo_indptr[r])
        ids = b.request_pages(r)
        # append: the oracle's page writer on the pre-append copy, bit-exact
        local_indptr = np.array([0, len(ids)], np.int32)
        local_ids = np.arange(len(ids), dtype=np.int32)
        ref_pages = OP.kv_append(before[r].copy(), [qo], [kv], local_indptr, local_ids,
                                 kn[q0:q0 + qo], vn[q0:q0 + qo])
        assert pages_host(pool, ids).tobytes() == ref_pages.tobytes(), f"append request {r}"
        # logical K/V for the oracle: cached prefix (device draw) + new rows
        toks = [t for t in (PREFILL_TOKENS if qo > 1 else (0,)) if t < qo]
        pos = np.array([kv - qo + t for t in toks])
        for hk in range(b.H_kv):
            k_log = ref_pages[:, 0, hk].reshape(-1, b.D)[:kv]
            v_log = ref_pages[:, 1, hk].reshape(-1, b.D)[:kv]
            qr = bits_to_f64(qh[[q0 + t for t in toks]][:, hk * g:(hk + 1) * g])
            O, L = OA.attend(qr, bits_to_f64(k_log)[:, None, :], bits_to_f64(v_log)[:, None, :],
                             pos, b.sm_scale, True)
            got = out[[q0 + t for t in toks]][:, hk * g:(hk + 1) * g].cpu().numpy()
            got_l = lse[[q0 + t for t in toks]][:, hk * g:(hk + 1) * g].cpu().numpy()
            err = float(np.abs(got - O).max())
            worst = max(worst, err)
            assert err <= 2e-2, f"request {r} kv head {hk}: {err}"
            assert float(np.abs(got_l - L).max()) <= 5e-3
    print(f"long: worst sampled max_abs_err={worst:.3e}", flush=True)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()

    # pack the chunk request's 512 pages (128 MiB) and unpack them elsewhere
    ids = b.request_pages(0)
    nb = m.pd_kv_pack_bytes(desc, len(ids))
    assert nb == 128 * 2 ** 20
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
    scratch = torch.empty(4 * len(ids), dtype=torch.uint8, device="cuda")
    m.pd_kv_pack(desc, pool, b.num_pool_pages, ids, buf, scratch)
    torch.cuda.synchronize()
    assert buf.cpu().numpy().tobytes() == pages_host(pool, ids).tobytes()
    dst = np.random.default_rng(9).permutation(b.spare_pages)[:len(ids)].astype(np.int32)
    m.pd_kv_unpack(desc, pool, b.num_pool_pages, dst, buf, scratch)
    torch.cuda.synchronize()
    assert pages_host(pool, dst).tobytes() == buf.cpu().numpy().tobytes()
