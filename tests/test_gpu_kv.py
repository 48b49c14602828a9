"""GPU: KV append, pack and unpack are bit-exact against the oracle's page
operations (Perplexity, "Disaggregated prefill and decode", sections "KV
Messenger" and "Sharded KV Cache Transfers")."""
import functools

import numpy as np
import pytest
import torch

from oracle import paged_kv as OP
from tests.harness import DeviceRun, dev_array, host_array, pd
from workloads import make_batch

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def batch(wid, lengths=None, **kw):
    if lengths is not None:
        lengths = (list(lengths[0]), list(lengths[1]))
    return make_batch(wid, lengths=lengths, **kw)


CASES = [
    ("tiny", None, {}),
    ("decode", None, {}),
    ("prefill", None, {}),
    ("mixed", None, {}),
    ("mixed", ((1, 5, 2, 300, 0, 17, 64), (1, 100, 64, 300, 9, 1000, 64)), {}),
    ("long", ((3, 1, 70), (3, 200, 130)), dict(page_size=128)),
    ("tiny", ((7, 1), (50, 33)), dict(page_size=32, head_dim=128)),
    ("tiny", ((3, 2, 5, 0, 11), (10, 40, 70, 3, 11)), dict(heads=(12, 3))),   # 96 chunks per row
]


@pytest.mark.parametrize("wid,lengths,kw", CASES)
def test_append_bit_exact(wid, lengths, kw):
    b = batch(wid, lengths, **kw)
    print(f"append {wid} {lengths} {kw}", flush=True)
    run = DeviceRun(b)
    run.append()
    torch.cuda.synchronize()
    got = host_array(run.pool, b.np_dtype)
    ref = run.pool_host.copy()
    OP.kv_append(ref, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.k_new, b.v_new)
    assert got.tobytes() == ref.tobytes()


@pytest.mark.parametrize("wid,lengths,kw", CASES[:4] + [CASES[5]])
def test_pack_unpack_bit_exact(wid, lengths, kw):
    b = batch(wid, lengths, **kw)
    print(f"pack {wid} {lengths} {kw}", flush=True)
    m = pd()
    run = DeviceRun(b)
    run.append()
    # pack the first prefill-like request (most pages) and the whole tiny batch
    r = int(np.argmax(b.page_indptr[1:] - b.page_indptr[:-1]))
    ids = b.request_pages(r) if wid != "tiny" else b.page_indices
    n = len(ids)
    nbytes = m.pd_kv_pack_bytes(run.desc, n)
    assert nbytes == OP.pack_bytes(n, b.H_kv, b.ps, b.D, b.elt)
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    scratch = torch.empty(4 * n, dtype=torch.uint8, device="cuda")
    m.pd_kv_pack(run.desc, run.pool, b.num_pool_pages, ids, buf, scratch)
    torch.cuda.synchronize()
    pool_now = host_array(run.pool, b.np_dtype)
    ref = OP.kv_pack(pool_now, ids)
    assert buf.cpu().numpy().tobytes() == ref.tobytes()
    # unpack into a fresh NaN pool at different page ids (spares first)
    dst = np.concatenate([b.spare_pages, np.setdiff1d(np.arange(b.num_pool_pages), b.spare_pages)])[:n]
    dst = np.random.default_rng(5).permutation(dst).astype(np.int32)
    fresh = np.full_like(pool_now, np.nan) if b.dtype == "f32" else np.full_like(pool_now, 0x7FC0)
    pool2 = dev_array(fresh)
    m.pd_kv_unpack(run.desc, pool2, b.num_pool_pages, dst, buf, scratch)
    torch.cuda.synchronize()
    ref2 = OP.kv_unpack(fresh.copy(), dst, ref)
    got2 = host_array(pool2, b.np_dtype)
    assert got2.tobytes() == ref2.tobytes()
    # pack(unpack(buf)) == buf
    buf2 = torch.empty_like(buf)
    m.pd_kv_pack(run.desc, pool2, b.num_pool_pages, dst, buf2, scratch)
    torch.cuda.synchronize()
    assert torch.equal(buf, buf2)


def test_attention_reads_no_nan_from_poisoned_slots():
    """Spare pages and tail slots are NaN; outputs stay finite, and the
    attention launch leaves the pool untouched."""
    b = batch("mixed", ((1, 5, 2, 300, 0, 17, 64), (1, 100, 64, 300, 9, 1000, 64)))
    run = DeviceRun(b)
    run.append()
    torch.cuda.synchronize()
    before = run.pool.clone()
    run.attention()
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), run.pool.view(torch.int16))
    n = int(b.qo_indptr[-1])
    assert torch.isfinite(run.out[:n]).all() and torch.isfinite(run.lse[:n]).all()


@pytest.mark.parametrize("n", [896, 897, 1500])
def test_pack_unpack_long_id_lists(n):
    """Lists of up to 896 page ids travel in the kernel arguments, longer
    ones are staged to the scratch: both paths bit-exact (the scratch starts
    as garbage, so ids read from the wrong place would show)."""
    b = batch("mixed", None)
    print(f"pack {n} pages of the mixed batch", flush=True)
    m = pd()
    run = DeviceRun(b)
    run.append()
    assert len(b.page_indices) >= n
    ids = np.random.default_rng(n).permutation(b.page_indices)[:n].astype(np.int32)
    buf = torch.empty(m.pd_kv_pack_bytes(run.desc, n), dtype=torch.uint8, device="cuda")
    scratch = torch.full((4 * n,), 0xFF, dtype=torch.uint8, device="cuda")
    m.pd_kv_pack(run.desc, run.pool, b.num_pool_pages, ids, buf, scratch)
    torch.cuda.synchronize()
    pool_now = host_array(run.pool, b.np_dtype)
    ref = OP.kv_pack(pool_now, ids)
    assert buf.cpu().numpy().tobytes() == ref.tobytes()
    dst = np.random.default_rng(n + 1).permutation(b.num_pool_pages)[:n].astype(np.int32)
    fresh = np.full_like(pool_now, 0x7FC0)
    pool2 = dev_array(fresh)
    scratch.fill_(0xFF)
    m.pd_kv_unpack(run.desc, pool2, b.num_pool_pages, dst, buf, scratch)
    torch.cuda.synchronize()
    assert host_array(pool2, b.np_dtype).tobytes() == OP.kv_unpack(fresh.copy(), dst, ref).tobytes()
