"""GPU: head-range (sharded) and multi-layer transfers are bit-exact against
the oracle's page operations; the per-layer completion counters count once
per layer and call, also across HIP-graph replays (Perplexity, "Disaggregated
prefill and decode", sections "Sharded KV Cache Transfers" and "KV
Messenger")."""
import functools
import threading
import time

import numpy as np
import pytest
import torch

from oracle import paged_kv as OP
from tests.harness import desc_of, dev_array, host_array, pd, prefix_pool
from workloads import BF16_NAN, make_batch

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def batch(wid):
    return make_batch(wid)


@functools.lru_cache(maxsize=None)
def pool_of(wid):
    return prefix_pool(batch(wid))


def scratch_for(n):
    return torch.empty(max(4 * n, 4), dtype=torch.uint8, device="cuda")


def pool_bytes(t):
    return t.view(torch.uint8).cpu().numpy().tobytes()


@pytest.mark.parametrize("wid,h0,h1", [("tiny", 0, 2), ("tiny", 1, 2), ("mixed", 0, 8), ("mixed", 3, 7),
                                       ("mixed", 7, 8), ("prefill", 10, 31)])
def test_pack_unpack_heads_bit_exact(wid, h0, h1):
    b = batch(wid)
    print(f"pack_heads {wid} [{h0}, {h1})", flush=True)
    m = pd()
    d = desc_of(b)
    host = pool_of(wid)
    pool = dev_array(host)
    rng = np.random.default_rng(11)
    ids = rng.permutation(np.asarray(b.page_indices))[:min(40, len(b.page_indices))].astype(np.int32)
    n = len(ids)
    nbytes = m.pd_kv_pack_heads_bytes(d, n, h0, h1)
    assert nbytes == OP.pack_heads_bytes(n, h0, h1, b.ps, b.D, b.elt)
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    scr = scratch_for(n)
    m.pd_kv_pack_heads(d, pool, b.num_pool_pages, ids, h0, h1, buf, scr)
    torch.cuda.synchronize()
    want = OP.kv_pack_heads(host, ids, h0, h1)
    assert buf.cpu().numpy().tobytes() == want.tobytes()
    dst = rng.permutation(np.asarray(b.spare_pages))[:n].astype(np.int32)
    if len(dst) < n:   # small workloads: unpack over other live pages instead
        dst = rng.permutation(b.num_pool_pages)[:n].astype(np.int32)
    m.pd_kv_unpack_heads(d, pool, b.num_pool_pages, dst, h0, h1, buf, scr)
    torch.cuda.synchronize()
    ref = OP.kv_unpack_heads(host.copy(), dst, h0, h1, want)
    assert pool_bytes(pool) == ref.tobytes()


@pytest.mark.parametrize("s,dd", [(2, 4), (4, 2), (8, 1), (1, 8), (2, 2), (8, 8)])
def test_reshard_between_tp_degrees(s, dd):
    """Every destination rank's pool equals the oracle's rebuild: the library's
    transfer table, pack_heads on the sources, unpack_heads on the targets."""
    b = batch("mixed")
    print(f"reshard 8 heads {s} -> {dd}", flush=True)
    m = pd()
    H = b.H_kv
    full = pool_of("mixed")
    P = full.shape[0]
    rng = np.random.default_rng(s * 10 + dd)
    r = int(np.argmax(b.page_indptr[1:] - b.page_indptr[:-1]))
    ids_src = np.asarray(b.request_pages(r), np.int32)
    P2 = len(ids_src) + 13
    ids_dst = rng.permutation(P2)[:len(ids_src)].astype(np.int32)
    src_h = [np.ascontiguousarray(full[:, :, k * (H // s):(k + 1) * (H // s)]) for k in range(s)]
    dst_h = [np.full((P2, 2, H // dd, b.ps, b.D), BF16_NAN, np.uint16) for _ in range(dd)]
    src = [dev_array(a) for a in src_h]
    dst = [dev_array(a) for a in dst_h]
    n = len(ids_src)
    scr = scratch_for(n)
    table = m.pd_kv_shard_transfers(H, s, dd)
    assert table == OP.shard_transfers(H, s, dd)
    for (sr, dr, a0, a1, b0, b1) in table:
        ds = m.make_desc(b.H_q // s, H // s, b.D, b.ps, b.dtype)
        dt = m.make_desc(b.H_q // dd, H // dd, b.D, b.ps, b.dtype)
        buf = torch.empty(m.pd_kv_pack_heads_bytes(ds, n, a0, a1), dtype=torch.uint8, device="cuda")
        m.pd_kv_pack_heads(ds, src[sr], P, ids_src, a0, a1, buf, scr)
        m.pd_kv_unpack_heads(dt, dst[dr], P2, ids_dst, b0, b1, buf, scr)
    torch.cuda.synchronize()
    OP.reshard(src_h, ids_src, dst_h, ids_dst, H)
    for q in range(dd):
        assert pool_bytes(dst[q]) == dst_h[q].tobytes(), f"destination rank {q}"


def layer_pools(shape, L, seed, dtype=np.uint16):
    rng = np.random.default_rng(seed)
    if dtype == np.uint16:
        return [rng.integers(0, 1 << 16, size=shape, dtype=np.uint16) for _ in range(L)]
    return [rng.standard_normal(shape).astype(np.float32) for _ in range(L)]


@pytest.mark.parametrize("wid,L,h0,h1", [("mixed", 3, 0, 8), ("mixed", 5, 2, 6), ("tiny", 2, 1, 2)])
def test_pack_unpack_layers_bit_exact_with_progress(wid, L, h0, h1):
    b = batch(wid)
    print(f"pack_layers {wid} L={L} [{h0}, {h1})", flush=True)
    m = pd()
    d = desc_of(b)
    P = 64
    shape = (P, 2, b.H_kv, b.ps, b.D)
    pools_h = layer_pools(shape, L, 5, b.np_dtype)
    pools = [dev_array(a) for a in pools_h]
    rng = np.random.default_rng(6)
    ids = rng.permutation(P)[:37].astype(np.int32)
    x = m.pd_xfer_plan(d, pools, P, ids, h0, h1)
    assert x.buffer_bytes == L * OP.pack_heads_bytes(len(ids), h0, h1, b.ps, b.D, b.elt)
    ws = torch.empty(x.workspace_bytes, dtype=torch.uint8, device="cuda")
    m.pd_xfer_upload(x, ws)
    buf = torch.empty(x.buffer_bytes, dtype=torch.uint8, device="cuda")
    prog = torch.zeros(L, dtype=torch.int32, pin_memory=True)
    m.pd_kv_pack_layers(x, ws, buf, prog)
    torch.cuda.synchronize()
    want = OP.kv_pack_layers(pools_h, ids, h0, h1)
    assert buf.cpu().numpy().tobytes() == want.tobytes()
    assert prog.tolist() == [1] * L
    m.pd_kv_pack_layers(x, ws, buf, prog)          # counters keep counting
    m.pd_kv_pack_layers(x, ws, buf)                # no progress array
    torch.cuda.synchronize()
    assert prog.tolist() == [2] * L
    assert buf.cpu().numpy().tobytes() == want.tobytes()
    # unpack on a "receiver": other pools, other page ids, a device-memory counter
    dst_h = layer_pools(shape, L, 7, b.np_dtype)
    dst = [dev_array(a) for a in dst_h]
    ids_dst = rng.permutation(P)[:37].astype(np.int32)
    x2 = m.pd_xfer_plan(d, dst, P, ids_dst, h0, h1)
    ws2 = torch.empty(x2.workspace_bytes, dtype=torch.uint8, device="cuda")
    m.pd_xfer_upload(x2, ws2)
    dprog = torch.zeros(L, dtype=torch.int32, device="cuda")
    m.pd_kv_unpack_layers(x2, ws2, buf, dprog)
    torch.cuda.synchronize()
    OP.kv_unpack_layers(dst_h, ids_dst, h0, h1, want)
    for layer in range(L):
        assert pool_bytes(dst[layer]) == dst_h[layer].tobytes(), f"layer {layer}"
    assert dprog.cpu().tolist() == [1] * L


def test_pack_layers_in_graph_replays():
    """Captured once, replayed three times with eager changes of the pools in
    between: every replay packs the current pools and bumps each counter."""
    b = batch("mixed")
    m = pd()
    d = desc_of(b)
    L, P = 4, 48
    shape = (P, 2, b.H_kv, b.ps, b.D)
    pools_h = layer_pools(shape, L, 21)
    pools = [dev_array(a) for a in pools_h]
    ids = np.random.default_rng(22).permutation(P)[:29].astype(np.int32)
    x = m.pd_xfer_plan(d, pools, P, ids, 0, b.H_kv)
    ws = torch.empty(x.workspace_bytes, dtype=torch.uint8, device="cuda")
    m.pd_xfer_upload(x, ws)
    buf = torch.zeros(x.buffer_bytes, dtype=torch.uint8, device="cuda")
    prog = torch.zeros(L, dtype=torch.int32, pin_memory=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up launch outside the capture
        m.pd_kv_pack_layers(x, ws, buf, prog)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert prog.tolist() == [1] * L
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.pd_kv_pack_layers(x, ws, buf, prog)
    torch.cuda.synchronize()
    assert prog.tolist() == [1] * L   # capture does not run the kernel
    for rep in range(3):
        rng = np.random.default_rng(100 + rep)
        for layer in range(L):      # eager work between replays
            pools_h[layer] = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
            pools[layer].copy_(dev_array(pools_h[layer]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"replay {rep}: progress {prog.tolist()}", flush=True)
        assert prog.tolist() == [2 + rep] * L
        assert buf.cpu().numpy().tobytes() == OP.kv_pack_layers(pools_h, ids, 0, b.H_kv).tobytes()


def test_progress_is_polled_by_a_host_thread():
    """A host thread polling the pinned counters sees every layer finish; the
    values only ever grow and end at one per layer."""
    b = make_batch("long", materialize=False)
    m = pd()
    d = desc_of(b)
    L, P, n = 16, 160, 128
    pools = [torch.empty((P, 2, b.H_kv, b.ps, b.D), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    for layer, t in enumerate(pools):
        t.view(torch.int16).fill_(layer)
    ids = np.arange(n, dtype=np.int32)[::-1].copy()
    x = m.pd_xfer_plan(d, pools, P, ids)
    ws = torch.empty(x.workspace_bytes, dtype=torch.uint8, device="cuda")
    m.pd_xfer_upload(x, ws)
    buf = torch.empty(x.buffer_bytes, dtype=torch.uint8, device="cuda")
    prog = torch.zeros(L, dtype=torch.int32, pin_memory=True)
    view = prog.numpy()
    seen, stop = [], threading.Event()

    def poll():
        last = None
        while not stop.is_set():
            cur = tuple(int(v) for v in view)
            if cur != last:
                seen.append(cur)
                last = cur
            if sum(cur) == L:
                break
        stop.set()

    torch.cuda.synchronize()
    th = threading.Thread(target=poll)
    th.start()
    m.pd_kv_pack_layers(x, ws, buf, prog)
    torch.cuda.synchronize()
    th.join(timeout=10)
    stop.set()
    assert tuple(int(v) for v in view) == (1,) * L
    assert seen[-1] == (1,) * L
    for a, c in zip(seen, seen[1:]):
        assert all(u <= v for u, v in zip(a, c))
    print(f"poller saw {len(seen)} distinct states (intermediate: "
          f"{sum(0 < sum(s) < L for s in seen)})", flush=True)
    got = buf.view(torch.int16).view(L, -1)[:, ::4096].cpu().numpy()
    assert all((got[layer] == layer).all() for layer in range(L))
