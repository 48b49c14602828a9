"""C-ABI boundary on the CPU: the library loads, exports every entry point the
header declares, rejects bad input with the documented status before doing
any device work, and the planner's work list covers the batch exactly."""
import ctypes
import os
import re

import numpy as np
import pytest

import decode_attention_kv_pd_amd as pd
from workloads import make_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pd_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pd_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "pd_plan" in names and "pd_kv_unpack" in names
    for n in names:
        assert hasattr(pd._lib, n), n
    assert set(names) == set(pd.EXPORTS)


def test_version_and_status_strings():
    assert "gfx950" in pd.version()
    assert pd._lib.pd_status_string(0) == b"PD_OK"
    assert pd._lib.pd_status_string(-3) == b"PD_ERR_OUT_OF_RANGE"


def desc(**kw):
    base = dict(num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=16, dtype="f32")
    base.update(kw)
    return pd.make_desc(**base)


def plan_args(qo=(3, 1), kv=(20, 17), ps=16, pool=10):
    qo, kv = list(qo), list(kv)
    npg = [(k + ps - 1) // ps for k in kv]
    indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    ids = np.arange(indptr[-1], dtype=np.int32)
    return qo, kv, indptr, ids, pool


def expect(status, fn, *a, **kw):
    with pytest.raises(pd.PdError) as e:
        fn(*a, **kw)
    assert e.value.name == status, str(e.value)
    assert len(pd._lib.pd_last_error()) > 0


def test_plan_accepts_valid_batch():
    qo, kv, ip, ids, pool = plan_args()
    p = pd.pd_plan(desc(), qo, kv, ip, ids, pool)
    s = p.stats()
    assert s.total_q_rows == 4 and s.batch == 2
    assert p.workspace_bytes > 0


@pytest.mark.parametrize("kw,status", [
    (dict(num_kv_heads=3), "PD_ERR_INVALID_ARG"),     # 4 % 3 != 0
    (dict(head_dim=96), "PD_ERR_UNSUPPORTED"),
    (dict(page_size=8), "PD_ERR_UNSUPPORTED"),
    (dict(dtype=7), "PD_ERR_UNSUPPORTED"),
    (dict(num_qo_heads=0), "PD_ERR_INVALID_ARG"),
    (dict(num_qo_heads=512, num_kv_heads=1), "PD_ERR_UNSUPPORTED"),
])
def test_plan_rejects_bad_desc(kw, status):
    qo, kv, ip, ids, pool = plan_args()
    expect(status, pd.pd_plan, desc(**kw), qo, kv, ip, ids, pool)


def test_plan_rejects_bad_batches():
    qo, kv, ip, ids, pool = plan_args()
    d = desc()
    expect("PD_ERR_INVALID_ARG", pd.pd_plan, d, [21, 1], kv, ip, ids, pool)        # qo > kv
    expect("PD_ERR_INVALID_ARG", pd.pd_plan, d, [-1, 1], kv, ip, ids, pool)        # negative
    expect("PD_ERR_INVALID_ARG", pd.pd_plan, d, qo, [20, 33], ip, ids, pool)       # page count
    bad = ids.copy(); bad[2] = bad[0]
    expect("PD_ERR_INVALID_ARG", pd.pd_plan, d, qo, kv, ip, bad, pool)             # duplicate page
    bad = ids.copy(); bad[1] = pool
    expect("PD_ERR_OUT_OF_RANGE", pd.pd_plan, d, qo, kv, ip, bad, pool)            # outside pool
    bad = ids.copy(); bad[1] = -5
    expect("PD_ERR_OUT_OF_RANGE", pd.pd_plan, d, qo, kv, ip, bad, pool)
    expect("PD_ERR_INVALID_ARG", pd.pd_plan, d, [], [], [0], [], pool)             # empty batch
    ip2 = ip.copy(); ip2[0] = 1
    expect("PD_ERR_INVALID_ARG", pd.pd_plan, d, qo, kv, ip2, ids, pool)


def test_plan_allows_empty_and_no_op_requests():
    d = desc()
    p = pd.pd_plan(d, [0, 0, 1], [0, 5, 1], [0, 0, 1, 2], [3, 4], 5)
    s = p.stats()
    assert s.total_q_rows == 1 and s.decode_row_groups == 2


class FakeTensor:
    """Host stand-in with a device-looking pointer: only for calls that must
    fail in argument checking before any device work."""

    def __init__(self, nbytes, ptr=0x1000):
        self._n, self._p = nbytes, ptr
        self.is_cuda = True

    def is_contiguous(self):
        return True

    def numel(self):
        return self._n

    def element_size(self):
        return 1

    def data_ptr(self):
        return self._p


def test_pack_unpack_reject_bad_lists_before_device_work():
    d = desc()
    pb = pd.pd_kv_pack_bytes(d, 1)
    pool, buf, scr = FakeTensor(10 * pb), FakeTensor(2 * pb), FakeTensor(8)
    for fn in (pd.pd_kv_pack, pd.pd_kv_unpack):
        expect("PD_ERR_OUT_OF_RANGE", fn, d, pool, 10, [0, 10], buf, scr, stream=0)
        expect("PD_ERR_INVALID_ARG", fn, d, pool, 10, [3, 3], buf, scr, stream=0)
        expect("PD_ERR_WORKSPACE", fn, d, pool, 10, [1, 2, 3], FakeTensor(3 * pb), scr, stream=0)
        expect("PD_ERR_WORKSPACE", fn, d, pool, 10, [1, 2], FakeTensor(pb), scr, stream=0)
        expect("PD_ERR_UNSUPPORTED", fn, desc(head_dim=80), pool, 10, [1], buf, scr, stream=0)


def test_pack_heads_reject_bad_arguments_before_device_work():
    d = desc(num_qo_heads=8, num_kv_heads=8)
    sb = pd.pd_kv_pack_heads_bytes(d, 1, 2, 5)
    assert sb == 2 * 3 * 16 * 64 * 4
    pool, buf, scr = FakeTensor(10 * pd.pd_kv_pack_bytes(d, 1)), FakeTensor(2 * sb), FakeTensor(8)
    for fn in (pd.pd_kv_pack_heads, pd.pd_kv_unpack_heads):
        for (h0, h1) in [(-1, 2), (3, 3), (5, 4), (0, 9)]:
            expect("PD_ERR_INVALID_ARG", fn, d, pool, 10, [1], h0, h1, buf, scr, stream=0)
        expect("PD_ERR_OUT_OF_RANGE", fn, d, pool, 10, [0, 10], 2, 5, buf, scr, stream=0)
        expect("PD_ERR_INVALID_ARG", fn, d, pool, 10, [3, 3], 2, 5, buf, scr, stream=0)
        expect("PD_ERR_WORKSPACE", fn, d, pool, 10, [1, 2, 3], 2, 5, buf, scr, stream=0)
        expect("PD_ERR_WORKSPACE", fn, d, pool, 10, [1, 2], 2, 5, FakeTensor(sb), scr, stream=0)
        expect("PD_ERR_WORKSPACE", fn, d, pool, 10, [1, 2], 2, 5, buf, FakeTensor(7), stream=0)


def test_pack_heads_bytes_formula():
    d = desc(num_qo_heads=64, num_kv_heads=8, head_dim=128, page_size=64, dtype="bf16")
    assert pd.pd_kv_pack_heads_bytes(d, 512, 0, 8) == pd.pd_kv_pack_bytes(d, 512)
    assert pd.pd_kv_pack_heads_bytes(d, 512, 0, 4) == 64 * 2 ** 20
    assert pd.pd_kv_pack_heads_bytes(d, 3, 7, 8) == 3 * 2 * 64 * 128 * 2
    assert pd.pd_kv_pack_heads_bytes(d, 3, 4, 4) == 0
    assert pd.pd_kv_pack_heads_bytes(d, 3, 0, 9) == 0


@pytest.mark.parametrize("H,s,d", [(8, 1, 1), (8, 2, 2), (8, 4, 2), (8, 8, 1), (8, 2, 4), (8, 1, 8),
                                   (6, 2, 3), (6, 3, 2), (64, 8, 2), (1, 1, 1)])
def test_shard_transfers_match_oracle(H, s, d):
    from oracle import paged_kv as OP
    assert pd.pd_kv_shard_transfers(H, s, d) == OP.shard_transfers(H, s, d)


def test_shard_transfers_errors():
    expect("PD_ERR_UNSUPPORTED", pd.pd_kv_shard_transfers, 8, 3, 1)
    expect("PD_ERR_UNSUPPORTED", pd.pd_kv_shard_transfers, 8, 16, 8)   # replicated heads
    expect("PD_ERR_INVALID_ARG", pd.pd_kv_shard_transfers, 8, 0, 1)
    n = pd.ctypes.c_int32(-1)
    arr = (pd.pd_head_transfer * 1)()
    st = pd._lib.pd_kv_shard_transfers(8, 4, 2, arr, 1, pd.ctypes.byref(n))
    assert pd.STATUS[st] == "PD_ERR_WORKSPACE" and n.value == 4


def test_xfer_plan_sizes_and_errors():
    d = desc(num_qo_heads=8, num_kv_heads=8)
    pools = [0x10000, 0x20000, 0x30000]
    x = pd.pd_xfer_plan(d, pools, 10, [4, 1, 7], 2, 6)
    assert x.buffer_bytes == 3 * 3 * 2 * 4 * 16 * 64 * 4
    assert x.workspace_bytes >= 3 * 8 + 3 * 4 + 3 * 4
    full = pd.pd_xfer_plan(d, pools, 10, [4, 1, 7])
    assert full.buffer_bytes == 3 * pd.pd_kv_pack_bytes(d, 3)
    expect("PD_ERR_INVALID_ARG", pd.pd_xfer_plan, d, [], 10, [1])
    expect("PD_ERR_INVALID_ARG", pd.pd_xfer_plan, d, [0x1000, 0], 10, [1])
    expect("PD_ERR_INVALID_ARG", pd.pd_xfer_plan, d, pools, 10, [1], 3, 3)
    expect("PD_ERR_INVALID_ARG", pd.pd_xfer_plan, d, pools, 10, [1, 1])
    expect("PD_ERR_OUT_OF_RANGE", pd.pd_xfer_plan, d, pools, 10, [10])
    expect("PD_ERR_UNSUPPORTED", pd.pd_xfer_plan, desc(head_dim=80), pools, 10, [1])
    expect("PD_ERR_WORKSPACE", pd.pd_xfer_upload, x, FakeTensor(x.workspace_bytes - 1), stream=0)
    expect("PD_ERR_WORKSPACE", pd.pd_kv_pack_layers, x, FakeTensor(x.workspace_bytes),
           FakeTensor(x.buffer_bytes - 1), stream=0)
    expect("PD_ERR_WORKSPACE", pd.pd_kv_unpack_layers, x, FakeTensor(x.workspace_bytes),
           FakeTensor(x.buffer_bytes - 1), stream=0)


def test_upload_rejects_small_workspace():
    qo, kv, ip, ids, pool = plan_args()
    p = pd.pd_plan(desc(), qo, kv, ip, ids, pool)
    expect("PD_ERR_WORKSPACE", pd.pd_plan_upload, p, FakeTensor(p.workspace_bytes - 1), stream=0)


def test_pack_bytes_formula():
    assert pd.pd_kv_pack_bytes(desc(), 7) == 7 * 2 * 2 * 16 * 64 * 4
    assert pd.pd_kv_pack_bytes(desc(num_qo_heads=64, num_kv_heads=8, head_dim=128, page_size=64,
                                    dtype="bf16"), 512) == 128 * 2 ** 20
    assert pd.pd_kv_pack_bytes(desc(), -1) == 0


# ------------------------------------------------------------- planner cover
MAX_DECODE_ROWS = 64   # rows of a (request, KV head) that the decode role takes


def check_cover(b, plan):
    """Every (request, query head, row) is computed exactly once: prefill
    tiles see exactly their causal key range; a decode row group's chunks
    tile [0, kv), every chunk's units cover the group's rows once, each unit
    writes the partial slots the merge group reads; the queues hold every
    unit once, each queue one kind of unit, and the two halves of a 64-row
    group's chunk sit in adjacent wavefronts of one block."""
    g = b.H_q // b.H_kv
    pf, du, mg, dq = plan.work_items(0), plan.work_items(1), plan.work_items(2), plan.work_items(4)[:, 0]
    seen = {}
    for (r, hk, q0, nq, kv_end, *_rest) in pf:
        qo, kv = int(b.qo_lens[r]), int(b.kv_lens[r])
        assert qo * g > MAX_DECODE_ROWS
        assert nq * g <= 256 and 0 <= q0 and q0 + nq <= qo
        assert kv_end == (kv - qo + q0 + nq if b.causal else kv)
        for t in range(q0, q0 + nq):
            for h in range(hk * g, hk * g + g):
                seen[(r, h, t)] = seen.get((r, h, t), 0) + 1
    # queues
    assert dq[0] == 0 and dq[-1] == len(du) and (np.diff(dq) >= 0).all()
    for s in range(len(dq) - 1):
        q = du[dq[s]:dq[s + 1]]
        if len(q):
            assert len(set(q[:, 6].tolist())) == 1, "a queue mixes unit kinds"
    slot_of_unit = np.repeat(np.arange(len(dq) - 1), np.diff(dq))
    pos_in_queue = np.concatenate([np.arange(n) for n in np.diff(dq)]) if len(du) else np.zeros(0, int)
    units = {}
    used_slots = set()
    first_half = {(r, hk, k0, k1): i for i, (r, hk, k0, k1, _p, c0, _n, _z) in enumerate(du.tolist()) if c0 == 0}
    paired = [bool(dq[s] < dq[s + 1] and du[dq[s], 7] == 1) for s in range(len(dq) - 1)]
    assert paired == sorted(paired, reverse=True), "paired queues take the first slots"
    for s in range(len(dq) - 1):
        q = du[dq[s]:dq[s + 1]]
        if len(q) and q[0, 7] == 1 and q[0, 5] == 0:
            # a paired queue: the next slot (same block) runs the same units, rows 32..63
            q2 = du[dq[s + 1]:dq[s + 2]]
            assert s % 2 == 0 and len(q2) == len(q)
            assert (q2[:, :4] == q[:, :4]).all() and (q2[:, 5] == 32).all() and (q2[:, 7] == 1).all()
    for i, (r, hk, k0, k1, part, c0, ncg, pair) in enumerate(du.tolist()):
        qo, kv = int(b.qo_lens[r]), int(b.kv_lens[r])
        rows = qo * g
        assert 1 <= rows <= MAX_DECODE_ROWS
        assert k0 % 32 == 0 and 0 <= k0 < k1 <= kv
        assert ncg == (1 if rows <= 16 else 2) and c0 % 32 == 0 and c0 < rows
        assert pair == (1 if rows > 32 else 0)
        units.setdefault((r, hk), []).append((k0, k1, part, c0, ncg, i))
        for n in range(c0, min(rows, c0 + 16 * ncg)):
            assert part + n - c0 not in used_slots
            used_slots.add(part + n - c0)
        if c0 == 32:   # the second half of a 64-row group's chunk: next wavefront, same block, same position
            t = first_half[(r, hk, k0, k1)]
            assert slot_of_unit[i] == slot_of_unit[t] + 1 and slot_of_unit[t] % 2 == 0
            assert pos_in_queue[i] == pos_in_queue[t]
    groups = {}
    for (r, hk, p0, n) in mg.tolist():
        assert (r, hk) not in groups
        groups[(r, hk)] = (p0, n)
    assert set(groups) == set(units)
    for (r, hk), us in units.items():
        qo, kv = int(b.qo_lens[r]), int(b.kv_lens[r])
        rows = qo * g
        p0, n = groups[(r, hk)]
        chunks = sorted({(k0, k1) for k0, k1, *_ in us})
        assert len(chunks) == n
        assert chunks[0][0] == 0 and chunks[-1][1] == kv
        assert all(chunks[i][1] == chunks[i + 1][0] for i in range(n - 1))
        for ci, (k0, k1) in enumerate(chunks):
            covered = []
            for (a0, a1, part, c0, ncg, _i) in us:
                if (a0, a1) != (k0, k1):
                    continue
                assert part == p0 + ci * rows + c0
                covered += list(range(c0, min(rows, c0 + 16 * ncg)))
            assert sorted(covered) == list(range(rows))
        for t in range(qo):
            for h in range(hk * g, hk * g + g):
                seen[(r, h, t)] = seen.get((r, h, t), 0) + 1
    n_rows = sum(n * int(b.qo_lens[r]) * g for (r, hk), (p0, n) in groups.items())
    assert used_slots == set(range(n_rows))
    expect_keys = {(r, h, t) for r in range(b.B) for h in range(b.H_q) for t in range(int(b.qo_lens[r]))}
    assert set(seen) == expect_keys
    assert all(v == 1 for v in seen.values())


@pytest.mark.parametrize("wid,kw", [
    ("tiny", {}),
    ("decode", {}),
    ("prefill", {}),
    ("mixed", {}),
    ("long", {}),
    ("mixed", dict(lengths=([1, 5, 2, 300, 0, 17], [1, 100, 64, 300, 9, 1000]))),
    ("tiny", dict(lengths=([4, 16, 1], [4, 40, 1]), heads=(8, 2))),
    ("tiny", dict(lengths=([33, 3], [33, 70]), causal=False)),
    ("long", dict(lengths=([1, 3, 9], [5000, 64, 9]), heads=(24, 8))),
    ("long", dict(lengths=([1, 1, 2, 4, 8, 9, 1], [20000, 33, 700, 4000, 64, 900, 17000]), heads=(64, 8))),
    ("long", dict(lengths=([1, 1, 1], [17000, 40, 1200]), heads=(64, 1))),
    ("long", dict(lengths=([1, 1, 2], [17000, 40, 1200]), heads=(32, 1))),
    ("mixed", dict(lengths=([1, 300, 1, 4, 1], [5000, 800, 70, 3000, 1]), heads=(32, 2))),
])
def test_planner_covers_batch(wid, kw):
    b = make_batch(wid, materialize=False, **kw)
    d = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype, b.causal)
    plan = pd.pd_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages)
    check_cover(b, plan)
    big = int(b.kv_lens.astype(np.int64).sum()) > 1_000_000   # keep the per-unit Python check small
    for chunk in ((2048, 4096) if big else (32, 100, 4096)):
        plan = pd.pd_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages,
                          decode_chunk_keys=chunk)
        check_cover(b, plan)


def test_planner_work_figures_match_closed_forms():
    """prefill flops = 4 D H_q x visible pairs; decode bytes = K + V read."""
    # the tiny workload's 713,728 algorithmic prefill flops (pairs 136 + 561):
    assert 4 * 64 * 4 * (16 * 17 // 2 + 33 * 34 // 2) == 713_728
    # its 16-token request has 32 rows (g = 2), few enough for the decode role;
    # the plan counts the flops of the rows it gives to prefill tiles
    for wid, flops, dbytes in [("tiny", 4 * 64 * 4 * 561, (16 + 40) * 2 * 2 * 64 * 4),
                               ("prefill", 21_516_779_520, 0)]:
        b = make_batch(wid, materialize=False)
        d = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype)
        s = pd.pd_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages).stats()
        pairs = sum(q * (k - q) + q * (q + 1) // 2 for q, k in zip(b.qo_lens.tolist(), b.kv_lens.tolist())
                    if q * (b.H_q // b.H_kv) > MAX_DECODE_ROWS)
        assert s.prefill_flops == 4 * b.D * b.H_q * pairs
        assert s.prefill_flops == flops and s.decode_kv_bytes == dbytes
    b = make_batch("long", materialize=False)
    d = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype)
    s = pd.pd_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages).stats()
    assert s.prefill_flops == 7_696_715_612_160
    assert s.decode_kv_bytes == 256 * 32768 * 2 * 8 * 128 * 2


@pytest.mark.parametrize("order", [0, 1])
def test_block_map_covers_work_and_keeps_xcd_affinity(order):
    """Every prefill tile and decode block appears once in the launch order;
    block i runs on XCD i % 8, and all tiles of one (request, KV head) land
    on the same XCD (the long workload's 8 KV heads on 8 different XCDs)."""
    b = make_batch("long", materialize=False)
    d = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype)
    plan = pd.pd_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages,
                      block_order=order)
    pf, dq, bmap = plan.work_items(0), plan.work_items(4), plan.work_items(3)[:, 0]
    n_db = (len(dq) - 1 + 7) // 8   # eight decode queues (one per wavefront) per block
    assert sorted(bmap[bmap >= 0].tolist()) == list(range(len(pf)))
    assert sorted((-bmap[bmap < 0] - 1).tolist()) == list(range(n_db))
    xcd_of_head = {}
    for pos, v in enumerate(bmap):
        if v >= 0:
            xcd_of_head.setdefault(int(pf[v][1]), set()).add(pos % 8)
    assert all(len(v) == 1 for v in xcd_of_head.values())
    assert len({next(iter(v)) for v in xcd_of_head.values()}) == 8
    if order == 0:   # interleaved (default): decode blocks appear before the last prefill tile
        first_d = int(np.argmax(bmap < 0))
        assert first_d < len(pf)
    else:            # prefill tiles first
        assert (bmap[:len(pf)] >= 0).all()


def test_decode_chunks_of_mixed_launches():
    """Mixed launches: with a prefill tile per CU or more, decode groups are
    cut into chunks whose block of eight streams about as long as the mean
    prefill tile runs (the long workload: four chunks per group graded
    about 8192 keys, longest first, 1024 decode blocks), one chunk per
    queue, queues longest first; with fewer tiles the decode
    runs in one round of queues on the free CUs unless that round would
    outlast the longest tile (the mixed workload's 63 decodes on 128 CUs
    would: chunks), and a small decode batch beside a 128-token prompt keeps
    its one round (queues of several pieces)."""
    def plan_of(b):
        d = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype, b.causal)
        return pd.pd_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages)
    b = make_batch("long", materialize=False)
    p = plan_of(b)
    du, dq, bmap = p.work_items(1), p.work_items(4)[:, 0], p.work_items(3)[:, 0]
    n = du[:, 3] - du[:, 2]
    assert (np.diff(dq) == 1).all() and (bmap < 0).sum() == 1024
    assert len(set(n.tolist())) == 4 and (abs(n - 8192) <= 0.1 * 8192).all()
    assert (np.diff(n) <= 0).all()                                   # longest first
    for r, hk in {(int(a), int(c)) for a, c in du[:, :2]}:
        pieces = sorted(du[(du[:, 0] == r) & (du[:, 1] == hk), 2:4].tolist())
        assert len(pieces) == 4 and pieces[0][0] == 0 and pieces[-1][1] == int(b.kv_lens[r])
        assert [q[1] - q[0] for q in pieces] == sorted([q[1] - q[0] for q in pieces], reverse=True)
    check_cover(b, p)
    b = make_batch("mixed", materialize=False)
    p = plan_of(b)
    du, dq = p.work_items(1), p.work_items(4)[:, 0]
    assert (np.diff(dq) == 1).all() and (du[:, 3] - du[:, 2]).max() <= 512
    check_cover(b, p)
    b = make_batch("mixed", materialize=False, lengths=([128] + [1] * 32, [128] * 33))
    p = plan_of(b)
    dq = p.work_items(4)[:, 0]
    assert np.diff(dq).max() > 1
    check_cover(b, p)


def test_prefill_block_shape_for_short_prompts():
    """Prefill-only launches of short caches run 128-row tiles (4-wavefront
    blocks, two per CU); 8 keeps 256-row tiles; a launch with decode rows,
    or a cache past 4096 keys without the option, keeps 256-row tiles."""
    def plan_of(wid, **kw):
        lengths = kw.pop("lengths", None)
        b = make_batch(wid, materialize=False, lengths=lengths)
        d = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype, b.causal)
        return b, pd.pd_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages, **kw)
    b, p = plan_of("prefill")
    pf = p.work_items(0)
    assert len(pf) == 1280 and (pf[:, 3] <= 128).all()   # g = 1: 128 tokens per tile
    check_cover(b, p)
    b, p = plan_of("prefill", prefill_block_waves=8)
    assert len(p.work_items(0)) == 640
    check_cover(b, p)
    b, p = plan_of("prefill", lengths=([300, 600], [300, 5000]))
    assert (p.work_items(0)[:, 3] > 128).any()            # 5000 cached keys: 256-row tiles
    b, p = plan_of("prefill", lengths=([300, 600], [300, 5000]), prefill_block_waves=4)
    assert (p.work_items(0)[:, 3] <= 128).all()
    check_cover(b, p)
    b, p = plan_of("mixed", prefill_block_waves=4)         # decode rows in the launch
    assert (p.work_items(0)[:, 3] * 4 > 128).any()
    check_cover(b, p)
    with pytest.raises(pd.PdError):
        plan_of("prefill", prefill_block_waves=2)


@pytest.mark.parametrize("chunk", [2_147_483_647, 2_147_483_000, 2_147_483_616, 1 << 30, 40, 31])
def test_decode_chunk_option_near_int32_max_still_covers_every_row(chunk):
    """A decode_chunk_keys option near INT32_MAX is clamped, not wrapped: the
    plan still gives every decode row group at least one key chunk and the
    chunks tile [0, kv) exactly (no merge group without partial results)."""
    b = make_batch("mixed", materialize=False,
                   lengths=([1, 1, 4, 1, 300], [4096, 33, 1500, 1, 300]))
    d = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype, b.causal)
    plan = pd.pd_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages,
                      decode_chunk_keys=chunk)
    check_cover(b, plan)
    mg = plan.work_items(2)
    assert (mg[:, 3] >= 1).all()
    s = plan.stats()
    assert 32 <= s.decode_chunk_keys <= 4096 + 31


# ------------------------------------------------- the no-allocation call
def test_noalloc_rejects_before_any_device_work():
    """Checks that need no device: an oversized plan, an MLA plan and a lone
    k_new are refused with the documented status before anything runs."""
    b = make_batch("long", materialize=False)
    d = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype, b.causal)
    big = pd.pd_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages,
                     decode_chunk_keys=32)
    assert big.workspace_bytes > pd.NOALLOC_SCRATCH_BYTES
    expect("PD_ERR_WORKSPACE", pd.pd_attention_run_noalloc, big, None, None, None, stream=0)
    fits = pd.pd_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages)
    assert fits.workspace_bytes <= pd.NOALLOC_SCRATCH_BYTES   # the long workload fits
    st = pd._lib.pd_attention_run_noalloc(fits.handle, None, None, ctypes.c_void_p(256), None, None, None, None)
    assert pd.STATUS[st] == "PD_ERR_INVALID_ARG"
    from workloads import make_mla_batch
    m = make_mla_batch("mla_tiny", materialize=False)
    md = pd.make_mla_desc(m.H, m.ps, m.causal, m.sm_scale)
    mp = pd.pd_mla_plan(md, m.qo_lens, m.kv_lens, m.page_indptr, m.page_indices, m.num_pool_pages)
    expect("PD_ERR_INVALID_ARG", pd.pd_attention_run_noalloc, mp, None, None, None, stream=0)
    assert pd.STATUS[pd._lib.pd_attention_run_noalloc(None, None, None, None, None, None, None, None)] == \
        "PD_ERR_INVALID_ARG"


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define PD_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", text)
    assert m and int(m.group(1)) * 2 ** 20 == pd.NOALLOC_SCRATCH_BYTES
