"""Host side of the latent-cache (MLA) path: argument checks, the planner's
work list and figures, and the rejections that happen before any device work
(CPU only; needs the built library, no GPU)."""
import numpy as np
import pytest

import decode_attention_kv_pd_amd as pd
from tests.test_host_abi import FakeTensor, expect
from workloads import make_mla_batch


def mdesc(**kw):
    base = dict(num_qo_heads=16, page_size=16)
    base.update(kw)
    return pd.make_mla_desc(**base)


def plan_of(b, **kw):
    d = pd.make_mla_desc(b.H, b.ps, b.causal, b.sm_scale)
    return pd.pd_mla_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages, **kw)


def test_page_bytes_formula():
    assert pd.pd_mla_page_bytes(mdesc(page_size=64)) == 64 * 576 * 2
    assert pd.pd_mla_page_bytes(mdesc(page_size=16)) == 16 * 576 * 2


@pytest.mark.parametrize("kw,status", [
    (dict(kv_lora_rank=256), "PD_ERR_UNSUPPORTED"),
    (dict(qk_rope_dim=32), "PD_ERR_UNSUPPORTED"),
    (dict(num_qo_heads=8), "PD_ERR_UNSUPPORTED"),
    (dict(num_qo_heads=24), "PD_ERR_UNSUPPORTED"),
    (dict(num_qo_heads=144), "PD_ERR_UNSUPPORTED"),
    (dict(page_size=8), "PD_ERR_UNSUPPORTED"),
    (dict(sm_scale=0.0), "PD_ERR_INVALID_ARG"),
    (dict(sm_scale=float("nan")), "PD_ERR_INVALID_ARG"),
])
def test_plan_rejects_bad_desc(kw, status):
    expect(status, pd.pd_mla_plan, mdesc(**kw), [1], [5], [0, 1], [0], 2)


def test_plan_rejects_bad_dtype_and_causal():
    d = mdesc()
    d.dtype = pd.PD_F32
    expect("PD_ERR_UNSUPPORTED", pd.pd_mla_plan, d, [1], [5], [0, 1], [0], 2)
    d = mdesc()
    d.causal = 2
    expect("PD_ERR_INVALID_ARG", pd.pd_mla_plan, d, [1], [5], [0, 1], [0], 2)


def test_plan_rejects_bad_batches():
    d = mdesc()
    expect("PD_ERR_INVALID_ARG", pd.pd_mla_plan, d, [3], [2], [0, 1], [0], 4)          # qo > kv
    expect("PD_ERR_INVALID_ARG", pd.pd_mla_plan, d, [1], [40], [0, 2], [0, 1], 4)      # 3 pages needed
    expect("PD_ERR_INVALID_ARG", pd.pd_mla_plan, d, [1, 1], [5, 5], [0, 1, 2], [1, 1], 4)  # duplicate id
    expect("PD_ERR_OUT_OF_RANGE", pd.pd_mla_plan, d, [1], [5], [0, 1], [9], 4)         # outside the pool
    expect("PD_ERR_INVALID_ARG", pd.pd_mla_plan, d, [-1], [5], [0, 1], [0], 4)


def rows_per_block(H):
    """Query rows per block: 8 wavefronts of 16 rows at 128 heads, else 4."""
    return 128 if H >= 128 else 64


def check_cover(b, plan):
    """Every (request, row group) has its keys [0, kv) covered exactly once
    by its blocks; split groups use distinct partial slots that their merge
    group lists in chunk order, unsplit groups write straight to out."""
    items, mg = plan.work_items(1), plan.work_items(2)
    H, R = b.H, rows_per_block(b.H)
    groups = {}
    for req, rg, k0, k1, part, *_ in items.tolist():
        groups.setdefault((req, rg), []).append((k0, k1, part))
    want = {(r, g) for r in range(b.B) for g in range(-(-int(b.qo_lens[r]) * H // R))}
    assert set(groups) == want
    mgs = {(r, g): (p0, n) for r, g, p0, n in mg.tolist()}
    used = set()
    for (r, g), chunks in groups.items():
        chunks.sort()
        kv = int(b.kv_lens[r])
        assert chunks[0][0] == 0 and chunks[-1][1] == kv
        assert all(chunks[i][1] == chunks[i + 1][0] for i in range(len(chunks) - 1))
        assert all(k0 % 32 == 0 for k0, _, _ in chunks)
        if len(chunks) == 1:
            assert chunks[0][2] == -1 and (r, g) not in mgs
        else:
            p0, n = mgs[(r, g)]
            assert n == len(chunks)
            assert [c[2] for c in chunks] == list(range(p0, p0 + n))
            used.update(range(p0, p0 + n))
    assert len(used) == sum(n for _, n in mgs.values())


@pytest.mark.parametrize("wid,kw", [
    ("mla_tiny", {}),
    ("mla_tp8", {}),
    ("mla_dp", {}),
    ("mla_tiny", dict(lengths=([1, 2, 0, 4, 1], [1, 77, 5, 4, 3000]), heads=48)),
    ("mla_tiny", dict(lengths=([2, 1], [2000, 33]), heads=128, page_size=128)),
])
def test_planner_covers_batch(wid, kw):
    b = make_mla_batch(wid, materialize=False, **kw)
    check_cover(b, plan_of(b))
    for chunk in (32, 100, 1024):
        check_cover(b, plan_of(b, decode_chunk_keys=chunk))


def test_plan_figures():
    b = make_mla_batch("mla_dp", materialize=False)
    p = plan_of(b)
    s = p.stats()
    assert s.decode_kv_bytes == int(b.kv_lens.astype(np.int64).sum()) * 576 * 2
    assert s.decode_row_groups == b.B and s.prefill_tiles == 0   # 128 heads: one 128-row group
    assert s.decode_units == len(p.work_items(1))
    n_parts = int(p.work_items(2)[:, 3].sum())
    assert p.workspace_bytes >= n_parts * 128 * (512 + 1) * 4


def test_blocks_of_one_key_chunk_share_an_xcd():
    """With two new tokens of 128 heads (two 128-row groups) each key chunk
    of a request is read by two blocks; in a balanced batch they sit one
    dispatch round apart on the same XCD (block i runs on XCD i % 8)."""
    b = make_mla_batch("mla_dp", materialize=False, lengths=([2] * 64, [4096] * 64))
    items = plan_of(b, decode_chunk_keys=1024).work_items(1)
    pos = {}
    for i, (req, rg, k0, *_rest) in enumerate(items.tolist()):
        pos.setdefault((req, k0), []).append(i)
    assert all(len(v) == 2 for v in pos.values())
    assert all(v[0] % 8 == v[1] % 8 and v[1] - v[0] == 8 for v in pos.values())


def test_calls_reject_the_other_kind_of_plan():
    b = make_mla_batch("mla_tiny", materialize=False)
    mp = plan_of(b)
    dp = pd.pd_plan(pd.make_desc(4, 2, 64, 16, "f32"), [1], [5], [0, 1], [0], 2)
    ws, t = FakeTensor(1 << 20), FakeTensor(1 << 20, ptr=0x2000)
    expect("PD_ERR_INVALID_ARG", pd.pd_attention_run, mp, ws, t, t, t, stream=0)
    expect("PD_ERR_INVALID_ARG", pd.pd_kv_append, mp, ws, t, t, t, stream=0)
    expect("PD_ERR_INVALID_ARG", pd.pd_mla_attention_run, dp, ws, t, t, t, stream=0)
    expect("PD_ERR_INVALID_ARG", pd.pd_mla_kv_append, dp, ws, t, t, stream=0)


def test_pack_unpack_reject_bad_lists_before_device_work():
    d = mdesc()
    pb = pd.pd_mla_page_bytes(d)
    pool, buf, scr = FakeTensor(10 * pb), FakeTensor(2 * pb), FakeTensor(8)
    for fn in (pd.pd_mla_kv_pack, pd.pd_mla_kv_unpack):
        expect("PD_ERR_OUT_OF_RANGE", fn, d, pool, 10, [0, 10], buf, scr, stream=0)
        expect("PD_ERR_INVALID_ARG", fn, d, pool, 10, [3, 3], buf, scr, stream=0)
        expect("PD_ERR_WORKSPACE", fn, d, pool, 10, [1, 2, 3], FakeTensor(3 * pb), scr, stream=0)
        expect("PD_ERR_WORKSPACE", fn, d, pool, 10, [1, 2], FakeTensor(pb), scr, stream=0)
        expect("PD_ERR_UNSUPPORTED", fn, mdesc(kv_lora_rank=128), pool, 10, [1], buf, scr, stream=0)


def test_chunk_length_fills_one_dispatch_round():
    """At 64 requests x U{1024..8192} keys the planner's chunk length gives
    at most one block per CU (one dispatch round) while still splitting the
    long requests; asking for fewer CUs gives longer chunks."""
    for wid in ("mla_tp8", "mla_dp"):
        b = make_mla_batch(wid, materialize=False)
        p = plan_of(b)
        s = p.stats()
        assert 128 < s.decode_units <= 256
        assert s.decode_chunk_keys < int(b.kv_lens.max())
        q = plan_of(b, num_cus=64)
        assert q.stats().decode_chunk_keys > s.decode_chunk_keys
        check_cover(b, q)


@pytest.mark.parametrize("chunk", [2_147_483_647, 2_147_483_000, 1 << 30, 33])
def test_decode_chunk_option_near_int32_max_still_covers_every_row(chunk):
    """The latent planner clamps a huge decode_chunk_keys instead of wrapping
    it: every (request, row group) still has blocks covering [0, kv)."""
    for wid, kw in (("mla_tiny", {}), ("mla_tiny", dict(lengths=([2, 1], [2000, 33]), heads=128,
                                                         page_size=128))):
        b = make_mla_batch(wid, materialize=False, **kw)
        check_cover(b, plan_of(b, decode_chunk_keys=chunk))
