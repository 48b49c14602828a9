"""Pins of the page-level oracle (append / gather / pack / unpack) and of the
transfer-size arithmetic, CPU only."""
import json
import os

import numpy as np
import pytest

from oracle import paged_kv as P
from workloads import make_batch, nan_pool, BF16_NAN

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pack_bytes_matches_survey_transfer_example():
    """kwkr.cn survey, section 5.1: 2048 tokens of OPT-175B KV at 4.5 MB per
    token over 8 x 64 GB/s links take about 17.6 ms."""
    g = json.load(open(os.path.join(GOLDEN, "kv_transfer_opt175b.json")))
    m, pr = g["model"], g["printed"]
    ps = 16
    pages = pr["tokens"] // ps
    per_layer = P.pack_bytes(pages, m["kv_heads"], ps, m["head_dim"], m["elt_bytes"])
    total = per_layer * m["layers"]
    assert total / pr["tokens"] == pr["mb_per_token"] * 2 ** 20
    t_ms = total / (pr["links"] * pr["gb_per_s_per_link"] * 2 ** 30) * 1e3
    assert round(t_ms, 1) == pr["latency_ms"]


def test_pack_bytes_closed_form():
    assert P.pack_bytes(7, 2, 16, 64, 4) == 114688          # the tiny workload
    assert P.pack_bytes(512, 8, 64, 128, 2) == 128 * 2 ** 20  # 32768 tokens, 8 heads


def test_hnd_page_and_head_slices_are_contiguous():
    """Each page is one contiguous image and each head's K (or V) slice of a
    page is one contiguous run, in the C-ordered pool."""
    b = make_batch("tiny", materialize=False)
    pool = np.zeros(b.pool_shape, np.float32)
    idx = np.arange(pool.size).reshape(pool.shape)
    page_elems = 2 * b.H_kv * b.ps * b.D
    for p in (0, 3):
        flat = idx[p].ravel()
        assert flat[0] == p * page_elems and np.all(np.diff(flat) == 1)
        for kvh in range(2):
            for h in range(b.H_kv):
                s = idx[p, kvh, h].ravel()
                assert np.all(np.diff(s) == 1) and s.size == b.ps * b.D


@pytest.mark.parametrize("wid,lengths", [
    ("tiny", None),
    ("tiny", ([1, 16, 17, 3, 0], [1, 16, 40, 33, 5])),
    ("mixed", ([9, 1, 1], [9, 17, 64])),
])
def test_append_then_gather_roundtrip(wid, lengths):
    b = make_batch(wid, lengths=lengths)
    pool = nan_pool(b)
    for r in range(b.B):
        kv, qo = int(b.kv_lens[r]), int(b.qo_lens[r])
        s = int(b.kv_indptr[r])
        P.write_prefix(pool, b.page_indptr, b.page_indices, r,
                       b.k[s:s + kv - qo], b.v[s:s + kv - qo])
    P.kv_append(pool, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices,
                b.k_new, b.v_new)
    for r in range(b.B):
        kv = int(b.kv_lens[r])
        s = int(b.kv_indptr[r])
        k, v = P.gather(pool, b.page_indptr, b.page_indices, r, kv)
        assert k.tobytes() == b.k[s:s + kv].tobytes()
        assert v.tobytes() == b.v[s:s + kv].tobytes()
    # spare pages and tail slots stay NaN
    nanbits = pool.view(np.uint16 if b.dtype == "bf16" else np.uint32)
    for p in b.spare_pages:
        if b.dtype == "bf16":
            assert np.all(pool[p] == BF16_NAN)
        else:
            assert np.all(np.isnan(pool[p]))
    for r in range(b.B):
        kv = int(b.kv_lens[r])
        if kv % b.ps:
            last = b.request_pages(r)[-1]
            tail = pool[last, :, :, kv % b.ps:, :]
            assert np.all(np.isnan(tail.astype(np.float32))) if b.dtype == "f32" else np.all(tail == BF16_NAN)
    del nanbits


def test_append_only_touches_new_positions():
    b = make_batch("tiny")
    pool = nan_pool(b)
    before = pool.copy()
    P.kv_append(pool, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.k_new, b.v_new)
    changed = np.argwhere(~np.isnan(pool[..., 0]))     # (page, kv, head, slot)
    expect = set()
    for r in range(b.B):
        kv, qo = int(b.kv_lens[r]), int(b.qo_lens[r])
        for t in range(kv - qo, kv):
            page, slot = P.token_slot(b.page_indptr, b.page_indices, b.ps, r, t)
            for kvh in range(2):
                for h in range(b.H_kv):
                    expect.add((page, kvh, h, slot))
    assert set(map(tuple, changed.tolist())) == expect
    assert np.isnan(before).all()


def test_pack_unpack_identity_and_relocation():
    b = make_batch("tiny")
    rng = np.random.default_rng(3)
    pool = rng.standard_normal(b.pool_shape).astype(np.float32)
    ids = b.request_pages(1)
    buf = P.kv_pack(pool, ids)
    assert buf.nbytes == P.pack_bytes(len(ids), b.H_kv, b.ps, b.D, 4)
    # buffer is the page images in list order
    assert buf.tobytes() == b"".join(pool[p].tobytes() for p in ids)
    # unpack into other pages, then pack them again: same bytes
    dst = b.spare_pages[:1].tolist() + b.request_pages(0).tolist() + b.request_pages(2).tolist()[:2]
    dst = np.asarray(dst[:len(ids)], np.int32)
    pool2 = np.full_like(pool, np.nan)
    P.kv_unpack(pool2, dst, buf)
    assert P.kv_pack(pool2, dst).tobytes() == buf.tobytes()
    # pages not in the destination list are untouched
    others = sorted(set(range(b.num_pool_pages)) - set(dst.tolist()))
    assert np.isnan(pool2[others]).all()
