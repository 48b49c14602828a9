"""Pins of the oracle's sharded (head-range) and multi-layer transfers, CPU only.

The post's section "Sharded KV Cache Transfers": when the prefiller splits the
KV heads over more tensor-parallel ranks than the decoder, the decoder's full
pages are rebuilt from the halves (more generally, the head ranges) sent by
several prefiller ranks; when the decoder has more ranks, each receives a part
of a source page; the decoder has to know the prefiller's split to count the
writes it waits for.  HND pages make every such head range of a page two
contiguous runs (its K part and its V part).

The pins: a rebuild of every destination rank's pages checked against plain
numpy head slicing of the unsharded pool, closed-form write counts, coverage
and disjointness of the ranges, the contiguity of a head slice in the pool's
flat order, and planted mistakes that the pins must catch.
"""
import os
import types

import numpy as np
import pytest

from oracle import paged_kv as P


def random_pool(rng, pages, H, ps=4, D=8):
    return rng.standard_normal((pages, 2, H, ps, D)).astype(np.float32)


def rebuild_ok(M, H, s, d, seed=0):
    """Shard an H-head pool over s source ranks, move it with M.reshard to d
    destination ranks (other page ids), compare with numpy head slicing."""
    rng = np.random.default_rng(seed)
    full = random_pool(rng, 12, H)
    ids_src = rng.permutation(12)[:7]
    ids_dst = rng.permutation(20)[:7]
    per_s, per_d = H // s, H // d
    src = [np.ascontiguousarray(full[:, :, r * per_s:(r + 1) * per_s]) for r in range(s)]
    dst = [np.full((20, 2, per_d, 4, 8), np.nan, np.float32) for _ in range(d)]
    M.reshard(src, ids_src, dst, ids_dst, H)
    for q in range(d):
        want = full[ids_src][:, :, q * per_d:(q + 1) * per_d]
        if not np.array_equal(dst[q][ids_dst], want):
            return False
        untouched = np.setdiff1d(np.arange(20), ids_dst)
        if not np.isnan(dst[q][untouched]).all():
            return False
    return True


SPLITS = [(8, 1, 1), (8, 2, 2), (8, 4, 2), (8, 8, 1), (8, 2, 4), (8, 1, 8), (8, 2, 8),
          (6, 2, 3), (6, 3, 2), (4, 4, 4)]


@pytest.mark.parametrize("H,s,d", SPLITS)
def test_reshard_rebuilds_every_destination_page(H, s, d):
    assert rebuild_ok(P, H, s, d)


@pytest.mark.parametrize("H,s,d", SPLITS)
def test_transfer_ranges_cover_each_rank_once(H, s, d):
    t = P.shard_transfers(H, s, d)
    for q in range(d):
        got = sorted(h for (_, dd, _, _, b0, b1) in t if dd == q for h in range(b0, b1))
        assert got == list(range(H // d))
    for r in range(s):
        got = sorted(h for (ss, _, a0, a1, _, _) in t if ss == r for h in range(a0, a1))
        assert got == list(range(H // s))
    assert sum(a1 - a0 for (_, _, a0, a1, _, _) in t) == H
    assert all(a1 - a0 == b1 - b0 > 0 for (_, _, a0, a1, b0, b1) in t)


@pytest.mark.parametrize("H,s,d", [c for c in SPLITS if c[1] % c[2] == 0 or c[2] % c[1] == 0])
def test_expected_writes_closed_form(H, s, d):
    """A destination page receives s / d writes when the prefiller has more
    ranks (each a 1/(s/d) share of the heads: the halves of the post for
    s = 2d), one write when the decoder has at least as many."""
    t = P.shard_transfers(H, s, d)
    want = s // d if s >= d else 1
    for q in range(d):
        writes = [x for x in t if x[1] == q]
        assert len(writes) == want
        assert all(x[5] - x[4] == (H // d) // want for x in writes)


def test_uneven_split_6_heads_2_to_3():
    """6 heads, 2 -> 3 ranks: rank 1 of the decoder takes one head from each
    source rank (two writes); ranks 0 and 2 take two heads from one source."""
    assert P.shard_transfers(6, 2, 3) == [(0, 0, 0, 2, 0, 2), (0, 1, 2, 3, 0, 1),
                                         (1, 1, 0, 1, 1, 2), (1, 2, 1, 3, 0, 2)]


def test_shards_must_divide_heads():
    with pytest.raises(ValueError):
        P.shard_transfers(8, 3, 1)


def test_head_slice_is_two_contiguous_runs_per_page():
    """In the C-ordered HND pool, heads [h0, h1) of a page are one run in the
    K half and one in the V half (the whole page when h0 = 0, h1 = H)."""
    pages, H, ps, D = 3, 8, 4, 8
    idx = np.arange(pages * 2 * H * ps * D).reshape(pages, 2, H, ps, D)
    for (h0, h1) in [(0, 8), (2, 5), (7, 8)]:
        flat = P.kv_pack_heads(idx, [1], h0, h1).reshape(-1)
        runs = 1 + int(np.count_nonzero(np.diff(flat) != 1))
        assert runs == (1 if (h0, h1) == (0, H) else 2)
        assert flat.size * 4 == P.pack_heads_bytes(1, h0, h1, ps, D, 4)


def test_pack_heads_of_all_heads_is_the_page_image():
    rng = np.random.default_rng(3)
    pool = random_pool(rng, 9, 4)
    ids = [5, 0, 7]
    assert np.array_equal(P.kv_pack_heads(pool, ids, 0, 4), P.kv_pack(pool, ids))


def test_unpack_heads_leaves_other_heads():
    rng = np.random.default_rng(4)
    pool = random_pool(rng, 6, 8)
    before = pool.copy()
    buf = rng.standard_normal((2, 2, 3, 4, 8)).astype(np.float32)
    P.kv_unpack_heads(pool, [4, 1], 2, 5, buf)
    assert np.array_equal(pool[[4, 1]][:, :, 2:5], buf)
    keep = np.ones(pool.shape, bool)
    keep[[4, 1], :, 2:5] = False
    assert np.array_equal(pool[keep], before[keep])


def test_layers_are_stacked_in_layer_order():
    rng = np.random.default_rng(5)
    pools = [random_pool(rng, 5, 4) for _ in range(3)]
    buf = P.kv_pack_layers(pools, [3, 1], 1, 3)
    assert buf.shape == (3, 2, 2, 2, 4, 8)
    for layer in range(3):
        assert np.array_equal(buf[layer], pools[layer][[3, 1]][:, :, 1:3])
    dst = [np.zeros_like(p) for p in pools]
    P.kv_unpack_layers(dst, [0, 4], 1, 3, buf)
    for layer in range(3):
        assert np.array_equal(dst[layer][[0, 4]][:, :, 1:3], pools[layer][[3, 1]][:, :, 1:3])


SRC = open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "paged_kv.py")).read()
MUTANTS = {
    "dst_range_not_rebased": ("lo - Dh[0], hi - Dh[0]", "lo, hi"),
    "src_range_not_rebased": ("lo - S[0], hi - S[0]", "lo, hi"),
    "heads_interleaved": ("return list(range(rank * per, (rank + 1) * per))",
                          "return list(range(rank, H_kv, shards))"),
    "v_half_from_k": ("out[i, half, j] = pool[int(p), half, h]", "out[i, half, j] = pool[int(p), 0, h]"),
    "unpack_heads_shifted": ("pool[int(p), half, h] = buf[i, half, j]", "pool[int(p), half, j] = buf[i, half, j]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_sharding_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1
    mod = types.ModuleType("paged_mutant")
    exec(compile(SRC.replace(old, new), "paged_mutant", "exec"), mod.__dict__)
    caught = False
    for (H, s, d) in SPLITS:
        try:
            if not rebuild_ok(mod, H, s, d):
                caught = True
        except (AssertionError, IndexError, ValueError):
            caught = True
    assert caught
