"""Page-level KV-cache operations on a numpy pool -- test infrastructure.

Pool layout ("HND" pages): one pool per layer, shaped
``[num_pages, 2, H_kv, page_size, D]``: for each page, the K half then the V
half; inside each half, head-major, then token slot, then head_dim.  So

  * a whole page is one contiguous image (one write moves a page), and
  * each KV head's slice of a page is contiguous (a head shard of a page is
    one write too).

This is the Perplexity post's HND layout (section "Sharded KV Cache
Transfers": heads placed before tokens so that a page copies with a single
write, unlike NHD which interleaves heads inside each token).  Token t of
request r lives in page ``page_indices[page_indptr[r] + t // page_size]`` at
slot ``t % page_size``.

The operations:
  kv_append   write each request's qo new tokens at positions [kv - qo, kv)
              -- KV entries are appended to the cache before attention reads
              them (post, section "KV Messenger")
  gather      read a request's logical K/V back out of its pages
  kv_pack     copy whole pages, in list order, into one contiguous buffer
              -- transfers move whole pages and their count is proportional
              to the pages sent (post, sections "KV Messenger" and "Sharded
              KV Cache Transfers"); a whole request at once is the
              request-level granularity of the kwkr.cn survey, section 5.4
  kv_unpack   copy the buffer's page images into (possibly different)
              destination pages -- the decoder allocates its own pages
              (post, section "KV Messenger")
  pack_bytes  size of a packed buffer

Sharded transfers (post, section "Sharded KV Cache Transfers"): when the
prefiller and the decoder split the KV heads over different numbers of
tensor-parallel ranks, a page is split or rebuilt by moving head ranges of it.
  kv_pack_heads / kv_unpack_heads   the same copies restricted to KV heads
              [h0, h1) of each page (K slice then V slice of each page)
  shard_heads, shard_transfers      which head range of a page goes from
              which source rank to which destination rank; a destination page
              expects one write per transfer that targets its rank
  kv_pack_layers / kv_unpack_layers the copies for several layers' pools at
              once, layer after layer -- transfers of a layer may start as
              soon as that layer's KV has been appended (post, section "KV
              Messenger")

All copies are exact: the arrays are moved as stored (fp32 values or bf16 bit
patterns), never converted.
"""
from __future__ import annotations

import numpy as np


def pack_bytes(n_pages: int, H_kv: int, page_size: int, head_dim: int,
               elt_bytes: int) -> int:
    """Bytes of ``n_pages`` page images: n * 2 (K and V) * H_kv * ps * D * elt."""
    return int(n_pages) * 2 * int(H_kv) * int(page_size) * int(head_dim) * int(elt_bytes)


def token_slot(page_indptr, page_indices, page_size, r, t):
    """(page id, slot) holding token t of request r."""
    page = int(page_indices[int(page_indptr[r]) + t // page_size])
    return page, t % page_size


def kv_append(pool, qo_lens, kv_lens, page_indptr, page_indices, k_new, v_new):
    """Write the new tokens of every request into the pool (in place).

    k_new, v_new: [sum qo, H_kv, D], request after request, each request's
    rows in token order; request r's rows go to positions kv_r - qo_r + i."""
    ps = pool.shape[3]
    row = 0
    for r in range(len(qo_lens)):
        qo, kv = int(qo_lens[r]), int(kv_lens[r])
        for i in range(qo):
            page, slot = token_slot(page_indptr, page_indices, ps, r, kv - qo + i)
            pool[page, 0, :, slot, :] = k_new[row]
            pool[page, 1, :, slot, :] = v_new[row]
            row += 1
    return pool


def write_prefix(pool, page_indptr, page_indices, r, k_rows, v_rows):
    """Place tokens [0, n) of request r (used to fill a cache before a step)."""
    ps = pool.shape[3]
    for t in range(k_rows.shape[0]):
        page, slot = token_slot(page_indptr, page_indices, ps, r, t)
        pool[page, 0, :, slot, :] = k_rows[t]
        pool[page, 1, :, slot, :] = v_rows[t]
    return pool


def gather(pool, page_indptr, page_indices, r, kv):
    """Logical K, V [kv, H_kv, D] of request r, read token by token."""
    ps = pool.shape[3]
    H_kv, D = pool.shape[2], pool.shape[4]
    k = np.empty((kv, H_kv, D), pool.dtype)
    v = np.empty((kv, H_kv, D), pool.dtype)
    for t in range(kv):
        page, slot = token_slot(page_indptr, page_indices, ps, r, t)
        k[t] = pool[page, 0, :, slot, :]
        v[t] = pool[page, 1, :, slot, :]
    return k, v


def kv_pack(pool, page_ids):
    """Contiguous buffer of the listed pages' images, in list order."""
    out = np.empty((len(page_ids),) + pool.shape[1:], pool.dtype)
    for i, p in enumerate(page_ids):
        out[i] = pool[int(p)]
    return out


def kv_unpack(pool, page_ids, buf):
    """Write buffer page i into pool page ``page_ids[i]`` (in place)."""
    for i, p in enumerate(page_ids):
        pool[int(p)] = buf[i]
    return pool


def pack_heads_bytes(n_pages: int, h0: int, h1: int, page_size: int, head_dim: int,
                     elt_bytes: int) -> int:
    """Bytes of the head-[h0, h1) slices of ``n_pages`` pages (K and V)."""
    return pack_bytes(n_pages, h1 - h0, page_size, head_dim, elt_bytes)


def kv_pack_heads(pool, page_ids, h0, h1):
    """Buffer [n, 2, h1 - h0, ps, D]: KV heads [h0, h1) of the listed pages."""
    out = np.empty((len(page_ids), 2, h1 - h0) + pool.shape[3:], pool.dtype)
    for i, p in enumerate(page_ids):
        for half in range(2):
            for j, h in enumerate(range(h0, h1)):
                out[i, half, j] = pool[int(p), half, h]
    return out


def kv_unpack_heads(pool, page_ids, h0, h1, buf):
    """Write buffer page i into KV heads [h0, h1) of pool page ``page_ids[i]``
    (in place); the other heads of the page are left as they are."""
    for i, p in enumerate(page_ids):
        for half in range(2):
            for j, h in enumerate(range(h0, h1)):
                pool[int(p), half, h] = buf[i, half, j]
    return pool


def kv_pack_layers(pools, page_ids, h0, h1):
    """Buffer [L, n, 2, h1 - h0, ps, D]: layer after layer, the head slices of
    the listed pages of each layer's pool."""
    return np.stack([kv_pack_heads(pool, page_ids, h0, h1) for pool in pools])


def kv_unpack_layers(pools, page_ids, h0, h1, buf):
    """Inverse of kv_pack_layers, in place in every layer's pool."""
    for layer, pool in enumerate(pools):
        kv_unpack_heads(pool, page_ids, h0, h1, buf[layer])
    return pools


def shard_heads(H_kv: int, shards: int, rank: int) -> list:
    """KV heads held by ``rank`` when H_kv heads are split evenly and in order
    over ``shards`` tensor-parallel ranks (contiguous blocks of heads)."""
    if shards < 1 or H_kv % shards:
        raise ValueError("the shards must divide the KV heads")
    per = H_kv // shards
    return list(range(rank * per, (rank + 1) * per))


def shard_transfers(H_kv: int, src_shards: int, dst_shards: int) -> list:
    """Every (source rank, destination rank) pair whose heads overlap, with the
    overlap as local head ranges on both sides:
    (src_rank, dst_rank, src_h0, src_h1, dst_h0, dst_h1).  Found by
    intersecting the head sets; each overlap is a contiguous range."""
    out = []
    for s in range(src_shards):
        S = shard_heads(H_kv, src_shards, s)
        for d in range(dst_shards):
            Dh = shard_heads(H_kv, dst_shards, d)
            common = sorted(set(S) & set(Dh))
            if not common:
                continue
            assert common == list(range(common[0], common[-1] + 1))
            lo, hi = common[0], common[-1] + 1
            out.append((s, d, lo - S[0], hi - S[0], lo - Dh[0], hi - Dh[0]))
    return out


def reshard(src_pools, page_ids_src, dst_pools, page_ids_dst, H_kv):
    """Apply shard_transfers: for every transfer, pack the head slice on the
    source rank and unpack it into the destination rank's pages (in place)."""
    for s, d, a0, a1, b0, b1 in shard_transfers(H_kv, len(src_pools), len(dst_pools)):
        buf = kv_pack_heads(src_pools[s], page_ids_src, a0, a1)
        kv_unpack_heads(dst_pools[d], page_ids_dst, b0, b1, buf)
    return dst_pools
