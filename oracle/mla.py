"""float64 reference for MLA (multi-head latent attention) decode over a
latent KV cache -- test infrastructure.  Only ``tests/``, the smoke check and
the benchmark's CPU baseline import it; the HIP path shares no code with it.

What the pages fix (Perplexity, "Disaggregated prefill and decode", section
"DeepSeek-R1" under "Disaggregated Deployments"): DeepSeek's MLA
compresses all KV heads of a token into a single latent vector, so tensor
parallelism cannot split the cache by heads.  Every rank holds the same
latent cache, and the heads are only separated after decompression.  The
pages give no dimensions and no formula.

Reading taken (the plainest one that matches the pages): the absorbed form of
MLA decode.  The up-projection of the keys is folded into the query, and the
up-projection of the values is applied after attention, outside this step.
Per cached token j the cache holds one row

    row_j = [ c_j (d_c latent entries) ; kr_j (d_r entries of the shared
              rotary key) ]

and a query row (token t, head h) brings q = [ qc (d_c) ; qr (d_r) ].  Then

    S_j   = scale * ( <qc, c_j> + <qr, kr_j> ) = scale * <q, row_j>
    O     = sum_j softmax(S)_j c_j                     (d_c entries)
    LSE   = m + ln sum_j exp(S_j - m),  m = max_j S_j

over the visible keys: j <= kv - qo + t when causal (the new tokens sit at
the end of the cache), else all kv keys.  So this is one-KV-head attention
whose key is the whole row and whose value is the row's first d_c entries.
The dimensions used by the workloads (d_c = 512, d_r = 64, 16 or 128 query
heads, scale 1 / sqrt(192)) are DeepSeek-V3's published configuration, not
the pages'.

The absorbed form is checked against the expanded multi-head form (per-head
keys W_UK c_j with the shared rotary key appended, per-head values W_UV c_j)
in ``tests/test_oracle_mla.py``.

Pool layout: ``[num_pages, page_size, d_c + d_r]``: one row per token slot,
so a page is one contiguous image, and every rank's copy is the same image.
Token t of request r lives in page ``page_indices[page_indptr[r] + t //
page_size]`` at slot ``t % page_size``.
"""
from __future__ import annotations

import math

import numpy as np

ROW_BLOCK = 256


def mla_attend(q, rows, positions, d_c, sm_scale, causal=True):
    """Absorbed MLA attention of query rows against one request's cache.

    q          [n, H, d_c + d_r] float64 query rows (absorbed latent part,
               then rotary part)
    rows       [kv, d_c + d_r]   float64 cache rows, position j at index j
    positions  [n] absolute positions of the query rows (kv - qo + t)
    Returns (O [n, H, d_c], LSE [n, H]) in float64.
    """
    q = np.asarray(q, np.float64)
    rows = np.asarray(rows, np.float64)
    positions = np.asarray(positions, np.int64)
    n, H, width = q.shape
    kv = rows.shape[0]
    if rows.shape[1] != width:
        raise ValueError("query and cache rows differ in width")
    values = rows[:, :d_c]
    O = np.empty((n, H, d_c), np.float64)
    L = np.empty((n, H), np.float64)
    key_pos = np.arange(kv)
    for i in range(n):
        visible = key_pos <= positions[i] if causal else np.ones(kv, bool)
        for h0 in range(0, H, ROW_BLOCK):
            h1 = min(H, h0 + ROW_BLOCK)
            S = sm_scale * (q[i, h0:h1, :] @ rows.T)          # [heads, kv]
            S = np.where(visible[None, :], S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            w = np.exp(S - m)
            den = w.sum(axis=1, keepdims=True)
            O[i, h0:h1, :] = (w @ values) / den
            L[i, h0:h1] = m[:, 0] + np.log(den[:, 0])
    return O, L


def request_positions(qo: int, kv: int) -> np.ndarray:
    """Absolute positions of a request's qo new rows over kv cached keys."""
    return np.arange(kv - qo, kv, dtype=np.int64)


def mla_attend_brute(q, rows, positions, d_c, sm_scale, causal=True):
    """The same definition with Python floats, ``math.exp`` and
    ``math.fsum``, for tiny inputs.  q: nested [n][H][w]; rows: nested
    [kv][w].  Returns (O nested [n][H][d_c], LSE nested [n][H])."""
    out, lse = [], []
    for i, qi in enumerate(q):
        row_o, row_l = [], []
        for qh in qi:
            keys = [j for j in range(len(rows)) if (not causal) or j <= positions[i]]
            s = [sm_scale * math.fsum(float(a) * float(b) for a, b in zip(qh, rows[j])) for j in keys]
            top = max(s)
            w = [math.exp(x - top) for x in s]
            den = math.fsum(w)
            row_o.append([math.fsum(w[k] * float(rows[j][d]) for k, j in enumerate(keys)) / den
                          for d in range(d_c)])
            row_l.append(top + math.log(den))
        out.append(row_o)
        lse.append(row_l)
    return out, lse


def mla_batch(q, rows, qo_lens, kv_lens, d_c, sm_scale, causal=True):
    """All requests of a ragged batch.  q [sum qo, H, w]; rows [sum kv, w]
    (each request's logical cache, concatenated).  Returns (O, LSE)."""
    qo_lens = np.asarray(qo_lens, np.int64)
    kv_lens = np.asarray(kv_lens, np.int64)
    n, H, _ = np.asarray(q).shape
    O = np.empty((n, H, d_c), np.float64)
    L = np.empty((n, H), np.float64)
    qa = ka = 0
    for qo, kv in zip(qo_lens, kv_lens):
        qo, kv = int(qo), int(kv)
        if qo:
            O[qa:qa + qo], L[qa:qa + qo] = mla_attend(q[qa:qa + qo], rows[ka:ka + kv],
                                                      request_positions(qo, kv), d_c, sm_scale, causal)
        qa += qo
        ka += kv
    return O, L


# ------------------------------------------------------------ latent pool
def mla_append(pool, new_rows, qo_lens, kv_lens, page_indptr, page_indices):
    """Write each request's qo new rows (token-major, [sum qo, w]) at its
    positions [kv - qo, kv).  The cache entries exist before attention reads
    them (post, section "KV Messenger").  Returns the pool (modified)."""
    ps = pool.shape[1]
    a = 0
    for r, (qo, kv) in enumerate(zip(qo_lens, kv_lens)):
        pages = page_indices[page_indptr[r]:page_indptr[r + 1]]
        for t in range(int(kv) - int(qo), int(kv)):
            pool[pages[t // ps], t % ps, :] = new_rows[a]
            a += 1
    return pool


def mla_gather(pool, page_indptr, page_indices, r, kv):
    """Request r's logical cache rows [kv, w] read back out of its pages."""
    ps = pool.shape[1]
    pages = page_indices[page_indptr[r]:page_indptr[r + 1]]
    return np.stack([pool[pages[t // ps], t % ps, :] for t in range(int(kv))]) if kv else pool[:0, 0, :]


def mla_pack(pool, page_ids):
    """Whole pages in list order, one contiguous buffer [n, ps, w].  Every
    rank holds the same latent pages, so a page travels whole, from any one
    rank (post, section "Sharded KV Cache Transfers")."""
    return np.stack([pool[int(i)] for i in page_ids]) if len(page_ids) else pool[:0]


def mla_unpack(pool, page_ids, buf):
    """The buffer's page images written into the destination pages."""
    for k, i in enumerate(page_ids):
        pool[int(i)] = buf[k]
    return pool
