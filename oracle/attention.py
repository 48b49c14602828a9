"""float64 reference attention over logical (unpaged) K/V -- test infrastructure.

Definition (scaled-dot-product softmax attention, grouped-query heads):

  for a request with qo query rows over kv cached keys, query head h reads
  KV head hk = h // g with g = H_q / H_kv (contiguous head groups);
  query row i sits at absolute position p_i = kv - qo + i;
  visible keys J_i = {j : j <= p_i} when causal, else all kv keys;
  S_ij = scale * <Q[i, h], K[j, hk]>;   m_i = max_{j in J_i} S_ij
  O[i, h] = sum_{j in J_i} exp(S_ij - m_i) V[j, hk] / sum_{j in J_i} exp(S_ij - m_i)
  LSE[i, h] = m_i + ln sum_{j in J_i} exp(S_ij - m_i)

Sources (no formula is printed on the pages; this is the plainest reading):
  * attention cost grows with kv_len for both prefill and decode, decode
    requests carry one token (qo_len = 1), prefill carries many (large
    qo_len) -- Perplexity, "Disaggregated prefill and decode", section
    "Prefill vs Decode performance";
  * a chunk of a chunked prefill attends over all prior KV -- same section,
    and the kwkr.cn survey, section 8 (chunked prefill re-reads the earlier
    KV cache for every chunk);
  * KV entries are appended before attention reads them -- post, section
    "KV Messenger";
  * the decoder's first step replays the prompt's last token against the
    cache the prefiller built -- post, section "Speculative Decoding";
  * grouped-query attention -- post, section "Qwen3-Coder".

Only numpy is used; row blocks bound memory, nothing else is reordered.
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 512


def attend(q, k, v, positions, sm_scale, causal=True):
    """Attention of query rows against one request's logical cache.

    q          [n, H_q, D]   float64 query rows
    k, v       [kv, H_kv, D] float64 keys / values, position j at index j
    positions  [n] absolute positions of the query rows (kv - qo + i)
    Returns (O [n, H_q, D], LSE [n, H_q]) in float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    positions = np.asarray(positions, np.int64)
    n, H_q, D = q.shape
    kv, H_kv, _ = k.shape
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    g = H_q // H_kv
    O = np.empty((n, H_q, D), np.float64)
    L = np.empty((n, H_q), np.float64)
    key_pos = np.arange(kv)
    for r0 in range(0, n, ROW_BLOCK):
        r1 = min(n, r0 + ROW_BLOCK)
        if causal:
            visible = key_pos[None, :] <= positions[r0:r1, None]
        else:
            visible = np.ones((r1 - r0, kv), bool)
        for h in range(H_q):
            hk = h // g
            S = sm_scale * (q[r0:r1, h, :] @ k[:, hk, :].T)
            S = np.where(visible, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            w = np.exp(S - m)
            den = w.sum(axis=1, keepdims=True)
            O[r0:r1, h, :] = (w @ v[:, hk, :]) / den
            L[r0:r1, h] = m[:, 0] + np.log(den[:, 0])
    return O, L


def request_positions(qo: int, kv: int) -> np.ndarray:
    """Absolute positions of a request's qo new rows over kv cached keys."""
    return np.arange(kv - qo, kv, dtype=np.int64)


def attention_batch(q, k, v, qo_lens, kv_lens, sm_scale, causal=True,
                    qo_indptr=None, kv_indptr=None):
    """Ragged batch: q [sum qo, H_q, D]; k, v [sum kv, H_kv, D] (logical,
    request after request).  Returns (O [sum qo, H_q, D], LSE [sum qo, H_q])."""
    qo_lens = np.asarray(qo_lens, np.int64)
    kv_lens = np.asarray(kv_lens, np.int64)
    if qo_indptr is None:
        qo_indptr = np.concatenate([[0], np.cumsum(qo_lens)])
    if kv_indptr is None:
        kv_indptr = np.concatenate([[0], np.cumsum(kv_lens)])
    n = int(qo_indptr[-1])
    H_q, D = q.shape[1], q.shape[2]
    O = np.zeros((n, H_q, D), np.float64)
    L = np.zeros((n, H_q), np.float64)
    for r in range(len(qo_lens)):
        qo, kv = int(qo_lens[r]), int(kv_lens[r])
        if qo == 0:
            continue
        a, b = int(qo_indptr[r]), int(qo_indptr[r + 1])
        c, d = int(kv_indptr[r]), int(kv_indptr[r + 1])
        O[a:b], L[a:b] = attend(q[a:b], k[c:d], v[c:d],
                                request_positions(qo, kv), sm_scale, causal)
    return O, L
