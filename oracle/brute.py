"""Scalar pure-Python attention for tiny inputs -- test infrastructure.

The same definition as ``oracle.attention`` (scaled-dot-product softmax over
the visible keys, causal mask aligned to the end of the cache, query head h
reading KV head h // (H_q / H_kv)), written with Python floats, ``math.exp``
and ``math.fsum``.  It shares no code with ``oracle.attention`` so that the
two can check each other.  Sources: Perplexity, "Disaggregated prefill and
decode", sections "Prefill vs Decode performance" and "Qwen3-Coder".
"""
from __future__ import annotations

import math


def attend_brute(q, k, v, positions, sm_scale, causal=True):
    """q: nested [n][H_q][D]; k, v: nested [kv][H_kv][D]; positions: [n].
    Returns (O nested [n][H_q][D], LSE nested [n][H_q]) as Python floats."""
    n = len(q)
    H_q = len(q[0]) if n else 0
    kv = len(k)
    H_kv = len(k[0]) if kv else 1
    D = len(q[0][0]) if n else 0
    group = H_q // H_kv
    out, lse = [], []
    for i in range(n):
        row_o, row_l = [], []
        for h in range(H_q):
            hk = h // group
            keys = [j for j in range(kv) if (not causal) or j <= positions[i]]
            s = []
            for j in keys:
                acc = 0.0
                for d in range(D):
                    acc += float(q[i][h][d]) * float(k[j][hk][d])
                s.append(sm_scale * acc)
            top = max(s)
            w = [math.exp(x - top) for x in s]
            den = math.fsum(w)
            o = []
            for d in range(D):
                o.append(math.fsum(w[t] * float(v[keys[t]][hk][d])
                                   for t in range(len(keys))) / den)
            row_o.append(o)
            row_l.append(top + math.log(den))
        out.append(row_o)
        lse.append(row_l)
    return out, lse
