"""Pins of the float64 oracle against things other than itself (CPU only).

* brute force: the scalar pure-Python definition on tiny inputs, including
  the whole tiny workload (3 requests, 4/2 heads, head_dim 64);
* a library routine: torch's CPU scaled_dot_product_attention in float64 with
  an explicit end-aligned causal mask, and scipy's logsumexp for the LSE;
* closed forms: one visible key returns its V row; uniform V returns V; a
  zero query averages the visible V rows; equal keys average V; one dominant
  logit returns that key's V row;
* invariants: chunked prefill equals full prefill; a decode step equals the
  last row of the equivalent prefill (the held-back-token handoff); GQA equals
  MHA over replicated KV heads; shifting every key by the same vector changes
  nothing; O is affine in V.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention as A
from oracle import brute as Bf
from workloads import make_batch


def rand(rng, *shape):
    return rng.standard_normal(shape)


def to_nested(a):
    return a.tolist()


# ------------------------------------------------------------- brute force
@pytest.mark.parametrize("qo,kv,Hq,Hkv,D,causal", [
    (1, 1, 1, 1, 4, True),
    (3, 3, 2, 1, 8, True),
    (2, 7, 4, 2, 8, True),
    (5, 9, 3, 3, 16, False),
    (1, 13, 6, 2, 8, True),
    (4, 4, 8, 1, 4, True),
])
def test_brute_vs_oracle_small(qo, kv, Hq, Hkv, D, causal):
    rng = np.random.default_rng(1234 + qo * 31 + kv)
    q, k, v = rand(rng, qo, Hq, D), rand(rng, kv, Hkv, D), rand(rng, kv, Hkv, D)
    pos = A.request_positions(qo, kv)
    s = 1.0 / math.sqrt(D)
    O, L = A.attend(q, k, v, pos, s, causal)
    Ob, Lb = Bf.attend_brute(to_nested(q), to_nested(k), to_nested(v), pos.tolist(), s, causal)
    np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-12)


def test_brute_vs_oracle_tiny_workload():
    b = make_batch("tiny")
    q, k, v = b.to_f64(b.q), b.to_f64(b.k), b.to_f64(b.v)
    O, L = A.attention_batch(q, k, v, b.qo_lens, b.kv_lens, b.sm_scale, True)
    for r in range(b.B):
        qa, qb = b.qo_indptr[r], b.qo_indptr[r + 1]
        ka, kb = b.kv_indptr[r], b.kv_indptr[r + 1]
        pos = A.request_positions(int(b.qo_lens[r]), int(b.kv_lens[r]))
        Ob, Lb = Bf.attend_brute(to_nested(q[qa:qb]), to_nested(k[ka:kb]),
                                 to_nested(v[ka:kb]), pos.tolist(), b.sm_scale, True)
        np.testing.assert_allclose(O[qa:qb], np.array(Ob), rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[qa:qb], np.array(Lb), rtol=0, atol=1e-12)


# ------------------------------------------------------------ library pins
def torch_sdpa_end_aligned(q, k, v, qo, kv, scale, causal):
    """torch CPU float64 SDPA with an explicit mask: row i sees keys j <=
    kv - qo + i (torch's own is_causal aligns to the start, so the mask is
    built by hand)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    g = Hq // Hkv
    kk = np.repeat(k, g, axis=1)   # contiguous head groups
    vv = np.repeat(v, g, axis=1)
    tq = torch.from_numpy(q).permute(1, 0, 2).contiguous()
    tk = torch.from_numpy(kk).permute(1, 0, 2).contiguous()
    tv = torch.from_numpy(vv).permute(1, 0, 2).contiguous()
    i = torch.arange(qo)[:, None]
    j = torch.arange(kv)[None, :]
    mask = (j <= i + (kv - qo)) if causal else torch.ones(qo, kv, dtype=torch.bool)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("qo,kv,Hq,Hkv,D,causal", [
    (64, 64, 4, 4, 64, True),
    (40, 200, 8, 2, 128, True),
    (1, 333, 8, 1, 64, True),
    (17, 50, 6, 3, 32, False),
    (128, 128, 4, 1, 128, True),
])
def test_oracle_vs_torch_sdpa(qo, kv, Hq, Hkv, D, causal):
    rng = np.random.default_rng(99 + qo + kv)
    q, k, v = rand(rng, qo, Hq, D), rand(rng, kv, Hkv, D), rand(rng, kv, Hkv, D)
    s = 1.0 / math.sqrt(D)
    O, L = A.attend(q, k, v, A.request_positions(qo, kv), s, causal)
    ref = torch_sdpa_end_aligned(q, k, v, qo, kv, s, causal)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    # LSE against scipy's logsumexp of the visible scaled logits
    g = Hq // Hkv
    for i in range(0, qo, max(1, qo // 7)):
        for h in range(Hq):
            vis = (kv - qo + i + 1) if causal else kv
            logits = s * (k[:vis, h // g, :] @ q[i, h, :])
            assert abs(L[i, h] - scipy.special.logsumexp(logits)) < 1e-12


def test_torch_is_causal_equals_end_aligned_when_square():
    """When qo == kv both alignments coincide; checks the hand-made mask."""
    rng = np.random.default_rng(5)
    q, k, v = rand(rng, 33, 2, 16), rand(rng, 33, 2, 16), rand(rng, 33, 2, 16)
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2) for x in (q, k, v))
    o1 = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.25)
    o2 = torch_sdpa_end_aligned(q, k, v, 33, 33, 0.25, True)
    np.testing.assert_allclose(o1.permute(1, 0, 2).numpy(), o2, atol=1e-13)


# ------------------------------------------------------------ closed forms
def test_single_key_returns_v():
    rng = np.random.default_rng(7)
    q, k, v = rand(rng, 1, 4, 64), rand(rng, 1, 2, 64), rand(rng, 1, 2, 64)
    O, L = A.attend(q, k, v, [0], 0.125, True)
    for h in range(4):
        np.testing.assert_array_equal(O[0, h], v[0, h // 2])
        assert L[0, h] == pytest.approx(0.125 * q[0, h] @ k[0, h // 2], abs=1e-14)


def test_first_row_of_causal_prefill_sees_one_key():
    rng = np.random.default_rng(8)
    q, k, v = rand(rng, 9, 2, 8), rand(rng, 9, 1, 8), rand(rng, 9, 1, 8)
    O, _ = A.attend(q, k, v, A.request_positions(9, 9), 0.3, True)
    np.testing.assert_array_equal(O[0, 0], v[0, 0])
    np.testing.assert_array_equal(O[0, 1], v[0, 0])


def test_uniform_v_returns_v():
    rng = np.random.default_rng(9)
    q, k = rand(rng, 12, 4, 32), rand(rng, 40, 2, 32)
    row = rand(rng, 2, 32)
    v = np.broadcast_to(row, (40, 2, 32)).copy()
    O, _ = A.attend(q, k, v, A.request_positions(12, 40), 0.2, True)
    for h in range(4):
        np.testing.assert_allclose(O[:, h], np.broadcast_to(row[h // 2], (12, 32)), atol=1e-14)


def test_zero_query_averages_visible_v():
    rng = np.random.default_rng(10)
    k, v = rand(rng, 20, 1, 16), rand(rng, 20, 1, 16)
    q = np.zeros((5, 1, 16))
    O, L = A.attend(q, k, v, A.request_positions(5, 20), 1.0, True)
    for i in range(5):
        vis = 20 - 5 + i + 1
        np.testing.assert_allclose(O[i, 0], v[:vis, 0].mean(axis=0), atol=1e-14)
        assert L[i, 0] == pytest.approx(math.log(vis), abs=1e-14)


def test_equal_keys_average_v():
    rng = np.random.default_rng(11)
    q, v = rand(rng, 3, 2, 16), rand(rng, 30, 2, 16)
    k = np.broadcast_to(rand(rng, 1, 2, 16), (30, 2, 16)).copy()
    O, _ = A.attend(q, k, v, A.request_positions(3, 30), 0.25, False)
    for h in range(2):
        np.testing.assert_allclose(O[:, h], np.broadcast_to(v[:, h].mean(axis=0), (3, 16)), atol=1e-13)


def test_dominant_logit_selects_its_value():
    rng = np.random.default_rng(12)
    D = 8
    k = rand(rng, 64, 1, D) * 0.01
    v = rand(rng, 64, 1, D)
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    k[37, 0, 0] = 80.0   # logit 80 above all others (others < 0.1)
    O, _ = A.attend(q, k, v, [63], 1.0, True)
    bound = 64 * math.exp(-79.0) * np.abs(v).max()
    assert np.abs(O[0, 0] - v[37, 0]).max() <= bound + 1e-15


# -------------------------------------------------------------- invariants
@pytest.mark.parametrize("L_total,c", [(37, 10), (64, 63), (50, 1), (96, 32)])
def test_chunked_prefill_equals_full(L_total, c):
    rng = np.random.default_rng(20 + c)
    q, k, v = rand(rng, L_total, 4, 16), rand(rng, L_total, 2, 16), rand(rng, L_total, 2, 16)
    s = 0.25
    Of, Lf = A.attend(q, k, v, A.request_positions(L_total, L_total), s, True)
    O1, L1 = A.attend(q[:c], k[:c], v[:c], A.request_positions(c, c), s, True)
    O2, L2 = A.attend(q[c:], k, v, A.request_positions(L_total - c, L_total), s, True)
    np.testing.assert_allclose(np.concatenate([O1, O2]), Of, atol=1e-13)
    np.testing.assert_allclose(np.concatenate([L1, L2]), Lf, atol=1e-13)


@pytest.mark.parametrize("L_total", [1, 2, 17, 100])
def test_decode_step_equals_last_prefill_row(L_total):
    rng = np.random.default_rng(30 + L_total)
    q, k, v = rand(rng, L_total, 8, 16), rand(rng, L_total, 2, 16), rand(rng, L_total, 2, 16)
    Of, Lf = A.attend(q, k, v, A.request_positions(L_total, L_total), 0.25, True)
    Od, Ld = A.attend(q[-1:], k, v, A.request_positions(1, L_total), 0.25, True)
    np.testing.assert_allclose(Od[0], Of[-1], atol=1e-13)
    np.testing.assert_allclose(Ld[0], Lf[-1], atol=1e-13)


def test_gqa_equals_replicated_mha():
    rng = np.random.default_rng(40)
    g = 4
    q, k, v = rand(rng, 11, 8, 16), rand(rng, 30, 2, 16), rand(rng, 30, 2, 16)
    pos = A.request_positions(11, 30)
    O1, L1 = A.attend(q, k, v, pos, 0.3, True)
    kk, vv = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    O2, L2 = A.attend(q, kk, vv, pos, 0.3, True)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


def test_key_shift_invariance():
    rng = np.random.default_rng(41)
    q, k, v = rand(rng, 6, 2, 16), rand(rng, 25, 2, 16), rand(rng, 25, 2, 16)
    pos = A.request_positions(6, 25)
    O1, _ = A.attend(q, k, v, pos, 0.25, True)
    shift = rand(rng, 1, 2, 16)
    O2, _ = A.attend(q, k + shift, v, pos, 0.25, True)
    np.testing.assert_allclose(O1, O2, atol=1e-12)


def test_value_affine():
    rng = np.random.default_rng(42)
    q, k, v = rand(rng, 6, 4, 16), rand(rng, 25, 2, 16), rand(rng, 25, 2, 16)
    pos = A.request_positions(6, 25)
    O1, _ = A.attend(q, k, v, pos, 0.25, True)
    O2, _ = A.attend(q, k, 3.0 * v - 2.0, pos, 0.25, True)
    np.testing.assert_allclose(O2, 3.0 * O1 - 2.0, atol=1e-12)


def test_batch_is_per_request():
    """The ragged batch is the concatenation of independent requests, and a
    request with qo = 0 produces no rows."""
    b = make_batch("tiny", lengths=([5, 0, 1, 7], [9, 16, 3, 7]))
    q, k, v = b.to_f64(b.q), b.to_f64(b.k), b.to_f64(b.v)
    O, L = A.attention_batch(q, k, v, b.qo_lens, b.kv_lens, b.sm_scale)
    assert O.shape[0] == 13
    for r in range(b.B):
        qa, qb = b.qo_indptr[r], b.qo_indptr[r + 1]
        ka, kb = b.kv_indptr[r], b.kv_indptr[r + 1]
        if qb == qa:
            continue
        Or, Lr = A.attend(q[qa:qb], k[ka:kb], v[ka:kb],
                          A.request_positions(int(b.qo_lens[r]), int(b.kv_lens[r])), b.sm_scale)
        np.testing.assert_array_equal(O[qa:qb], Or)
        np.testing.assert_array_equal(L[qa:qb], Lr)
