"""Pins of the MLA oracle (``oracle.mla``) against things other than itself
(CPU only).

* absorption identity: the absorbed latent form equals expanded multi-head
  attention, computed by the separately pinned ``oracle.attention.attend``.
  The expanded form uses per-head keys [W_UK_h c_j ; kr_j], per-head values
  W_UV_h c_j, and queries [qn_h ; qr_h].  Absorbed: q = [W_UK_h^T qn_h ; qr_h],
  O_h = W_UV_h (latent output).  This is the reason MLA decode can read the
  latent rows directly.
* brute force: the scalar Python twin on tiny inputs;
* closed forms: one key returns its latent row; equal latent rows return
  that row; a zero query averages the visible latent rows; a dominant logit
  returns its row;
* invariants: a two-token step's second row equals a one-token step over
  the same cache, and its first row never sees the newest key (the causal
  mask sits at the end of the cache); latent pages round-trip through
  append / gather and pack / unpack bit for bit;
* planted mistakes in the oracle's source are caught by these pins.
"""
import math
import os
import types

import numpy as np
import pytest

from oracle import attention as A
from oracle import mla as M
from workloads import make_mla_batch


def rand(rng, *shape):
    return rng.standard_normal(shape)


def expanded_vs_absorbed(M_, rng, n, H, kv, d_c, d_r, d_n, d_v, causal=True, qo=None):
    """Returns (O_absorbed projected by W_UV, O_expanded, L_absorbed, L_expanded)."""
    c = rand(rng, kv, d_c)
    kr = rand(rng, kv, d_r)
    W_UK = rand(rng, H, d_n, d_c) / math.sqrt(d_c)
    W_UV = rand(rng, H, d_v, d_c) / math.sqrt(d_c)
    qn = rand(rng, n, H, d_n)
    qr = rand(rng, n, H, d_r)
    scale = 1.0 / math.sqrt(d_n + d_r)
    pos = M.request_positions(n if qo is None else qo, kv)
    # expanded: MHA with H KV heads of width d_n + d_r (V zero-padded)
    K = np.concatenate([np.einsum("hnc,jc->jhn", W_UK, c), np.repeat(kr[:, None, :], H, axis=1)], axis=2)
    V = np.zeros((kv, H, d_n + d_r))
    V[:, :, :d_v] = np.einsum("hvc,jc->jhv", W_UV, c)
    Q = np.concatenate([qn, qr], axis=2)
    Oe, Le = A.attend(Q, K, V, pos, scale, causal)
    # absorbed: one latent row per token
    q_abs = np.concatenate([np.einsum("hnc,ihn->ihc", W_UK, qn), qr], axis=2)
    rows = np.concatenate([c, kr], axis=1)
    Ol, Ll = M_.mla_attend(q_abs, rows, pos, d_c, scale, causal)
    Oa = np.einsum("hvc,ihc->ihv", W_UV, Ol)
    return Oa, Oe[:, :, :d_v], Ll, Le


@pytest.mark.parametrize("n,H,kv,d_c,d_r,d_n,d_v,causal", [
    (1, 4, 9, 16, 8, 12, 10, True),
    (3, 2, 11, 24, 4, 8, 8, True),
    (2, 3, 7, 16, 8, 12, 6, False),
    (1, 16, 40, 512, 64, 128, 128, True),     # DeepSeek-V3 widths, 16 heads
])
def test_absorption_identity(n, H, kv, d_c, d_r, d_n, d_v, causal):
    rng = np.random.default_rng(100 + n * 7 + kv)
    Oa, Oe, La, Le = expanded_vs_absorbed(M, rng, n, H, kv, d_c, d_r, d_n, d_v, causal)
    np.testing.assert_allclose(Oa, Oe, rtol=0, atol=1e-10)
    np.testing.assert_allclose(La, Le, rtol=0, atol=1e-10)


@pytest.mark.parametrize("qo,kv,H,d_c,d_r,causal", [
    (1, 1, 2, 8, 4, True),
    (2, 9, 3, 8, 4, True),
    (3, 5, 2, 6, 2, False),
    (1, 13, 4, 16, 8, True),
])
def test_brute_vs_oracle(qo, kv, H, d_c, d_r, causal):
    rng = np.random.default_rng(7 + qo + 11 * kv)
    q, rows = rand(rng, qo, H, d_c + d_r), rand(rng, kv, d_c + d_r)
    pos = M.request_positions(qo, kv)
    s = 1.0 / math.sqrt(d_c + d_r)
    O, L = M.mla_attend(q, rows, pos, d_c, s, causal)
    Ob, Lb = M.mla_attend_brute(q.tolist(), rows.tolist(), pos.tolist(), d_c, s, causal)
    np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-12)


def test_brute_on_tiny_workload_requests():
    """The parity workload's first two requests (kv 1 and kv 77 with two new
    tokens) at full width, two heads, against the scalar twin."""
    b = make_mla_batch("mla_tiny")
    q, rows = b.to_f64(b.q), b.to_f64(b.rows)
    for r in (0, 1):
        qa, qb = int(b.qo_indptr[r]), int(b.qo_indptr[r + 1])
        ka, kb = int(b.kv_indptr[r]), int(b.kv_indptr[r + 1])
        pos = M.request_positions(qb - qa, kb - ka)
        O, L = M.mla_attend(q[qa:qb, :2], rows[ka:kb], pos, b.d_c, b.sm_scale)
        Ob, Lb = M.mla_attend_brute(q[qa:qb, :2].tolist(), rows[ka:kb].tolist(), pos.tolist(), b.d_c,
                                    b.sm_scale)
        np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-12)


# ------------------------------------------------------------ closed forms
D_C, D_R = 32, 8


def test_single_key_returns_its_latent_row():
    rng = np.random.default_rng(3)
    q, rows = rand(rng, 1, 5, D_C + D_R), rand(rng, 1, D_C + D_R)
    O, L = M.mla_attend(q, rows, [0], D_C, 0.3)
    np.testing.assert_allclose(O[0], np.repeat(rows[:, :D_C], 5, axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(L[0], 0.3 * (q[0] @ rows[0]), rtol=0, atol=1e-13)


def test_equal_latent_rows_return_that_row():
    rng = np.random.default_rng(4)
    rows = rand(rng, 20, D_C + D_R)
    rows[:, :D_C] = rows[0, :D_C]            # same latent, different rotary keys
    O, _ = M.mla_attend(rand(rng, 3, 4, D_C + D_R), rows, M.request_positions(3, 20), D_C, 0.2)
    np.testing.assert_allclose(O, np.broadcast_to(rows[0, :D_C], O.shape), rtol=0, atol=1e-13)


def test_zero_query_averages_visible_latent_rows():
    rng = np.random.default_rng(5)
    rows = rand(rng, 12, D_C + D_R)
    O, L = M.mla_attend(np.zeros((2, 3, D_C + D_R)), rows, M.request_positions(2, 12), D_C, 0.5)
    np.testing.assert_allclose(O[0], np.broadcast_to(rows[:11, :D_C].mean(0), (3, D_C)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(O[1], np.broadcast_to(rows[:, :D_C].mean(0), (3, D_C)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(L, [[math.log(11)] * 3, [math.log(12)] * 3], rtol=0, atol=1e-14)


def test_dominant_rotary_logit_returns_its_row():
    """The logit gap comes from the rotary part alone, so a dropped rotary
    term would miss the dominant key."""
    rng = np.random.default_rng(6)
    kv = 30
    rows = rand(rng, kv, D_C + D_R) * 0.01
    q = np.zeros((1, 1, D_C + D_R))
    q[0, 0, D_C] = 1.0
    rows[17, D_C] = 400.0                     # logit 0.25 * 400 = 100 above the rest
    O, _ = M.mla_attend(q, rows, [kv - 1], D_C, 0.25)
    np.testing.assert_allclose(O[0, 0], rows[17, :D_C], rtol=0, atol=1e-30 + kv * math.exp(-90))


# ------------------------------------------------------------- invariants
def test_two_token_step_rows():
    """Row 1 of a two-token step equals a one-token step over the same
    cache; row 0 ignores the newest key (changing it leaves row 0 alone)."""
    rng = np.random.default_rng(8)
    kv = 25
    q, rows = rand(rng, 2, 4, D_C + D_R), rand(rng, kv, D_C + D_R)
    O2, L2 = M.mla_attend(q, rows, M.request_positions(2, kv), D_C, 0.3)
    O1, L1 = M.mla_attend(q[1:], rows, M.request_positions(1, kv), D_C, 0.3)
    np.testing.assert_allclose(O2[1], O1[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(L2[1], L1[0], rtol=0, atol=1e-14)
    rows2 = rows.copy()
    rows2[-1] = rand(rng, D_C + D_R) * 10
    O3, _ = M.mla_attend(q, rows2, M.request_positions(2, kv), D_C, 0.3)
    np.testing.assert_array_equal(O3[0], O2[0])
    assert np.abs(O3[1] - O2[1]).max() > 1e-3


def test_latent_pages_round_trip():
    b = make_mla_batch("mla_tiny", lengths=([1, 3, 2], [1, 40, 17]))
    pool = np.full(b.pool_shape, np.nan, np.float32)
    rows = b.to_f64(b.rows).astype(np.float32)
    # fill every cached row by appending each request's whole cache as new tokens
    for r in range(b.B):
        ka, kb = int(b.kv_indptr[r]), int(b.kv_indptr[r + 1])
        M.mla_append(pool, rows[ka:kb], [kb - ka], [kb - ka], b.page_indptr[r:r + 2] - b.page_indptr[r],
                     b.request_pages(r))
    for r in range(b.B):
        ka, kb = int(b.kv_indptr[r]), int(b.kv_indptr[r + 1])
        np.testing.assert_array_equal(M.mla_gather(pool, b.page_indptr, b.page_indices, r, kb - ka), rows[ka:kb])
    ids = b.page_indices[::-1].copy()
    buf = M.mla_pack(pool, ids)
    dst = np.zeros_like(pool)
    M.mla_unpack(dst, ids, buf)
    np.testing.assert_array_equal(np.isnan(dst[ids]), np.isnan(pool[ids]))
    np.testing.assert_array_equal(np.nan_to_num(dst[ids]), np.nan_to_num(pool[ids]))
    assert buf.nbytes == len(ids) * b.ps * b.width * 4


def test_batch_is_per_request():
    b = make_mla_batch("mla_tiny")
    q, rows = b.to_f64(b.q), b.to_f64(b.rows)
    O, L = M.mla_batch(q, rows, b.qo_lens, b.kv_lens, b.d_c, b.sm_scale)
    r = 2
    qa, ka = int(b.qo_indptr[r]), int(b.kv_indptr[r])
    O2, L2 = M.mla_attend(q[qa:qa + 1], rows[ka:ka + 300], [299], b.d_c, b.sm_scale)
    np.testing.assert_array_equal(O[qa], O2[0])
    np.testing.assert_array_equal(L[qa], L2[0])


# ------------------------------------------------------- planted mistakes
SRC = open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "mla.py")).read()

MUTANTS = {
    "rotary_term_dropped": ("S = sm_scale * (q[i, h0:h1, :] @ rows.T)",
                            "S = sm_scale * (q[i, h0:h1, :d_c] @ rows[:, :d_c].T)"),
    "value_from_rotary_end": ("values = rows[:, :d_c]", "values = rows[:, -d_c:]"),
    "mask_off_by_one": ("visible = key_pos <= positions[i]", "visible = key_pos < positions[i] + 2"),
    "start_aligned_causal": ("np.arange(kv - qo, kv, dtype=np.int64)", "np.arange(0, qo, dtype=np.int64)"),
    "scale_dropped": ("S = sm_scale * (", "S = ("),
    "lse_without_max": ("L[i, h0:h1] = m[:, 0] + np.log", "L[i, h0:h1] = np.log"),
    "not_normalised": ("O[i, h0:h1, :] = (w @ values) / den", "O[i, h0:h1, :] = (w @ values)"),
}


def load_variant(src):
    mod = types.ModuleType("mla_mutant")
    exec(compile(src, "mla_mutant", "exec"), mod.__dict__)
    return mod


def pins_pass(Mv) -> bool:
    rng = np.random.default_rng(21)
    ok = True
    for args in [(1, 4, 9, 16, 8, 12, 10, True), (3, 2, 11, 24, 4, 8, 8, True)]:
        Oa, Oe, La, Le = expanded_vs_absorbed(Mv, rng, *args)
        ok &= np.allclose(Oa, Oe, atol=1e-10) and np.allclose(La, Le, atol=1e-10)
    q, rows = rand(rng, 2, 3, 12), rand(rng, 9, 12)
    pos = Mv.request_positions(2, 9)
    O, L = Mv.mla_attend(q, rows, pos, 8, 0.4, True)
    Ob, Lb = M.mla_attend_brute(q.tolist(), rows.tolist(), list(range(7, 9)), 8, 0.4, True)
    ok &= np.allclose(O, np.array(Ob), atol=1e-12) and np.allclose(L, np.array(Lb), atol=1e-12)
    Oz, Lz = Mv.mla_attend(np.zeros((1, 2, 12)), rows, [8], 8, 0.4)
    ok &= np.allclose(Oz[0], rows[:, :8].mean(0), atol=1e-14) and np.allclose(Lz, math.log(9), atol=1e-14)
    return bool(ok)


def test_unmutated_oracle_passes_the_pins():
    assert pins_pass(load_variant(SRC))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation site of {name} not found once"
    assert not pins_pass(load_variant(SRC.replace(old, new)))
