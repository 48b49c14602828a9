"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is the oracle's own source with one plausible slip (a dropped
term, a wrong index, a transposed operand, a shifted mask); the pins that
``test_oracle_pins`` applies -- brute force, torch SDPA with an end-aligned
mask, the decode-equals-last-row handoff and the closed forms -- are run
against the mutant and at least one of them must fail.
"""
import math
import os
import types

import numpy as np
import pytest
import torch

from oracle import brute as Bf

SRC = open(os.path.join(os.path.dirname(os.path.dirname(__file__)),
                        "oracle", "attention.py")).read()

MUTANTS = {
    "start_aligned_causal": ("np.arange(kv - qo, kv, dtype=np.int64)", "np.arange(0, qo, dtype=np.int64)"),
    "gqa_interleaved_heads": ("hk = h // g", "hk = h % H_kv"),
    "scale_dropped": ("S = sm_scale * (", "S = ("),
    "k_used_as_v": ("(w @ v[:, hk, :])", "(w @ k[:, hk, :])"),
    "mask_off_by_one": ("key_pos[None, :] <= positions", "key_pos[None, :] < positions"),
    "lse_without_max": ("L[r0:r1, h] = m[:, 0] + np.log", "L[r0:r1, h] = np.log"),
    "not_normalised": ("O[r0:r1, h, :] = (w @ v[:, hk, :]) / den", "O[r0:r1, h, :] = (w @ v[:, hk, :])"),
    "q_head_from_kv_head": ("S = sm_scale * (q[r0:r1, h, :]", "S = sm_scale * (q[r0:r1, hk, :]"),
    "scale_squared": ("S = sm_scale * (", "S = sm_scale * sm_scale * ("),
}


def load_variant(src):
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def pins_pass(A):
    """Run a compact set of the oracle pins against module A; True if all pass."""
    ok = True
    rng = np.random.default_rng(77)
    # brute force, GQA 4/2, chunk over prior keys
    for (qo, kv, Hq, Hkv, D) in [(3, 9, 4, 2, 8), (1, 6, 2, 1, 4)]:
        q = rng.standard_normal((qo, Hq, D))
        k = rng.standard_normal((kv, Hkv, D))
        v = rng.standard_normal((kv, Hkv, D))
        pos = A.request_positions(qo, kv)
        s = 1.0 / math.sqrt(D)
        O, L = A.attend(q, k, v, pos, s, True)
        Ob, Lb = Bf.attend_brute(q.tolist(), k.tolist(), v.tolist(),
                                 list(range(kv - qo, kv)), s, True)
        ok &= np.allclose(O, np.array(Ob), atol=1e-12) and np.allclose(L, np.array(Lb), atol=1e-12)
    # torch SDPA with an explicit end-aligned mask
    qo, kv, H, D = 5, 12, 2, 16
    q, k, v = (rng.standard_normal(s) for s in ((qo, H, D), (kv, H, D), (kv, H, D)))
    O, _ = A.attend(q, k, v, A.request_positions(qo, kv), 0.25, True)
    mask = torch.arange(kv)[None, :] <= torch.arange(qo)[:, None] + (kv - qo)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x).permute(1, 0, 2) for x in (q, k, v)), attn_mask=mask, scale=0.25)
    ok &= np.allclose(O, ref.permute(1, 0, 2).numpy(), atol=1e-12)
    # decode step equals last prefill row
    Of, _ = A.attend(q, k[:qo], v[:qo], A.request_positions(qo, qo), 0.25, True)
    Od, _ = A.attend(q[-1:], k[:qo], v[:qo], A.request_positions(1, qo), 0.25, True)
    ok &= np.allclose(Od[0], Of[-1], atol=1e-13)
    return bool(ok)


def test_unmutated_oracle_passes():
    assert pins_pass(load_variant(SRC))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name} not found"
    mutant = load_variant(SRC.replace(old, new))
    assert not pins_pass(mutant), f"pins did not catch mutant {name}"
