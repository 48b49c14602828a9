"""GPU: latent-cache (MLA) decode parity with the float64 oracle, through the
C ABI.  Bars as for the other bf16 paths (fp32 accumulation): max |O -
O_oracle| <= 2e-2 and |LSE - LSE_oracle| <= 5e-3 + 2^-20 max|LSE| (the
normaliser is the sum of the bf16-rounded softmax weights).

Cases: the parity workload (kv 1, a two-token step, kv 300); 16 to 128 heads;
page sizes 16 to 128; ragged lengths with tails; one-, two- and four-token
steps; non-causal; split-count invariance and bitwise determinism; a
sharpened softmax and logits rising along the cache (the rescale path), each
at 128 heads too (the 32-row kernel, whose output lives in accumulation
registers); and the two full-size decode workloads on sampled requests.  Appends and page
transfers are checked bit for bit, and NaN-poisoned spare pages and tail
slots are never read."""
import functools

import numpy as np
import pytest
import torch

import decode_attention_kv_pd_amd as pd
from oracle import mla as OM
from tests.harness import report
from workloads import (BF16_NAN, bf16_bits_to_f32, device_normal_, device_seed, f32_to_bf16_bits,
                       make_mla_batch)

pytestmark = pytest.mark.gpu

TOL = 2e-2


def lse_bar(L):
    return 5e-3 + 2.0 ** -20 * float(np.abs(L).max())


def host_pool(b, with_new=False):
    """bf16 bit pool: NaN everywhere, then each request's rows [0, kv - qo)
    (and the new rows too when with_new)."""
    pool = np.full(b.pool_shape, BF16_NAN, np.uint16)
    for r in range(b.B):
        ka, kv, qo = int(b.kv_indptr[r]), int(b.kv_lens[r]), int(b.qo_lens[r])
        n = kv if with_new else kv - qo
        if n:
            OM.mla_append(pool, b.rows[ka:ka + n], [n], [n], b.page_indptr[r:r + 2] - b.page_indptr[r],
                          b.request_pages(r))
    return pool


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


class MlaRun:
    def __init__(self, b, chunk=0):
        self.b = b
        d = pd.make_mla_desc(b.H, b.ps, b.causal, b.sm_scale)
        self.plan = pd.pd_mla_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages,
                                   decode_chunk_keys=chunk)
        self.ws = torch.empty(max(self.plan.workspace_bytes, 1), dtype=torch.uint8, device="cuda")
        pd.pd_plan_upload(self.plan, self.ws)
        n = int(b.qo_indptr[-1])
        self.out = torch.full((n, b.H, b.d_c), float("nan"), dtype=torch.float32, device="cuda")
        self.lse = torch.full((n, b.H), float("nan"), dtype=torch.float32, device="cuda")

    def step(self, pool=None):
        """Append the new rows into a pool holding the older ones, then attend."""
        b = self.b
        if pool is None:
            pool = to_dev(host_pool(b))
            pd.pd_mla_kv_append(self.plan, self.ws, pool, to_dev(b.new_rows))
        self.pool = pool
        pd.pd_mla_attention_run(self.plan, self.ws, to_dev(b.q), pool, self.out, self.lse)
        torch.cuda.synchronize()
        return self.out.cpu().numpy(), self.lse.cpu().numpy()


@functools.lru_cache(maxsize=None)
def oracle(key):
    b = BATCHES[key]
    return OM.mla_batch(b.to_f64(b.q), b.to_f64(b.rows), b.qo_lens, b.kv_lens, b.d_c, b.sm_scale, b.causal)


BATCHES = {}


def batch(name, **kw):
    key = (name, tuple(sorted((k, str(v)) for k, v in kw.items())))
    if key not in BATCHES:
        BATCHES[key] = make_mla_batch(name, **kw)
    return key, BATCHES[key]


def check(key, b, label, chunk=0):
    print(f"case {label}: B={b.B} H={b.H} ps={b.ps} causal={b.causal} qo={b.qo_lens.tolist()[:6]} "
          f"kv={b.kv_lens.tolist()[:6]} chunk={chunk}", flush=True)
    run = MlaRun(b, chunk)
    out, lse = run.step()
    O, L = oracle(key)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert report(label, out, O) <= TOL
    assert np.abs(lse - L).max() <= lse_bar(L)
    return run, out, lse


def test_tiny_workload_and_append_bits():
    key, b = batch("mla_tiny")
    run, _, _ = check(key, b, "mla_tiny")
    got = run.pool.cpu().numpy().view(np.uint16)
    want = host_pool(b, with_new=True)
    np.testing.assert_array_equal(got, want)   # appended rows bit-exact, NaN elsewhere untouched


RAGGED = [
    dict(lengths=([1, 1, 1, 1, 1], [1, 33, 64, 65, 1000]), heads=32),
    dict(lengths=([2, 1, 3], [2, 300, 129]), heads=48),
    dict(lengths=([1, 4, 1], [700, 95, 31]), heads=64, page_size=32),
    dict(lengths=([1, 2], [2049, 517]), heads=128, page_size=64),
    dict(lengths=([1, 1, 2], [5000, 17, 130]), heads=16, page_size=128),
    dict(lengths=([2, 1, 0, 1], [90, 40, 7, 1]), heads=16, causal=False),
    dict(lengths=([3, 1], [40, 1]), heads=128, causal=False),
    dict(lengths=([4, 2, 1], [4, 70, 33]), heads=128, page_size=16),
    dict(lengths=([1, 1, 3], [40000, 129, 2500]), heads=128, page_size=128),   # long cache, big pages
]


@pytest.mark.parametrize("idx", range(len(RAGGED)))
def test_ragged_parity(idx):
    key, b = batch("mla_tiny", **RAGGED[idx])
    check(key, b, f"mla_ragged{idx}")


@pytest.mark.parametrize("chunk", [32, 96, 1024])
def test_split_count_invariance(chunk):
    key, b = batch("mla_tiny", lengths=([1, 2, 1], [3000, 1500, 777]), heads=128, page_size=64)
    out0, _ = MlaRun(b).step()
    _, out1, _ = check(key, b, f"mla_split{chunk}", chunk=chunk)
    assert np.abs(out1 - out0).max() <= 2 * TOL


@pytest.mark.parametrize("heads", [64, 128])
def test_bitwise_deterministic_for_a_fixed_plan(heads):
    _, b = batch("mla_tiny", lengths=([1, 1, 2], [4000, 900, 300]), heads=heads)
    run = MlaRun(b, chunk=256)
    first = run.step()
    for _ in range(3):
        again = run.step(run.pool)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])


@pytest.mark.parametrize("heads", [32, 128])
def test_sharpened_softmax(heads):
    key, b = batch("mla_tiny", lengths=([1, 2, 1], [400, 1000, 33]), heads=heads, q_gain=8.0)
    check(key, b, f"mla_sharp{heads}")


def rising(b, nats_per_key):
    """Logits rising along each request's keys through the rotary part:
    q_rot[0] = 8, key j's rot[0] += r j with 8 r scale = nats_per_key."""
    q = bf16_bits_to_f32(b.q).copy()
    rows = bf16_bits_to_f32(b.rows).copy()
    q[:, :, b.d_c] = 8.0
    r = nats_per_key / (8.0 * b.sm_scale)
    for i in range(b.B):
        s, e = int(b.kv_indptr[i]), int(b.kv_indptr[i + 1])
        rows[s:e, b.d_c] += np.float32(r) * np.arange(e - s, dtype=np.float32)
    b.q, b.rows = f32_to_bf16_bits(q), f32_to_bf16_bits(rows)
    return b


@pytest.mark.parametrize("heads", [16, 128])
@pytest.mark.parametrize("nats", [1.0, 0.05])
def test_rising_logits(nats, heads):
    """The running max moves many times per block: the rescale of the
    accumulated output (for 128 heads, the accumulation-register path)."""
    key, b = batch("mla_tiny", lengths=([1, 2, 1], [600, 300, 2000]), heads=heads, rep=int(nats * 100))
    rising(b, nats)
    oracle.cache_clear()
    check(key, b, f"mla_rising{nats}_h{heads}")


@pytest.mark.parametrize("heads", [16, 128])
def test_one_dominant_key_is_reproduced(heads):
    """One key whose logit is 60 nats above the rest: O equals its latent row
    (bf16 values, exactly representable) to fp32 rounding."""
    key, b = batch("mla_tiny", lengths=([1], [777]), heads=heads, rep=5)
    q = bf16_bits_to_f32(b.q).copy()
    rows = bf16_bits_to_f32(b.rows).copy()
    q[:] = 0.0
    q[:, :, b.d_c] = 1.0
    rows[:, b.d_c] = 0.0
    rows[400, b.d_c] = 60.0 / b.sm_scale
    b.q, b.rows = f32_to_bf16_bits(q), f32_to_bf16_bits(rows)
    oracle.cache_clear()
    run, out, _ = check(key, b, "mla_dominant")
    want = bf16_bits_to_f32(b.rows[400, :b.d_c])
    assert np.abs(out[0] - want[None, :]).max() <= 1e-6 * max(1.0, float(np.abs(want).max()))


def test_pack_unpack_bit_exact():
    _, b = batch("mla_tiny", lengths=([1, 1], [100, 300]), heads=16, page_size=16)
    d = pd.make_mla_desc(b.H, b.ps)
    pool_h = host_pool(b, with_new=True)
    pool = to_dev(pool_h)
    ids = b.page_indices[::-1].copy()
    pb = pd.pd_mla_page_bytes(d)
    buf = torch.zeros(len(ids) * pb, dtype=torch.uint8, device="cuda")
    scr = torch.zeros(4 * len(ids), dtype=torch.uint8, device="cuda")
    pd.pd_mla_kv_pack(d, pool, b.num_pool_pages, ids, buf, scr)
    torch.cuda.synchronize()
    got = buf.cpu().numpy().view(np.uint16).reshape(len(ids), b.ps, b.width)
    np.testing.assert_array_equal(got, OM.mla_pack(pool_h, ids))
    dst = torch.zeros_like(pool)
    dst_ids = np.random.default_rng(3).permutation(b.num_pool_pages)[:len(ids)].astype(np.int32)
    pd.pd_mla_kv_unpack(d, dst, b.num_pool_pages, dst_ids, buf, scr)
    torch.cuda.synchronize()
    want = OM.mla_unpack(np.zeros_like(pool_h), dst_ids, OM.mla_pack(pool_h, ids))
    np.testing.assert_array_equal(dst.cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("name", ["mla_tp8", "mla_dp"])
def test_full_size_sampled(name):
    """The full decode workloads in the launch configuration the benchmark
    times (inputs drawn on the device), checked on sampled requests."""
    b = make_mla_batch(name, materialize=False)
    print(f"case {name}: B={b.B} H={b.H} total kv={int(b.kv_lens.sum())}", flush=True)
    pool = device_normal_(torch.empty(b.pool_shape, dtype=torch.bfloat16, device="cuda"), device_seed(b.wid, 0, 0))
    n = int(b.qo_indptr[-1])
    q = device_normal_(torch.empty((n, b.H, b.width), dtype=torch.bfloat16, device="cuda"), device_seed(b.wid, 0, 1))
    d = pd.make_mla_desc(b.H, b.ps, b.causal, b.sm_scale)
    plan = pd.pd_mla_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages)
    ws = torch.empty(max(plan.workspace_bytes, 1), dtype=torch.uint8, device="cuda")
    pd.pd_plan_upload(plan, ws)
    out = torch.empty((n, b.H, b.d_c), dtype=torch.float32, device="cuda")
    lse = torch.empty((n, b.H), dtype=torch.float32, device="cuda")
    pd.pd_mla_attention_run(plan, ws, q, pool, out, lse)
    torch.cuda.synchronize()
    out_h, lse_h = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(out_h).all() and np.isfinite(lse_h).all()
    pool_h = pool.view(torch.int16).cpu().numpy().view(np.uint16)
    q_h = q.view(torch.int16).cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(11)
    for r in sorted(rng.choice(b.B, size=3, replace=False).tolist()) + [int(np.argmax(b.kv_lens))]:
        kv = int(b.kv_lens[r])
        rows = OM.mla_gather(pool_h, b.page_indptr, b.page_indices, r, kv)
        qa = int(b.qo_indptr[r])
        O, L = OM.mla_attend(bf16_bits_to_f32(q_h[qa:qa + 1]).astype(np.float64),
                             bf16_bits_to_f32(rows).astype(np.float64), [kv - 1], b.d_c, b.sm_scale)
        assert report(f"{name}[r={r} kv={kv}]", out_h[qa:qa + 1], O) <= TOL
        assert np.abs(lse_h[qa:qa + 1] - L).max() <= lse_bar(L)
