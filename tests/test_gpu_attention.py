"""GPU: attention parity with the float64 oracle, element by element.

Bars: max |O - O_oracle| <= 1e-4 for fp32 inputs and <= 2e-2 for bf16 inputs
(fp32 accumulation); LSE within 1e-4 (fp32) / 5e-3 (bf16: the kernels
normalise by the sum of the bf16-rounded softmax weights, whose log differs
from the exact log-sum-exp by at most ln(1 + 2^-8) < 3.9e-3), plus
2^-20 max|LSE|: the LSE carries the absolute rounding error of the fp32
logits it is made of, a few fp32 ulps of their magnitude (negligible for
N(0,1) data, about 3e-4 where logits reach 300 nats).  Cases span the
five seeded workloads (the long one at reduced length here; full length in
test_gpu_long), several tiles and ragged tails, every supported head_dim,
page size and GQA group, causal and non-causal, qo = 0 requests, the
decode unit widths (qo * g = 16 / 17, 32 / 33, 64 / 65: one 16-row column
group, two, two wavefronts of two, then prefill tiles), and a sharpened
softmax."""
import functools

import numpy as np
import pytest
import torch

from oracle import attention as OA
from tests.harness import DeviceRun, oracle_outputs, pd, report, tolerance
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_batch

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def batch(wid, lengths=None, **kw):
    if lengths is not None:
        lengths = (list(lengths[0]), list(lengths[1]))
    return make_batch(wid, lengths=lengths, **kw)


def lse_tol(b):
    return 1e-4 if b.dtype == "f32" else 5e-3


def check(b, name, chunk=0):
    print(f"case {name}: B={b.B} H={b.H_q}/{b.H_kv} D={b.D} ps={b.ps} {b.dtype} "
          f"causal={b.causal} rows={int(b.qo_indptr[-1])} chunk={chunk}", flush=True)
    out, lse = DeviceRun(b, decode_chunk_keys=chunk).step()
    O, L = oracle_outputs(b)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    err = report(name, out, O)
    assert err <= tolerance(b)
    assert np.abs(lse - L).max() <= lse_tol(b) + 2.0 ** -20 * np.abs(L).max()
    return out, lse


@pytest.mark.parametrize("wid", ["tiny", "decode", "prefill", "mixed"])
def test_workload_parity(wid):
    check(batch(wid), wid)


RAGGED = [
    # (workload for dtype/shape defaults, lengths, overrides)
    ("tiny", ((1, 2, 3, 17, 64, 0), (1, 9, 40, 17, 64, 30)), {}),
    ("tiny", ((4, 5, 1), (4, 70, 129)), dict(heads=(16, 4))),          # qo*g = 16 / 20 / 4
    ("tiny", ((33, 1), (50, 100)), dict(causal=False)),
    ("tiny", ((20, 1, 3), (100, 300, 31)), dict(head_dim=128, page_size=64)),
    ("mixed", ((1, 2, 4, 5), (33, 65, 1000, 4000)), {}),                 # qo*g = 4 .. 20
    ("mixed", ((1, 16, 17, 100), (1, 16, 17, 100)), dict(heads=(16, 16))),
    ("mixed", ((1, 1, 200), (5000, 31, 1000)), dict(heads=(16, 1), page_size=128)),
    ("mixed", ((300, 1, 3), (300, 777, 64)), dict(heads=(24, 8), page_size=32)),
    ("mixed", ((129, 1), (257, 257)), dict(head_dim=64, page_size=64)),
    ("mixed", ((70, 1, 2), (90, 333, 65)), dict(causal=False)),
    ("prefill", ((513, 1), (1000, 1)), dict(heads=(8, 8))),
    ("long", ((1000, 1, 1), (3000, 3000, 64)), dict(heads=(64, 8))),    # long at reduced size
    ("long", ((48, 2), (96, 4100)), dict(heads=(128, 1), page_size=16)),  # g = 128
    # wide decode row groups (qo * g of 17 .. 64 rows: 32-row units, and two
    # 32-row units per chunk side by side above 32 rows) over long caches
    ("long", ((1, 1, 1), (16500, 700, 33)), dict(heads=(256, 8))),       # g = 32
    ("long", ((1, 1), (17000, 900)), dict(heads=(64, 1))),               # g = 64
    ("long", ((4, 4, 1, 2), (16400, 500, 3000, 90)), dict(heads=(64, 8))),  # qo = 4 at g = 8
    ("mixed", ((1, 3, 8, 1, 9), (2500, 4100, 300, 60, 700)), dict(heads=(64, 8))),  # 8/24/64/8/72 rows
    ("mixed", ((1, 1, 2), (3000, 70, 1500)), dict(heads=(33, 1))),         # 33 / 33 / 66 rows
    ("mixed", ((1, 3, 2), (1800, 2000, 45)), dict(heads=(48, 3))),         # 16 / 48 / 32 rows
    ("tiny", ((5, 9, 2), (40, 300, 17)), dict(heads=(28, 4))),             # fp32: 35 / 63 / 14 rows
    # paired 64-row groups at head_dim 64 and page 16 (their four shared V
    # stages are 4 KiB each), with a 33-row group beside them
    ("mixed", ((1, 1, 1), (5000, 37, 1200)), dict(heads=(64, 1), head_dim=64, page_size=16)),
    ("mixed", ((1, 3), (2100, 900)), dict(heads=(33, 3), head_dim=64)),   # 11 / 33 rows
]


@pytest.mark.parametrize("idx", range(len(RAGGED)))
def test_ragged_parity(idx):
    wid, lengths, kw = RAGGED[idx]
    check(batch(wid, lengths, **kw), f"ragged{idx}")


def rising_logits(b, nats_per_key: float = 1.0):
    """Make the logits rise along each request's keys: Q[..., 0] = 8 and
    K[j, :, 0] += r j with 8 r sm_scale = nats_per_key.  At one nat per key
    every 64-key tile's maximum exceeds the running maximum by about 92 in
    log2 units, so the speculative softmax must rescale O and l at every
    tile of every prefill row and every step of every decode row."""
    to32 = lambda a: a.astype(np.float32) if b.dtype == "f32" else bf16_bits_to_f32(a)
    back = lambda a: a.astype(np.float32) if b.dtype == "f32" else f32_to_bf16_bits(a)
    q, k = to32(b.q).copy(), to32(b.k).copy()
    q[:, :, 0] = 8.0
    r = nats_per_key / (8.0 * b.sm_scale)
    for i in range(b.B):
        s, e = int(b.kv_indptr[i]), int(b.kv_indptr[i + 1])
        k[s:e, :, 0] += np.float32(r) * np.arange(e - s, dtype=np.float32)[:, None]
    b.q, b.k = back(q), back(k)
    return b


@pytest.mark.parametrize("nats", [1.0, 0.05])
def test_rising_logits(nats):
    """The rescale path of the speculative softmax on every tile (1 nat per
    key) and on some tiles only (0.05 nat per key: about 4.6 log2 units per
    tile, so a rescale every dozen or so tiles), prefill and decode rows."""
    check(rising_logits(make_batch("mixed", lengths=((300, 1, 2), (300, 2000, 900)), heads=(16, 4)), nats),
          f"rising{nats}")
    check(rising_logits(make_batch("tiny", lengths=((40, 1), (100, 300))), nats), f"rising{nats}_f32")
    check(rising_logits(make_batch("mixed", lengths=((1, 1, 3), (2000, 333, 900)), heads=(64, 2)), nats),
          f"rising{nats}_wide")


@pytest.mark.parametrize("log2_scale,nats", [(20, 1.0), (40, 0.6)])
def test_large_values_scale_exactly(log2_scale, nats):
    """V times 2^k (exact in bf16) under rising logits: every output row is
    the unscaled run's times 2^k bit for bit and the LSE is unchanged.  At
    0.6 nat per key a 64-key tile raises the logits by about 38 nats, below
    the speculative softmax's rescale trigger (weights of 2^64), so weights
    up to about 2^55 multiply values up to 2^44 in the fp32 accumulators; the
    exact scaling shows that nothing overflows or rounds differently.  The
    scaled-back rows meet the usual bar against the oracle."""
    def make():
        return rising_logits(make_batch("mixed", lengths=((300, 1, 2), (300, 2000, 900)), heads=(16, 4)), nats)
    base, big = make(), make()
    big.v = f32_to_bf16_bits(bf16_bits_to_f32(big.v) * np.float32(2.0 ** log2_scale))
    assert np.array_equal(bf16_bits_to_f32(big.v), bf16_bits_to_f32(base.v) * np.float32(2.0 ** log2_scale))
    out0, lse0 = DeviceRun(base).step()
    out1, lse1 = DeviceRun(big).step()
    assert np.isfinite(out1).all()
    assert np.array_equal(out1, out0 * np.float32(2.0 ** log2_scale))
    assert np.array_equal(lse1.view(np.uint32), lse0.view(np.uint32))
    O, _ = oracle_outputs(base)
    assert report(f"large{log2_scale}", out1 / np.float32(2.0 ** log2_scale), O) <= tolerance(base)


def test_sharpened_softmax():
    """Q scaled by 8: logits of order 8, far from uniform weights."""
    check(batch("mixed", ((200, 1, 1), (260, 900, 33)), q_gain=8.0), "sharp")
    check(batch("tiny", ((16, 1), (33, 40)), q_gain=8.0), "sharp_f32")


@pytest.mark.parametrize("chunk", [32, 96, 512])
def test_split_count_invariance(chunk):
    # 16-row, 32-row and paired 64-row decode units (a forced chunk gives one
    # unit per queue: the paired queues then hold a single unit each)
    for heads in ((32, 8), (64, 2), (128, 2)):
        b = batch("mixed", ((1, 2, 1, 3), (4000, 3000, 2048, 700)), heads=heads)
        out0, _ = DeviceRun(b).step()
        out1, _ = check(b, f"split{chunk}_{heads}", chunk=chunk)
        assert np.abs(out1 - out0).max() <= 2 * tolerance(b)


QUEUE_CASES = [
    # (workload, lengths, overrides, planner CUs, chunk): few CUs give every
    # wavefront a long span of keys crossing many row groups (requests,
    # heads, unit kinds), so its queue holds many units
    ("mixed", ((1, 2, 1, 3, 1, 0, 1), (4000, 3000, 2048, 700, 1, 5, 33)), {}, 1, 0),
    ("mixed", ((1, 3, 8, 1, 2), (2500, 4100, 300, 60, 900)), dict(heads=(64, 8)), 2, 0),
    ("mixed", ((1, 1, 1, 1), (3000, 95, 1500, 40)), dict(heads=(64, 1)), 1, 0),
    ("decode", None, {}, 4, 0),
    ("tiny", ((5, 9, 2, 1), (40, 300, 17, 100)), dict(heads=(28, 4)), 1, 0),
]


@pytest.mark.parametrize("idx", range(len(QUEUE_CASES)))
def test_decode_queues_of_many_units(idx):
    wid, lengths, kw, cus, chunk = QUEUE_CASES[idx]
    b = batch(wid, lengths, **kw)
    run = DeviceRun(b, decode_chunk_keys=chunk, num_cus=cus)
    dq = run.plan.work_items(4)[:, 0]
    assert np.diff(dq).max() >= 3, "the case should queue several units per wavefront"
    print(f"case queues{idx}: {len(dq) - 1} queues, up to {np.diff(dq).max()} units each", flush=True)
    out, lse = run.step()
    O, L = oracle_outputs(b)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert report(f"queues{idx}", out, O) <= tolerance(b)
    assert np.abs(lse - L).max() <= lse_tol(b) + 2.0 ** -20 * np.abs(L).max()


PREFILL4_CASES = [
    # prefill-only batches in 128-row tiles of 4-wavefront blocks (two blocks
    # per CU): g = 1 / 4 / 32 (32 / 4 tokens per tile), head_dim 64,
    # non-causal, chunks over cached keys, caches past the automatic limit
    ("prefill", None, {}),                                                  # the 8 x 512 workload (default plan)
    ("prefill", ((300, 513, 129, 700), (300, 513, 129, 700)), dict(heads=(8, 8))),
    ("prefill", ((257, 90), (1000, 800)), dict(heads=(16, 4))),             # chunked prefill over cached keys
    ("prefill", ((400, 70), (400, 900)), dict(heads=(8, 2), causal=False)),
    ("prefill", ((320, 513), (320, 513)), dict(heads=(8, 8), head_dim=64, page_size=64)),
    ("prefill", ((37, 300), (900, 5000)), dict(heads=(32, 1), page_size=64)),  # g = 32: 4-token tiles
    ("prefill", ((3000, 65), (9000, 100)), dict(heads=(8, 8))),             # long caches, a 65-row tail tile
]


@pytest.mark.parametrize("idx", range(len(PREFILL4_CASES)))
def test_prefill_four_wave_blocks(idx):
    wid, lengths, kw = PREFILL4_CASES[idx]
    b = batch(wid, lengths, **kw)
    run = DeviceRun(b, prefill_block_waves=4)
    pf = run.plan.work_items(0)
    assert len(pf) and (pf[:, 3] * (b.H_q // b.H_kv) <= 128).all()
    print(f"case pf4_{idx}: {len(pf)} tiles of <= 128 rows", flush=True)
    out, lse = run.step()
    O, L = oracle_outputs(b)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert report(f"pf4_{idx}", out, O) <= tolerance(b)
    assert np.abs(lse - L).max() <= lse_tol(b) + 2.0 ** -20 * np.abs(L).max()
    # 256-row tiles of 8-wavefront blocks give the same rows to rounding
    out8, _ = DeviceRun(b, prefill_block_waves=8).step()
    assert np.abs(out8 - out).max() <= tolerance(b)


def test_bitwise_deterministic_for_a_fixed_plan():
    b = batch("mixed", ((300, 1, 1, 2), (300, 4000, 1500, 700)))
    run = DeviceRun(b)
    run.append()
    run.attention()
    torch.cuda.synchronize()
    first = run.out.clone(), run.lse.clone()
    for _ in range(3):
        run.attention()
    torch.cuda.synchronize()
    assert torch.equal(first[0], run.out) and torch.equal(first[1], run.lse)


def test_decode_step_equals_last_prefill_row():
    """The held-back-token handoff (post, section "Speculative Decoding"): a
    decode step over the cache of a prefill equals that prefill's last row."""
    L = 777
    full = batch("mixed", ((L,), (L,)))
    dec = make_batch("mixed", lengths=([1], [L]))
    dec.q = full.q[-1:].copy()
    dec.k, dec.v = full.k, full.v
    out_f, lse_f = DeviceRun(full).step()
    out_d, lse_d = DeviceRun(dec).step()
    O, L_ = OA.attend(full.to_f64(full.q[-1:]), full.to_f64(full.k), full.to_f64(full.v), [L - 1],
                      full.sm_scale)
    assert np.abs(out_d[0] - O[0]).max() <= tolerance(full)
    assert np.abs(out_f[-1] - O[0]).max() <= tolerance(full)
    assert np.abs(out_d[0] - out_f[-1]).max() <= 2 * tolerance(full)
    assert np.abs(lse_d[0] - lse_f[-1]).max() <= 2 * lse_tol(full)


def test_chunked_prefill_equals_full():
    """Prefill in two chunks (the second attending over the first's KV)
    equals one prefill (kwkr.cn survey, section 8)."""
    L, c = 600, 250
    full = batch("mixed", ((L,), (L,)))
    out_f, _ = DeviceRun(full).step()
    second = make_batch("mixed", lengths=([L - c], [L]))
    second.q = full.q[c:].copy()
    second.k, second.v = full.k, full.v
    out_2, _ = DeviceRun(second).step()
    first = make_batch("mixed", lengths=([c], [c]))
    first.q = full.q[:c].copy()
    first.k, first.v = full.k[:c].copy(), full.v[:c].copy()
    out_1, _ = DeviceRun(first).step()
    got = np.concatenate([out_1, out_2])
    O, _ = oracle_outputs(full)
    assert np.abs(got - O).max() <= tolerance(full)
    assert np.abs(got - out_f).max() <= 2 * tolerance(full)


@pytest.mark.parametrize("cus", [16, 64])
def test_mixed_launch_chunked_decode(cus):
    """A prompt with a prefill tile per CU or more beside decodes of 1, 5
    and 9 tokens (16-row, 32-row and paired 64-row groups at g = 4): the
    decode groups are cut into chunks sized to the prefill tiles (many
    pieces per group, a ragged last piece) and interleaved with the tiles;
    every row at parity."""
    qo = [512, 1, 1, 5, 1, 9, 1, 1, 1]
    kv = [512, 3000, 5000, 700, 1500, 4100, 257, 33, 2049]
    b = batch("mixed", (tuple(qo), tuple(kv)))
    run = DeviceRun(b, num_cus=cus)
    dq = run.plan.work_items(4)[:, 0]
    assert (np.diff(dq) == 1).all() and len(dq) > 100        # one chunk per queue, many chunks
    print(f"case chunked_{cus}: {len(dq) - 1} decode units", flush=True)
    out, lse = run.step()
    O, L = oracle_outputs(b)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert report(f"chunked_{cus}", out, O) <= tolerance(b)
    assert np.abs(lse - L).max() <= lse_tol(b) + 2.0 ** -20 * np.abs(L).max()


@pytest.mark.parametrize("L", [128, 1024])
def test_interference_sweep_batches(L):
    """The interference sweep's 1PnD batch (one causal prompt of L tokens
    plus decodes over caches of L tokens, the mixed workload's shapes) at
    parity, and its decode-only / prefill-only halves equal to the mixed
    launch's rows (kwkr.cn survey, section 2)."""
    n = 8
    qo, kv = [L] + [1] * n, [L] * (n + 1)
    b = make_batch("mixed", lengths=(qo, kv))
    out_m, lse_m = check(b, f"sweep{L}")
    for keep in ("decode", "prefill"):
        sel = np.array([keep == "prefill"] + [keep == "decode"] * n)
        part = make_batch("mixed", lengths=(list(np.where(sel, qo, 0)), kv))
        part.q = b.q[np.repeat(sel, qo)].copy()
        part.k, part.v = b.k, b.v
        out_p, _ = DeviceRun(part).step()
        rows = np.repeat(sel, qo)
        assert np.abs(out_p - out_m[rows]).max() <= 2 * tolerance(b)


def test_step_in_graph_replays():
    """The whole step (append, the attention launch and its merge, pack and
    unpack of a request's pages) captured once in a HIP graph and replayed
    three times, with the pool restored and the outputs poisoned eagerly in
    between: every replay equals the eager step bit for bit (the step holds
    kernel launches only, with the page ids in the transfer's arguments, so
    it can be captured; post, section "KV Messenger")."""
    b = batch("mixed")
    m = pd()
    run = DeviceRun(b)
    pool0 = run.pool.clone()
    ids = b.request_pages(0)
    dst = np.random.default_rng(3).permutation(b.spare_pages)[:len(ids)].astype(np.int32)
    assert 0 < len(ids) <= len(dst)
    nbytes = m.pd_kv_pack_bytes(run.desc, len(ids))
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    scratch = torch.empty(4 * len(ids), dtype=torch.uint8, device="cuda")

    def step():
        run.append()
        run.attention()
        m.pd_kv_pack(run.desc, run.pool, b.num_pool_pages, ids, buf, scratch)
        m.pd_kv_unpack(run.desc, run.pool, b.num_pool_pages, dst, buf, scratch)

    step()  # eager reference (also loads every kernel before the capture)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (run.out, run.lse, buf, run.pool)]
    n = int(b.qo_indptr[-1])
    O, _ = oracle_outputs(b)
    assert report("graph eager", run.out[:n].cpu().numpy(), O) <= tolerance(b)
    g = torch.cuda.CUDAGraph()
    run.pool.copy_(pool0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        run.pool.copy_(pool0)           # eager work between replays
        run.out.fill_(float("nan"))
        run.lse.fill_(float("nan"))
        buf.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = [torch.equal(a.view(torch.uint8), r.view(torch.uint8))
                for a, r in zip((run.out, run.lse, buf, run.pool), ref)]
        print(f"replay {rep}: out/lse/buf/pool bitwise equal {same}", flush=True)
        assert all(same)
