#!/usr/bin/env python3
"""Benchmark of the ragged paged-attention hot path on one MI355X.

One step = the whole path over one batch of the long-context workload (an
8192-token causal chunk over 24576 cached tokens plus 256 single-token
decodes over 32768 cached tokens; 64 query / 8 KV heads, head_dim 128, bf16,
page size 64; pool of 138164 pages = 36.2 GB, drawn on the device):

  pd_plan + pd_plan_upload   host planning of the ragged batch, table upload
  pd_kv_append               8448 new K/V rows into their pages
  pd_attention_run           prefill tiles + split-KV decode units in one
                             launch, then the partial-result merge
  pd_kv_pack / pd_kv_unpack  the chunk request's 512 pages (128 MiB) into a
                             transfer buffer and back into other pages

It is the one workload whose step exercises every part of the path.  Inputs
are resident in HBM before the timed region.  W warm-up steps, then K timed
steps between device synchronisations; per-phase times come from HIP events
recorded on the launch stream (torch's current stream, which the binding
launches on).  Each step streams the 34 GB decode cache, which evicts the L2
and the MALL by itself.

Afterwards, untimed legs measure:
  * decode-only and prefill-only plans over the same pool (per-phase GB/s and
    TFLOP/s, interference ratio);
  * the decode (64 x kv U{512..4096}, 40/40 heads), prefill (8 x 512 causal,
    40/40 heads) and mixed (one 1024-token prefill + 63 decodes, 32/8 heads)
    workloads;
  * transfers, the interference sweep and the latent-cache decode;
  * the CPU oracle on a bounded sample, over a process pool.
Every leg times one call per repetition with HIP events after reading a
1 GiB buffer (so L2 and MALL start cold), and reports median, min and p90;
calls shorter than 50 us are also timed as 100 back-to-back launches.

Prints one JSON line.  ``value`` is the step's attainment of the MI355X
roofline in percent: the ideal time of the step's algorithmic work at peak
(attention launch: max of its decode bytes / 8 TB/s and its prefill flops /
2.5 PFLOP/s; append, pack, unpack: bytes / 8 TB/s) divided by the measured
time per step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E, 8 TB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, 2.5 PFLOP/s
METRIC = "decode attn HBM GB/s + prefill attn TFLOP/s (% of MI355X peak), 1 GPU"
SHORT_MS = 0.05              # calls shorter than this are also timed back to back
B2B_LAUNCHES = 100


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--reps", type=int, default=20, help="timed repetitions of each leg")
    ap.add_argument("--leg-warmup", type=int, default=5, help="untimed calls before each leg")
    ap.add_argument("--no-phases", action="store_true", help="skip the decode-only / prefill-only legs")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the decode / prefill / mixed workload legs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-transfers", action="store_true",
                    help="skip the pack / unpack, head-range and multi-layer transfer legs")
    ap.add_argument("--layers", type=int, default=8, help="layers of the multi-layer pack leg")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the interference / chunked-prefill sweep")
    ap.add_argument("--sweep-decodes", type=int, default=32, help="decodes in the 1PnD sweep batches")
    ap.add_argument("--no-mla", action="store_true", help="skip the latent-cache (MLA) decode legs")
    ap.add_argument("--loop", choices=("prefill", "decode", "mixed"), default=None,
                    help="only run one attention launch kind of the workload back to back for "
                         "--loop-seconds (for sampling board power and clocks from another process)")
    ap.add_argument("--loop-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle processes (0: the host's available cores, at most 16)")
    ap.add_argument("--cpu-decode-rows", type=int, default=8, help="decode rows per oracle process")
    ap.add_argument("--cpu-prefill-rows", type=int, default=6, help="prefill-chunk rows per oracle process")
    return ap.parse_args()


def algorithmic_work(b, elt=2):
    """What the method must move or compute, not the dense work it avoids.
    Decode requests (qo = 1) read their K/V once, read Q and write O (fp32):
    decode bytes.  Prefill requests (qo > 1) do 4 D flops per visible
    (query, key) pair per query head: prefill flops; their compulsory bytes
    are Q, K/V and O.  Append reads and writes each new row."""
    dec_bytes = pre_bytes = flops = 0
    for qo, kv in zip(b.qo_lens.tolist(), b.kv_lens.tolist()):
        if qo == 0:
            continue
        kvb = 2 * kv * b.H_kv * b.D * elt
        qob = qo * b.H_q * b.D * (elt + 4)
        if qo == 1:
            dec_bytes += kvb + qob
        else:
            pre_bytes += kvb + qob
            pairs = qo * (kv - qo) + qo * (qo + 1) // 2 if b.causal else qo * kv
            flops += 4 * b.D * b.H_q * pairs
    rows = int(b.qo_lens.sum())
    append_bytes = 2 * (2 * rows * b.H_kv * b.D * elt)
    return dict(decode_bytes=dec_bytes, prefill_bytes=pre_bytes, prefill_flops=flops,
                append_bytes=append_bytes)


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed PMC summary
    (FETCH_SIZE and WRITE_SIZE runs, calibrated on the pack kernel's known
    copy size), or None when the kernels or the planner (which decides the
    launch's blocks and their order) changed since the counters were taken:
    the summary records both sources' hashes."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attention_long_pmc_traffic.txt")
    csrc = os.path.join(ROOT, "decode_attention_kv_pd_amd", "csrc")
    if workload != "long" or not os.path.exists(path):
        return None

    def digest(name):
        return hashlib.sha256(open(os.path.join(csrc, name), "rb").read()).hexdigest()[:16]

    want = {"attention_sha256_16": digest("attention.hip"), "planner_sha256_16": digest("api.cpp")}
    for line in open(path):
        if line.startswith("TRAFFIC "):
            kv = dict(t.split("=", 1) for t in line.split()[1:])
            if all(kv.get(k) == v for k, v in want.items()):
                return int(kv["bytes_per_launch"])
    return None


def spread(ts):
    ts = np.asarray(ts, np.float64)
    return {"median": round(float(np.median(ts)), 4), "min": round(float(ts.min()), 4),
            "p90": round(float(np.percentile(ts, 90)), 4), "mean": round(float(ts.mean()), 4),
            "reps": int(ts.size)}


class Meter:
    """Times device calls with HIP events on torch's current stream, which is
    the stream the binding launches on."""

    def __init__(self, torch, reps, warmup, flush_bytes=1 << 30):
        self.torch = torch
        self.reps = reps
        self.warmup = warmup
        self.flush_buf = torch.ones(flush_bytes // 4, dtype=torch.int32, device="cuda")
        self.flush_out = torch.empty((), dtype=torch.int64, device="cuda")

    def flush(self):
        # reads 1 GiB (a sum): replaces the L2 of every XCD and the MALL with
        # clean lines, so the timed call neither hits its own data nor pays for
        # writing back someone else's
        self.torch.sum(self.flush_buf, 0, dtype=self.torch.int64, out=self.flush_out)

    def time(self, fn, flush=True, b2b=None):
        torch = self.torch
        for _ in range(self.warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(self.reps):
            if flush:
                self.flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        r = spread(ts)
        r["flushed"] = bool(flush)
        if b2b or (b2b is None and r["median"] < SHORT_MS):
            if flush:
                self.flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(B2B_LAUNCHES):
                fn()
            e1.record()
            torch.cuda.synchronize()
            r["b2b100_ms"] = round(e0.elapsed_time(e1) / B2B_LAUNCHES, 4)
        return r


# ------------------------------------------------------------------ CPU oracle
def _cpu_worker(idx, barrier, out_q, spec):
    """One oracle process: draws its share of the sample (the workload's
    distribution), waits for every process, then times its oracle calls."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as OA
    from workloads import bf16_bits_to_f32, f32_to_bf16_bits

    rng = np.random.default_rng(np.random.SeedSequence([2026, spec["wid"], 99, idx]))

    def draw(*shape):
        return bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))).astype(np.float64)

    kv, qo, H_q, H_kv, D = spec["kv"], spec["qo"], spec["H_q"], spec["H_kv"], spec["D"]
    k, v = draw(kv, H_kv, D), draw(kv, H_kv, D)           # one cache, shared by this process's rows
    qd = draw(spec["n_dec"], H_q, D)
    toks = rng.integers(0, qo, size=spec["n_pre"])         # prefill-chunk rows at random positions
    qp = draw(spec["n_pre"], H_q, D)
    with threadpool_limits(limits=1):
        barrier.wait(timeout=300)
        t0 = time.perf_counter()
        for i in range(spec["n_dec"]):
            OA.attend(qd[i:i + 1], k, v, np.array([kv - 1]), spec["scale"], True)
        t1 = time.perf_counter()
        for i in range(spec["n_pre"]):
            OA.attend(qp[i:i + 1], k, v, np.array([kv - qo + int(toks[i])]), spec["scale"], True)
        t2 = time.perf_counter()
    dec_bytes = spec["n_dec"] * (2 * kv * H_kv * D * 2 + H_q * D * 6)
    flops = int(sum(4 * D * H_q * (kv - qo + int(t) + 1) for t in toks))
    out_q.put((idx, t0, t1, t2, dec_bytes, flops))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(b, workers, n_dec, n_pre):
    """The float64 oracle timed on the host's cores: `workers` processes
    (one BLAS thread each), each computing n_dec decode rows (64 heads over a
    32768-token cache) and n_pre rows of the 8192-token chunk (64 heads, over
    its causal key range).  Throughput = the sample's work over the wall time
    from the moment every process has its inputs drawn to the moment the last
    one finishes, in the step's unit."""
    import multiprocessing as mp

    if workers <= 0:
        try:
            avail = len(os.sched_getaffinity(0))
        except AttributeError:
            avail = os.cpu_count() or 1
        workers = max(1, min(avail, 16))
    spec = {"wid": b.wid, "kv": int(b.kv_lens[0]), "qo": int(b.qo_lens[0]), "H_q": b.H_q, "H_kv": b.H_kv,
            "D": b.D, "scale": b.sm_scale, "n_dec": n_dec, "n_pre": n_pre}
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(workers)
    q = ctx.Queue()
    procs = [ctx.Process(target=_cpu_worker, args=(i, barrier, q, spec)) for i in range(workers)]
    for p in procs:
        p.start()
    res = [q.get(timeout=900) for _ in procs]
    for p in procs:
        p.join()
    t_start = min(r[1] for r in res)
    t_dec_end = max(r[2] for r in res)
    t_end = max(r[3] for r in res)
    dec_bytes = sum(r[4] for r in res)
    flops = sum(r[5] for r in res)
    secs = t_end - t_start
    ideal = dec_bytes / (PEAK_HBM_GBPS * 1e9) + flops / (PEAK_BF16_TFLOPS * 1e12)
    busy = sum(r[3] - r[1] for r in res)
    return {"value": 100.0 * ideal / secs, "unit": "% of MI355X peak", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{workers} processes x ({n_dec} decode rows x {b.H_q} heads over {spec['kv']} keys + "
                      f"{n_pre} chunk rows x {b.H_q} heads at random chunk positions); float64 numpy "
                      f"oracle, one BLAS thread per process, each process with its own drawn cache",
            "seconds": round(secs, 3), "cpu_seconds": round(busy, 3),
            "decode_GBps": round(dec_bytes / max(t_dec_end - t_start, 1e-9) / 1e9, 4),
            "prefill_TFLOPs": round(flops / max(t_end - t_dec_end, 1e-9) / 1e12, 6)}


# ------------------------------------------------------------------- helpers
def device_inputs(torch, b, pd, salt=0):
    """Pool, Q, new K/V, outputs of a workload, drawn on the device."""
    from workloads import device_normal_, device_seed
    n = max(int(b.qo_lens.sum()), 1)
    t = {"pool": device_normal_(torch.empty(b.pool_shape, dtype=torch.bfloat16, device="cuda"),
                                device_seed(b.wid, salt, 0)),
         "q": device_normal_(torch.empty((n, b.H_q, b.D), dtype=torch.bfloat16, device="cuda"),
                             device_seed(b.wid, salt, 1)),
         "k_new": device_normal_(torch.empty((n, b.H_kv, b.D), dtype=torch.bfloat16, device="cuda"),
                                 device_seed(b.wid, salt, 2)),
         "v_new": device_normal_(torch.empty((n, b.H_kv, b.D), dtype=torch.bfloat16, device="cuda"),
                                 device_seed(b.wid, salt, 3)),
         "out": torch.empty((n, b.H_q, b.D), dtype=torch.float32, device="cuda"),
         "lse": torch.empty((n, b.H_q), dtype=torch.float32, device="cuda")}
    return t


def sub_plan(pd, torch, b, desc, sel, q, **kw):
    """Plan, workspace, Q rows and outputs for the requests selected by `sel`
    (the others get qo = 0), over the same pool."""
    qo = np.where(sel, b.qo_lens, 0).astype(np.int32)
    p = pd.pd_plan(desc, qo, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages, **kw)
    ws = torch.empty(max(p.workspace_bytes, 1), dtype=torch.uint8, device="cuda")
    pd.pd_plan_upload(p, ws)
    idx = np.concatenate([np.arange(b.qo_indptr[r], b.qo_indptr[r + 1]) for r in range(b.B) if sel[r]])
    qs = q[torch.as_tensor(idx, device="cuda")].contiguous()
    o = torch.empty((len(idx), b.H_q, b.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((len(idx), b.H_q), dtype=torch.float32, device="cuda")
    return p, ws, qs, o, lse


def roofline_entry(w, t_ms):
    """Per-phase figures of one attention call of t_ms against MI355X peaks."""
    hbm_ms = w["decode_bytes"] / (PEAK_HBM_GBPS * 1e9) * 1e3
    mfma_ms = w["prefill_flops"] / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    return {"decode_GBps": round(w["decode_bytes"] / (t_ms * 1e-3) / 1e9, 1),
            "prefill_TFLOPs": round(w["prefill_flops"] / (t_ms * 1e-3) / 1e12, 1),
            "roofline_frac_strict": round(max(hbm_ms, mfma_ms) / t_ms, 4),
            "roofline_frac_sum": round((hbm_ms + mfma_ms) / t_ms, 4)}


# --------------------------------------------------- decode / prefill / mixed
def config_legs(args, pd, torch, meter):
    """The decode, prefill and mixed workloads, each on its own pool: append
    and attention timed per call (flushed caches), with per-phase rates, the
    prefill workload's attainable rate (its compulsory Q, K/V and O bytes
    make it HBM-bound when the caches are cold) and, for the mixed workload,
    decode-only and prefill-only plans and the interference ratio."""
    from workloads import make_batch

    res = {}
    for wid in ("decode", "prefill", "mixed"):
        b = make_batch(wid, materialize=False)
        desc = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype, b.causal, b.sm_scale)
        t = device_inputs(torch, b, pd)
        w = algorithmic_work(b)
        h0 = time.perf_counter()
        plan = pd.pd_plan(desc, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages)
        plan_ms = (time.perf_counter() - h0) * 1e3
        ws = torch.empty(max(plan.workspace_bytes, 1), dtype=torch.uint8, device="cuda")
        pd.pd_plan_upload(plan, ws)
        app = meter.time(lambda: pd.pd_kv_append(plan, ws, t["pool"], t["k_new"], t["v_new"]))
        # the short prompts are also timed back to back (warm L2, MALL and TLB),
        # which separates the cold-cache cost from the kernel's own
        att = meter.time(lambda: pd.pd_attention_run(plan, ws, t["q"], t["pool"], t["out"], t["lse"]),
                         b2b=True if wid == "prefill" else None)
        assert torch.isfinite(t["out"]).all().item(), f"{wid}: non-finite attention output"
        st = plan.stats()
        e = {"shape": f"B {b.B}, H {b.H_q}/{b.H_kv}, D {b.D}, page {b.ps}, bf16",
             "plan_host_ms": round(plan_ms, 4),
             "plan": {"prefill_tiles": st.prefill_tiles, "decode_units": st.decode_units,
                      "decode_chunk_keys": st.decode_chunk_keys},
             "append_ms": app, "append_GBps": round(w["append_bytes"] / (app["median"] * 1e-3) / 1e9, 1),
             "attention_ms": att}
        tm = att["median"]
        if wid == "decode":
            gbps = w["decode_bytes"] / (tm * 1e-3) / 1e9
            e.update({"decode_bytes": w["decode_bytes"], "GBps": round(gbps, 1),
                      "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4), "target_ms_at_70pct":
                      round(w["decode_bytes"] / (0.7 * PEAK_HBM_GBPS * 1e9) * 1e3, 4)})
        elif wid == "prefill":
            tf = w["prefill_flops"] / (tm * 1e-3) / 1e12
            t_mfma = w["prefill_flops"] / (PEAK_BF16_TFLOPS * 1e12) * 1e3
            t_hbm = w["prefill_bytes"] / (PEAK_HBM_GBPS * 1e9) * 1e3
            t_att = max(t_mfma, t_hbm)
            e.update({"prefill_flops": w["prefill_flops"], "compulsory_bytes": w["prefill_bytes"],
                      "TFLOPs": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                      "attainable_ms": round(t_att, 4), "frac_of_attainable": round(t_att / tm, 4)})
            if "b2b100_ms" in att:
                e["frac_of_attainable_b2b"] = round(t_att / att["b2b100_ms"], 4)
        else:
            e.update({"decode_bytes": w["decode_bytes"], "prefill_flops": w["prefill_flops"]})
            e.update(roofline_entry(w, tm))
            dec = b.qo_lens == 1
            for name, sel in (("decode_only", dec), ("prefill_only", ~dec)):
                p, wsp, qs, o, lse = sub_plan(pd, torch, b, desc, sel, t["q"])
                r = meter.time(lambda: pd.pd_attention_run(p, wsp, qs, t["pool"], o, lse))
                if name == "decode_only":
                    r["GBps"] = round(w["decode_bytes"] / (r["median"] * 1e-3) / 1e9, 1)
                    r["frac_of_peak"] = round(r["GBps"] / PEAK_HBM_GBPS, 4)
                else:
                    r["TFLOPs"] = round(w["prefill_flops"] / (r["median"] * 1e-3) / 1e12, 1)
                    r["frac_of_peak"] = round(r["TFLOPs"] / PEAK_BF16_TFLOPS, 4)
                e[name] = r
                p.close()
            e["interference_ratio"] = round(tm / e["decode_only"]["median"], 3)
            e["mixed_vs_sum"] = round(tm / (e["decode_only"]["median"] + e["prefill_only"]["median"]), 3)
        res[wid] = e
        plan.close()
        del t, ws
        torch.cuda.synchronize()
        print(f"[bench] {wid} workload leg done", file=sys.stderr, flush=True)
    res["wide_decode"] = wide_decode_legs(pd, torch, meter)
    return res


def wide_decode_legs(pd, torch, meter):
    """Decode rows of more than 16 query rows per KV head (post, sections
    "Speculative Decoding": multi-token steps, and "Prefill vs Decode
    performance": decode spread over kv_len): 64 requests over 16384-token
    caches, 8 KV heads, head_dim 128, page 64, bf16, with 32 query heads per
    KV head (g = 32), 64 (g = 64), and 4-token steps at g = 8 (32 rows).
    Algorithmic bytes: K/V read once plus Q and O."""
    from workloads import make_batch

    res = {}
    for name, heads, qo in (("g32", (256, 8), 1), ("g64", (512, 8), 1), ("qo4_g8", (64, 8), 4)):
        n = 64
        b = make_batch("long", lengths=([qo] * n, [16384] * n), heads=heads, materialize=False)
        desc = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype, b.causal, b.sm_scale)
        t = device_inputs(torch, b, pd, salt=7)
        plan = pd.pd_plan(desc, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages)
        ws = torch.empty(max(plan.workspace_bytes, 1), dtype=torch.uint8, device="cuda")
        pd.pd_plan_upload(plan, ws)
        r = meter.time(lambda: pd.pd_attention_run(plan, ws, t["q"], t["pool"], t["out"], t["lse"]))
        assert torch.isfinite(t["out"]).all().item(), f"{name}: non-finite attention output"
        nbytes = 2 * int(b.kv_lens.astype(np.int64).sum()) * b.H_kv * b.D * 2 + int(b.qo_lens.sum()) * b.H_q * b.D * 6
        gbps = nbytes / (r["median"] * 1e-3) / 1e9
        st = plan.stats()
        res[name] = {"shape": f"64 x (qo {qo}, kv 16384), H {b.H_q}/{b.H_kv} (rows per KV head {qo * b.H_q // b.H_kv})",
                     "ms": r, "bytes": nbytes, "GBps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
                     "decode_units": st.decode_units, "prefill_tiles": st.prefill_tiles,
                     "chunk_keys": st.decode_chunk_keys}
        plan.close()
        del t, ws
        torch.cuda.synchronize()
    print(f"[bench] wide decode legs done", file=sys.stderr, flush=True)
    return res


# ------------------------------------------------------------------ transfers
def transfer_legs(args, pd, torch, meter, b, desc, pool, pack_ids, unpack_ids):
    """Pack / unpack of the chunk request's pages (whole pages, then half of
    the KV heads: what a rank sends when the decoder has twice the
    prefiller's TP degree), timed per call after a cache flush, and a
    multi-layer pack of the same page count over `--layers` layer pools in
    one launch, with per-layer progress counters in pinned host memory
    polled from the host.  Bytes are read + written."""
    from workloads import device_normal_, device_seed

    out = {}
    n = len(pack_ids)
    nb = pd.pd_kv_pack_bytes(desc, n)
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
    scr = torch.empty(4 * n, dtype=torch.uint8, device="cuda")
    r = meter.time(lambda: pd.pd_kv_pack(desc, pool, b.num_pool_pages, pack_ids, buf, scr))
    out["pack"] = {"pages": n, "bytes": nb, "ms": r, "GBps": round(2 * nb / (r["median"] * 1e-3) / 1e9, 1)}
    r = meter.time(lambda: pd.pd_kv_unpack(desc, pool, b.num_pool_pages, unpack_ids, buf, scr))
    out["unpack"] = {"ms": r, "GBps": round(2 * nb / (r["median"] * 1e-3) / 1e9, 1)}
    del buf
    h1 = b.H_kv // 2
    nb = pd.pd_kv_pack_heads_bytes(desc, n, 0, h1)
    hbuf = torch.empty(nb, dtype=torch.uint8, device="cuda")
    r = meter.time(lambda: pd.pd_kv_pack_heads(desc, pool, b.num_pool_pages, pack_ids, 0, h1, hbuf, scr))
    out["pack_heads"] = {"heads": [0, h1], "pages": n, "bytes": nb, "ms": r,
                         "GBps": round(2 * nb / (r["median"] * 1e-3) / 1e9, 1)}
    r = meter.time(lambda: pd.pd_kv_unpack_heads(desc, pool, b.num_pool_pages, unpack_ids, 0, h1, hbuf, scr))
    out["unpack_heads"] = {"ms": r, "GBps": round(2 * nb / (r["median"] * 1e-3) / 1e9, 1)}
    del hbuf

    L = args.layers
    P = n + 16
    pools = [device_normal_(torch.empty((P, 2, b.H_kv, b.ps, b.D), dtype=torch.bfloat16, device="cuda"),
                            device_seed(b.wid, 1, 10 + layer)) for layer in range(L)]
    ids = np.random.default_rng(8).permutation(P)[:n].astype(np.int32)
    x = pd.pd_xfer_plan(desc, pools, P, ids)
    ws = torch.empty(x.workspace_bytes, dtype=torch.uint8, device="cuda")
    pd.pd_xfer_upload(x, ws)
    lbuf = torch.empty(x.buffer_bytes, dtype=torch.uint8, device="cuda")
    prog = torch.zeros(L, dtype=torch.int32, pin_memory=True)
    r = meter.time(lambda: pd.pd_kv_pack_layers(x, ws, lbuf, prog))
    # the host polls the counters during one more launch (the launch returns
    # at once; the polling loop runs in this thread, so no lock stands between
    # the launch and the first read)
    torch.cuda.synchronize()
    view = prog.numpy()
    start = view.copy()
    flips = [None] * L
    t_launch = time.perf_counter()
    pd.pd_kv_pack_layers(x, ws, lbuf, prog)
    deadline = t_launch + 5.0
    while any(f is None for f in flips) and time.perf_counter() < deadline:
        now = time.perf_counter()
        for layer in range(L):
            if flips[layer] is None and view[layer] != start[layer]:
                flips[layer] = now
    torch.cuda.synchronize()
    t_sync = time.perf_counter()
    ready = [round((f - t_launch) * 1e6, 1) if f is not None else None for f in flips]
    out["pack_layers"] = {"layers": L, "pages_per_layer": n, "bytes": x.buffer_bytes, "ms": r,
                          "GBps": round(2 * x.buffer_bytes / (r["median"] * 1e-3) / 1e9, 1),
                          "host_seen_layer_ready_us": ready,
                          "host_launch_to_sync_us": round((t_sync - t_launch) * 1e6, 1)}
    x.close()
    del pools, lbuf
    torch.cuda.synchronize()
    return out


def interference_sweep(args, pd, torch):
    """Kernel-level analogue of the interference comparison in the kwkr.cn
    survey, section 2 (one prefill batched with n decodes, "1PnD", against the
    n decodes alone, "nD", and the prefill alone), over prompt lengths, and of
    its section 8 remark that every chunk of a chunked prefill re-reads all
    earlier KV.  Shapes of the mixed workload (H 32/8, D 128, page 16, bf16);
    each decode's cache holds as many tokens as the prompt.  Times are the
    attention launch + merge, averaged over back-to-back launches."""
    from workloads import device_normal_, device_seed, make_batch

    reps = 20

    def per_launch(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def setup(b, qo, kv, page_indptr, page_indices):
        desc = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype, b.causal, b.sm_scale)
        plan = pd.pd_plan(desc, qo, kv, page_indptr, page_indices, b.num_pool_pages)
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
        pd.pd_plan_upload(plan, ws)
        rows = max(int(np.sum(qo)), 1)
        q = device_normal_(torch.empty((rows, b.H_q, b.D), dtype=torch.bfloat16, device="cuda"), 5)
        o = torch.empty((rows, b.H_q, b.D), dtype=torch.float32, device="cuda")
        lse = torch.empty((rows, b.H_q), dtype=torch.float32, device="cuda")
        return plan, ws, q, o, lse

    n = args.sweep_decodes
    res = {"shapes": "H 32/8, D 128, page 16, bf16; decode caches as long as the prompt",
           "decodes": n, "points": [], "chunked": []}
    for L in (128, 256, 512, 1024, 2048, 4096):
        qo = np.array([L] + [1] * n, np.int32)
        kv = np.array([L] * (n + 1), np.int32)
        b = make_batch("mixed", lengths=(qo, kv), materialize=False)
        pool = device_normal_(torch.empty(b.pool_shape, dtype=torch.bfloat16, device="cuda"), device_seed(4, L, 0))
        pt = {"prompt": L}
        for name, sel in (("1PnD", qo), ("nD", np.array([0] + [1] * n, np.int32)),
                          ("prefill_only", np.array([L] + [0] * n, np.int32))):
            plan, ws, q, o, lse = setup(b, sel, kv, b.page_indptr, b.page_indices)
            pt[name + "_us"] = round(per_launch(lambda: pd.pd_attention_run(plan, ws, q, pool, o, lse)) * 1e3, 2)
            plan.close()
        pt["ratio_vs_nD"] = round(pt["1PnD_us"] / pt["nD_us"], 3)
        pt["ratio_vs_sum"] = round(pt["1PnD_us"] / (pt["nD_us"] + pt["prefill_only_us"]), 3)
        res["points"].append(pt)
        del pool
    # chunked prefill of one 4096-token prompt: chunk c attends over the
    # c + 1 chunks' keys (all earlier KV re-read)
    P = 4096
    b = make_batch("mixed", lengths=([P], [P]), materialize=False)
    pool = device_normal_(torch.empty(b.pool_shape, dtype=torch.bfloat16, device="cuda"), device_seed(4, 0, 1))
    kv_token_bytes = 2 * b.H_kv * b.D * 2
    for C in (256, 512, 1024, 2048, 4096):
        legs = []
        for c in range(P // C):
            kv_c = (c + 1) * C
            npg = -(-kv_c // b.ps)
            legs.append(setup(b, np.array([C], np.int32), np.array([kv_c], np.int32),
                              np.array([0, npg], np.int32), np.asarray(b.page_indices[:npg])))

        def run_all():
            for (plan, ws, q, o, lse) in legs:
                pd.pd_attention_run(plan, ws, q, pool, o, lse)

        t = per_launch(run_all)
        res["chunked"].append({"prompt": P, "chunk": C, "launches": len(legs), "us": round(t * 1e3, 2),
                               "kv_bytes_read": sum((c + 1) * C for c in range(P // C)) * kv_token_bytes})
        for leg in legs:
            leg[0].close()
    single = res["chunked"][-1]["us"]
    for r in res["chunked"]:
        r["time_vs_single"] = round(r["us"] / single, 3)
        r["kv_reread_factor"] = round(r["kv_bytes_read"] / (P * kv_token_bytes), 2)
    del pool
    torch.cuda.synchronize()
    return res


def mla_legs(args, pd, torch, meter):
    """Latent-cache (MLA) decode legs, untimed by the step: the two DeepSeek
    decode workloads (one TP-8 rank with 16 query heads, one data-parallel
    attention rank with 128; 64 requests, caches of 1024..8192 tokens, page
    size 64, pools drawn on the device).  Per workload: pd_mla_kv_append of
    the 64 new latent rows, pd_mla_attention_run (attention + merge), and
    pd_mla_kv_pack / pd_mla_kv_unpack of the longest request's pages.
    Algorithmic work: latent rows read once per request + Q read + O and LSE
    written (bytes); 2 (576 + 512) flops per (query row, visible key)."""
    from workloads import device_normal_, device_seed, make_mla_batch

    def timed(fn):
        return meter.time(fn)

    res = {}
    for name in ("mla_tp8", "mla_dp"):
        b = make_mla_batch(name, materialize=False)
        pool = device_normal_(torch.empty(b.pool_shape, dtype=torch.bfloat16, device="cuda"), device_seed(b.wid, 0, 0))
        n = int(b.qo_indptr[-1])
        q = device_normal_(torch.empty((n, b.H, b.width), dtype=torch.bfloat16, device="cuda"), device_seed(b.wid, 0, 1))
        rows_new = device_normal_(torch.empty((n, b.width), dtype=torch.bfloat16, device="cuda"), device_seed(b.wid, 0, 2))
        d = pd.make_mla_desc(b.H, b.ps, b.causal, b.sm_scale)
        plan = pd.pd_mla_plan(d, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages)
        ws = torch.empty(max(plan.workspace_bytes, 1), dtype=torch.uint8, device="cuda")
        pd.pd_plan_upload(plan, ws)
        out = torch.empty((n, b.H, b.d_c), dtype=torch.float32, device="cuda")
        lse = torch.empty((n, b.H), dtype=torch.float32, device="cuda")
        r_app = timed(lambda: pd.pd_mla_kv_append(plan, ws, pool, rows_new))
        r_attn = timed(lambda: pd.pd_mla_attention_run(plan, ws, q, pool, out, lse))
        t_app, t_attn = r_app["median"], r_attn["median"]
        keys = int(b.kv_lens.astype(np.int64).sum())
        nbytes = keys * b.width * 2 + n * b.H * (b.width * 2 + b.d_c * 4 + 4)
        flops = keys * b.H * 2 * (b.width + b.d_c)           # qo = 1: every cached key is visible
        ideal = max(nbytes / (PEAK_HBM_GBPS * 1e9), flops / (PEAK_BF16_TFLOPS * 1e12))
        r = int(np.argmax(b.kv_lens))
        ids = b.request_pages(r)
        pb = pd.pd_mla_page_bytes(d)
        buf = torch.empty(len(ids) * pb, dtype=torch.uint8, device="cuda")
        scr = torch.empty(4 * len(ids), dtype=torch.uint8, device="cuda")
        t_pack = timed(lambda: pd.pd_mla_kv_pack(d, pool, b.num_pool_pages, ids, buf, scr))["median"]
        t_unpack = timed(lambda: pd.pd_mla_kv_unpack(d, pool, b.num_pool_pages, ids, buf, scr))["median"]
        st = plan.stats()
        res[name] = {
            "shape": f"B {b.B}, H {b.H}, latent {b.d_c} + rotary {b.d_r}, page {b.ps}, bf16, kv 1024..8192",
            "attention_ms": r_attn, "blocks": st.decode_units, "chunk_keys": st.decode_chunk_keys,
            "GBps": round(nbytes / (t_attn * 1e-3) / 1e9, 1),
            "TFLOPs": round(flops / (t_attn * 1e-3) / 1e12, 1),
            "hbm_frac": round(nbytes / (t_attn * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "mfma_frac": round(flops / (t_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "roofline_frac": round(ideal / (t_attn * 1e-3), 4),
            "append_ms": r_app,
            "pack_pages": len(ids), "pack_GBps": round(2 * len(ids) * pb / (t_pack * 1e-3) / 1e9, 1),
            "unpack_GBps": round(2 * len(ids) * pb / (t_unpack * 1e-3) / 1e9, 1),
        }
        plan.close()
        del pool, q, rows_new, out, lse, ws, buf, scr
    torch.cuda.synchronize()
    return res


def power_loop(args, pd, torch, b, desc, pool, q):
    """--loop: one launch kind (prefill-only, decode-only or the mixed launch)
    back to back for --loop-seconds, so that the board's power and clocks
    can be read meanwhile (e.g. `amd-smi metric -p -c`); prints one JSON line
    with the launches and their mean time."""
    dec = b.qo_lens == 1
    sel = {"prefill": ~dec, "decode": dec, "mixed": np.ones(b.B, bool)}[args.loop]
    p, wsp, qs, o, ls = sub_plan(pd, torch, b, desc, sel, q)
    torch.cuda.synchronize()
    print(f"[bench] {args.loop} launches back to back for {args.loop_seconds} s", file=sys.stderr, flush=True)
    n, t0 = 0, time.time()
    while time.time() - t0 < args.loop_seconds:
        for _ in range(20):
            pd.pd_attention_run(p, wsp, qs, pool, o, ls)
        torch.cuda.synchronize()
        n += 20
    dt = time.time() - t0
    print(json.dumps({"loop": args.loop, "launches": n, "seconds": round(dt, 2),
                      "ms_per_launch": round(dt / n * 1e3, 4)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(no multi-GPU sharding is implemented).", file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_attention_kv_pd_amd as pd
    from workloads import make_batch

    torch.cuda.set_device(0)
    dev = "cuda"
    b = make_batch(args.workload, materialize=False)
    if b.dtype != "bf16":
        raise SystemExit("bench.py times bf16 workloads")
    desc = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype, b.causal, b.sm_scale)
    work = algorithmic_work(b)
    n_rows = int(b.qo_lens.sum())

    # ---- device-resident inputs
    t = device_inputs(torch, b, pd)
    pool, q, k_new, v_new, out, lse = (t[k] for k in ("pool", "q", "k_new", "v_new", "out", "lse"))
    if args.loop:
        return power_loop(args, pd, torch, b, desc, pool, q)
    r_pack = int(np.argmax(b.qo_lens))
    pack_ids = b.request_pages(r_pack)
    unpack_ids = np.random.default_rng(7).permutation(b.spare_pages)[:len(pack_ids)].astype(np.int32)
    n_pack = len(pack_ids)
    pack_nbytes = pd.pd_kv_pack_bytes(desc, n_pack)
    buf = torch.empty(pack_nbytes, dtype=torch.uint8, device=dev)
    scratch = torch.empty(4 * n_pack, dtype=torch.uint8, device=dev)
    plan0 = pd.pd_plan(desc, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages)
    stats = plan0.stats()
    ws = torch.empty(plan0.workspace_bytes, dtype=torch.uint8, device=dev)
    assert stats.prefill_flops == work["prefill_flops"]
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    plan_host_s = 0.0
    keep = []

    def step(i=None):
        nonlocal plan_host_s
        t0 = time.perf_counter()
        plan = pd.pd_plan(desc, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages)
        pd.pd_plan_upload(plan, ws)
        plan_host_s += time.perf_counter() - t0
        e = ev[i] if i is not None else None
        if e: e[0].record()
        pd.pd_kv_append(plan, ws, pool, k_new, v_new)
        if e: e[1].record()
        pd.pd_attention_run(plan, ws, q, pool, out, lse)
        if e: e[2].record()
        pd.pd_kv_pack(desc, pool, b.num_pool_pages, pack_ids, buf, scratch)
        if e: e[3].record()
        pd.pd_kv_unpack(desc, pool, b.num_pool_pages, unpack_ids, buf, scratch)
        if e: e[4].record()
        keep.append(plan)
        if len(keep) > 2:
            keep.pop(0).close()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    plan_host_s = 0.0
    print(f"[bench] warm-up done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    def phase(a, c):
        return spread([ev[i][a].elapsed_time(ev[i][c]) for i in range(args.steps)])

    s_append, s_attn, s_pack, s_unpack = phase(0, 1), phase(1, 2), phase(2, 3), phase(3, 4)
    t_attn = s_attn["mean"]     # average launch duration over the timed steps
    assert torch.isfinite(out).all().item(), "non-finite attention output"
    print(f"[bench] timed steps: {ms_step:.4f} ms/step, attention launch avg {t_attn:.4f} ms",
          file=sys.stderr, flush=True)

    # ---- roofline of the dominant launch (pd_attention_run: mixed kernel + merge).
    # Algorithmic bytes: the decode requests' K/V read once, their Q read and
    # O written; the prefill chunk's compulsory bytes are reported beside them.
    attn_hbm_ms = work["decode_bytes"] / (PEAK_HBM_GBPS * 1e9) * 1e3
    attn_mfma_ms = work["prefill_flops"] / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    bound = "hbm" if attn_hbm_ms >= attn_mfma_ms else "mfma"
    if bound == "hbm":
        achieved, peak, unit = work["decode_bytes"] / (t_attn * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"
    else:
        achieved, peak, unit = work["prefill_flops"] / (t_attn * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    pack_bytes_rw = 2 * pack_nbytes
    ideal_ms = (max(attn_hbm_ms, attn_mfma_ms)
                + (work["append_bytes"] + 2 * pack_bytes_rw) / (PEAK_HBM_GBPS * 1e9) * 1e3)
    value = 100.0 * ideal_ms / ms_step

    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "% of MI355X peak (roofline time of the step)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, drawn on the device)",
        "config": {"workload": "long-context mixed batch: 1 causal chunk qo 8192 over kv 32768 + 256 "
                               "decodes kv 32768, H 64/8, D 128, page 64, pack/unpack 512 pages",
                   "batch": b.B, "q_rows": n_rows, "pool_pages": b.num_pool_pages,
                   "pool_GB": round(b.num_pool_pages * b.page_bytes / 1e9, 2)},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": measured_traffic(args.workload),
                     "kernel": "pd_attention_run (attn_bf16_kernel + merge_kernel)",
                     "algorithmic_bytes": work["decode_bytes"],
                     "prefill_compulsory_bytes": work["prefill_bytes"],
                     "algorithmic_flops": work["prefill_flops"],
                     "mfma_frac": round(work["prefill_flops"] / (t_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "frac_sum_form": round((attn_hbm_ms + attn_mfma_ms) / t_attn, 4),
                     "avg_ms": round(t_attn, 4)},
        "phases_ms": {"plan_host": round(plan_host_s * 1e3 / args.steps, 4), "append": s_append,
                      "attention": s_attn, "pack": s_pack, "unpack": s_unpack},
        "append_GBps": round(work["append_bytes"] / (s_append["mean"] * 1e-3) / 1e9, 1),
        "pack_GBps": round(pack_bytes_rw / (s_pack["mean"] * 1e-3) / 1e9, 1),
        "unpack_GBps": round(pack_bytes_rw / (s_unpack["mean"] * 1e-3) / 1e9, 1),
        "plan": {"prefill_tiles": stats.prefill_tiles, "decode_units": stats.decode_units,
                 "decode_chunk_keys": stats.decode_chunk_keys},
    }
    for p in keep:
        p.close()
    keep.clear()
    meter = Meter(torch, args.reps, args.leg_warmup)

    # ---- per-phase legs: decode-only and prefill-only plans over the same pool
    if not args.no_phases:
        dec = b.qo_lens == 1
        legs = {}
        for name, sel in (("decode_only", dec), ("prefill_only", ~dec)):
            p, wsp, qs, os_, ls = sub_plan(pd, torch, b, desc, sel, q)
            r = meter.time(lambda: pd.pd_attention_run(p, wsp, qs, pool, os_, ls))
            tm = r["median"]
            if name == "decode_only":
                gbps = work["decode_bytes"] / (tm * 1e-3) / 1e9
                r.update({"GBps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)})
            else:
                tf = work["prefill_flops"] / (tm * 1e-3) / 1e12
                r.update({"TFLOPs": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
            legs[name] = r
            p.close()
            del wsp, qs, os_, ls
        # the same mixed batch with every prefill tile launched before the decode blocks
        p, wsp, qs, os_, ls = sub_plan(pd, torch, b, desc, np.ones(b.B, bool), q, block_order=1)
        legs["mixed_prefill_first_order_ms"] = meter.time(lambda: pd.pd_attention_run(p, wsp, qs, pool, os_, ls))
        p.close()
        del wsp, qs, os_, ls
        legs["interference_ratio"] = round(t_attn / legs["decode_only"]["median"], 3)
        legs["mixed_vs_sum"] = round(t_attn / (legs["decode_only"]["median"] + legs["prefill_only"]["median"]), 3)
        result["phases"] = legs
        result["decode_attn_GBps"] = legs["decode_only"]["GBps"]
        result["prefill_attn_TFLOPs"] = legs["prefill_only"]["TFLOPs"]
        print(f"[bench] phase legs done", file=sys.stderr, flush=True)

    if not args.no_transfers:
        result["transfers"] = transfer_legs(args, pd, torch, meter, b, desc, pool, pack_ids, unpack_ids)
        print(f"[bench] transfer legs done", file=sys.stderr, flush=True)

    del t, pool, q, k_new, v_new, out, lse, buf, scratch, ws
    torch.cuda.synchronize()

    if not args.no_configs:
        result["workloads"] = config_legs(args, pd, torch, meter)

    if not args.no_mla:
        result["mla_decode"] = mla_legs(args, pd, torch, meter)
        print(f"[bench] MLA legs done", file=sys.stderr, flush=True)

    if not args.no_sweep:
        result["interference_sweep"] = interference_sweep(args, pd, torch)
        print(f"[bench] interference sweep done", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(b, args.cpu_workers, args.cpu_decode_rows, args.cpu_prefill_rows)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
