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

It is the one workload whose step exercises every part of the path; the
other workloads are parity cases of the test suite.  Inputs are resident in
HBM before the timed region.  W warm-up steps, then K timed steps between
device synchronisations; per-phase times come from HIP events recorded on the
launch stream.  Afterwards, untimed legs run decode-only and prefill-only
plans over the same pool (per-phase GB/s and TFLOP/s, interference ratio),
and the CPU oracle is timed on a bounded sample of the same workload.

Prints one JSON line.  ``value`` is the step's attainment of the MI355X
roofline in percent: the ideal time of the step's algorithmic work at peak
(attention launch: max of its HBM bytes / 8 TB/s and its prefill flops /
2.5 PFLOP/s; append, pack, unpack: bytes / 8 TB/s) divided by the measured
time per step.
"""
from __future__ import annotations

import argparse
import json
import math
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--phase-reps", type=int, default=5)
    ap.add_argument("--no-phases", action="store_true", help="skip the decode-only / prefill-only legs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-transfers", action="store_true",
                    help="skip the head-range and multi-layer transfer legs")
    ap.add_argument("--layers", type=int, default=8, help="layers of the multi-layer pack leg")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the interference / chunked-prefill sweep")
    ap.add_argument("--sweep-decodes", type=int, default=32, help="decodes in the 1PnD sweep batches")
    ap.add_argument("--no-mla", action="store_true", help="skip the latent-cache (MLA) decode legs")
    ap.add_argument("--cpu-decode-requests", type=int, default=60)
    ap.add_argument("--cpu-prefill-tokens", type=int, default=40)
    return ap.parse_args()


def algorithmic_work(b, elt=2):
    """Bytes and flops the method must move / compute (not the dense work
    it avoids): decode rows read their K/V once plus Q, write O (fp32) and
    LSE; prefill flops count visible (query, key) pairs only (4 D flops per
    pair per query head); the prefill request's compulsory bytes are its
    Q, K/V and O.  Append reads and writes each new row; pack / unpack read
    and write each page."""
    g = b.H_q // b.H_kv
    dec_bytes = pre_bytes = 0
    flops = 0
    for qo, kv in zip(b.qo_lens.tolist(), b.kv_lens.tolist()):
        if qo == 0:
            continue
        kvb = 2 * kv * b.H_kv * b.D * elt
        qob = qo * b.H_q * (b.D * elt + b.D * 4 + 4)
        if qo * g <= 16:
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
    copy size), or None when the kernel source changed since the counters
    were taken (the summary records the source hash)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attention_long_pmc_traffic.txt")
    src = os.path.join(ROOT, "decode_attention_kv_pd_amd", "csrc", "attention.hip")
    if workload != "long" or not os.path.exists(path):
        return None
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    for line in open(path):
        if line.startswith("TRAFFIC "):
            kv = dict(t.split("=", 1) for t in line.split()[1:])
            if kv.get("attention_sha256_16") == digest:
                return int(kv["bytes_per_launch"])
    return None


def cpu_baseline(b, n_dec, n_tok):
    """Time the float64 oracle on a bounded sample of the workload: n_dec
    decode requests (all heads, full 32768-token cache) and n_tok tokens of
    the prefill chunk (all heads).  Inputs are drawn on the host with the
    workload's distribution; only the oracle call is timed, with BLAS held to
    one thread."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as OA
    from workloads import f32_to_bf16_bits, bf16_bits_to_f32

    rng = np.random.default_rng(np.random.SeedSequence([2026, b.wid, 99]))
    g = b.H_q // b.H_kv

    def draw(*shape):
        return bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))).astype(np.float64)

    secs = 0.0
    dec_bytes = pre_flops = 0
    kv = int(b.kv_lens[0])
    k, v = draw(kv, b.H_kv, b.D), draw(kv, b.H_kv, b.D)   # one cache, reused by every sampled request
    with threadpool_limits(limits=1):
        for i in range(n_dec + 1):
            if i < n_dec:     # a decode request: one row, all heads
                q = draw(1, b.H_q, b.D)
                pos = np.array([kv - 1])
                dec_bytes += 2 * kv * b.H_kv * b.D * 2 + b.H_q * (b.D * 2 + b.D * 4 + 4)
            else:             # prefill tokens spread over the chunk
                qo = int(b.qo_lens[0])
                toks = np.linspace(0, qo - 1, n_tok).astype(np.int64)
                q = draw(n_tok, b.H_q, b.D)
                pos = kv - qo + toks
                pre_flops += int(4 * b.D * b.H_q * (pos + 1).sum())
            t0 = time.perf_counter()
            OA.attend(q, k, v, pos, b.sm_scale, True)
            secs += time.perf_counter() - t0
    ideal = dec_bytes / (PEAK_HBM_GBPS * 1e9) + pre_flops / (PEAK_BF16_TFLOPS * 1e12)
    return {"value": 100.0 * ideal / secs, "unit": "% of MI355X peak", "cores": 1, "kind": "oracle",
            "sample": f"{n_dec} decode rows x {b.H_q} heads over {kv} keys + {n_tok} prefill-chunk "
                      f"rows x {b.H_q} heads (float64 numpy oracle, 1 BLAS thread; one drawn cache "
                      f"shared by the sampled rows)",
            "seconds": round(secs, 3), "decode_GBps": dec_bytes / secs / 1e9 if n_dec else None,
            "prefill_TFLOPs": pre_flops / secs / 1e12 if n_tok else None}


def transfer_legs(args, pd, torch, b, desc, pool, pack_ids, unpack_ids):
    """Head-range pack / unpack of the chunk request's pages (half of the KV
    heads: what a rank sends when the decoder has twice the prefiller's TP
    degree), and a multi-layer pack of the same page count over `--layers`
    layer pools in one launch, with per-layer progress counters in pinned
    host memory polled from the host.  Bytes are read + written."""
    from workloads import device_normal_, device_seed

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    out = {}
    n = len(pack_ids)
    h1 = b.H_kv // 2
    nb = pd.pd_kv_pack_heads_bytes(desc, n, 0, h1)
    hbuf = torch.empty(nb, dtype=torch.uint8, device="cuda")
    scr = torch.empty(4 * n, dtype=torch.uint8, device="cuda")
    pd.pd_kv_pack_heads(desc, pool, b.num_pool_pages, pack_ids, 0, h1, hbuf, scr)
    t = timed(lambda: pd.pd_kv_pack_heads(desc, pool, b.num_pool_pages, pack_ids, 0, h1, hbuf, scr),
              args.phase_reps)
    out["pack_heads"] = {"heads": [0, h1], "pages": n, "bytes": nb, "ms": round(t, 4),
                         "GBps": round(2 * nb / (t * 1e-3) / 1e9, 1)}
    t = timed(lambda: pd.pd_kv_unpack_heads(desc, pool, b.num_pool_pages, unpack_ids, 0, h1, hbuf, scr),
              args.phase_reps)
    out["unpack_heads"] = {"ms": round(t, 4), "GBps": round(2 * nb / (t * 1e-3) / 1e9, 1)}
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
    pd.pd_kv_pack_layers(x, ws, lbuf, prog)
    torch.cuda.synchronize()
    t = timed(lambda: pd.pd_kv_pack_layers(x, ws, lbuf, prog), args.phase_reps)
    # the host polls the counters during one more launch (the launch returns
    # at once; the polling loop runs in this thread, so no lock stands between
    # the launch and the first read)
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
    out["pack_layers"] = {"layers": L, "pages_per_layer": n, "bytes": x.buffer_bytes, "ms": round(t, 4),
                          "GBps": round(2 * x.buffer_bytes / (t * 1e-3) / 1e9, 1),
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


def mla_legs(args, pd, torch):
    """Latent-cache (MLA) decode legs, untimed by the step: the two DeepSeek
    decode workloads (one TP-8 rank with 16 query heads, one data-parallel
    attention rank with 128; 64 requests, caches of 1024..8192 tokens, page
    size 64, pools drawn on the device).  Per workload: pd_mla_kv_append of
    the 64 new latent rows, pd_mla_attention_run (attention + merge), and
    pd_mla_kv_pack / pd_mla_kv_unpack of the longest request's pages.
    Algorithmic work: latent rows read once per request + Q read + O and LSE
    written (bytes); 2 (576 + 512) flops per (query row, visible key)."""
    from workloads import device_normal_, device_seed, make_mla_batch

    reps = args.phase_reps * 4

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

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
        t_app = timed(lambda: pd.pd_mla_kv_append(plan, ws, pool, rows_new))
        t_attn = timed(lambda: pd.pd_mla_attention_run(plan, ws, q, pool, out, lse))
        keys = int(b.kv_lens.astype(np.int64).sum())
        nbytes = keys * b.width * 2 + n * b.H * (b.width * 2 + b.d_c * 4 + 4)
        flops = keys * b.H * 2 * (b.width + b.d_c)           # qo = 1: every cached key is visible
        ideal = max(nbytes / (PEAK_HBM_GBPS * 1e9), flops / (PEAK_BF16_TFLOPS * 1e12))
        r = int(np.argmax(b.kv_lens))
        ids = b.request_pages(r)
        pb = pd.pd_mla_page_bytes(d)
        buf = torch.empty(len(ids) * pb, dtype=torch.uint8, device="cuda")
        scr = torch.empty(4 * len(ids), dtype=torch.uint8, device="cuda")
        t_pack = timed(lambda: pd.pd_mla_kv_pack(d, pool, b.num_pool_pages, ids, buf, scr))
        t_unpack = timed(lambda: pd.pd_mla_kv_unpack(d, pool, b.num_pool_pages, ids, buf, scr))
        st = plan.stats()
        res[name] = {
            "shape": f"B {b.B}, H {b.H}, latent {b.d_c} + rotary {b.d_r}, page {b.ps}, bf16, kv 1024..8192",
            "attention_ms": round(t_attn, 4), "blocks": st.decode_units, "chunk_keys": st.decode_chunk_keys,
            "GBps": round(nbytes / (t_attn * 1e-3) / 1e9, 1),
            "TFLOPs": round(flops / (t_attn * 1e-3) / 1e12, 1),
            "hbm_frac": round(nbytes / (t_attn * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "mfma_frac": round(flops / (t_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "roofline_frac": round(ideal / (t_attn * 1e-3), 4),
            "append_us": round(t_app * 1e3, 2),
            "pack_pages": len(ids), "pack_GBps": round(2 * len(ids) * pb / (t_pack * 1e-3) / 1e9, 1),
            "unpack_GBps": round(2 * len(ids) * pb / (t_unpack * 1e-3) / 1e9, 1),
        }
        plan.close()
        del pool, q, rows_new, out, lse, ws, buf, scr
    torch.cuda.synchronize()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(no multi-GPU sharding is implemented).", file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_attention_kv_pd_amd as pd
    from workloads import device_normal_, device_seed, make_batch

    torch.cuda.set_device(0)
    dev = "cuda"
    b = make_batch(args.workload, materialize=False)
    if b.dtype != "bf16":
        raise SystemExit("bench.py times bf16 workloads")
    desc = pd.make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype, b.causal, b.sm_scale)
    work = algorithmic_work(b)
    n_rows = int(b.qo_lens.sum())

    # ---- device-resident inputs
    pool = device_normal_(torch.empty(b.pool_shape, dtype=torch.bfloat16, device=dev), device_seed(b.wid, 0, 0))
    q = device_normal_(torch.empty((n_rows, b.H_q, b.D), dtype=torch.bfloat16, device=dev), device_seed(b.wid, 0, 1))
    k_new = device_normal_(torch.empty((n_rows, b.H_kv, b.D), dtype=torch.bfloat16, device=dev), device_seed(b.wid, 0, 2))
    v_new = device_normal_(torch.empty((n_rows, b.H_kv, b.D), dtype=torch.bfloat16, device=dev), device_seed(b.wid, 0, 3))
    out = torch.empty((n_rows, b.H_q, b.D), dtype=torch.float32, device=dev)
    lse = torch.empty((n_rows, b.H_q), dtype=torch.float32, device=dev)
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
    attn_bytes = work["decode_bytes"] + work["prefill_bytes"]
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

    def avg(a, c):
        return float(np.mean([ev[i][a].elapsed_time(ev[i][c]) for i in range(args.steps)]))

    t_append, t_attn, t_pack, t_unpack = avg(0, 1), avg(1, 2), avg(2, 3), avg(3, 4)
    assert torch.isfinite(out).all().item(), "non-finite attention output"

    # ---- roofline of the dominant launch (pd_attention_run: mixed kernel + merge)
    attn_hbm_ms = attn_bytes / (PEAK_HBM_GBPS * 1e9) * 1e3
    attn_mfma_ms = work["prefill_flops"] / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    bound = "hbm" if attn_hbm_ms >= attn_mfma_ms else "mfma"
    if bound == "hbm":
        achieved, peak, unit = attn_bytes / (t_attn * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"
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
                     "algorithmic_bytes": attn_bytes, "algorithmic_flops": work["prefill_flops"],
                     "mfma_frac": round(work["prefill_flops"] / (t_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "avg_ms": round(t_attn, 4)},
        "phases_ms": {"plan_host": round(plan_host_s * 1e3 / args.steps, 4), "append": round(t_append, 4),
                      "attention": round(t_attn, 4), "pack": round(t_pack, 4), "unpack": round(t_unpack, 4)},
        "append_GBps": round(work["append_bytes"] / (t_append * 1e-3) / 1e9, 1),
        "pack_GBps": round(pack_bytes_rw / (t_pack * 1e-3) / 1e9, 1),
        "unpack_GBps": round(pack_bytes_rw / (t_unpack * 1e-3) / 1e9, 1),
        "plan": {"prefill_tiles": stats.prefill_tiles, "decode_units": stats.decode_units,
                 "decode_chunk_keys": stats.decode_chunk_keys},
    }

    # ---- per-phase legs: decode-only and prefill-only plans over the same pool
    if not args.no_phases:
        dec = b.qo_lens * (b.H_q // b.H_kv) <= 16
        legs = {}
        for name, sel in (("decode_only", dec), ("prefill_only", ~dec)):
            qo = np.where(sel, b.qo_lens, 0).astype(np.int32)
            p = pd.pd_plan(desc, qo, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages)
            wsp = torch.empty(max(p.workspace_bytes, 1), dtype=torch.uint8, device=dev)
            pd.pd_plan_upload(p, wsp)
            # rows of the selected requests only: pack their q rows first
            idx = np.concatenate([np.arange(b.qo_indptr[r], b.qo_indptr[r + 1]) for r in range(b.B) if sel[r]])
            qs = q[torch.as_tensor(idx, device=dev)].contiguous()
            os_ = torch.empty((len(idx), b.H_q, b.D), dtype=torch.float32, device=dev)
            ls = torch.empty((len(idx), b.H_q), dtype=torch.float32, device=dev)
            pd.pd_attention_run(p, wsp, qs, pool, os_, ls)
            torch.cuda.synchronize()
            ts = []
            for _ in range(args.phase_reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                pd.pd_attention_run(p, wsp, qs, pool, os_, ls)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            t = float(np.median(ts))
            if name == "decode_only":
                gbps = work["decode_bytes"] / (t * 1e-3) / 1e9
                legs[name] = {"ms": round(t, 4), "GBps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}
            else:
                tf = work["prefill_flops"] / (t * 1e-3) / 1e12
                legs[name] = {"ms": round(t, 4), "TFLOPs": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
            p.close()
            del wsp, qs, os_, ls
        # the same mixed batch with every prefill tile launched before the decode blocks
        p = pd.pd_plan(desc, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices, b.num_pool_pages,
                       block_order=1)
        pd.pd_plan_upload(p, ws)
        pd.pd_attention_run(p, ws, q, pool, out, lse)
        torch.cuda.synchronize()
        ts = []
        for _ in range(args.phase_reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            pd.pd_attention_run(p, ws, q, pool, out, lse)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        legs["mixed_prefill_first_order_ms"] = round(float(np.median(ts)), 4)
        p.close()
        legs["interference_ratio"] = round(t_attn / legs["decode_only"]["ms"], 3)
        legs["mixed_vs_sum"] = round(t_attn / (legs["decode_only"]["ms"] + legs["prefill_only"]["ms"]), 3)
        result["phases"] = legs
        result["decode_attn_GBps"] = legs["decode_only"]["GBps"]
        result["prefill_attn_TFLOPs"] = legs["prefill_only"]["TFLOPs"]
        print(f"[bench] phase legs done", file=sys.stderr, flush=True)

    if not args.no_transfers:
        result["transfers"] = transfer_legs(args, pd, torch, b, desc, pool, pack_ids, unpack_ids)
        print(f"[bench] transfer legs done", file=sys.stderr, flush=True)

    if not args.no_mla:
        result["mla_decode"] = mla_legs(args, pd, torch)
        print(f"[bench] MLA legs done", file=sys.stderr, flush=True)

    if not args.no_sweep:
        result["interference_sweep"] = interference_sweep(args, pd, torch)
        print(f"[bench] interference sweep done", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(b, args.cpu_decode_requests, args.cpu_prefill_tokens)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
