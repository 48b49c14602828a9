"""Test-side driver: moves a seeded workload onto the GPU, runs the library
through its C ABI (Python binding), and computes what the oracle says.

Inputs come from ``workloads``; the expected values come from ``oracle``
only.  Nothing here computes attention itself.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import attention as OA
from oracle import paged_kv as OP
from workloads import Batch, nan_pool


def pd():
    import decode_attention_kv_pd_amd as m
    return m


def dev_array(a: np.ndarray, device="cuda"):
    """numpy fp32 or bf16-bit (uint16) array -> GPU tensor holding the same bytes."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


def host_array(t: torch.Tensor, like: np.dtype) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if like == np.uint16:
        return a.view(np.uint16)
    return a


def prefix_pool(b: Batch) -> np.ndarray:
    """NaN pool holding tokens [0, kv - qo) of every request (the cache as it
    stands before this step's append), built by the oracle's page writer."""
    pool = nan_pool(b)
    for r in range(b.B):
        kv, qo = int(b.kv_lens[r]), int(b.qo_lens[r])
        s = int(b.kv_indptr[r])
        if kv - qo > 0:
            OP.write_prefix(pool, b.page_indptr, b.page_indices, r,
                            b.k[s:s + kv - qo], b.v[s:s + kv - qo])
    return pool


def desc_of(b: Batch):
    return pd().make_desc(b.H_q, b.H_kv, b.D, b.ps, b.dtype, b.causal, b.sm_scale)


class DeviceRun:
    """One step of the path on the GPU for a materialised batch."""

    def __init__(self, b: Batch, decode_chunk_keys: int = 0, pool: np.ndarray = None,
                 device="cuda", num_cus: int = 0, prefill_block_waves: int = 0):
        m = pd()
        self.b = b
        self.desc = desc_of(b)
        self.plan = m.pd_plan(self.desc, b.qo_lens, b.kv_lens, b.page_indptr, b.page_indices,
                              b.num_pool_pages, decode_chunk_keys=decode_chunk_keys, num_cus=num_cus,
                              prefill_block_waves=prefill_block_waves)
        self.ws = torch.empty(max(self.plan.workspace_bytes, 1), dtype=torch.uint8, device=device)
        m.pd_plan_upload(self.plan, self.ws)
        self.pool_host = prefix_pool(b) if pool is None else pool
        self.pool = dev_array(self.pool_host, device)
        self.q = dev_array(b.q, device)
        self.k_new = dev_array(b.k_new, device)
        self.v_new = dev_array(b.v_new, device)
        n = int(b.qo_indptr[-1])
        self.out = torch.full((max(n, 1), b.H_q, b.D), float("nan"), dtype=torch.float32, device=device)
        self.lse = torch.full((max(n, 1), b.H_q), float("nan"), dtype=torch.float32, device=device)

    def append(self):
        pd().pd_kv_append(self.plan, self.ws, self.pool, self.k_new, self.v_new)

    def attention(self):
        pd().pd_attention_run(self.plan, self.ws, self.q, self.pool, self.out, self.lse)

    def step(self):
        self.append()
        self.attention()
        torch.cuda.synchronize()
        n = int(self.b.qo_indptr[-1])
        return self.out[:n].cpu().numpy(), self.lse[:n].cpu().numpy()


def oracle_outputs(b: Batch):
    """float64 O, LSE of the whole batch from the oracle."""
    return OA.attention_batch(b.to_f64(b.q), b.to_f64(b.k), b.to_f64(b.v), b.qo_lens, b.kv_lens,
                              b.sm_scale, b.causal, b.qo_indptr, b.kv_indptr)


def tolerance(b: Batch) -> float:
    """Max-abs bar for O: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs with
    fp32 accumulation."""
    return 1e-4 if b.dtype == "f32" else 2e-2


def report(name, got, ref):
    err = np.abs(got.astype(np.float64) - ref)
    rms = np.sqrt(np.mean((got - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30)
    print(f"[{name}] max_abs_err={err.max():.3e} rel_rms={rms:.3e} max|ref|={np.abs(ref).max():.3f}",
          flush=True)
    return float(err.max())
