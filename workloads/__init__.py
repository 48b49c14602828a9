"""Seeded synthetic inputs for ragged paged attention.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It only draws random numbers and does page-pool bookkeeping
(which page belongs to which request); it holds none of the attention, append
or pack arithmetic.  Both the CPU oracle and the HIP path consume what it
produces, and neither imports the other.

Workloads (all values i.i.d. N(0, 1), causal, softmax scale 1/sqrt(head_dim)):

  tiny      3 requests, (qo, kv) = (16, 16), (33, 33), (1, 40); 4 query / 2 KV
            heads, head_dim 64, fp32, page size 16
  decode    64 requests, qo 1, kv uniform in [512, 4096]; 40 / 40 heads,
            head_dim 128, bf16, page size 16
  prefill   8 requests, qo = kv = 512; 40 / 40 heads, head_dim 128, bf16,
            page size 16
  mixed     1 request qo = kv = 1024 plus 63 requests qo 1, kv uniform in
            [1024, 2048]; 32 / 8 heads, head_dim 128, bf16, page size 16
  long      1 chunk qo 8192 over kv 32768 plus 256 requests qo 1, kv 32768;
            64 / 8 heads, head_dim 128, bf16, page size 64

These sizes follow the workloads that the Perplexity post "Disaggregated
prefill and decode" (section "Prefill vs Decode performance") and the kwkr.cn
PD-disaggregation survey (sections 2-3 and 8) reason about: ragged batches of
long causal prefills, chunked prefills over prior KV, and single-token decodes
over long caches, with GQA (post, section "Qwen3-Coder") and pages in HND
order (post, section "Sharded KV Cache Transfers").

Random stream: numpy ``SeedSequence([2026, workload_id, rep])``, drawn in the
fixed order lengths, pool permutation, Q, K, V.  bf16 values are the fp32
draws rounded to nearest even.  The pool holds exactly the pages the batch
needs plus 5 % spare pages, randomly permuted; spare pages and the unused tail
slots of each request's last page are NaN so that any read of them shows up.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

SEED_ROOT = 2026

WORKLOADS = {
    1: dict(name="tiny", H_q=4, H_kv=2, D=64, ps=16, dtype="f32"),
    2: dict(name="decode", H_q=40, H_kv=40, D=128, ps=16, dtype="bf16"),
    3: dict(name="prefill", H_q=40, H_kv=40, D=128, ps=16, dtype="bf16"),
    4: dict(name="mixed", H_q=32, H_kv=8, D=128, ps=16, dtype="bf16"),
    5: dict(name="long", H_q=64, H_kv=8, D=128, ps=64, dtype="bf16"),
}
NAME_TO_ID = {v["name"]: k for k, v in WORKLOADS.items()}

BF16_NAN = np.uint16(0x7FC0)


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns
    the 16-bit patterns as uint16.  NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ lengths
def _lengths(wid: int, rng: np.random.Generator):
    if wid == 1:
        qo = [16, 33, 1]
        kv = [16, 33, 40]
    elif wid == 2:
        kv = rng.integers(512, 4096, size=64, endpoint=True).tolist()
        qo = [1] * 64
    elif wid == 3:
        qo = [512] * 8
        kv = [512] * 8
    elif wid == 4:
        kv = [1024] + rng.integers(1024, 2048, size=63, endpoint=True).tolist()
        qo = [1024] + [1] * 63
    elif wid == 5:
        qo = [8192] + [1] * 256
        kv = [32768] * 257
    else:
        raise ValueError(f"unknown workload {wid}")
    return np.asarray(qo, np.int32), np.asarray(kv, np.int32)


@dataclasses.dataclass
class Batch:
    """One ragged batch.  Arrays are numpy; ``q``, ``k_new``, ``v_new`` and the
    logical K/V hold fp32 values for f32 workloads and bf16 bit patterns
    (uint16) for bf16 workloads."""

    wid: int
    name: str
    H_q: int
    H_kv: int
    D: int
    ps: int
    dtype: str
    causal: bool
    sm_scale: float
    qo_lens: np.ndarray
    kv_lens: np.ndarray
    page_indptr: np.ndarray
    page_indices: np.ndarray
    num_pool_pages: int
    spare_pages: np.ndarray
    # materialised values (None when generated on the device)
    q: Optional[np.ndarray] = None          # [sum qo, H_q, D]
    k: Optional[np.ndarray] = None          # [sum kv, H_kv, D] logical, per request
    v: Optional[np.ndarray] = None
    kv_indptr: Optional[np.ndarray] = None  # [B + 1] into k / v
    qo_indptr: Optional[np.ndarray] = None  # [B + 1] into q

    @property
    def B(self) -> int:
        return int(self.qo_lens.shape[0])

    @property
    def elt(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.uint16

    @property
    def pool_shape(self):
        return (self.num_pool_pages, 2, self.H_kv, self.ps, self.D)

    @property
    def page_bytes(self) -> int:
        return 2 * self.H_kv * self.ps * self.D * self.elt

    def to_f64(self, a: np.ndarray) -> np.ndarray:
        """Exact values of stored elements as float64."""
        if self.dtype == "f32":
            return np.asarray(a, np.float32).astype(np.float64)
        return bf16_bits_to_f32(a).astype(np.float64)

    def new_rows(self, a: np.ndarray) -> np.ndarray:
        """Rows [kv - qo, kv) of each request's logical K or V: the tokens a
        step appends, in token-major order [sum qo, H_kv, D]."""
        parts = []
        for r in range(self.B):
            s = int(self.kv_indptr[r])
            kv, qo = int(self.kv_lens[r]), int(self.qo_lens[r])
            parts.append(a[s + kv - qo: s + kv])
        return np.concatenate(parts, axis=0)

    @property
    def k_new(self):
        return self.new_rows(self.k)

    @property
    def v_new(self):
        return self.new_rows(self.v)

    def request_pages(self, r: int) -> np.ndarray:
        return self.page_indices[self.page_indptr[r]:self.page_indptr[r + 1]]


def seed_sequence(wid: int, rep: int = 0) -> np.random.SeedSequence:
    return np.random.SeedSequence([SEED_ROOT, wid, rep])


def make_batch(wid, rep: int = 0, materialize: bool = True,
               q_gain: float = 1.0, lengths=None, heads=None,
               head_dim=None, page_size=None, dtype=None, causal=True,
               spare_frac: float = 0.05) -> Batch:
    """Build a workload.  ``wid`` is a workload id or name.  ``lengths``
    (qo_lens, kv_lens) and the shape keywords override the defaults, which
    the tests use for small ragged cases.  ``q_gain`` scales Q before
    rounding (a sharpened softmax)."""
    if isinstance(wid, str):
        wid = NAME_TO_ID[wid]
    spec = dict(WORKLOADS[wid])
    if heads is not None:
        spec["H_q"], spec["H_kv"] = heads
    if head_dim is not None:
        spec["D"] = head_dim
    if page_size is not None:
        spec["ps"] = page_size
    if dtype is not None:
        spec["dtype"] = dtype
    rng = np.random.default_rng(seed_sequence(wid, rep))
    # (1) lengths
    qo, kv = _lengths(wid, rng)
    if lengths is not None:
        qo = np.asarray(lengths[0], np.int32)
        kv = np.asarray(lengths[1], np.int32)
    ps = spec["ps"]
    npages = (kv.astype(np.int64) + ps - 1) // ps
    total = int(npages.sum())
    # (2) pool permutation
    pool = max(total + 1, int(math.ceil(total * (1.0 + spare_frac))))
    perm = rng.permutation(pool).astype(np.int32)
    page_indptr = np.zeros(len(qo) + 1, np.int32)
    page_indptr[1:] = np.cumsum(npages)
    page_indices = perm[:total].copy()
    spare = perm[total:].copy()
    b = Batch(wid=wid, name=spec["name"], H_q=spec["H_q"], H_kv=spec["H_kv"],
              D=spec["D"], ps=ps, dtype=spec["dtype"], causal=bool(causal),
              sm_scale=1.0 / math.sqrt(spec["D"]), qo_lens=qo, kv_lens=kv,
              page_indptr=page_indptr, page_indices=page_indices,
              num_pool_pages=pool, spare_pages=spare)
    b.qo_indptr = np.zeros(len(qo) + 1, np.int64)
    b.qo_indptr[1:] = np.cumsum(qo)
    b.kv_indptr = np.zeros(len(kv) + 1, np.int64)
    b.kv_indptr[1:] = np.cumsum(kv)
    if not materialize:
        return b
    # (3) Q, (4) K, (5) V
    nq, nk = int(b.qo_indptr[-1]), int(b.kv_indptr[-1])
    q = rng.standard_normal((nq, b.H_q, b.D), dtype=np.float32)
    if q_gain != 1.0:
        q *= np.float32(q_gain)
    k = rng.standard_normal((nk, b.H_kv, b.D), dtype=np.float32)
    v = rng.standard_normal((nk, b.H_kv, b.D), dtype=np.float32)
    if b.dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    b.q, b.k, b.v = q, k, v
    return b


def nan_pool(b: Batch) -> np.ndarray:
    """A pool whose every element is NaN (fp32 NaN or the bf16 quiet NaN)."""
    if b.dtype == "f32":
        return np.full(b.pool_shape, np.nan, np.float32)
    return np.full(b.pool_shape, BF16_NAN, np.uint16)


def device_normal_(t, seed: int):
    """Fill a torch tensor (any device, fp32 or bf16) with N(0, 1) draws from
    torch's counter-based generator seeded with ``seed``.  Used for the
    workloads too large to draw on the host; bf16 is torch's rounding of its
    fp32 draws (round to nearest even)."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed))
    t.normal_(0.0, 1.0, generator=g)
    return t


def device_seed(wid: int, rep: int, stream: int) -> int:
    """64-bit seed for the device generator, derived from the same seed
    sequence as the host draws (``stream`` separates Q / K-V / new tokens)."""
    ss = np.random.SeedSequence([SEED_ROOT, wid, rep, 1000 + stream])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


# ------------------------------------------------------------ MLA workloads
# Latent KV cache (multi-head latent attention, post section "DeepSeek-R1"
# under "Disaggregated Deployments"): one row of d_c + d_r values per token,
# shared by every query head.  Dimensions are DeepSeek-V3's published
# configuration (latent 512, rotary key 64, 128 query heads, softmax scale
# 1 / sqrt(128 + 64)); the pages give none.
#
#   mla_tiny  3 requests, (qo, kv) = (1, 1), (2, 77), (1, 300); 16 heads,
#             page size 16 (parity sizes)
#   mla_tp8   64 decode requests, kv uniform in [1024, 8192]; 16 heads: one
#             rank of an 8-way tensor-parallel decoder, which still holds the
#             whole latent cache
#   mla_dp    the same requests with all 128 heads: one rank of a
#             data-parallel attention decoder
MLA_WORKLOADS = {
    6: dict(name="mla_tiny", H=16, ps=16),
    7: dict(name="mla_tp8", H=16, ps=64),
    8: dict(name="mla_dp", H=128, ps=64),
}
MLA_NAME_TO_ID = {v["name"]: k for k, v in MLA_WORKLOADS.items()}
MLA_D_C = 512
MLA_D_R = 64


@dataclasses.dataclass
class MlaBatch:
    """One ragged MLA batch.  ``q`` [sum qo, H, d_c + d_r] and the logical
    cache ``rows`` [sum kv, d_c + d_r] hold bf16 bit patterns (uint16)."""

    wid: int
    name: str
    H: int
    d_c: int
    d_r: int
    ps: int
    causal: bool
    sm_scale: float
    qo_lens: np.ndarray
    kv_lens: np.ndarray
    page_indptr: np.ndarray
    page_indices: np.ndarray
    num_pool_pages: int
    spare_pages: np.ndarray
    q: Optional[np.ndarray] = None
    rows: Optional[np.ndarray] = None
    kv_indptr: Optional[np.ndarray] = None
    qo_indptr: Optional[np.ndarray] = None

    @property
    def B(self) -> int:
        return int(self.qo_lens.shape[0])

    @property
    def width(self) -> int:
        return self.d_c + self.d_r

    @property
    def pool_shape(self):
        return (self.num_pool_pages, self.ps, self.width)

    @property
    def page_bytes(self) -> int:
        return self.ps * self.width * 2

    def to_f64(self, a: np.ndarray) -> np.ndarray:
        return bf16_bits_to_f32(a).astype(np.float64)

    @property
    def new_rows(self) -> np.ndarray:
        """Rows [kv - qo, kv) of each request's cache, token-major."""
        parts = []
        for r in range(self.B):
            s = int(self.kv_indptr[r])
            kv, qo = int(self.kv_lens[r]), int(self.qo_lens[r])
            parts.append(self.rows[s + kv - qo: s + kv])
        return np.concatenate(parts, axis=0)

    def request_pages(self, r: int) -> np.ndarray:
        return self.page_indices[self.page_indptr[r]:self.page_indptr[r + 1]]


def _mla_lengths(wid: int, rng: np.random.Generator):
    if wid == 6:
        return np.asarray([1, 2, 1], np.int32), np.asarray([1, 77, 300], np.int32)
    if wid in (7, 8):
        kv = rng.integers(1024, 8192, size=64, endpoint=True)
        return np.ones(64, np.int32), kv.astype(np.int32)
    raise ValueError(f"unknown MLA workload {wid}")


def make_mla_batch(wid, rep: int = 0, materialize: bool = True, lengths=None, heads=None,
                   page_size=None, causal=True, q_gain: float = 1.0,
                   spare_frac: float = 0.05) -> MlaBatch:
    """Build an MLA workload (id or name).  Random stream
    ``SeedSequence([2026, wid, rep])`` drawn in the order lengths, pool
    permutation, Q, cache rows; values N(0, 1) rounded to bf16 (nearest
    even).  Spare pages and tail slots are left for the caller to poison."""
    if isinstance(wid, str):
        wid = MLA_NAME_TO_ID[wid]
    spec = dict(MLA_WORKLOADS[wid])
    if heads is not None:
        spec["H"] = heads
    if page_size is not None:
        spec["ps"] = page_size
    rng = np.random.default_rng(seed_sequence(wid, rep))
    qo, kv = _mla_lengths(wid, rng)
    if lengths is not None:
        qo = np.asarray(lengths[0], np.int32)
        kv = np.asarray(lengths[1], np.int32)
    ps = spec["ps"]
    npages = (kv.astype(np.int64) + ps - 1) // ps
    total = int(npages.sum())
    pool = max(total + 1, int(math.ceil(total * (1.0 + spare_frac))))
    perm = rng.permutation(pool).astype(np.int32)
    page_indptr = np.zeros(len(qo) + 1, np.int32)
    page_indptr[1:] = np.cumsum(npages)
    b = MlaBatch(wid=wid, name=spec["name"], H=spec["H"], d_c=MLA_D_C, d_r=MLA_D_R, ps=ps,
                 causal=bool(causal), sm_scale=1.0 / math.sqrt(128 + MLA_D_R), qo_lens=qo, kv_lens=kv,
                 page_indptr=page_indptr, page_indices=perm[:total].copy(), num_pool_pages=pool,
                 spare_pages=perm[total:].copy())
    b.qo_indptr = np.zeros(len(qo) + 1, np.int64)
    b.qo_indptr[1:] = np.cumsum(qo)
    b.kv_indptr = np.zeros(len(kv) + 1, np.int64)
    b.kv_indptr[1:] = np.cumsum(kv)
    if not materialize:
        return b
    nq, nk = int(b.qo_indptr[-1]), int(b.kv_indptr[-1])
    q = rng.standard_normal((nq, b.H, b.width), dtype=np.float32)
    if q_gain != 1.0:
        q *= np.float32(q_gain)
    rows = rng.standard_normal((nk, b.width), dtype=np.float32)
    b.q, b.rows = f32_to_bf16_bits(q), f32_to_bf16_bits(rows)
    return b
