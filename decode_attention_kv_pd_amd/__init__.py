"""Python binding of libpd_attn.so, the MI355X (gfx950) ragged paged-attention
library.  Argument marshalling only: every step of the path runs in the
library's HIP kernels; torch supplies device memory and the current stream.

The names mirror the C entry points of include/pd_attn.h:

  pd_plan(desc, qo_lens, kv_lens, page_indptr, page_indices, num_pool_pages,
          decode_chunk_keys=0, num_cus=0, block_order=0,
          prefill_block_waves=0)                   -> Plan  (host only)
  pd_plan_upload(plan, ws, stream=None)
  pd_kv_append(plan, ws, kv_pool, k_new, v_new, stream=None)
  pd_attention_run(plan, ws, q, kv_pool, out, lse=None, stream=None)
  pd_attention_run_noalloc(plan, q, kv_pool, out, lse=None, k_new=None, v_new=None, stream=None)
  pd_kv_pack_bytes(desc, n_pages)                   -> int
  pd_kv_pack(desc, kv_pool, num_pool_pages, page_ids, buf, scratch, stream=None)
  pd_kv_unpack(desc, kv_pool, num_pool_pages, page_ids, buf, scratch, stream=None)
  pd_kv_pack_heads_bytes(desc, n_pages, h0, h1)     -> int
  pd_kv_pack_heads(desc, kv_pool, num_pool_pages, page_ids, h0, h1, buf, scratch, stream=None)
  pd_kv_unpack_heads(desc, kv_pool, num_pool_pages, page_ids, h0, h1, buf, scratch, stream=None)
  pd_kv_shard_transfers(num_kv_heads, src_shards, dst_shards) -> list of 6-tuples
  pd_xfer_plan(desc, kv_pools, num_pool_pages, page_ids, h0=0, h1=None) -> XferPlan (host only)
  pd_xfer_upload(xfer, ws, stream=None)
  pd_kv_pack_layers(xfer, ws, buf, progress=None, stream=None)
  pd_kv_unpack_layers(xfer, ws, buf, progress=None, stream=None)
  pd_mla_page_bytes(mdesc)                          -> int
  pd_mla_plan(mdesc, qo_lens, kv_lens, page_indptr, page_indices, num_pool_pages,
              decode_chunk_keys=0, num_cus=0)     -> Plan  (host only)
  pd_mla_kv_append(plan, ws, kv_pool, rows_new, stream=None)
  pd_mla_attention_run(plan, ws, q, kv_pool, out, lse=None, stream=None)
  pd_mla_kv_pack(mdesc, kv_pool, num_pool_pages, page_ids, buf, scratch, stream=None)
  pd_mla_kv_unpack(mdesc, kv_pool, num_pool_pages, page_ids, buf, scratch, stream=None)

Device arguments are torch tensors (contiguous, on the GPU); host arrays are
anything numpy can turn into int32.  Errors raise PdError carrying the
library's status and message.  Importing this module fails loudly when the
library has not been built: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree library; PD_ATTN_LIB names another build of it (for instance one
# whose host code carries sanitizers, see build.py)
LIB_PATH = os.environ.get("PD_ATTN_LIB") or os.path.join(_HERE, "libpd_attn.so")

PD_F32 = 0
PD_BF16 = 1

STATUS = {0: "PD_OK", -1: "PD_ERR_INVALID_ARG", -2: "PD_ERR_UNSUPPORTED",
          -3: "PD_ERR_OUT_OF_RANGE", -4: "PD_ERR_WORKSPACE", -5: "PD_ERR_HIP",
          -6: "PD_ERR_NO_MEMORY"}


class PdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class pd_attn_desc(ctypes.Structure):
    _fields_ = [("num_qo_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class pd_mla_desc(ctypes.Structure):
    _fields_ = [("num_qo_heads", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
                ("qk_rope_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class pd_plan_options(ctypes.Structure):
    _fields_ = [("decode_chunk_keys", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("block_order", ctypes.c_int32), ("prefill_block_waves", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 4)]


class pd_plan_stats(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("total_q_rows", ctypes.c_int32),
                ("prefill_tiles", ctypes.c_int32), ("decode_units", ctypes.c_int32),
                ("decode_row_groups", ctypes.c_int32), ("decode_chunk_keys", ctypes.c_int32),
                ("prefill_flops", ctypes.c_int64), ("decode_kv_bytes", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64)]


EXPORTS = ("pd_plan", "pd_plan_workspace_bytes", "pd_plan_upload", "pd_plan_get_stats",
           "pd_plan_free", "pd_plan_work_items", "pd_kv_append", "pd_attention_run", "pd_attention_run_noalloc", "pd_kv_pack_bytes",
           "pd_kv_pack", "pd_kv_unpack", "pd_kv_pack_heads_bytes", "pd_kv_pack_heads", "pd_kv_unpack_heads",
           "pd_kv_shard_transfers", "pd_xfer_plan", "pd_xfer_buffer_bytes", "pd_xfer_workspace_bytes",
           "pd_xfer_upload", "pd_kv_pack_layers", "pd_kv_unpack_layers", "pd_xfer_free",
           "pd_mla_page_bytes", "pd_mla_plan", "pd_mla_kv_append", "pd_mla_attention_run", "pd_mla_kv_pack",
           "pd_mla_kv_unpack", "pd_status_string", "pd_last_error", "pd_version")


class pd_head_transfer(ctypes.Structure):
    _fields_ = [("src_rank", ctypes.c_int32), ("dst_rank", ctypes.c_int32),
                ("src_h0", ctypes.c_int32), ("src_h1", ctypes.c_int32),
                ("dst_h0", ctypes.c_int32), ("dst_h1", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python decode_attention_kv_pd_amd/build.py` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, VP = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    pI32 = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "pd_plan": (I32, [ctypes.POINTER(pd_attn_desc), I32, pI32, pI32, pI32, pI32, I32,
                          ctypes.POINTER(pd_plan_options), ctypes.POINTER(P)]),
        "pd_plan_workspace_bytes": (SZ, [P]),
        "pd_plan_upload": (I32, [P, VP, SZ, VP]),
        "pd_plan_get_stats": (I32, [P, ctypes.POINTER(pd_plan_stats)]),
        "pd_plan_free": (None, [P]),
        "pd_plan_work_items": (I32, [P, I32, pI32, I32]),
        "pd_kv_append": (I32, [P, VP, VP, VP, VP, VP]),
        "pd_attention_run": (I32, [P, VP, VP, VP, VP, VP, VP]),
        "pd_attention_run_noalloc": (I32, [P, VP, VP, VP, VP, VP, VP, VP]),
        "pd_kv_pack_bytes": (SZ, [ctypes.POINTER(pd_attn_desc), I32]),
        "pd_kv_pack": (I32, [ctypes.POINTER(pd_attn_desc), VP, I32, pI32, I32, VP, SZ, VP, SZ, VP]),
        "pd_kv_unpack": (I32, [ctypes.POINTER(pd_attn_desc), VP, I32, pI32, I32, VP, SZ, VP, SZ, VP]),
        "pd_kv_pack_heads_bytes": (SZ, [ctypes.POINTER(pd_attn_desc), I32, I32, I32]),
        "pd_kv_pack_heads": (I32, [ctypes.POINTER(pd_attn_desc), VP, I32, pI32, I32, I32, I32, VP, SZ, VP, SZ,
                                   VP]),
        "pd_kv_unpack_heads": (I32, [ctypes.POINTER(pd_attn_desc), VP, I32, pI32, I32, I32, I32, VP, SZ, VP, SZ,
                                     VP]),
        "pd_kv_shard_transfers": (I32, [I32, I32, I32, ctypes.POINTER(pd_head_transfer), I32, pI32]),
        "pd_xfer_plan": (I32, [ctypes.POINTER(pd_attn_desc), I32, ctypes.POINTER(VP), I32, pI32, I32, I32, I32,
                               ctypes.POINTER(P)]),
        "pd_xfer_buffer_bytes": (SZ, [P]),
        "pd_xfer_workspace_bytes": (SZ, [P]),
        "pd_xfer_upload": (I32, [P, VP, SZ, VP]),
        "pd_kv_pack_layers": (I32, [P, VP, VP, SZ, VP, VP]),
        "pd_kv_unpack_layers": (I32, [P, VP, VP, SZ, VP, VP]),
        "pd_xfer_free": (None, [P]),
        "pd_mla_page_bytes": (SZ, [ctypes.POINTER(pd_mla_desc)]),
        "pd_mla_plan": (I32, [ctypes.POINTER(pd_mla_desc), I32, pI32, pI32, pI32, pI32, I32,
                              ctypes.POINTER(pd_plan_options), ctypes.POINTER(P)]),
        "pd_mla_kv_append": (I32, [P, VP, VP, VP, VP]),
        "pd_mla_attention_run": (I32, [P, VP, VP, VP, VP, VP, VP]),
        "pd_mla_kv_pack": (I32, [ctypes.POINTER(pd_mla_desc), VP, I32, pI32, I32, VP, SZ, VP, SZ, VP]),
        "pd_mla_kv_unpack": (I32, [ctypes.POINTER(pd_mla_desc), VP, I32, pI32, I32, VP, SZ, VP, SZ, VP]),
        "pd_status_string": (ctypes.c_char_p, [I32]),
        "pd_last_error": (ctypes.c_char_p, []),
        "pd_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def _check(status: int):
    if status != 0:
        raise PdError(status, _lib.pd_last_error().decode())


def version() -> str:
    return _lib.pd_version().decode()


def make_desc(num_qo_heads, num_kv_heads, head_dim, page_size, dtype, causal=True,
              sm_scale=None) -> pd_attn_desc:
    if isinstance(dtype, str):
        dtype = {"f32": PD_F32, "bf16": PD_BF16}[dtype]
    if sm_scale is None:
        sm_scale = 1.0 / float(head_dim) ** 0.5
    return pd_attn_desc(int(num_qo_heads), int(num_kv_heads), int(head_dim), int(page_size),
                        int(dtype), int(bool(causal)), float(sm_scale))


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, nbytes=None):
    """Device pointer of a contiguous GPU tensor (optionally size-checked)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")
    return ctypes.c_void_p(t.data_ptr())


@dataclass
class PlanStats:
    batch: int
    total_q_rows: int
    prefill_tiles: int
    decode_units: int
    decode_row_groups: int
    decode_chunk_keys: int
    prefill_flops: int
    decode_kv_bytes: int
    workspace_bytes: int


class Plan:
    """Owns a pd_plan_t; freed on close() or garbage collection."""

    def __init__(self, handle, desc):
        self._h = handle
        self.desc = desc

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan is closed")
        return self._h

    @property
    def workspace_bytes(self) -> int:
        return int(_lib.pd_plan_workspace_bytes(self.handle))

    def stats(self) -> PlanStats:
        s = pd_plan_stats()
        _check(_lib.pd_plan_get_stats(self.handle, ctypes.byref(s)))
        return PlanStats(*(getattr(s, f) for f, _ in pd_plan_stats._fields_))

    def work_items(self, kind: int) -> np.ndarray:
        """The plan's work list: kind 0 prefill tiles [n, 8], 1 decode units
        [n, 8], 2 merge groups [n, 4], 3 launch block map [n, 1], 4 decode
        queue offsets [n, 1] (see pd_plan_work_items)."""
        width = {0: 8, 1: 8, 2: 4, 3: 1, 4: 1}.get(int(kind), 8)
        n = _lib.pd_plan_work_items(self.handle, int(kind), None, 0)
        if n < 0:
            _check(n)
        out = np.zeros((max(n, 1), width), np.int32)
        got = _lib.pd_plan_work_items(self.handle, int(kind),
                                      out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n)
        if got < 0:
            _check(got)
        return out[:n]

    def close(self):
        if self._h is not None:
            _lib.pd_plan_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def pd_plan(desc, qo_lens, kv_lens, page_indptr, page_indices, num_pool_pages,
            decode_chunk_keys: int = 0, num_cus: int = 0, block_order: int = 0,
            prefill_block_waves: int = 0) -> Plan:
    qo, pqo = _i32(qo_lens)
    kv, pkv = _i32(kv_lens)
    ip, pip = _i32(page_indptr)
    pi, ppi = _i32(page_indices)
    if len(qo) != len(kv) or len(ip) != len(qo) + 1:
        raise ValueError("qo_lens / kv_lens / page_indptr lengths disagree")
    opts = pd_plan_options(int(decode_chunk_keys), int(num_cus), int(block_order), int(prefill_block_waves))
    h = ctypes.c_void_p()
    _check(_lib.pd_plan(ctypes.byref(desc), len(qo), pqo, pkv, pip, ppi if len(pi) else None,
                        int(num_pool_pages), ctypes.byref(opts), ctypes.byref(h)))
    return Plan(h, desc)


def pd_plan_upload(plan: Plan, ws, stream=None):
    _check(_lib.pd_plan_upload(plan.handle, _dev(ws, "ws"), ws.numel() * ws.element_size(),
                               _stream(stream)))


def pd_kv_append(plan: Plan, ws, kv_pool, k_new, v_new, stream=None):
    _check(_lib.pd_kv_append(plan.handle, _dev(ws, "ws"), _dev(kv_pool, "kv_pool"),
                             _dev(k_new, "k_new"), _dev(v_new, "v_new"), _stream(stream)))


def pd_attention_run(plan: Plan, ws, q, kv_pool, out, lse=None, stream=None):
    _check(_lib.pd_attention_run(plan.handle, _dev(ws, "ws"), _dev(q, "q"), _dev(kv_pool, "kv_pool"),
                                 _dev(out, "out"), _dev(lse, "lse"), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024   # PD_NOALLOC_SCRATCH_BYTES


def pd_attention_run_noalloc(plan: Plan, q, kv_pool, out, lse=None, k_new=None, v_new=None, stream=None):
    """pd_attention_run (after pd_kv_append when k_new / v_new are given)
    over the library's static device scratch: no workspace, no upload."""
    _check(_lib.pd_attention_run_noalloc(plan.handle, _dev(q, "q"), _dev(kv_pool, "kv_pool"),
                                         _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(out, "out"),
                                         _dev(lse, "lse"), _stream(stream)))


def pd_kv_pack_bytes(desc, n_pages: int) -> int:
    return int(_lib.pd_kv_pack_bytes(ctypes.byref(desc), int(n_pages)))


def pd_kv_pack(desc, kv_pool, num_pool_pages, page_ids, buf, scratch, stream=None):
    ids, pids = _i32(page_ids)
    _check(_lib.pd_kv_pack(ctypes.byref(desc), _dev(kv_pool, "kv_pool"), int(num_pool_pages), pids,
                           len(ids), _dev(buf, "buf"), buf.numel() * buf.element_size(),
                           _dev(scratch, "scratch"), scratch.numel() * scratch.element_size(),
                           _stream(stream)))


def pd_kv_unpack(desc, kv_pool, num_pool_pages, page_ids, buf, scratch, stream=None):
    ids, pids = _i32(page_ids)
    _check(_lib.pd_kv_unpack(ctypes.byref(desc), _dev(kv_pool, "kv_pool"), int(num_pool_pages), pids,
                             len(ids), _dev(buf, "buf"), buf.numel() * buf.element_size(),
                             _dev(scratch, "scratch"), scratch.numel() * scratch.element_size(),
                             _stream(stream)))


def pd_kv_pack_heads_bytes(desc, n_pages: int, h0: int, h1: int) -> int:
    return int(_lib.pd_kv_pack_heads_bytes(ctypes.byref(desc), int(n_pages), int(h0), int(h1)))


def pd_kv_pack_heads(desc, kv_pool, num_pool_pages, page_ids, h0, h1, buf, scratch, stream=None):
    ids, pids = _i32(page_ids)
    _check(_lib.pd_kv_pack_heads(ctypes.byref(desc), _dev(kv_pool, "kv_pool"), int(num_pool_pages), pids,
                                 len(ids), int(h0), int(h1), _dev(buf, "buf"), buf.numel() * buf.element_size(),
                                 _dev(scratch, "scratch"), scratch.numel() * scratch.element_size(),
                                 _stream(stream)))


def pd_kv_unpack_heads(desc, kv_pool, num_pool_pages, page_ids, h0, h1, buf, scratch, stream=None):
    ids, pids = _i32(page_ids)
    _check(_lib.pd_kv_unpack_heads(ctypes.byref(desc), _dev(kv_pool, "kv_pool"), int(num_pool_pages), pids,
                                   len(ids), int(h0), int(h1), _dev(buf, "buf"),
                                   buf.numel() * buf.element_size(), _dev(scratch, "scratch"),
                                   scratch.numel() * scratch.element_size(), _stream(stream)))


def pd_kv_shard_transfers(num_kv_heads: int, src_shards: int, dst_shards: int) -> list:
    """[(src_rank, dst_rank, src_h0, src_h1, dst_h0, dst_h1), ...]"""
    n = ctypes.c_int32(0)
    _check(_lib.pd_kv_shard_transfers(int(num_kv_heads), int(src_shards), int(dst_shards), None, 0,
                                      ctypes.byref(n)))
    arr = (pd_head_transfer * max(n.value, 1))()
    _check(_lib.pd_kv_shard_transfers(int(num_kv_heads), int(src_shards), int(dst_shards), arr, n.value,
                                      ctypes.byref(n)))
    return [tuple(getattr(arr[i], f) for f, _ in pd_head_transfer._fields_) for i in range(n.value)]


class XferPlan:
    """Owns a pd_xfer_t; freed on close() or garbage collection."""

    def __init__(self, handle, desc, num_layers):
        self._h = handle
        self.desc = desc
        self.num_layers = num_layers

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("transfer plan is closed")
        return self._h

    @property
    def buffer_bytes(self) -> int:
        return int(_lib.pd_xfer_buffer_bytes(self.handle))

    @property
    def workspace_bytes(self) -> int:
        return int(_lib.pd_xfer_workspace_bytes(self.handle))

    def close(self):
        if self._h is not None:
            _lib.pd_xfer_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def pd_xfer_plan(desc, kv_pools, num_pool_pages, page_ids, h0=0, h1=None) -> XferPlan:
    """kv_pools: list of per-layer pool tensors (GPU) or raw device addresses."""
    ptrs = (ctypes.c_void_p * max(len(kv_pools), 1))()
    for i, t in enumerate(kv_pools):
        ptrs[i] = t if isinstance(t, int) else _dev(t, f"kv_pools[{i}]").value
    ids, pids = _i32(page_ids)
    h1 = desc.num_kv_heads if h1 is None else h1
    h = ctypes.c_void_p()
    _check(_lib.pd_xfer_plan(ctypes.byref(desc), len(kv_pools), ptrs, int(num_pool_pages),
                             pids if len(ids) else None, len(ids), int(h0), int(h1), ctypes.byref(h)))
    return XferPlan(h, desc, len(kv_pools))


def pd_xfer_upload(xfer: XferPlan, ws, stream=None):
    _check(_lib.pd_xfer_upload(xfer.handle, _dev(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)))


def _progress_ptr(progress):
    """Address of a progress array: a pinned host tensor or a GPU tensor."""
    if progress is None:
        return None
    if not progress.is_contiguous() or progress.element_size() != 4:
        raise ValueError("progress must be a contiguous 32-bit tensor")
    if not progress.is_cuda and not progress.is_pinned():
        raise ValueError("progress on the host must be pinned (pin_memory=True)")
    return ctypes.c_void_p(progress.data_ptr())


def pd_kv_pack_layers(xfer: XferPlan, ws, buf, progress=None, stream=None):
    _check(_lib.pd_kv_pack_layers(xfer.handle, _dev(ws, "ws"), _dev(buf, "buf"), buf.numel() * buf.element_size(),
                                  _progress_ptr(progress), _stream(stream)))


def pd_kv_unpack_layers(xfer: XferPlan, ws, buf, progress=None, stream=None):
    _check(_lib.pd_kv_unpack_layers(xfer.handle, _dev(ws, "ws"), _dev(buf, "buf"),
                                    buf.numel() * buf.element_size(), _progress_ptr(progress),
                                    _stream(stream)))


# ------------------------------------------------------------ latent (MLA) cache
def make_mla_desc(num_qo_heads, page_size, causal=True, sm_scale=None, kv_lora_rank=512,
                  qk_rope_dim=64) -> pd_mla_desc:
    """sm_scale defaults to 1/sqrt(128 + qk_rope_dim) (DeepSeek-V3's query-key
    head width)."""
    if sm_scale is None:
        sm_scale = 1.0 / float(128 + qk_rope_dim) ** 0.5
    return pd_mla_desc(int(num_qo_heads), int(kv_lora_rank), int(qk_rope_dim), int(page_size), PD_BF16,
                       int(bool(causal)), float(sm_scale))


def pd_mla_page_bytes(mdesc) -> int:
    return int(_lib.pd_mla_page_bytes(ctypes.byref(mdesc)))


def pd_mla_plan(mdesc, qo_lens, kv_lens, page_indptr, page_indices, num_pool_pages,
                decode_chunk_keys: int = 0, num_cus: int = 0) -> Plan:
    qo, pqo = _i32(qo_lens)
    kv, pkv = _i32(kv_lens)
    ip, pip = _i32(page_indptr)
    pi, ppi = _i32(page_indices)
    if len(qo) != len(kv) or len(ip) != len(qo) + 1:
        raise ValueError("qo_lens / kv_lens / page_indptr lengths disagree")
    opts = pd_plan_options(int(decode_chunk_keys), int(num_cus), 0)
    h = ctypes.c_void_p()
    _check(_lib.pd_mla_plan(ctypes.byref(mdesc), len(qo), pqo, pkv, pip, ppi if len(pi) else None,
                            int(num_pool_pages), ctypes.byref(opts), ctypes.byref(h)))
    return Plan(h, mdesc)


def pd_mla_kv_append(plan: Plan, ws, kv_pool, rows_new, stream=None):
    _check(_lib.pd_mla_kv_append(plan.handle, _dev(ws, "ws"), _dev(kv_pool, "kv_pool"), _dev(rows_new, "rows_new"),
                                 _stream(stream)))


def pd_mla_attention_run(plan: Plan, ws, q, kv_pool, out, lse=None, stream=None):
    _check(_lib.pd_mla_attention_run(plan.handle, _dev(ws, "ws"), _dev(q, "q"), _dev(kv_pool, "kv_pool"),
                                     _dev(out, "out"), _dev(lse, "lse"), _stream(stream)))


def pd_mla_kv_pack(mdesc, kv_pool, num_pool_pages, page_ids, buf, scratch, stream=None):
    ids, pids = _i32(page_ids)
    _check(_lib.pd_mla_kv_pack(ctypes.byref(mdesc), _dev(kv_pool, "kv_pool"), int(num_pool_pages), pids, len(ids),
                               _dev(buf, "buf"), buf.numel() * buf.element_size(), _dev(scratch, "scratch"),
                               scratch.numel() * scratch.element_size(), _stream(stream)))


def pd_mla_kv_unpack(mdesc, kv_pool, num_pool_pages, page_ids, buf, scratch, stream=None):
    ids, pids = _i32(page_ids)
    _check(_lib.pd_mla_kv_unpack(ctypes.byref(mdesc), _dev(kv_pool, "kv_pool"), int(num_pool_pages), pids,
                                 len(ids), _dev(buf, "buf"), buf.numel() * buf.element_size(),
                                 _dev(scratch, "scratch"), scratch.numel() * scratch.element_size(),
                                 _stream(stream)))
