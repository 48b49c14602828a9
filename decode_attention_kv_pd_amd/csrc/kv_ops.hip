// HIP KV-cache copy kernels for gfx950 (MI355X, CDNA4): the append of new
// K/V rows into their pages, and page transfers (pack / unpack of whole pages
// or of a range of KV heads, for one or several layers, with per-layer
// completion counters).
//
// What is copied follows the Perplexity post "Disaggregated prefill and
// decode": K/V are appended to the paged cache before attention reads them
// and copies of a layer's pages may start right after its append (section
// "KV Messenger"); pages hold heads before tokens, so a page and each head
// range of it are contiguous runs, and differently sharded ranks exchange
// head ranges of pages (section "Sharded KV Cache Transfers").  Every copy is
// bit-exact (16-byte moves of the stored bytes).
//
// Layout recap (see include/pd_attn.h): pool [pages][2][H_kv][ps][D],
// k_new / v_new [rows][H_kv][D].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "pd_internal.hpp"

namespace pdk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Planner tables are read through the constant address space (wave-uniform
// reads become scalar loads).
#define CONST_AS __attribute__((address_space(4)))
template <class T>
__device__ __forceinline__ T ldc(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "dword-sized tables");
  T out;
  const CONST_AS int32_t* src = (const CONST_AS int32_t*)p;
  int32_t* dst = (int32_t*)&out;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) dst[i] = src[i];
  return out;
}

// ------------------------------------------------------------------------
// KV append: the new rows are cut into 16-byte chunks (a row is 2 H_kv heads
// of D elements, K then V); a block copies `rows_per_block` consecutive rows
// (about 16 KB), each thread four chunks at a time (loads, then stores).  The
// (page, slot) of every row comes from the planner's row table.
// ------------------------------------------------------------------------
constexpr int kAppendBatch = 4;

__global__ __launch_bounds__(kBlockThreads) void append_kernel(AppendParams p) {
  const int cph = p.D * p.elt / 16;             // chunks per head row
  const int cpr = 2 * p.H_kv * cph;             // chunks per token row
  const int row0 = blockIdx.x * p.rows_per_block;
  const int nrows = min(p.rows_per_block, p.total_rows - row0);
  const int nchunks = nrows * cpr;
  const int64_t page_bytes = (int64_t)cpr * 16 * p.ps;
  for (int c0 = threadIdx.x; c0 < nchunks; c0 += kBlockThreads * kAppendBatch) {
    u32x4 v[kAppendBatch];
    char* dst[kAppendBatch];
#pragma unroll
    for (int k = 0; k < kAppendBatch; ++k) {
      const int c = c0 + k * kBlockThreads;
      dst[k] = nullptr;
      if (c < nchunks) {
        const int r = c / cpr, rem = c - r * cpr;
        const int kvsel = rem / (p.H_kv * cph), hc = rem - kvsel * (p.H_kv * cph);  // head * cph + part
        const int row = row0 + r;
        const int2 at = p.rowpos[row];                                                // (page, slot)
        const char* src = (const char*)(kvsel ? p.v_new : p.k_new) + ((int64_t)row * p.H_kv * cph + hc) * 16;
        const int hh = hc / cph, part = hc - hh * cph;
        dst[k] = (char*)p.pool + at.x * page_bytes + ((int64_t)((kvsel * p.H_kv + hh) * p.ps + at.y) * cph + part) * 16;
        v[k] = *(const u32x4*)src;
      }
    }
#pragma unroll
    for (int k = 0; k < kAppendBatch; ++k)
      if (dst[k]) *(u32x4*)dst[k] = v[k];
  }
}

// ------------------------------------------------------------------------
// Page transfers (pack / unpack, whole pages or a range of KV heads, one or
// several layers).  The slice of page p moved for layer l is its K part then
// its V part, each seg_bytes long at seg_off in its half (HND: a head range
// of a half is one contiguous run); in the buffer it sits at ((l * n + i) *
// 2 + half) * seg_bytes.  Items of work are (page i, 64 KiB slab y, layer
// l): 16 chunks of 16 B per thread, all loads of a slab before its stores.
// ------------------------------------------------------------------------
constexpr int kPackChunksPerThread = 16;
constexpr int64_t kSlabChunks = (int64_t)kBlockThreads * kPackChunksPerThread;

// Plain single-layer transfers: a grid of at most kXferBlocks blocks strides
// over the (page, slab) items; loads and stores carry the non-temporal hint
// (every byte is read once and written once).  The page ids come from the
// kernel arguments when they fit there (no upload before the launch) or from
// device memory.  Measured on MI355X (512 pages of 256 KiB out of a
// 4096-page pool, after a 1 GiB flush): pack 50 vs 54-55 us with one block
// per (page, slab), unpack 53 vs 55 us; the ids in the arguments save the
// 5-10 us that their upload added in front of every call.
constexpr int kXferBlocks = 1024;
struct XferInlineIds {
  int32_t id[kXferInlineIds];
};

template <class Ids>
__device__ __forceinline__ void xfer_plain(const XferParams& p, const Ids& ids) {
  const int64_t segc = p.seg_bytes / 16;
  const int64_t ny = (2 * segc + kSlabChunks - 1) / kSlabChunks;
  const int64_t items = (int64_t)p.n * ny;
  for (int64_t w = blockIdx.x; w < items; w += gridDim.x) {
    const int i = (int)(w / ny);
    const int64_t y = w - (int64_t)i * ny;
    const int64_t page = ids(i);
    char* buf = p.buf + (int64_t)i * 2 * p.seg_bytes;
    char* pg = (char*)p.pool0 + page * p.page_bytes + p.seg_off;
    const int64_t cs = y * kSlabChunks;  // first chunk of the slab
    const int64_t c0 = cs + threadIdx.x;
    u32x4 v[kPackChunksPerThread];
    if (cs + kSlabChunks <= segc || (cs >= segc && cs + kSlabChunks <= 2 * segc)) {
      // the whole slab lies in one half: one contiguous run on both sides
      const int64_t pc = cs < segc ? cs * 16 : p.half_bytes + (cs - segc) * 16;
      const char* src = (p.to_buffer ? pg + pc : buf + cs * 16) + 16 * threadIdx.x;
      char* dst = (p.to_buffer ? buf + cs * 16 : pg + pc) + 16 * threadIdx.x;
#pragma unroll
      for (int k = 0; k < kPackChunksPerThread; ++k)
        v[k] = __builtin_nontemporal_load((const u32x4*)(src + 16 * k * kBlockThreads));
#pragma unroll
      for (int k = 0; k < kPackChunksPerThread; ++k)
        __builtin_nontemporal_store(v[k], (u32x4*)(dst + 16 * k * kBlockThreads));
      continue;
    }
#pragma unroll
    for (int k = 0; k < kPackChunksPerThread; ++k) {
      const int64_t c = c0 + k * kBlockThreads;
      if (c < 2 * segc) {
        const int64_t pc = c < segc ? c * 16 : p.half_bytes + (c - segc) * 16;
        v[k] = __builtin_nontemporal_load((const u32x4*)(p.to_buffer ? pg + pc : buf + c * 16));
      }
    }
#pragma unroll
    for (int k = 0; k < kPackChunksPerThread; ++k) {
      const int64_t c = c0 + k * kBlockThreads;
      if (c < 2 * segc) {
        const int64_t pc = c < segc ? c * 16 : p.half_bytes + (c - segc) * 16;
        __builtin_nontemporal_store(v[k], (u32x4*)(p.to_buffer ? buf + c * 16 : pg + pc));
      }
    }
  }
}

__global__ __launch_bounds__(kBlockThreads) void xfer_plain_kernel(XferParams p) {
  xfer_plain(p, [&](int i) { return p.page_ids[i]; });
}
__global__ __launch_bounds__(kBlockThreads) void xfer_inline_kernel(XferParams p, XferInlineIds ids) {
  xfer_plain(p, [&](int i) { return ids.id[i]; });
}

// Multi-layer transfers with per-layer completion: block (page i, slab y,
// layer l); grid order makes the blocks of layer 0 dispatch first.  The
// copies are written through to memory (stores coherent at system scope, so
// no L2 write-back is needed to publish them), each block counts itself
// done once its stores are acknowledged, and the last block of layer l to
// finish resets that layer's block counter (so the next call starts from
// zero without a memset) and, with a progress array, adds one to
// progress[l] with a system-scope release store.
// Measured on MI355X (512 pages of 256 KiB, 8 layers): 5.1 TB/s read +
// written with 64 KiB slabs against 2.7 TB/s with 16 KiB slabs (each block
// waits for its stores to be acknowledged before it retires).  (A release
// fence per block after plain stores, instead of write-through, ran at 0.24
// TB/s: the L2 write-back it implies is per block.)

// 16-byte vector store written through to memory (coherent at system scope).
__device__ __forceinline__ void store16_sys(char* p, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}

__global__ __launch_bounds__(kBlockThreads) void xfer_layers_kernel(XferParams p) {
  const int i = blockIdx.x;
  const int l = blockIdx.z;
  const int64_t page = p.page_ids[i];
  char* pool = (char*)(p.layers ? p.layers[l] : p.pool0);
  const int64_t segc = p.seg_bytes / 16;
  char* buf = p.buf + ((int64_t)l * p.n + i) * 2 * p.seg_bytes;
  char* pg = pool + page * p.page_bytes + p.seg_off;
  const int64_t c0 = (int64_t)blockIdx.y * kSlabChunks + threadIdx.x;
  u32x4 v[kPackChunksPerThread];
#pragma unroll
  for (int k = 0; k < kPackChunksPerThread; ++k) {
    const int64_t c = c0 + k * kBlockThreads;
    if (c < 2 * segc) {
      const int64_t pc = c < segc ? c * 16 : p.half_bytes + (c - segc) * 16;
      v[k] = *(const u32x4*)(p.to_buffer ? pg + pc : buf + c * 16);
    }
  }
#pragma unroll
  for (int k = 0; k < kPackChunksPerThread; ++k) {
    const int64_t c = c0 + k * kBlockThreads;
    if (c < 2 * segc) {
      const int64_t pc = c < segc ? c * 16 : p.half_bytes + (c - segc) * 16;
      store16_sys(p.to_buffer ? buf + c * 16 : pg + pc, v[k]);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores have reached memory
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t blocks = gridDim.x * gridDim.y;
    const uint32_t prev = __hip_atomic_fetch_add(p.done + l, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == blocks - 1) {
      __hip_atomic_store(p.done + l, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (p.progress) {
        __threadfence_system();
        const uint32_t n = __hip_atomic_load(p.progress + l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(p.progress + l, n + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  if (p.total_rows == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((p.total_rows + p.rows_per_block - 1) / p.rows_per_block);
  hipLaunchKernelGGL(append_kernel, dim3(blocks), dim3(kBlockThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_xfer(const XferParams& p, const int32_t* host_ids, hipStream_t s) {
  if (p.n == 0 || p.L == 0) return hipSuccess;
  if (p.done) {
    const unsigned ny = (unsigned)((2 * p.seg_bytes / 16 + kSlabChunks - 1) / kSlabChunks);
    hipLaunchKernelGGL(xfer_layers_kernel, dim3(p.n, ny, p.L), dim3(kBlockThreads), 0, s, p);
    return hipGetLastError();
  }
  const int64_t items = (int64_t)p.n * ((2 * p.seg_bytes / 16 + kSlabChunks - 1) / kSlabChunks);
  const unsigned blocks = (unsigned)std::min<int64_t>(items, kXferBlocks);
  if (host_ids && p.n <= kXferInlineIds) {
    XferInlineIds ids;
    std::copy(host_ids, host_ids + p.n, ids.id);
    hipLaunchKernelGGL(xfer_inline_kernel, dim3(blocks), dim3(kBlockThreads), 0, s, p, ids);
  } else {
    hipLaunchKernelGGL(xfer_plain_kernel, dim3(blocks), dim3(kBlockThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace pdk
