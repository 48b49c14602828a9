// Device code shared by the MLA decode kernels (mla.hip: 16 query rows per
// wavefront on 16x16x32 products; mla_wide.hip: 32 rows per wavefront on
// 32x32x16 products): the staging of 32-key steps of the latent cache in
// LDS by direct loads, and LDS reads and waits issued from inline asm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "pd_internal.hpp"

namespace pdk {
namespace {

// A block: 4 wavefronts (one per SIMD), one key range, 32 keys per step.  A step's rows are staged in LDS as four
// Lds<128> tiles (the latent entries 0-127, 128-255, 256-383, 384-511) and
// one Lds<64> tile (the rotary key), the layout whose 16-byte reads (score
// operand) and transposed reads (value operand) are bank-conflict free at
// 128 columns.  Four stages are in flight.
struct MlaCfg {
  static constexpr int KEYS = 32;
  static constexpr int QUARTER = Lds<128>::bytes(KEYS);
  static constexpr int ROPE = 4 * QUARTER;
  static constexpr int STAGE = ROPE + Lds<64>::bytes(KEYS);
  static constexpr int NSTAGE = 4;
  static constexpr int LDS_BYTES = NSTAGE * STAGE;
  static constexpr int KS = kMlaWidth / 32;                     // 32-wide k-steps of S (16 latent, 2 rotary)
  static constexpr int DB = kMlaLatent / 16;                    // 16-row d-blocks of O^T
  static constexpr int LAT_LOADS = 4 * (KEYS / Lds<128>::RPB);  // 1 KiB block loads of a step (latent)
  static constexpr int LOADS = LAT_LOADS + KEYS / Lds<64>::RPB; // ... and rotary
  static constexpr int LOADS_PER_WAVE = 9;  // 8 latent + 1 rotary block loads per wavefront
};
static_assert(MlaCfg::LAT_LOADS == 32 && MlaCfg::LOADS == 4 * MlaCfg::LOADS_PER_WAVE, "stage loads split over the wavefronts");
static_assert(MlaCfg::LDS_BYTES <= 160 * 1024, "LDS of one block");
static_assert(Lds<128>::RPB == 4 && Lds<64>::RPB == 8, "tile geometry");

// Direct global->LDS load of 16 bytes per lane from a wave-uniform base plus
// a 32-bit lane offset (the scalar-base form of the load; see load_lds16).
__device__ __forceinline__ void load_lds16_sbase(const char* base, uint32_t off, LDS_AS char* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}

// Page id of key `key` of a request (clamped to its last key).
__device__ __forceinline__ int mla_page(const MlaParams& p, const ReqInfo& ri, int key) {
  return ldc(p.page_indices + ri.page_start + (min(key, ri.kv - 1) >> p.ps_shift));
}

// A step whose 32 keys are all valid: keys b .. b + 15 are consecutive
// slots of page pgA and b + 16 .. b + 31 of page pgB (pages hold >= 16
// aligned keys), so each of its loads is a wave-uniform base plus a
// loop-invariant lane offset (the scalar-base form of the load).
struct MlaFullStep {
  const char* baseA;  // cache row of key b
  const char* baseB;  // cache row of key b + 16
  LDS_AS char* st;    // stage
};
__device__ __forceinline__ MlaFullStep mla_full_step(const MlaParams& p, int b, int pgA, int pgB, LDS_AS char* st) {
  constexpr int64_t RB = 2 * kMlaWidth;  // bytes per cache row
  const char* pool = (const char*)p.pool;
  const int psm = p.ps - 1;
  return {pool + ((int64_t)pgA * p.ps + (b & psm)) * RB, pool + ((int64_t)pgB * p.ps + ((b + 16) & psm)) * RB, st};
}

// Load I (0..8) of wavefront w's share of a full step: I < 8 the latent
// load (tile I / 2, rows 4 (w + 4 (I % 2)) .. +3), I = 8 the rotary load
// (rows 8 w .. +7).  The loads can be issued one at a time.
template <int I>
__device__ __forceinline__ void mla_issue_full(const MlaFullStep& f, int w, int lane) {
  constexpr int64_t RB = 2 * kMlaWidth;
  if constexpr (I < 8) {
    constexpr int q4 = I / 2;
    const int jb = w + 4 * (I % 2);
    const uint32_t off = (4 * w + Lds<128>::dma_row(lane)) * RB + 256 * q4 + 16 * Lds<128>::dma_chunk(lane);
    load_lds16_sbase(I % 2 ? f.baseB : f.baseA, off, f.st + q4 * MlaCfg::QUARTER + jb * Lds<128>::BLOCK);
  } else {
    const uint32_t off = (8 * (w % 2) + Lds<64>::dma_row(lane)) * RB + 2 * kMlaLatent + 16 * Lds<64>::dma_chunk(lane);
    load_lds16_sbase(w < 2 ? f.baseA : f.baseB, off, f.st + MlaCfg::ROPE + w * Lds<64>::BLOCK);
  }
}

// Wavefront w's share (latent loads i = 0..7: tile i / 2, rows 4 (w + 4 (i
// % 2)) .. +3; then one rotary load, rows 8 w .. +7) of the 36 block loads
// of the step at key b into stage `st`.  pgA / pgB are the pages of keys b
// .. b + 15 and b + 16 .. b + 31.  Keys >= kv (only in a request's last
// step) are read from key kv - 1 instead: finite data, masked later, and
// tail slots are never read.
__device__ __forceinline__ void mla_issue(const MlaParams& p, const ReqInfo& ri, int b, int pgA, int pgB,
                                          int w, int lane, LDS_AS char* st) {
  const char* pool = (const char*)p.pool;
  const int kvm1 = ri.kv - 1;
  const int psm = p.ps - 1;
  constexpr int64_t RB = 2 * kMlaWidth;  // bytes per cache row
  if (b + 32 <= ri.kv) {
    const MlaFullStep f = mla_full_step(p, b, pgA, pgB, st);
    mla_issue_full<0>(f, w, lane);
    mla_issue_full<1>(f, w, lane);
    mla_issue_full<2>(f, w, lane);
    mla_issue_full<3>(f, w, lane);
    mla_issue_full<4>(f, w, lane);
    mla_issue_full<5>(f, w, lane);
    mla_issue_full<6>(f, w, lane);
    mla_issue_full<7>(f, w, lane);
    mla_issue_full<8>(f, w, lane);
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q4 = i / 2, jb = w + 4 * (i % 2);
    const int row = 4 * jb + Lds<128>::dma_row(lane);
    const int key = min(b + row, kvm1);
    const int page = jb < 4 ? pgA : pgB;
    load_lds16(pool + ((int64_t)page * p.ps + (key & psm)) * RB + 256 * q4 + 16 * Lds<128>::dma_chunk(lane),
               st + q4 * MlaCfg::QUARTER + jb * Lds<128>::BLOCK);
  }
  {
    const int row = 8 * w + Lds<64>::dma_row(lane);
    const int key = min(b + row, kvm1);
    const int page = w < 2 ? pgA : pgB;
    load_lds16(pool + ((int64_t)page * p.ps + (key & psm)) * RB + 2 * kMlaLatent + 16 * Lds<64>::dma_chunk(lane),
               st + MlaCfg::ROPE + w * Lds<64>::BLOCK);
  }
}

// 16-byte LDS read issued from inline asm, so that the compiler neither
// reorders it nor waits for it: the caller waits with lgkm_wait_for.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16_asm(const LDS_AS char* p) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field");
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(p), "n"(OFF) : "memory");
  return v;
}

// Wait until the LDS read that produced `v` has landed, given that LATER
// reads were issued after it.  LDS reads complete in issue order, so at most
// LATER outstanding LGKM operations means this one is done, whatever else
// (scalar loads) is in flight.  Tying `v` to the wait keeps its consumer
// after it.
template <int LATER>
__device__ __forceinline__ void lgkm_wait_for(u32x4& v) {
  static_assert(LATER >= 0 && LATER < 16, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(LATER));
}

// Transposed 8-byte LDS read issued from inline asm (see lds_read16_asm).
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16_asm(const LDS_AS char* p) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field");
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(p), "n"(OFF) : "memory");
  return v;
}

// Wait for this wavefront's loads of the current step, with `later_steps`
// (<= 2) later steps' loads (LPW each) still allowed in flight.
template <int LPW>
__device__ __forceinline__ void mla_wait_loads(int later_steps) {
  if (later_steps >= 2)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPW) : "memory");
  else if (later_steps == 1)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace
}  // namespace pdk
