// Device helpers shared by the attention kernels (attention.hip) and the MLA
// decode kernel (mla.hip) for gfx950 (MI355X, CDNA4): vector types, MFMA and
// LDS wrappers, direct global->LDS loads, lane reductions, the speculative
// softmax's range test, and the LDS tile layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ int uniform_i(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Read-only planner tables (work items, request rows, page table) are read
// through the constant address space, so wave-uniform reads become scalar
// loads instead of vector loads followed by a full vmcnt wait.
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

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Transposed LDS read of 16-bit elements: in each 16-lane group, lane j
// addresses row j/4, columns 4*(j%4)..+3 of a 4-row block and receives column
// j of that block (rows 0..3), two elements per dword.
__device__ __forceinline__ u32x2 lds_read_tr16(const LDS_AS char* p) {
  bf16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
  return __builtin_bit_cast(u32x2, t);
}

__device__ __forceinline__ u32x4 lds_read16(const LDS_AS char* p) { return *(const LDS_AS u32x4*)p; }

// 16 bytes per lane, global -> LDS without passing through VGPRs
// (global_load_lds_dwordx4).  `lds` is the wave-uniform base of a 1 KiB
// destination, passed in M0; lane i lands at lds + 16 * i.
// Issued from inline asm: the compiler's own wait insertion treats every LDS
// read that follows a direct-to-LDS load as possibly aliasing it and waits
// for all loads in flight (vmcnt(0)), which would wait for the prefetches of
// later tiles too.  The kernels instead wait for exactly the loads they need
// (s_waitcnt vmcnt(n) before the barrier that publishes a tile).  The s_nop
// is the wait state a write of M0 needs before a direct-to-LDS load reads it.
__device__ __forceinline__ void load_lds16(const void* src, LDS_AS char* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}
// The same with the non-temporal hint, for the decode role's V stream (read
// once).  Measured on MI355X over the long workload: decode-only 9 % faster,
// the mixed launch 1 % faster.  (The same hint on the decode K loads into
// registers made the mixed launch 8 % slower, so they keep the default.)
__device__ __forceinline__ void load_lds16_nt(const void* src, LDS_AS char* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "{m0}"(m0) : "memory");
}

// N 16-byte fragments 64 bytes apart (src, src + 64, ...) into registers,
// issued from inline asm.  The loads are asynchronous and invisible to the
// compiler: it takes the registers as written when the asm ends, so the
// caller must wait for them itself (s_waitcnt vmcnt) and then pin them
// (pin_regs) before any instruction reads them.  Used where the compiler's
// own wait insertion, which cannot count the direct-to-LDS loads above,
// would otherwise wait for loads of later steps as well.
template <int N>
__device__ __forceinline__ void load_frags64(const void* src, u32x4 (&f)[N]);
template <>
__device__ __forceinline__ void load_frags64<4>(const void* src, u32x4 (&f)[4]) {
  asm volatile(
      "global_load_dwordx4 %0, %4, off\n\t"
      "global_load_dwordx4 %1, %4, off offset:64\n\t"
      "global_load_dwordx4 %2, %4, off offset:128\n\t"
      "global_load_dwordx4 %3, %4, off offset:192"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
      : "v"(src));
}
template <>
__device__ __forceinline__ void load_frags64<2>(const void* src, u32x4 (&f)[2]) {
  asm volatile(
      "global_load_dwordx4 %0, %2, off\n\t"
      "global_load_dwordx4 %1, %2, off offset:64"
      : "=&v"(f[0]), "=&v"(f[1])
      : "v"(src));
}
// After the s_waitcnt that covers their loads: from here on the compiler
// sees the registers as defined by this (empty) asm, which it keeps after the
// wait, so no read of them can move above it.
template <int N>
__device__ __forceinline__ void pin_regs(u32x4 (&f)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(f[i]));
}

// Reductions across lane l and lane l ^ 32 / l ^ 16 (v_permlane*_swap).
__device__ __forceinline__ float max_x32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_x16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// True when any of the packed bf16 P values is >= 2^64, inf or NaN (P >= 0,
// so the bit patterns order like the values).
template <int N>
__device__ __forceinline__ bool p_out_of_range(const uint32_t (&pk)[N]) {
  u16x2 m = __builtin_bit_cast(u16x2, pk[0]);
#pragma unroll
  for (int i = 1; i < N; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, pk[i]));
  return max(m.x, m.y) > 0x5F7F;
}
constexpr uint32_t kBf16OnesPair = 0x3F803F80u;  // two bf16 1.0
__device__ __forceinline__ bool wave_any(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0; }

// Speculative softmax: P = exp2(s * c - m_ref * c) is computed against the
// reference maximum m_ref of earlier tiles, without this tile's row maximum.
// Only when some P of the tile is >= 2^64 (or inf / NaN, which is also how
// the first tile, m_ref = -inf, is caught) is the row maximum taken, O and l
// rescaled and P recomputed.  m_ref never exceeds the true running maximum,
// so P never underflows more than with an exact maximum, and P < 2^64 stays
// far inside the bf16 / fp32 range.  The normaliser l is the sum of the same
// bf16-rounded P that multiply V (v_dot2 against bf16 ones in the prefill
// role, an extra MFMA against an all-ones operand in the decode role), so O
// is a convex combination of V rows whatever m_ref is, and a single dominant
// key is reproduced exactly.

// LDS tile layout (K and V tiles of the prefill role, V stages of the decode
// role).  Rows of D bf16 go into 1 KiB load blocks of RPB = 512 / D rows,
// filled by one direct global->LDS load each (lane l lands at slot l, 16
// bytes).  Blocks are 1056 bytes apart (32 bytes of padding).
//   * Slot 4 q + i of a block holds row r = q % RPB, chunk 4 (q / RPB) +
//     (i ^ (r & 1)): each group of four lanes of the load fetches 64
//     contiguous bytes of one row.  The direct loads move data at several
//     times the rate of a layout whose neighbouring lanes fetch different
//     rows (measured on MI355X: 130 vs 38 GB/s per CU from L2).
//   * LDS has 64 banks of 4 bytes on gfx950.  The 1056-byte block stride and
//     the chunk swizzle (i ^ (r & 1)) keep the reads of both roles on distinct
//     banks at head_dim 128: the K reads (16 bytes per lane, consecutive rows
//     on consecutive lanes) and the transposed V reads (4 rows x 32 bytes per
//     16 lanes).  At head_dim 64 the K reads are two-way.
//   * Every read address is a per-lane constant plus an immediate: chunk
//     steps of 2 keep the swizzle bit (see chunk_step).
template <int D>
struct Lds {
  static constexpr int RPB = 512 / D;
  static constexpr int BLOCK = 1056;
  static constexpr int ROW_BYTES = 2 * D;
  __device__ static constexpr int off(int row, int chunk) {
    const int r = row % RPB;
    return (row / RPB) * BLOCK + 16 * (4 * (RPB * (chunk / 4) + r) + ((chunk % 4) ^ (r & 1)));
  }
  // off(row, c0 + 2 k) - off(row, c0) for c0 in {0, 1} (the same for every row).
  __device__ static constexpr int chunk_step(int k) { return 64 * RPB * (k / 2) + 32 * (k % 2); }
  // Row (in the block) and chunk that lane l of a block load fetches.
  __device__ static constexpr int dma_row(int l) { return (l / 4) % RPB; }
  __device__ static constexpr int dma_chunk(int l) { return 4 * (l / (4 * RPB)) + ((l % 4) ^ (dma_row(l) & 1)); }
  static constexpr int bytes(int rows) { return rows / RPB * BLOCK; }
  // Lane l of a block load lands where off() places its row and chunk, and
  // chunk_step matches off() for every row.
  __device__ static constexpr bool consistent() {
    for (int l = 0; l < 64; ++l)
      if (off(dma_row(l), dma_chunk(l)) != 16 * l) return false;
    for (int row = 0; row < 64; ++row)
      for (int c0 = 0; c0 < 2; ++c0)
        for (int k = 0; 2 * k + c0 < D / 8; ++k)
          if (off(row, c0 + 2 * k) - off(row, c0) != chunk_step(k)) return false;
    return true;
  }
};
static_assert(Lds<128>::consistent() && Lds<64>::consistent(), "LDS tile layout");

}  // namespace
}  // namespace pdk
