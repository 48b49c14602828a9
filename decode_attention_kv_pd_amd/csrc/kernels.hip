// HIP kernels for gfx950 (MI355X, CDNA4): KV append, page pack/unpack,
// ragged paged attention (causal prefill tiles on bf16 MFMA and split-KV
// decode units in one launch), and the merge of split-KV partial results.
//
// What is computed follows the Perplexity post "Disaggregated prefill and
// decode": requests with many query tokens (prefill, compute bound) and
// requests with one query token over a long cache (decode, bound by reading
// the cache) are batched into one step; attention is spread over requests and
// over kv_len (section "Prefill vs Decode performance"); K/V are appended to
// paged caches whose pages hold heads before tokens (sections "KV Messenger"
// and "Sharded KV Cache Transfers"); whole pages move between devices
// (section "KV Messenger").  The attention formula is standard scaled
// dot-product softmax with the causal mask aligned to the end of the cache.
//
// Layout recap (see include/pd_attn.h): pool [pages][2][H_kv][ps][D],
// q [rows][H_q][D], k_new / v_new [rows][H_kv][D], out fp32 [rows][H_q][D].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pd_internal.hpp"

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

// 4 x 16 transposed LDS read: in each 16-lane group, lane j addresses row j/4,
// columns 4*(j%4)..+3 of a 4-row block of 16-bit elements and receives column
// j of that block (rows 0..3), two elements per dword.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  bf16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
  return __builtin_bit_cast(u32x2, t);
}

// 16 bytes per lane, global -> LDS without passing through VGPRs.  `lds` is
// the wave-uniform base of a 1 KiB destination; lane i lands at lds + 16 * i.
__device__ __forceinline__ void load_lds16(const void* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, (LDS_AS void*)lds, 16, 0, 0);
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

// LDS swizzles (16-byte chunks within a row of D bf16 elements).
// K rows are read 16 bytes per lane, eight consecutive rows per LDS cycle:
// XOR with row % 8 spreads them over eight chunk positions.
__device__ __forceinline__ int swz_k(int row) { return row & 7; }
// V rows are read by the 4 x 16 transposed read (4 rows x 32 bytes per
// 16-lane group): XOR with 2 * (row % 4) keeps each 32-byte pair together and
// moves the four rows to four different pairs.
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 1; }

// ------------------------------------------------------------------------
// Decode role: one wavefront computes one DecodeItem (<= 16 query rows of
// one KV head over keys [k0, k1)), 32 keys per step.
//   S^T[key][col] = K Q^T on v_mfma_f32_16x16x32_bf16 (K from global straight
//   into the A operand; Q^T held in registers as the B operand);
//   online softmax per column across the four 16-lane groups;
//   O^T[d][col] += V^T P^T on the same MFMA, V staged through LDS by direct
//   global->LDS loads and read back transposed; P^T comes from the S
//   accumulators without any lane exchange (key order inside the 32-key step
//   is permuted identically in both operands).
// ------------------------------------------------------------------------
template <int D>
struct DecodeCfg {
  static constexpr int KS = D / 32;               // 32-wide k-steps of S
  static constexpr int DB = D / 16;               // 16-row d-blocks of O^T
  static constexpr int ROW_BYTES = 2 * D;
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;            // rows per 1 KiB load
  static constexpr int VLOADS = 32 / RPI;         // V loads per 32-key step
  static constexpr int STAGE_BYTES = 32 * ROW_BYTES;
  static constexpr int WAVE_LDS = 2 * STAGE_BYTES;
};

template <int D>
__device__ __forceinline__ void decode_issue(const AttnParams& p, const ReqInfo& ri, int hk, int b,
                                             int lane, u32x4 (&kf)[2][D / 32], char* stage) {
  using C = DecodeCfg<D>;
  const uint16_t* pool = (const uint16_t*)p.pool;
  const int32_t* pages = p.page_indices + ri.page_start;
  const int kvm1 = ri.kv - 1;
  const int psm = p.ps - 1;
  const int n = lane & 15, q = lane >> 4;
  int64_t kbase[2], vbase[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int j0 = b + 16 * sb;
    const int page = pages[min(j0, kvm1) / p.ps];  // wave-uniform
    kbase[sb] = (int64_t)page * p.page_elems + (int64_t)hk * p.ps * D;
    vbase[sb] = (int64_t)page * p.page_elems + (int64_t)(p.H_kv + hk) * p.ps * D;
    const int row = min(j0 + n, kvm1) & psm;
    const uint16_t* kp = pool + kbase[sb] + (int64_t)row * D + 8 * q;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kf[sb][ks] = *(const u32x4*)(kp + 32 * ks);
  }
#pragma unroll
  for (int i = 0; i < C::VLOADS; ++i) {
    const int R = i * C::RPI + lane / C::CPR;  // row of the 32-key step
    const int pc = lane % C::CPR;
    const int c = pc ^ swz_v(R);
    const int sb = (i * C::RPI) >> 4;
    const int row = min(b + R, kvm1) & psm;
    const uint16_t* vp = pool + vbase[sb] + (int64_t)row * D + 8 * c;
    load_lds16(vp, stage + i * 1024);
  }
}

// One 32-key step of a decode unit: issue the next step's loads (K into
// `kn`, V into LDS stage `sn`), wait for this step's, then S, softmax, PV.
template <int D>
__device__ __forceinline__ void decode_step(const AttnParams& p, const ReqInfo& ri, int hk, int b, int k1,
                                            int lim, int lane, const u32x4 (&qf)[D / 32],
                                            const u32x4 (&kc)[2][D / 32], u32x4 (&kn)[2][D / 32],
                                            const char* st, char* sn, float& m_run, float& l_run,
                                            f32x4 (&oacc)[D / 16]) {
  using C = DecodeCfg<D>;
  const int q = lane >> 4;
  const float cl = p.c_log2;
  const int nb = b + 32;
  if (nb < k1) {
    decode_issue<D>(p, ri, hk, nb, lane, kn, sn);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * C::KS + C::VLOADS) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  // S^T for keys b + 16 sb + 4 q + i, column n
  f32x4 s[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) s[sb] = mfma16(kc[sb][ks], qf[ks], s[sb]);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = b + 16 * sb + 4 * q + i;
      if (key >= lim) s[sb][i] = -INFINITY;
      mx = fmaxf(mx, s[sb][i]);
    }
  mx = max_x16(mx);
  mx = max_x32(mx);
  const float m_new = fmaxf(m_run, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = fast_exp2((m_run - m_use) * cl);
  const float mc = m_use * cl;
  float psum = 0.f;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[sb][i] = fast_exp2(__builtin_fmaf(s[sb][i], cl, -mc));
      psum += s[sb][i];
    }
  l_run = l_run * alpha + psum;
  m_run = m_new;
  u32x4 pb = {pack_bf16(s[0][0], s[0][1]), pack_bf16(s[0][2], s[0][3]),
              pack_bf16(s[1][0], s[1][1]), pack_bf16(s[1][2], s[1][3])};
  // V^T[d = 16 db + j][keys 4q + e, 16 + 4q + e] from the transposed read
  const int j = lane & 15;
  const int r1 = 4 * q + (j >> 2);
  const int r2 = r1 + 16;
  const int half = (j & 1) * 8;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const int c = 2 * db + ((j & 3) >> 1);
    u32x2 a1 = lds_read_tr16(st + r1 * C::ROW_BYTES + ((c ^ swz_v(r1)) << 4) + half);
    u32x2 a2 = lds_read_tr16(st + r2 * C::ROW_BYTES + ((c ^ swz_v(r2)) << 4) + half);
    u32x4 a = {a1[0], a1[1], a2[0], a2[1]};
    oacc[db] = oacc[db] * alpha;
    oacc[db] = mfma16(a, pb, oacc[db]);
  }
}

template <int D>
__device__ void decode_unit(const AttnParams& p, int unit, char* lds) {
  using C = DecodeCfg<D>;
  const int lane = threadIdx.x & 63;
  const DecodeItem it = p.du[unit];
  const ReqInfo ri = p.req[it.req];
  const int g = p.g;
  const int nrows = ri.qo * g;
  const int n = lane & 15, q = lane >> 4;
  const bool col_ok = n < nrows;
  const int t = col_ok ? n / g : 0;
  const int h = it.hk * g + (col_ok ? n % g : 0);
  const int lim = min(it.k1, p.causal ? ri.kv - ri.qo + t + 1 : ri.kv);

  u32x4 qf[C::KS];
  {
    const uint16_t* qp = (const uint16_t*)p.q + ((int64_t)(ri.qo_start + t) * p.H_q + h) * D + 8 * q;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 v = *(const u32x4*)(qp + 32 * ks);
      qf[ks] = col_ok ? v : u32x4{0, 0, 0, 0};
    }
  }

  f32x4 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  u32x4 kf0[2][C::KS], kf1[2][C::KS];
  decode_issue<D>(p, ri, it.hk, it.k0, lane, kf0, lds);
  for (int b = it.k0;;) {
    decode_step<D>(p, ri, it.hk, b, it.k1, lim, lane, qf, kf0, kf1, lds, lds + C::STAGE_BYTES, m_run,
                   l_run, oacc);
    b += 32;
    if (b >= it.k1) break;
    decode_step<D>(p, ri, it.hk, b, it.k1, lim, lane, qf, kf1, kf0, lds + C::STAGE_BYTES, lds, m_run,
                   l_run, oacc);
    b += 32;
    if (b >= it.k1) break;
  }
  // columns: sum the four 16-lane groups
  float l_tot = sum_x16(l_run);
  l_tot = sum_x32(l_tot);
  if (col_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* po = p.part_o + ((int64_t)it.part * kDecodeCols + n) * D + 4 * q;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) *(f32x4*)(po + 16 * db) = oacc[db] * inv;
    if (q == 0)
      p.part_lse[(int64_t)it.part * kDecodeCols + n] =
          l_tot > 0.f ? m_run * p.sm_scale + __logf(l_tot) : -INFINITY;
  }
}

// ------------------------------------------------------------------------
// Prefill role: one 256-thread block computes one PrefillItem (<= 128 query
// rows: tokens x the g heads of one KV head) over 64-key tiles.
//   Wave w owns query rows 32 w .. 32 w + 31 (the N index of both products).
//   S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16; Q^T stays in
//   registers; K and V tiles are staged in LDS (double buffered, direct
//   global->LDS loads, one 16-row page group per wave); K is read back 16
//   bytes per lane, V with the transposed read; P^T is the S accumulator
//   re-packed to bf16 in place.  Only tiles that cross the causal diagonal
//   (or the end of the cache) are masked.
// ------------------------------------------------------------------------
template <int D>
struct PrefillCfg {
  static constexpr int KS = D / 16;     // 16-wide k-steps of S
  static constexpr int DB = D / 32;     // 32-row d-blocks of O^T
  static constexpr int ROW_BYTES = 2 * D;
  static constexpr int CPR = D / 8;
  static constexpr int RPI = 64 / CPR;  // rows per 1 KiB load
  static constexpr int LOADS = 16 / RPI;
  static constexpr int TILE_BYTES = 64 * ROW_BYTES;
  static constexpr int LDS_BYTES = 4 * TILE_BYTES;  // K, V x 2 buffers
};

template <int D>
__device__ __forceinline__ void prefill_issue(const AttnParams& p, const ReqInfo& ri, int hk,
                                              int kv_end, int kbase, int w, int lane, char* kbuf,
                                              char* vbuf) {
  using C = PrefillCfg<D>;
  const uint16_t* pool = (const uint16_t*)p.pool;
  const int32_t* pages = p.page_indices + ri.page_start;
  const int last = kv_end - 1;
  const int j0 = kbase + 16 * w;
  const int page = pages[min(j0, last) / p.ps];
  const int64_t kb = (int64_t)page * p.page_elems + (int64_t)hk * p.ps * D;
  const int64_t vb = (int64_t)page * p.page_elems + (int64_t)(p.H_kv + hk) * p.ps * D;
  const int psm = p.ps - 1;
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int R0 = 16 * w + i * C::RPI;
    const int R = R0 + lane / C::CPR;
    const int pc = lane % C::CPR;
    const int row = min(kbase + R, last) & psm;
    load_lds16(pool + kb + (int64_t)row * D + 8 * (pc ^ swz_k(R)), kbuf + R0 * C::ROW_BYTES);
    load_lds16(pool + vb + (int64_t)row * D + 8 * (pc ^ swz_v(R)), vbuf + R0 * C::ROW_BYTES);
  }
}

template <int D>
__device__ void prefill_tile(const AttnParams& p, int item, char* lds) {
  using C = PrefillCfg<D>;
  const int lane = threadIdx.x & 63;
  const int w = uniform_i(threadIdx.x >> 6);
  const PrefillItem it = p.pf[item];
  const ReqInfo ri = p.req[it.req];
  const int g = p.g;
  const int rows = it.nq * g;
  const int nloc = lane & 31;
  const int h2 = lane >> 5;
  const int n = 32 * w + nloc;
  const bool row_ok = n < rows;
  const int t = row_ok ? n / g : 0;
  const int h = it.hk * g + (row_ok ? n % g : 0);
  const int qpos0 = ri.kv - ri.qo + it.q0;  // absolute position of the tile's first token
  const int lim = p.causal ? qpos0 + t + 1 : ri.kv;
  const int tile_min_lim = p.causal ? qpos0 + 1 : it.kv_end;  // smallest limit of any row
  const int64_t qrow = (int64_t)(ri.qo_start + it.q0 + t) * p.H_q + h;

  u32x4 qf[C::KS];
  {
    const uint16_t* qp = (const uint16_t*)p.q + qrow * D + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 v = *(const u32x4*)(qp + 16 * ks);
      qf[ks] = row_ok ? v : u32x4{0, 0, 0, 0};
    }
  }
  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float cl = p.c_log2;

  char* kbuf[2] = {lds, lds + C::TILE_BYTES};
  char* vbuf[2] = {lds + 2 * C::TILE_BYTES, lds + 3 * C::TILE_BYTES};
  const int ntiles = (it.kv_end + 63) >> 6;
  prefill_issue<D>(p, ri, it.hk, it.kv_end, 0, w, lane, kbuf[0], vbuf[0]);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    const int kbase = kt * 64;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < ntiles)
      prefill_issue<D>(p, ri, it.hk, it.kv_end, kbase + 64, w, lane, kbuf[buf ^ 1], vbuf[buf ^ 1]);
    const char* kt_lds = kbuf[buf];
    const char* vt_lds = vbuf[buf];
    // S^T[key 32 kb + 8 jj + 4 h2 + i][query n] in s[kb][4 jj + i]
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const int R = 32 * kb + nloc;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int c = 2 * ks + h2;
        u32x4 a = *(const u32x4*)(kt_lds + R * C::ROW_BYTES + ((c ^ swz_k(R)) << 4));
        s[kb] = mfma32(a, qf[ks], s[kb]);
      }
    }
    if (kbase + 64 > tile_min_lim) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase + 32 * kb + 8 * (r >> 2) + 4 * h2 + (r & 3);
          if (key >= lim) s[kb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_x32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * cl);
    const float mc = m_use * cl;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], cl, -mc));
        psum += s[kb][r];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] = oacc[db] * alpha;
    // O^T += V^T P^T over the four 16-key k-steps
    const int G = lane >> 4;
    const int j = lane & 15;
    const int dhalf = G & 1;
    const int half = (j & 1) * 8;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        u32x4 pb = {pack_bf16(s[kb][8 * sp + 0], s[kb][8 * sp + 1]),
                    pack_bf16(s[kb][8 * sp + 2], s[kb][8 * sp + 3]),
                    pack_bf16(s[kb][8 * sp + 4], s[kb][8 * sp + 5]),
                    pack_bf16(s[kb][8 * sp + 6], s[kb][8 * sp + 7])};
        const int r1 = 32 * kb + 16 * sp + 4 * h2 + (j >> 2);
        const int r2 = r1 + 8;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int c = 4 * db + 2 * dhalf + ((j & 3) >> 1);
          u32x2 a1 = lds_read_tr16(vt_lds + r1 * C::ROW_BYTES + ((c ^ swz_v(r1)) << 4) + half);
          u32x2 a2 = lds_read_tr16(vt_lds + r2 * C::ROW_BYTES + ((c ^ swz_v(r2)) << 4) + half);
          u32x4 a = {a1[0], a1[1], a2[0], a2[1]};
          oacc[db] = mfma32(a, pb, oacc[db]);
        }
      }
  }
  const float l_tot = sum_x32(l_run);
  if (row_ok) {
    const float inv = 1.f / l_tot;
    float* op = p.out + qrow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 v = {oacc[db][4 * jj + 0], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2], oacc[db][4 * jj + 3]};
        *(f32x4*)(op + 32 * db + 8 * jj + 4 * h2) = v * inv;
      }
    if (h2 == 0 && p.lse) p.lse[qrow] = m_run * p.sm_scale + __logf(l_tot);
  }
}

// One launch for both roles: blocks [0, n_pf) are prefill tiles, the rest
// hold four decode units each (one per wavefront).
template <int D>
__global__ __launch_bounds__(kBlockThreads, 2) void attn_bf16_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char lds[PrefillCfg<D>::LDS_BYTES];
  static_assert(kWavesPerBlock * DecodeCfg<D>::WAVE_LDS <= PrefillCfg<D>::LDS_BYTES, "lds");
  const int b = blockIdx.x;
  if (b < p.n_pf) {
    prefill_tile<D>(p, b, lds);
  } else {
    const int w = uniform_i(threadIdx.x >> 6);
    const int unit = (b - p.n_pf) * kWavesPerBlock + w;
    if (unit < p.n_du) decode_unit<D>(p, unit, lds + w * DecodeCfg<D>::WAVE_LDS);
  }
}

// ------------------------------------------------------------------------
// fp32 inputs: the same work items computed with plain VALU code (one
// wavefront per query row, lanes over keys for the scores and over head_dim
// for the output).  Exact fp32 online softmax; no MFMA (fp32 is used for
// the small parity workload only).
// ------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Attention of one query row over keys [k0, k1) of request ri, KV head hk.
// Returns the normalised row in o (lane owns d = lane + 64 i) and its LSE.
template <int D>
__device__ void f32_row(const AttnParams& p, const ReqInfo& ri, int hk, const float* qv, int k0,
                        int k1, float (&o)[D / 64], float& lse) {
  constexpr int NO = D / 64;
  const int lane = threadIdx.x & 63;
  const float* pool = (const float*)p.pool;
  const int32_t* pages = p.page_indices + ri.page_start;
  float m = -INFINITY, l = 0.f;
#pragma unroll
  for (int i = 0; i < NO; ++i) o[i] = 0.f;
  for (int kb = k0; kb < k1; kb += 64) {
    const int j = kb + lane;
    float s = -INFINITY;
    if (j < k1) {
      const int64_t off = (int64_t)pages[j / p.ps] * p.page_elems + (int64_t)hk * p.ps * D +
                          (int64_t)(j % p.ps) * D;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(qv[d], pool[off + d], acc);
      s = acc * p.sm_scale;
    }
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = __expf(m - m_new);
    const float pr = (j < k1) ? __expf(s - m_new) : 0.f;
    l = l * alpha + wave_sum(pr);
#pragma unroll
    for (int i = 0; i < NO; ++i) o[i] *= alpha;
    const int cnt = min(64, k1 - kb);
    for (int jj = 0; jj < cnt; ++jj) {
      const float pj = __shfl(pr, jj);
      const int key = kb + jj;
      const int64_t off = (int64_t)pages[key / p.ps] * p.page_elems +
                          (int64_t)(p.H_kv + hk) * p.ps * D + (int64_t)(key % p.ps) * D;
#pragma unroll
      for (int i = 0; i < NO; ++i) o[i] = __builtin_fmaf(pj, pool[off + lane + 64 * i], o[i]);
    }
    m = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < NO; ++i) o[i] *= inv;
  lse = l > 0.f ? m + __logf(l) : -INFINITY;
}

template <int D>
__global__ __launch_bounds__(kBlockThreads) void attn_f32_kernel(AttnParams p) {
  constexpr int NO = D / 64;
  const int lane = threadIdx.x & 63;
  const int w = uniform_i(threadIdx.x >> 6);
  const int b = blockIdx.x;
  const float* qbase = (const float*)p.q;
  if (b < p.n_pf) {
    const PrefillItem it = p.pf[b];
    const ReqInfo ri = p.req[it.req];
    const int rows = it.nq * p.g;
    for (int n = w; n < rows; n += kWavesPerBlock) {
      const int t = n / p.g, h = it.hk * p.g + n % p.g;
      const int lim = p.causal ? ri.kv - ri.qo + it.q0 + t + 1 : ri.kv;
      const int64_t row = (int64_t)(ri.qo_start + it.q0 + t) * p.H_q + h;
      float o[NO], lse;
      f32_row<D>(p, ri, it.hk, qbase + row * D, 0, min(lim, it.kv_end), o, lse);
#pragma unroll
      for (int i = 0; i < NO; ++i) p.out[row * D + lane + 64 * i] = o[i];
      if (lane == 0 && p.lse) p.lse[row] = lse;
    }
  } else {
    const int unit = (b - p.n_pf) * kWavesPerBlock + w;
    if (unit >= p.n_du) return;
    const DecodeItem it = p.du[unit];
    const ReqInfo ri = p.req[it.req];
    const int nrows = ri.qo * p.g;
    for (int n = 0; n < nrows; ++n) {
      const int t = n / p.g, h = it.hk * p.g + n % p.g;
      const int lim = p.causal ? ri.kv - ri.qo + t + 1 : ri.kv;
      const int64_t row = (int64_t)(ri.qo_start + t) * p.H_q + h;
      float o[NO], lse;
      f32_row<D>(p, ri, it.hk, qbase + row * D, it.k0, min(lim, it.k1), o, lse);
      float* po = p.part_o + ((int64_t)it.part * kDecodeCols + n) * D;
#pragma unroll
      for (int i = 0; i < NO; ++i) po[lane + 64 * i] = o[i];
      if (lane == 0) p.part_lse[(int64_t)it.part * kDecodeCols + n] = lse;
    }
  }
}

// ------------------------------------------------------------------------
// Merge of split-KV partials: for each decode row, LSE* = max_i lse_i,
// w_i = exp(lse_i - LSE*), O = sum_i w_i o_i / sum_i w_i,
// LSE = LSE* + ln sum_i w_i; parts are visited in a fixed order.
// ------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kBlockThreads) void merge_kernel(AttnParams p) {
  const MergeGroup mg = p.mg[blockIdx.x];
  const ReqInfo ri = p.req[mg.req];
  const int nrows = ri.qo * p.g;
  constexpr int D4 = D / 4;
  for (int idx = threadIdx.x; idx < nrows * D4; idx += kBlockThreads) {
    const int n = idx / D4, d4 = idx % D4;
    const int t = n / p.g, h = mg.hk * p.g + n % p.g;
    float mx = -INFINITY;
    for (int i = 0; i < mg.nparts; ++i)
      mx = fmaxf(mx, p.part_lse[(int64_t)(mg.part0 + i) * kDecodeCols + n]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float sw = 0.f;
    for (int i = 0; i < mg.nparts; ++i) {
      const int64_t slot = (int64_t)(mg.part0 + i) * kDecodeCols + n;
      const float li = p.part_lse[slot];
      const float wi = (li == -INFINITY) ? 0.f : __expf(li - mx);
      const f32x4 oi = *(const f32x4*)(p.part_o + slot * D + 4 * d4);
      acc += oi * wi;
      sw += wi;
    }
    const int64_t row = (int64_t)(ri.qo_start + t) * p.H_q + h;
    *(f32x4*)(p.out + row * D + 4 * d4) = acc * (1.f / sw);
    if (d4 == 0 && p.lse) p.lse[row] = mx + __logf(sw);
  }
}

// ------------------------------------------------------------------------
// KV append: one block per new token row; 16-byte copies of each head's K
// and V row into (page, slot) of position kv - qo + i.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(kBlockThreads) void append_kernel(AppendParams p) {
  const int row = blockIdx.x;
  int lo = 0, hi = p.B - 1;  // last request with qo_indptr[r] <= row
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.qo_indptr[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const ReqInfo ri = p.req[lo];
  const int pos = ri.kv - ri.qo + (row - ri.qo_start);
  const int page = p.page_indices[ri.page_start + pos / p.ps];
  const int slot = pos % p.ps;
  const int64_t head_bytes = (int64_t)p.D * p.elt;
  const int cph = (int)(head_bytes / 16);
  const int64_t page_bytes = 2 * (int64_t)p.H_kv * p.ps * head_bytes;
  char* pool = (char*)p.pool + (int64_t)page * page_bytes;
  const int total = 2 * p.H_kv * cph;
  for (int c = threadIdx.x; c < total; c += kBlockThreads) {
    const int kvsel = c / (p.H_kv * cph);
    const int hh = (c / cph) % p.H_kv;
    const int cc = c % cph;
    const char* src = (const char*)(kvsel ? p.v_new : p.k_new) + ((int64_t)row * p.H_kv + hh) * head_bytes + cc * 16;
    char* dst = pool + (((int64_t)kvsel * p.H_kv + hh) * p.ps + slot) * head_bytes + cc * 16;
    *(u32x4*)dst = *(const u32x4*)src;
  }
}

// ------------------------------------------------------------------------
// Page pack / unpack: block (page i, 16 KiB slab), 16-byte copies.
// ------------------------------------------------------------------------
constexpr int kPackChunksPerThread = 4;
__global__ __launch_bounds__(kBlockThreads) void pack_kernel(PackParams p) {
  const int i = blockIdx.x;
  const int64_t page = p.page_ids[i];
  const int64_t cpp = p.page_bytes / 16;
  const char* src;
  char* dst;
  if (p.to_buffer) {
    src = (const char*)p.src + page * p.page_bytes;
    dst = (char*)p.dst + (int64_t)i * p.page_bytes;
  } else {
    src = (const char*)p.src + (int64_t)i * p.page_bytes;
    dst = (char*)p.dst + page * p.page_bytes;
  }
  const int64_t c0 = (int64_t)blockIdx.y * kBlockThreads * kPackChunksPerThread + threadIdx.x;
  u32x4 v[kPackChunksPerThread];
#pragma unroll
  for (int k = 0; k < kPackChunksPerThread; ++k) {
    const int64_t c = c0 + k * kBlockThreads;
    if (c < cpp) v[k] = *(const u32x4*)(src + c * 16);
  }
#pragma unroll
  for (int k = 0; k < kPackChunksPerThread; ++k) {
    const int64_t c = c0 + k * kBlockThreads;
    if (c < cpp) *(u32x4*)(dst + c * 16) = v[k];
  }
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int dtype, hipStream_t s) {
  const int blocks = p.n_pf + (p.n_du + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  if (dtype == 1) {
    if (p.D == 128)
      hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(blocks), dim3(kBlockThreads), 0, s, p);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(blocks), dim3(kBlockThreads), 0, s, p);
  } else {
    if (p.D == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(blocks), dim3(kBlockThreads), 0, s, p);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(blocks), dim3(kBlockThreads), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const AttnParams& p, hipStream_t s) {
  if (p.n_mg == 0) return hipSuccess;
  if (p.D == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(p.n_mg), dim3(kBlockThreads), 0, s, p);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3(p.n_mg), dim3(kBlockThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  if (p.total_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(p.total_rows), dim3(kBlockThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_pack(const PackParams& p, hipStream_t s) {
  if (p.n == 0) return hipSuccess;
  const int64_t cpp = p.page_bytes / 16;
  const int64_t per_block = (int64_t)kBlockThreads * kPackChunksPerThread;
  const unsigned ny = (unsigned)((cpp + per_block - 1) / per_block);
  hipLaunchKernelGGL(pack_kernel, dim3(p.n, ny), dim3(kBlockThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace pdk
