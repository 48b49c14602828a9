// HIP attention kernels for gfx950 (MI355X, CDNA4): ragged paged attention
// (causal prefill tiles on bf16 MFMA and split-KV decode units in one
// launch), the fp32 variant, and the merge of split-KV partial results.
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

#include "device_common.hpp"
#include "pd_internal.hpp"

namespace pdk {
namespace {

// Byte offset of (page, kv half, head) in the pool.
__device__ __forceinline__ int64_t page_head_off(const AttnParams& p, int page, int half, int hk) {
  return ((int64_t)page * p.page_elems + (int64_t)(half * p.H_kv + hk) * p.ps * p.D) * 2;
}

// ------------------------------------------------------------------------
// Decode role: a wavefront runs a queue of DecodeItems (units) one after the
// other.  A unit is up to 16 NCG query rows of one (request, KV head) over a
// key range [k0, k1), 32 keys per step:
//   S^T[key][col] = K Q^T on v_mfma_f32_16x16x32_bf16 (K from HBM straight
//   into the A operand; Q^T of each 16-row column group held in registers as
//   the B operand, loaded once per unit);
//   online softmax per column across the four 16-lane groups;
//   O^T[d][col] += V^T P^T on the same MFMA, V staged through a per-wave LDS
//   double buffer by direct global->LDS loads and read back transposed (one
//   read serves every column group); P^T comes from the S accumulators
//   without any lane exchange (key order inside the 32-key step is permuted
//   identically in both operands).
// Every step issues the next step's loads before it computes.  The issue is
// unconditional: the last step of a unit issues its own loads again (in
// bounds, never used), so every path through the step loop has the same
// loads in flight and the compiler's own waits never drain the prefetch.
// ------------------------------------------------------------------------
template <int D>
struct DecodeCfg {
  static constexpr int KS = D / 32;               // 32-wide k-steps of S
  static constexpr int DB = D / 16;               // 16-row d-blocks of O^T
  static constexpr int RPB = Lds<D>::RPB;
  static constexpr int VLOADS = 32 / RPB;         // V loads per 32-key step
  static constexpr int STAGE_BYTES = Lds<D>::bytes(32);
  static constexpr int WAVE_LDS = 2 * STAGE_BYTES;
};

// Page ids of the two 16-key groups of the 32-key step at key b (clamped to
// the request's last key, so a step past the end reads the last page).
__device__ __forceinline__ int2 decode_pages(const AttnParams& p, const ReqInfo& ri, int b) {
  const int32_t* pages = p.page_indices + ri.page_start;
  const int kvm1 = ri.kv - 1;
  return make_int2(ldc(pages + (min(b, kvm1) >> p.ps_shift)), ldc(pages + (min(b + 16, kvm1) >> p.ps_shift)));
}

// Loads of one 32-key step at key b, all from inline asm, so that the step
// loop alone decides how long to wait for them.  Keys >= kv (only in the
// request's last step) are read from row kv - 1 instead (finite data, masked
// later), so tail slots are never read.
// K fragments of the 16-key half sb into `kf` (KS loads); `page` holds key
// b + 16 sb.
template <int D>
__device__ __forceinline__ void decode_issue_k(const AttnParams& p, const ReqInfo& ri, int hk, int b, int page,
                                               int sb, int lane, u32x4 (&kf)[D / 32]) {
  using C = DecodeCfg<D>;
  const int n = lane & 15, q = lane >> 4;
  const char* kb = (const char*)p.pool + page_head_off(p, page, 0, hk);
  const int krow = min(b + 16 * sb + n, ri.kv - 1) & (p.ps - 1);
  load_frags64<C::KS>(kb + krow * 2 * D + 16 * q, kf);
}
// V rows of the 16-key half sb (keys b + 16 sb ...) into its part of the LDS
// stage (VLOADS / 2 loads); `page` holds key b + 16 sb.
template <int D>
__device__ __forceinline__ void decode_issue_v(const AttnParams& p, const ReqInfo& ri, int hk, int b, int page,
                                               int sb, int lane, LDS_AS char* stage) {
  using C = DecodeCfg<D>;
  const char* vb = (const char*)p.pool + page_head_off(p, page, 1, hk);
  const int kvm1 = ri.kv - 1;
  const int r = Lds<D>::dma_row(lane), c = Lds<D>::dma_chunk(lane);
#pragma unroll
  for (int i = 0; i < C::VLOADS / 2; ++i) {
    const int vrow = min(b + 16 * sb + i * C::RPB + r, kvm1) & (p.ps - 1);
    load_lds16_nt(vb + vrow * 2 * D + 16 * c, stage + (sb * (C::VLOADS / 2) + i) * Lds<D>::BLOCK);
  }
}
// K and V of both halves, half by half: 2 KS + VLOADS loads.
template <int D>
__device__ __forceinline__ void decode_issue(const AttnParams& p, const ReqInfo& ri, int hk, int b, int2 pg,
                                             int lane, u32x4 (&kf)[2][D / 32], LDS_AS char* stage) {
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    decode_issue_k<D>(p, ri, hk, b, sb ? pg.y : pg.x, sb, lane, kf[sb]);
    decode_issue_v<D>(p, ri, hk, b, sb ? pg.y : pg.x, sb, lane, stage);
  }
}

// Per-lane state of a unit: for column group j, this lane's column (lane &
// 15) is query row c0 + 16 j + (lane & 15) of the row group.
template <int NCG>
struct DecodeLanes {
  int q;          // 16-lane group
  int v_off;      // lane part of the transposed V read address
  int lim[NCG];   // keys < lim are visible to the lane's column
  int mask_from;  // smallest lim of any column of the unit (uniform)
};

template <int D, int NCG>
struct DecodeAcc {
  f32x4 o[NCG][D / 16];
  f32x4 l[NCG];    // column sums of the bf16 P (all four entries equal)
  float m[NCG];    // reference maximum of each column
};

// S, softmax and PV of the 32-key step at key b (K in kc, V in LDS stage st).
// `before_v` runs after the softmax, before the first read of the V stage.
template <int D, int NCG, class BeforeV>
__device__ __forceinline__ void decode_compute(const AttnParams& p, int b, const DecodeLanes<NCG>& ln,
                                               const u32x4 (&qf)[NCG][D / 32], const u32x4 (&kc)[2][D / 32],
                                               const LDS_AS char* st, DecodeAcc<D, NCG>& a, BeforeV&& before_v) {
  using C = DecodeCfg<D>;
  const float cl = p.c_log2;
  // S^T for keys b + 16 sb + 4 q + i, column lane & 15 of group j
  f32x4 s[NCG][2];
#pragma unroll
  for (int j = 0; j < NCG; ++j)
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[j][sb] = mfma16(kc[sb][0], qf[j][0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int ks = 1; ks < C::KS; ++ks) s[j][sb] = mfma16(kc[sb][ks], qf[j][ks], s[j][sb]);
    }
  if (b + 32 > ln.mask_from) {
#pragma unroll
    for (int j = 0; j < NCG; ++j)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (b + 16 * sb + 4 * ln.q + i >= ln.lim[j]) s[j][sb][i] = -INFINITY;
  }
  u32x4 pb[NCG];
#pragma unroll
  for (int j = 0; j < NCG; ++j) {
    uint32_t pk[4];
    {
      const float mc = a.m[j] * cl;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          pk[2 * sb + i] = pack_bf16(fast_exp2(__builtin_fmaf(s[j][sb][2 * i], cl, -mc)),
                                     fast_exp2(__builtin_fmaf(s[j][sb][2 * i + 1], cl, -mc)));
    }
    if (wave_any(p_out_of_range(pk))) {
      float mx = fmaxf(fmaxf(fmaxf(s[j][0][0], s[j][0][1]), fmaxf(s[j][0][2], s[j][0][3])),
                       fmaxf(fmaxf(s[j][1][0], s[j][1][1]), fmaxf(s[j][1][2], s[j][1][3])));
      mx = max_x16(mx);
      mx = max_x32(mx);
      const float m_new = fmaxf(a.m[j], mx);
      if (m_new != -INFINITY) {  // a column with no visible key yet keeps m = -inf
        const float alpha = fast_exp2((a.m[j] - m_new) * cl);  // m = -inf -> 0
        a.l[j] = a.l[j] * alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) a.o[j][db] = a.o[j][db] * alpha;
        a.m[j] = m_new;
      }
      const float mc = (a.m[j] == -INFINITY) ? 0.f : a.m[j] * cl;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          pk[2 * sb + i] = pack_bf16(fast_exp2(__builtin_fmaf(s[j][sb][2 * i], cl, -mc)),
                                     fast_exp2(__builtin_fmaf(s[j][sb][2 * i + 1], cl, -mc)));
    }
    pb[j] = u32x4{pk[0], pk[1], pk[2], pk[3]};
    a.l[j] = mfma16(u32x4{kBf16OnesPair, kBf16OnesPair, kBf16OnesPair, kBf16OnesPair}, pb[j], a.l[j]);
  }
  before_v();
  // V^T[d = 16 db + (lane & 15)][keys 4q + e, 16 + 4q + e]
  const LDS_AS char* vp = st + ln.v_off;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    const u32x2 a1 = lds_read_tr16(vp + Lds<D>::chunk_step(db));
    const u32x2 a2 = lds_read_tr16(vp + Lds<D>::chunk_step(db) + (16 / C::RPB) * Lds<D>::BLOCK);
    const u32x4 va = {a1[0], a1[1], a2[0], a2[1]};
#pragma unroll
    for (int j = 0; j < NCG; ++j) a.o[j][db] = mfma16(va, pb[j], a.o[j][db]);
  }
}

// One step of a unit at key b: issue the loads of the next step (this step's
// again when it is the unit's last: b + 32 >= k1) into kn / sn, wait for this
// step's, compute it.  Returns false after the unit's last step, with every
// load landed.
template <int D, int NCG>
__device__ __forceinline__ bool decode_step(const AttnParams& p, const ReqInfo& ri, int hk, int k1, int& b,
                                            int2& pg, int2& pg_next, int lane, const DecodeLanes<NCG>& ln,
                                            u32x4 (&qf)[NCG][D / 32], u32x4 (&kc)[2][D / 32],
                                            u32x4 (&kn)[2][D / 32], const LDS_AS char* st, LDS_AS char* sn,
                                            DecodeAcc<D, NCG>& a) {
  using C = DecodeCfg<D>;
  const int nb = b + 32;
  const bool more = nb < k1;
  decode_issue<D>(p, ri, hk, more ? nb : b, more ? pg_next : pg, lane, kn, sn);
  // this step's K and V (and the unit's Q, loaded before its first step)
  // have landed; the next step's loads stay in flight through the compute
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * C::KS + C::VLOADS) : "memory");
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) pin_regs(kc[sb]);
#pragma unroll
  for (int j = 0; j < NCG; ++j) pin_regs(qf[j]);
  const int2 pg_after = decode_pages(p, ri, nb + 32);  // scalar loads, used next step
  decode_compute<D, NCG>(p, b, ln, qf, kc, st, a, [] {});
  if (!more) {
    // the repeated loads have landed; kn stays live up to here, so that the
    // compiler places nothing else in its registers while they are in flight
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) pin_regs(kn[sb]);
    return false;
  }
  b = nb;
  pg = pg_next;
  pg_next = pg_after;
  return true;
}

// Start of a unit: Q^T fragments (inline-asm loads, covered by the first
// step's wait), the lanes' key limits, zero accumulators.  A column past the
// group's last row reads row 0's query: it computes a finite copy of that
// row, and its results are never stored.
template <int D, int NCG>
__device__ __forceinline__ void decode_unit_begin(const AttnParams& p, const DecodeItem& it, const ReqInfo& ri,
                                                  int lane, DecodeLanes<NCG>& ln, u32x4 (&qf)[NCG][D / 32],
                                                  DecodeAcc<D, NCG>& a) {
  using C = DecodeCfg<D>;
  const int n = lane & 15, q = lane >> 4;
  const int g = p.g;
  const int rows = ri.qo * g;
#pragma unroll
  for (int j = 0; j < NCG; ++j) {
    const int row = it.c0 + 16 * j + n;
    const bool ok = row < rows;
    const int t = ok ? row / g : 0;
    const int h = it.hk * g + (ok ? row % g : 0);
    ln.lim[j] = min(it.k1, p.causal ? ri.kv - ri.qo + t + 1 : ri.kv);
    const uint16_t* qp = (const uint16_t*)p.q + ((int64_t)(ri.qo_start + t) * p.H_q + h) * D + 8 * q;
    load_frags64<C::KS>(qp, qf[j]);
  }
  ln.mask_from = min(it.k1, p.causal ? ri.kv - ri.qo + it.c0 / g + 1 : ri.kv);
#pragma unroll
  for (int j = 0; j < NCG; ++j) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) a.o[j][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    a.l[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    a.m[j] = -INFINITY;
  }
}

// End of a unit: row c0 + 16 j + n to partial row part + 16 j + n.
template <int D, int NCG>
__device__ __forceinline__ void decode_unit_store(const AttnParams& p, const DecodeItem& it, int rows, int lane,
                                                  const DecodeAcc<D, NCG>& a) {
  using C = DecodeCfg<D>;
  const int n = lane & 15, q = lane >> 4;
#pragma unroll
  for (int j = 0; j < NCG; ++j) {
    if (it.c0 + 16 * j + n < rows) {
      const float l_tot = a.l[j][0];
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const int64_t pr = (int64_t)it.part + 16 * j + n;
      float* po = p.part_o + pr * D + 4 * q;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) *(f32x4*)(po + 16 * db) = a.o[j][db] * inv;
      if (q == 0) p.part_lse[pr] = l_tot > 0.f ? a.m[j] * p.sm_scale + __logf(l_tot) : -INFINITY;
    }
  }
}

template <int NCG>
__device__ __forceinline__ void decode_lanes_init(DecodeLanes<NCG>& ln, int lane, int v_off) {
  ln.q = lane >> 4;
  ln.v_off = v_off;
}

// A wavefront's queue: units [u0, u1), each written to its partial rows.
template <int D, int NCG>
__device__ void decode_queue(const AttnParams& p, int u0, int u1, LDS_AS char* lds) {
  using C = DecodeCfg<D>;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, q = lane >> 4;
  DecodeLanes<NCG> ln;
  decode_lanes_init(ln, lane, Lds<D>::off(4 * q + (n >> 2), (n & 3) >> 1) + 8 * (n & 1));
  u32x4 kf0[2][C::KS], kf1[2][C::KS];
  LDS_AS char* st0 = lds;
  LDS_AS char* st1 = lds + C::STAGE_BYTES;
  for (int u = u0; u < u1; ++u) {
    const DecodeUnit du = ldc(p.du + u);
    const DecodeItem& it = du.it;
    const ReqInfo& ri = du.ri;
    u32x4 qf[NCG][C::KS];
    DecodeAcc<D, NCG> a;
    decode_unit_begin<D, NCG>(p, it, ri, lane, ln, qf, a);
    int b = it.k0;
    int2 pg = decode_pages(p, ri, b);
    int2 pg_next = decode_pages(p, ri, b + 32);
    decode_issue<D>(p, ri, it.hk, b, pg, lane, kf0, st0);
    for (;;) {
      if (!decode_step<D, NCG>(p, ri, it.hk, it.k1, b, pg, pg_next, lane, ln, qf, kf0, kf1, st0, st1, a)) break;
      if (!decode_step<D, NCG>(p, ri, it.hk, it.k1, b, pg, pg_next, lane, ln, qf, kf1, kf0, st1, st0, a)) break;
    }
    decode_unit_store<D, NCG>(p, it, ri.qo * p.g, lane, a);
  }
}

// ------------------------------------------------------------------------
// Two wavefronts on one 64-row group (rows 0..31 and 32..63 of a (request,
// KV head) with more than 32 query rows) read the same keys.  They share
// their LDS as four V stages: each loads one 16-key half of every step's V
// rows, three steps ahead, and reads both halves; K goes to each one's
// registers one step ahead, as in the single-wavefront queue.  The pair runs
// the same units in the same order, so its steps are numbered alike (T,
// counted over the whole queue; step T uses stage T & 3).  Two counters per
// wavefront in LDS carry the handshake:
//   landed = T + 1 once its half of step T's V is in the stage (written
//            after the wait that covers those loads);
//   read   = T + 1 once its reads of stage T & 3 are issued (LDS executes a
//            wavefront's operations in order, so a later write to the stage
//            cannot overtake them).
// Before reading step T's V a wavefront waits for the partner's landed >=
// T + 1; before loading into stage (T + 3) & 3 (last read at step T - 1) it
// waits for the partner's read >= T.  Each wait only needs an event that the
// partner reaches without waiting for a later event of this wavefront, so
// the pair cannot deadlock; the waits are bounded all the same.
// ------------------------------------------------------------------------
constexpr int kPairSpinLimit = 1 << 16;  // s_sleep 1 rounds (~64 clocks each, ~4 ms in all) before a wait gives up

__device__ __forceinline__ void pair_wait(const volatile LDS_AS int32_t* f, int target) {
  for (int i = 0; i < kPairSpinLimit; ++i) {
    if (__builtin_amdgcn_readfirstlane(*f) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");  // nothing of the stage is read before the counter
}
__device__ __forceinline__ void pair_signal(volatile LDS_AS int32_t* f, int value) {
  asm volatile("" ::: "memory");  // after the stage reads / the covering wait
  *f = value;
}

// Page id of key b (clamped to the request's last key).
__device__ __forceinline__ int decode_page(const AttnParams& p, const ReqInfo& ri, int b) {
  return ldc(p.page_indices + ri.page_start + (min(b, ri.kv - 1) >> p.ps_shift));
}

struct PairState {
  volatile LDS_AS int32_t* mine;    // [0] landed, [1] read
  const volatile LDS_AS int32_t* theirs;
  LDS_AS char* stages;              // four stages of STAGE_BYTES
  int h;                            // the 16-key half this wavefront loads (= its row half)
  int T;                            // steps of the queue so far
};

// One step T at key b of a paired unit: issue K of the next step and this
// wavefront's V half of step T + 3 (the unit's last step again past its
// end), wait for this step's K and V half, compute.
template <int D>
__device__ __forceinline__ bool decode_step_pair(const AttnParams& p, const ReqInfo& ri, int hk, int k1, int blast,
                                                 int& b, int2& pg, int2& pg_next, int& vpg, int& vpg_next,
                                                 int lane, const DecodeLanes<2>& ln, u32x4 (&qf)[2][D / 32],
                                                 u32x4 (&kc)[2][D / 32], u32x4 (&kn)[2][D / 32], PairState& ps,
                                                 DecodeAcc<D, 2>& a) {
  using C = DecodeCfg<D>;
  const int nb = b + 32;
  const bool more = nb < k1;
  const int T = ps.T;
  {
    const int kb = more ? nb : b;
    const int2 kp = more ? pg_next : pg;
    decode_issue_k<D>(p, ri, hk, kb, kp.x, 0, lane, kn[0]);
    decode_issue_k<D>(p, ri, hk, kb, kp.y, 1, lane, kn[1]);
  }
  pair_wait(ps.theirs + 1, T);  // the partner has read stage (T + 3) & 3 at its step T - 1
  decode_issue_v<D>(p, ri, hk, min(b + 96, blast), vpg, ps.h, lane, ps.stages + ((T + 3) & 3) * C::STAGE_BYTES);
  // loads issued after this step's K: V half of T + 2, K of T + 1, V half of
  // T + 3 (2 KS + VLOADS); this step's V half is older still
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * C::KS + C::VLOADS) : "memory");
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) pin_regs(kc[sb]);
#pragma unroll
  for (int j = 0; j < 2; ++j) pin_regs(qf[j]);
  pair_signal(ps.mine, T + 1);
  const int2 pg_after = decode_pages(p, ri, nb + 32);             // K pages of the step after next
  // V page of step T + 5 (issued two steps from now, at step T + 2)
  const int vpg_after = decode_page(p, ri, min(b + 160, blast) + 16 * ps.h);
  decode_compute<D, 2>(p, b, ln, qf, kc, ps.stages + (T & 3) * C::STAGE_BYTES, a,
                       [&] { pair_wait(ps.theirs, T + 1); });
  pair_signal(ps.mine + 1, T + 1);
  ps.T = T + 1;
  if (!more) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) pin_regs(kn[sb]);
    return false;
  }
  b = nb;
  pg = pg_next;
  pg_next = pg_after;
  vpg = vpg_next;
  vpg_next = vpg_after;
  return true;
}

template <int D>
__device__ void decode_queue_pair(const AttnParams& p, int u0, int u1, PairState ps) {
  using C = DecodeCfg<D>;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, q = lane >> 4;
  DecodeLanes<2> ln;
  decode_lanes_init(ln, lane, Lds<D>::off(4 * q + (n >> 2), (n & 3) >> 1) + 8 * (n & 1));
  u32x4 kf0[2][C::KS], kf1[2][C::KS];
  for (int u = u0; u < u1; ++u) {
    const DecodeUnit du = ldc(p.du + u);
    const DecodeItem& it = du.it;
    const ReqInfo& ri = du.ri;
    u32x4 qf[2][C::KS];
    DecodeAcc<D, 2> a;
    decode_unit_begin<D, 2>(p, it, ri, lane, ln, qf, a);
    int b = it.k0;
    const int blast = it.k0 + ((it.k1 - it.k0 - 1) & ~31);  // key of the unit's last step
    int2 pg = decode_pages(p, ri, b);
    decode_issue_k<D>(p, ri, it.hk, b, pg.x, 0, lane, kf0[0]);
    decode_issue_k<D>(p, ri, it.hk, b, pg.y, 1, lane, kf0[1]);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int vb = min(b + 32 * k, blast);
      pair_wait(ps.theirs + 1, ps.T + k - 3);
      decode_issue_v<D>(p, ri, it.hk, vb, decode_page(p, ri, vb + 16 * ps.h), ps.h, lane,
                        ps.stages + ((ps.T + k) & 3) * C::STAGE_BYTES);
    }
    int2 pg_next = decode_pages(p, ri, b + 32);
    int vpg = decode_page(p, ri, min(b + 96, blast) + 16 * ps.h);
    int vpg_next = decode_page(p, ri, min(b + 128, blast) + 16 * ps.h);
    for (;;) {
      if (!decode_step_pair<D>(p, ri, it.hk, it.k1, blast, b, pg, pg_next, vpg, vpg_next, lane, ln, qf, kf0, kf1,
                               ps, a))
        break;
      if (!decode_step_pair<D>(p, ri, it.hk, it.k1, blast, b, pg, pg_next, vpg, vpg_next, lane, ln, qf, kf1, kf0,
                               ps, a))
        break;
    }
    decode_unit_store<D, 2>(p, it, ri.qo * p.g, lane, a);
  }
}

// ------------------------------------------------------------------------
// Prefill role: one 512-thread block computes one PrefillItem (<= 256 query
// rows: tokens x the g heads of one KV head) over 64-key tiles.
//   Wave w owns query rows 32 w .. 32 w + 31 (the N index of both products).
//   S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16; Q^T stays in
//   registers; K and V tiles are staged in LDS by direct global->LDS loads
//   (four buffers of each, each wave loading one 8-row group), read back 16
//   bytes per lane (K) and transposed (V); P^T is the S accumulator re-packed
//   to bf16 in place, and the row sums of the rounded P are v_dot2 sums.
//   Eight wavefronts share every K/V tile.  The loop is software-pipelined:
//   S of tile t + 1 runs on the MFMA pipe while the VALU computes the
//   softmax of tile t, then PV of tile t; the workgroup meets at a barrier
//   once per pair of tiles, so the two wavefronts of a SIMD need not run the
//   same phase at the same time.  Tiles that cross the causal diagonal (or
//   the end of the cache) run a masked copy.
// ------------------------------------------------------------------------
// W wavefronts per block: 8 (256-row tiles, four K and V buffers, one block
// per CU) or 4 (128-row tiles, two buffers, two blocks per CU; see
// prefill_tile4).
template <int D, int W = kAttnWaves>
struct PrefillCfg {
  static constexpr int KS = D / 16;     // 16-wide k-steps of S
  static constexpr int DB = D / 32;     // 32-row d-blocks of O^T
  static constexpr int RPB = Lds<D>::RPB;
  static constexpr int ROWS_PER_WAVE = 64 / W;        // K/V rows each wave loads per tile
  static constexpr int LOADS = ROWS_PER_WAVE / RPB;   // 1 KiB loads per wave per matrix per tile
  static constexpr int NBUF = W == 8 ? 4 : 2;         // K and V tile buffers
  static constexpr int TILE_BYTES = Lds<D>::bytes(64);
  static constexpr int LDS_BYTES = 2 * NBUF * TILE_BYTES;
  static_assert(LOADS >= 1 && (W == 8 || W == 4), "prefill block shape");
};

// Page id of wave w's row group of the tile at kbase (clamped to the tile's
// last key).
template <int D, int W = kAttnWaves>
__device__ __forceinline__ int prefill_page(const AttnParams& p, const ReqInfo& ri, int kv_end, int kbase,
                                            int w) {
  constexpr int RW = PrefillCfg<D, W>::ROWS_PER_WAVE;
  return ldc(p.page_indices + ri.page_start + (min(kbase + RW * w, kv_end - 1) >> p.ps_shift));
}

// Loads of one matrix (K or V: `half`) of the 64-key tile at kbase (wave w:
// its 8-row group, inside one page since pages hold >= 16 aligned rows).
// `full`: every row < kv_end; otherwise rows past kv_end - 1 are read from
// row kv_end - 1 (finite, masked later).
template <int D, int W = kAttnWaves>
__device__ __forceinline__ void prefill_issue(const AttnParams& p, int hk, int half, int kv_end, int kbase,
                                              int w, int page, int lane, bool full, LDS_AS char* dst) {
  using C = PrefillCfg<D, W>;
  const char* pool = (const char*)p.pool;
  const int psm = p.ps - 1;
  const int r = Lds<D>::dma_row(lane), c = Lds<D>::dma_chunk(lane);
  const int j0 = kbase + C::ROWS_PER_WAVE * w;
  LDS_AS char* d = dst + (C::ROWS_PER_WAVE / C::RPB) * w * Lds<D>::BLOCK;
  const char* base = pool + page_head_off(p, page, half, hk);
  if (full) {
    const char* b = base + (j0 & psm) * 2 * D + r * 2 * D + 16 * c;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) load_lds16(b + i * C::RPB * 2 * D, d + i * Lds<D>::BLOCK);
  } else {
    const int last = kv_end - 1;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int row = min(j0 + i * C::RPB + r, last) & psm;
      load_lds16(base + row * 2 * D + 16 * c, d + i * Lds<D>::BLOCK);
    }
  }
}
template <int D>
__device__ __forceinline__ void prefill_issue_k(const AttnParams& p, int hk, int kv_end, int kbase, int w,
                                                int page, int lane, bool full, LDS_AS char* dst) {
  prefill_issue<D>(p, hk, 0, kv_end, kbase, w, page, lane, full, dst);
}
template <int D>
__device__ __forceinline__ void prefill_issue_v(const AttnParams& p, int hk, int kv_end, int kbase, int w,
                                                int page, int lane, bool full, LDS_AS char* dst) {
  prefill_issue<D>(p, hk, 1, kv_end, kbase, w, page, lane, full, dst);
}

struct PrefillLanes {
  int h2;     // lane >> 5: which 4-key half of each 8-key group this lane holds
  int k_off;  // lane part of the K read address
  int v_off;  // lane part of the transposed V read address
};

// S^T = K Q^T for one 64-key tile in LDS: S^T[key 32 kb + 8 jj + 4 h2 + i]
// [query] lands in s[kb][4 jj + i].  The two accumulator chains are
// interleaved and K is read one k-step ahead.
template <int D>
__device__ __forceinline__ void prefill_scores(const LDS_AS char* kt, PrefillLanes ln,
                                               const u32x4 (&qf)[D / 16], f32x16 (&s)[2]) {
  using C = PrefillCfg<D>;
  constexpr int RPB = C::RPB;
  const LDS_AS char* kp = kt + ln.k_off;
  constexpr int KB1 = (32 / RPB) * Lds<D>::BLOCK;
  u32x4 a0 = lds_read16(kp), a1 = lds_read16(kp + KB1);
  u32x4 n0 = lds_read16(kp + Lds<D>::chunk_step(1)), n1 = lds_read16(kp + KB1 + Lds<D>::chunk_step(1));
  s[0] = mfma32(a0, qf[0], f32x16{});
  s[1] = mfma32(a1, qf[0], f32x16{});
#pragma unroll
  for (int ks = 1; ks < C::KS; ++ks) {
    a0 = n0;
    a1 = n1;
    if (ks + 1 < C::KS) {
      n0 = lds_read16(kp + Lds<D>::chunk_step(ks + 1));
      n1 = lds_read16(kp + KB1 + Lds<D>::chunk_step(ks + 1));
    }
    s[0] = mfma32(a0, qf[ks], s[0]);
    s[1] = mfma32(a1, qf[ks], s[1]);
  }
}

// Speculative softmax of one tile's scores (see kMaxTileSum above): returns
// P in bf16 pairs, in the key order of the PV operand (pk[kb][4 sp + i]).
// P = exp2(s c - mc) of one tile's scores, packed to bf16 in the key order of
// the PV operand (pk[kb][4 sp + i]); returns this lane's sum of the rounded
// P (v_dot2 against bf16 ones, two chains).
template <int D>
__device__ __forceinline__ float prefill_exp(const f32x16 (&s)[2], float cl, float mc, uint32_t (&pk)[2][8]) {
  float t[2] = {0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pk[kb][i] = pack_bf16(fast_exp2(__builtin_fmaf(s[kb][2 * i], cl, -mc)),
                            fast_exp2(__builtin_fmaf(s[kb][2 * i + 1], cl, -mc)));
      t[kb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[kb][i]),
                                              __builtin_bit_cast(bf16x2, kBf16OnesPair), t[kb], false);
    }
  return t[0] + t[1];
}

// FIRST: the wavefront's first key tile (tile 0; m_ref = -inf, O and the
// sums still zero).  The speculative pass would find every weight infinite
// and be redone, so the row maximum is taken at once: the same values as the
// general path's rescale branch (alpha = 0 there), one pass of exponentials.
// Every row sees key 0, so the maximum is finite.
template <int D, bool MASK, bool FIRST = false>
__device__ __forceinline__ void prefill_softmax(const AttnParams& p, f32x16 (&s)[2], int kbase, int lim,
                                                PrefillLanes ln, float& m_ref, float& lsum,
                                                f32x16 (&oacc)[D / 32], uint32_t (&pk)[2][8]) {
  using C = PrefillCfg<D>;
  const float cl = p.c_log2;
  if (MASK) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kbase + 32 * kb + 8 * (r >> 2) + 4 * ln.h2 + (r & 3) >= lim) s[kb][r] = -INFINITY;
  }
  if constexpr (FIRST) {
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    m_ref = max_x32(mx);
    lsum = prefill_exp<D>(s, cl, m_ref * cl, pk);
    return;
  }
  float ts = prefill_exp<D>(s, cl, m_ref * cl, pk);
  // Some P of the tile reached 2^64, or is inf / NaN (the first tile, with
  // m_ref = -inf): this lane's sum of them shows it.
  if (wave_any(!(ts < 0x1p64f))) {
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = max_x32(mx);
    const float m_new = fmaxf(m_ref, mx);
    const float alpha = fast_exp2((m_ref - m_new) * cl);  // m_ref = -inf -> 0
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] = oacc[db] * alpha;
    m_ref = m_new;
    ts = prefill_exp<D>(s, cl, m_ref * cl, pk);
  }
  lsum += ts;
}

// O^T += V^T P^T over the four 16-key k-steps of one tile.
template <int D>
__device__ __forceinline__ void prefill_pv(const LDS_AS char* vt, PrefillLanes ln, const uint32_t (&pk)[2][8],
                                           f32x16 (&oacc)[D / 32]) {
  using C = PrefillCfg<D>;
  constexpr int RPB = C::RPB;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      const u32x4 pb = {pk[kb][4 * sp + 0], pk[kb][4 * sp + 1], pk[kb][4 * sp + 2], pk[kb][4 * sp + 3]};
      const LDS_AS char* vp = vt + ln.v_off + ((32 * kb + 16 * sp) / RPB) * Lds<D>::BLOCK;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const u32x2 a1 = lds_read_tr16(vp + Lds<D>::chunk_step(2 * db));
        const u32x2 a2 = lds_read_tr16(vp + Lds<D>::chunk_step(2 * db) + (8 / RPB) * Lds<D>::BLOCK);
        const u32x4 a = {a1[0], a1[1], a2[0], a2[1]};
        oacc[db] = mfma32(a, pb, oacc[db]);
      }
    }
}

struct PrefillLoop {
  int ntiles, nfull;
  int pg[3];  // page ids of tiles t + 2, t + 3, t + 4 for the loads issued at the next even t
};

// One pipelined iteration t over the 64-key tile t (K and V tiles live in
// buffer t % 4).  The workgroup synchronises once per pair of tiles: at even
// t every wave waits for its loads of the pair issued at t - 2 (K(t+1),
// K(t+2), V(t), V(t+1): all it has in flight), the barrier publishes them,
// and the wave issues its part of K(t+3), K(t+4), V(t+2), V(t+3) into the
// buffers of tiles t - 1 and t, which every wave finished reading before
// that barrier.  Between barriers the two wavefronts that share a SIMD can
// drift apart by up to a tile, so one's softmax overlaps the other's
// matrix products.  Then S(t+1) on the MFMA pipe, the softmax of S(t) on the
// VALU, and PV(t).
template <int D, bool MASK, bool NEXT>
__device__ __forceinline__ void prefill_iter(const AttnParams& p, const ReqInfo& ri, const PrefillItem& it,
                                             int t, int w, int lane, int wnt, int lim, PrefillLanes ln,
                                             const u32x4 (&qf)[D / 16], LDS_AS char* kbuf, LDS_AS char* vbuf,
                                             PrefillLoop& L, f32x16 (&s_cur)[2], f32x16 (&s_next)[2],
                                             float& m_ref, float& lsum, f32x16 (&oacc)[D / 32]) {
  using C = PrefillCfg<D>;
  static_assert(C::NBUF == 4, "two tiles per barrier with one pair in flight");
  const int nt = L.ntiles;
  if ((t & 1) == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 2 < nt)
      prefill_issue_v<D>(p, it.hk, it.kv_end, (t + 2) * 64, w, L.pg[0], lane, t + 2 < L.nfull,
                         vbuf + ((t + 2) & 3) * C::TILE_BYTES);
    if (t + 3 < nt) {
      prefill_issue_k<D>(p, it.hk, it.kv_end, (t + 3) * 64, w, L.pg[1], lane, t + 3 < L.nfull,
                         kbuf + ((t + 3) & 3) * C::TILE_BYTES);
      prefill_issue_v<D>(p, it.hk, it.kv_end, (t + 3) * 64, w, L.pg[1], lane, t + 3 < L.nfull,
                         vbuf + ((t + 3) & 3) * C::TILE_BYTES);
    }
    if (t + 4 < nt)
      prefill_issue_k<D>(p, it.hk, it.kv_end, (t + 4) * 64, w, L.pg[2], lane, t + 4 < L.nfull,
                         kbuf + (t & 3) * C::TILE_BYTES);
  } else {
    // page ids for the loads of the next even iteration t + 1 (scalar loads)
#pragma unroll
    for (int j = 0; j < 3; ++j) L.pg[j] = prefill_page<D>(p, ri, it.kv_end, (t + 3 + j) * 64, w);
  }
  if (t < wnt) {  // the wave's rows see a key of tile t
    // S(t + 1) even when the wave will skip tile t + 1: one straight block
    // lets the compiler interleave these products with the softmax of tile t
    if (NEXT) prefill_scores<D>(kbuf + ((t + 1) & 3) * C::TILE_BYTES, ln, qf, s_next);  // NEXT: t + 1 < ntiles
    uint32_t pk[2][8];
    prefill_softmax<D, MASK>(p, s_cur, t * 64, lim, ln, m_ref, lsum, oacc, pk);
    prefill_pv<D>(vbuf + (t & 3) * C::TILE_BYTES, ln, pk, oacc);
  }
}

template <int D>
__device__ void prefill_tile(const AttnParams& p, const PrefillItem& it, const ReqInfo& ri, LDS_AS char* lds) {
  using C = PrefillCfg<D>;
  constexpr int RPB = C::RPB;
  const int lane = threadIdx.x & 63;
  const int w = uniform_i(threadIdx.x >> 6);
  const int g = p.g;
  const int rows = it.nq * g;
  const int nloc = lane & 31;
  // Row block of this wave.  Under a causal mask a wave skips the key tiles
  // that lie wholly above its rows (the last ones); the two wavefronts of a
  // SIMD (w and w + 4) take complementary row blocks (rb and 7 - rb), so the
  // skipped work is spread evenly over the SIMDs of short prompts.
  static_assert(kAttnWaves == 8, "row blocks are paired per SIMD for 8 wavefronts");
  const int rb = w < 4 ? w : 11 - w;
  const int n = 32 * rb + nloc;
  const bool row_ok = n < rows;
  const int t = row_ok ? n / g : 0;
  const int h = it.hk * g + (row_ok ? n % g : 0);
  const int qpos0 = ri.kv - ri.qo + it.q0;  // absolute position of the tile's first token
  const int lim = p.causal ? qpos0 + t + 1 : ri.kv;
  const int mask_from = p.causal ? qpos0 + 1 : it.kv_end;  // smallest limit of any row
  const int64_t qrow = (int64_t)(ri.qo_start + it.q0 + t) * p.H_q + h;

  PrefillLanes ln;
  ln.h2 = lane >> 5;
  ln.k_off = Lds<D>::off(nloc, ln.h2);
  {
    const int j = lane & 15, dhalf = (lane >> 4) & 1;
    ln.v_off = Lds<D>::off(4 * ln.h2 + (j >> 2), 2 * dhalf + ((j & 3) >> 1)) + 8 * (j & 1);
  }

  u32x4 qf[C::KS];
  {
    const uint16_t* qp = (const uint16_t*)p.q + qrow * D + 8 * ln.h2;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const u32x4 v = *(const u32x4*)(qp + 16 * ks);
      qf[ks] = row_ok ? v : u32x4{0, 0, 0, 0};
    }
  }
  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
  float m_ref = -INFINITY;
  float lsum = 0.f;  // this lane's share (half of the keys) of its row's sum of the bf16 P

  LDS_AS char* kbuf = lds;
  LDS_AS char* vbuf = lds + C::NBUF * C::TILE_BYTES;
  const int ntiles = (it.kv_end + 63) >> 6;
  const int nfull = it.kv_end >> 6;                                  // tiles with every row < kv_end
  const int nplain = min(ntiles, mask_from / 64);  // tiles whose keys all lie below every row's limit
  // prologue: K(0) V(0) K(1) V(1) K(2) and the page ids of the loads issued
  // at t = 0 (tiles 2, 3, 4); S(0)
  PrefillLoop L;
  L.ntiles = ntiles;
  L.nfull = nfull;
  for (int j = 0; j < 3 && j < ntiles; ++j) {
    prefill_issue_k<D>(p, it.hk, it.kv_end, j * 64, w, prefill_page<D>(p, ri, it.kv_end, j * 64, w), lane,
                       j < nfull, kbuf + j * C::TILE_BYTES);
    if (j < 2)
      prefill_issue_v<D>(p, it.hk, it.kv_end, j * 64, w, prefill_page<D>(p, ri, it.kv_end, j * 64, w), lane,
                         j < nfull, vbuf + j * C::TILE_BYTES);
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) L.pg[j] = prefill_page<D>(p, ri, it.kv_end, (2 + j) * 64, w);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // key tiles this wave computes: up to the limit of its last row (none for
  // a wave whose rows are all padding)
  int wnt = 0;
  if (32 * rb < rows) {
    const int tmax = min(32 * rb + 31, rows - 1) / g;
    wnt = (min(it.kv_end, p.causal ? qpos0 + tmax + 1 : it.kv_end) + 63) >> 6;
  }
  const bool active = wnt > 0;
  // Scores alternate between two register sets, sa holding S(kt) at the top
  // of each unrolled pair, so no iteration copies them.
  f32x16 sa[2], sb[2];
  if (active) prefill_scores<D>(kbuf, ln, qf, sa);
  // iterations with a next tile (unmasked, then masked), then the last one
  const int last = ntiles - 1;
  const int n1 = min(nplain, last);
  int kt = 0;
#define PD_PREFILL_ITER(MASK, NEXT, T, CUR, NXT)                                                            \
  prefill_iter<D, MASK, NEXT>(p, ri, it, T, w, lane, wnt, lim, ln, qf, kbuf, vbuf, L, CUR, NXT, m_ref, lsum, \
                              oacc)
  for (; kt + 1 < n1; kt += 2) {
    PD_PREFILL_ITER(false, true, kt, sa, sb);
    PD_PREFILL_ITER(false, true, kt + 1, sb, sa);
  }
  if (kt < n1) {
    PD_PREFILL_ITER(false, true, kt, sa, sb);
    ++kt;
    sa[0] = sb[0];
    sa[1] = sb[1];
  }
  for (; kt + 1 < last; kt += 2) {
    PD_PREFILL_ITER(true, true, kt, sa, sb);
    PD_PREFILL_ITER(true, true, kt + 1, sb, sa);
  }
  if (kt < last) {
    PD_PREFILL_ITER(true, true, kt, sa, sb);
    sa[0] = sb[0];
    sa[1] = sb[1];
  }
  if (last < nplain)
    PD_PREFILL_ITER(false, false, last, sa, sb);
  else
    PD_PREFILL_ITER(true, false, last, sa, sb);
#undef PD_PREFILL_ITER
  const float l_tot = sum_x32(lsum);
  if (row_ok) {
    const float inv = 1.f / l_tot;
    float* op = p.out + qrow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 v = {oacc[db][4 * jj + 0], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2], oacc[db][4 * jj + 3]};
        *(f32x4*)(op + 32 * db + 8 * jj + 4 * ln.h2) = v * inv;
      }
    if (ln.h2 == 0 && p.lse) p.lse[qrow] = m_ref * p.sm_scale + __logf(l_tot);
  }
}

// ------------------------------------------------------------------------
// Short prompts: 4-wavefront blocks of 128 query rows with two K and two V
// tile buffers (67.6 KB of LDS at head_dim 128), so that two blocks share a
// CU and one block's prologue (its cold Q and first K/V loads) overlaps the
// other's tiles.  One barrier per key tile: at the start of iteration t
// every wave waits for its loads of K(t+1) and V(t) (issued one iteration
// earlier), the barrier publishes them, and the wave issues K(t+2) into the
// buffer of K(t) (read by S(t) in iteration t - 1) and V(t+1) into the
// buffer of V(t - 1) (read by PV(t - 1)).  Then S(t+1), the softmax of t and
// PV(t), as in prefill_iter.  Each SIMD holds one wavefront of each of the
// two blocks, so no row-block pairing is needed; a wavefront still skips
// the key tiles wholly above its rows.
// ------------------------------------------------------------------------
constexpr int kPrefill4Waves = 4;
constexpr int kPrefill4Threads = 64 * kPrefill4Waves;
constexpr int kPrefill4Rows = 32 * kPrefill4Waves;

struct Prefill4Loop {
  int ntiles, nfull;
  int pk, pv;  // page ids of K(t + 2) and V(t + 1) for the loads of iteration t
};

template <int D, bool MASK, bool NEXT, bool FIRST = false>
__device__ __forceinline__ void prefill_iter4(const AttnParams& p, const ReqInfo& ri, const PrefillItem& it,
                                              int t, int w, int lane, int wnt, int lim, PrefillLanes ln,
                                              const u32x4 (&qf)[D / 16], LDS_AS char* kbuf, LDS_AS char* vbuf,
                                              Prefill4Loop& L, f32x16 (&s_cur)[2], f32x16 (&s_next)[2],
                                              float& m_ref, float& lsum, f32x16 (&oacc)[D / 32]) {
  constexpr int W = kPrefill4Waves;
  using C = PrefillCfg<D, W>;
  const int nt = L.ntiles;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (t + 2 < nt)
    prefill_issue<D, W>(p, it.hk, 0, it.kv_end, (t + 2) * 64, w, L.pk, lane, t + 2 < L.nfull,
                        kbuf + (t & 1) * C::TILE_BYTES);
  if (t + 1 < nt)
    prefill_issue<D, W>(p, it.hk, 1, it.kv_end, (t + 1) * 64, w, L.pv, lane, t + 1 < L.nfull,
                        vbuf + ((t + 1) & 1) * C::TILE_BYTES);
  // pages of the next iteration's loads: V(t + 2) lies in the tile of K(t + 2)
  L.pv = L.pk;
  L.pk = prefill_page<D, W>(p, ri, it.kv_end, (t + 3) * 64, w);
  if (t < wnt) {
    if (NEXT) prefill_scores<D>(kbuf + ((t + 1) & 1) * C::TILE_BYTES, ln, qf, s_next);
    uint32_t pk[2][8];
    prefill_softmax<D, MASK, FIRST>(p, s_cur, t * 64, lim, ln, m_ref, lsum, oacc, pk);
    prefill_pv<D>(vbuf + (t & 1) * C::TILE_BYTES, ln, pk, oacc);
  }
}

template <int D>
__device__ void prefill_tile4(const AttnParams& p, const PrefillItem& it, const ReqInfo& ri, LDS_AS char* lds) {
  constexpr int W = kPrefill4Waves;
  using C = PrefillCfg<D, W>;
  const int lane = threadIdx.x & 63;
  const int w = uniform_i(threadIdx.x >> 6);
  const int g = p.g;
  const int rows = it.nq * g;
  const int nloc = lane & 31;
  const int n = 32 * w + nloc;
  const bool row_ok = n < rows;
  const int t = row_ok ? n / g : 0;
  const int h = it.hk * g + (row_ok ? n % g : 0);
  const int qpos0 = ri.kv - ri.qo + it.q0;
  const int lim = p.causal ? qpos0 + t + 1 : ri.kv;
  const int mask_from = p.causal ? qpos0 + 1 : it.kv_end;
  const int64_t qrow = (int64_t)(ri.qo_start + it.q0 + t) * p.H_q + h;

  PrefillLanes ln;
  ln.h2 = lane >> 5;
  ln.k_off = Lds<D>::off(nloc, ln.h2);
  {
    const int j = lane & 15, dhalf = (lane >> 4) & 1;
    ln.v_off = Lds<D>::off(4 * ln.h2 + (j >> 2), 2 * dhalf + ((j & 3) >> 1)) + 8 * (j & 1);
  }
  u32x4 qf[C::KS];
  {
    const uint16_t* qp = (const uint16_t*)p.q + qrow * D + 8 * ln.h2;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const u32x4 v = *(const u32x4*)(qp + 16 * ks);
      qf[ks] = row_ok ? v : u32x4{0, 0, 0, 0};
    }
  }
  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
  float m_ref = -INFINITY;
  float lsum = 0.f;

  LDS_AS char* kbuf = lds;
  LDS_AS char* vbuf = lds + C::NBUF * C::TILE_BYTES;
  const int ntiles = (it.kv_end + 63) >> 6;
  const int nfull = it.kv_end >> 6;
  const int nplain = min(ntiles, mask_from / 64);
  // prologue: K(0) V(0) K(1), and the pages of iteration 0's loads
  Prefill4Loop L;
  L.ntiles = ntiles;
  L.nfull = nfull;
  {
    const int pg0 = prefill_page<D, W>(p, ri, it.kv_end, 0, w);
    prefill_issue<D, W>(p, it.hk, 0, it.kv_end, 0, w, pg0, lane, 0 < nfull, kbuf);
    prefill_issue<D, W>(p, it.hk, 1, it.kv_end, 0, w, pg0, lane, 0 < nfull, vbuf);
    const int pg1 = prefill_page<D, W>(p, ri, it.kv_end, 64, w);
    if (ntiles > 1) prefill_issue<D, W>(p, it.hk, 0, it.kv_end, 64, w, pg1, lane, 1 < nfull, kbuf + C::TILE_BYTES);
    L.pv = pg1;
    L.pk = prefill_page<D, W>(p, ri, it.kv_end, 128, w);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int wnt = 0;
  if (32 * w < rows) {
    const int tmax = min(32 * w + 31, rows - 1) / g;
    wnt = (min(it.kv_end, p.causal ? qpos0 + tmax + 1 : it.kv_end) + 63) >> 6;
  }
  f32x16 sa[2], sb[2];
  if (wnt > 0) prefill_scores<D>(kbuf, ln, qf, sa);
  const int last = ntiles - 1;
  const int n1 = min(nplain, last);
  int kt = 0;
#define PD_PREFILL4_ITER(MASK, NEXT, T, CUR, NXT)                                                            \
  prefill_iter4<D, MASK, NEXT>(p, ri, it, T, w, lane, wnt, lim, ln, qf, kbuf, vbuf, L, CUR, NXT, m_ref, lsum, \
                               oacc)
  // key tile 0 (with a next tile) on its own: its softmax takes the row
  // maximum at once.  (Short prompts have few key tiles, so the general
  // path's second pass over their first tile is a visible share of the
  // work: 8 x 512 prompts 0.0609-0.0614 against 0.0620-0.0627 ms, same
  // box.  The 8-wavefront kernel keeps the general path: there it measured
  // 1 % slower on the long mixed launch.)
  if (last > 0) {
    if (n1 > 0)
      prefill_iter4<D, false, true, true>(p, ri, it, 0, w, lane, wnt, lim, ln, qf, kbuf, vbuf, L, sa, sb, m_ref,
                                          lsum, oacc);
    else
      prefill_iter4<D, true, true, true>(p, ri, it, 0, w, lane, wnt, lim, ln, qf, kbuf, vbuf, L, sa, sb, m_ref,
                                         lsum, oacc);
    kt = 1;
    sa[0] = sb[0];
    sa[1] = sb[1];
  }
  for (; kt + 1 < n1; kt += 2) {
    PD_PREFILL4_ITER(false, true, kt, sa, sb);
    PD_PREFILL4_ITER(false, true, kt + 1, sb, sa);
  }
  if (kt < n1) {
    PD_PREFILL4_ITER(false, true, kt, sa, sb);
    ++kt;
    sa[0] = sb[0];
    sa[1] = sb[1];
  }
  for (; kt + 1 < last; kt += 2) {
    PD_PREFILL4_ITER(true, true, kt, sa, sb);
    PD_PREFILL4_ITER(true, true, kt + 1, sb, sa);
  }
  if (kt < last) {
    PD_PREFILL4_ITER(true, true, kt, sa, sb);
    sa[0] = sb[0];
    sa[1] = sb[1];
  }
  if (last < nplain)
    PD_PREFILL4_ITER(false, false, last, sa, sb);
  else
    PD_PREFILL4_ITER(true, false, last, sa, sb);
#undef PD_PREFILL4_ITER
  const float l_tot = sum_x32(lsum);
  if (row_ok) {
    const float inv = 1.f / l_tot;
    float* op = p.out + qrow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 v = {oacc[db][4 * jj + 0], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2], oacc[db][4 * jj + 3]};
        *(f32x4*)(op + 32 * db + 8 * jj + 4 * ln.h2) = v * inv;
      }
    if (ln.h2 == 0 && p.lse) p.lse[qrow] = m_ref * p.sm_scale + __logf(l_tot);
  }
}

// Prefill-only launches of 128-row tiles (the plan's launch records all hold
// one tile): two blocks per CU.
template <int D>
__global__ __launch_bounds__(kPrefill4Threads, 2) void attn_prefill4_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char lds_raw[PrefillCfg<D, kPrefill4Waves>::LDS_BYTES];
  const LaunchRec* rec = p.launch + blockIdx.x;
  prefill_tile4<D>(p, ldc((const PrefillItem*)rec->w), ldc((const ReqInfo*)(rec->w + 8)), (LDS_AS char*)lds_raw);
}

// One launch for both roles: the block map gives each block a prefill tile
// (v >= 0) or a decode block of eight unit queues, one per wavefront (v < 0).
// Decode blocks keep the paired queues' counters (two per wavefront) after
// the eight wavefronts' stages.
template <int D>
constexpr int decode_lds_bytes() {
  return kAttnWaves * DecodeCfg<D>::WAVE_LDS + 2 * kAttnWaves * (int)sizeof(int32_t);
}
template <int D>
constexpr int attn_lds_bytes() {
  return PrefillCfg<D>::LDS_BYTES > decode_lds_bytes<D>() ? PrefillCfg<D>::LDS_BYTES : decode_lds_bytes<D>();
}
template <int D>
__global__ __launch_bounds__(kAttnThreads, 1) void attn_bf16_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) char lds_raw[attn_lds_bytes<D>()];
  LDS_AS char* lds = (LDS_AS char*)lds_raw;
  const LaunchRec* rec = p.launch + blockIdx.x;
  const int w = uniform_i(threadIdx.x >> 6);
  // the record and this wavefront's queue offsets (meaningful for decode
  // blocks only) are loaded together: none depends on another
  const int v = ldc(&rec->v);
  const int u0 = ldc(rec->w + w), u1 = ldc(rec->w + w + 1);
  if (v >= 0) {
    prefill_tile<D>(p, ldc((const PrefillItem*)rec->w), ldc((const ReqInfo*)(rec->w + 8)), lds);
  } else {
    // Paired queues take the first slots of the launch; a block that holds
    // some zeroes their counters, and the barrier (taken by all eight
    // wavefronts or none) orders this before any wavefront's first wait.
    volatile LDS_AS int32_t* cnt = (volatile LDS_AS int32_t*)(lds + kAttnWaves * DecodeCfg<D>::WAVE_LDS);
    if (ldc(rec->w + 9)) {
      if ((threadIdx.x & 63) < 2) cnt[2 * w + (threadIdx.x & 63)] = 0;
      __syncthreads();
    }
    if (u0 < u1) {
      LDS_AS char* wl = lds + w * DecodeCfg<D>::WAVE_LDS;
      const DecodeItem first = ldc(&p.du[u0].it);
      if (first.pair) {
        // slots 2 i and 2 i + 1 of a block: rows 0..31 and 32..63
        const int h = w & 1;
        PairState ps{cnt + 2 * w, cnt + 2 * (w ^ 1), lds + (w & ~1) * DecodeCfg<D>::WAVE_LDS, h, 0};
        decode_queue_pair<D>(p, u0, u1, ps);
      } else if (first.ncg == 2) {
        decode_queue<D, 2>(p, u0, u1, wl);
      } else {
        decode_queue<D, 1>(p, u0, u1, wl);
      }
    }
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
__global__ __launch_bounds__(kAttnThreads) void attn_f32_kernel(AttnParams p) {
  constexpr int NO = D / 64;
  const int lane = threadIdx.x & 63;
  const int w = uniform_i(threadIdx.x >> 6);
  const LaunchRec* rec = p.launch + blockIdx.x;
  const int v = ldc(&rec->v);
  const float* qbase = (const float*)p.q;
  if (v >= 0) {
    const PrefillItem it = ldc((const PrefillItem*)rec->w);
    const ReqInfo ri = ldc((const ReqInfo*)(rec->w + 8));
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
    const int u1 = ldc(rec->w + w + 1);
    for (int u = ldc(rec->w + w); u < u1; ++u) {
      const DecodeUnit du = ldc(p.du + u);
      const DecodeItem& it = du.it;
      const ReqInfo& ri = du.ri;
      const int nrows = min(ri.qo * p.g, it.c0 + kDecodeCols * it.ncg);
      for (int n = it.c0; n < nrows; ++n) {
        const int t = n / p.g, h = it.hk * p.g + n % p.g;
        const int lim = p.causal ? ri.kv - ri.qo + t + 1 : ri.kv;
        const int64_t row = (int64_t)(ri.qo_start + t) * p.H_q + h;
        float o[NO], lse;
        f32_row<D>(p, ri, it.hk, qbase + row * D, it.k0, min(lim, it.k1), o, lse);
        const int64_t ps = (int64_t)it.part + (n - it.c0);
        float* po = p.part_o + ps * D;
#pragma unroll
        for (int i = 0; i < NO; ++i) po[lane + 64 * i] = o[i];
        if (lane == 0) p.part_lse[ps] = lse;
      }
    }
  }
}

// ------------------------------------------------------------------------
// Merge of split-KV partials: for each decode row, LSE* = max_i lse_i,
// w_i = exp(lse_i - LSE*), O = sum_i w_i o_i / sum_i w_i,
// LSE = LSE* + ln sum_i w_i; parts are visited in a fixed order.
// ------------------------------------------------------------------------
// Groups of at most kMergeBatch parts load every part's LSE and output at
// once (one round trip), then combine them in part order; larger groups
// take two passes over the parts.  Both orders of arithmetic are the same.
constexpr int kMergeBatch = 8;

template <int D>
__global__ __launch_bounds__(kBlockThreads) void merge_kernel(AttnParams p) {
  const MergeRec mg = ldc(p.mg + blockIdx.x);
  const int nrows = mg.nrows;
  constexpr int D4 = D / 4;
  for (int idx = threadIdx.x; idx < nrows * D4; idx += kBlockThreads) {
    const int n = idx / D4, d4 = idx % D4;
    const int t = n / p.g, h = mg.hk * p.g + n % p.g;
    const int64_t base = (int64_t)mg.part0 + n;
    const int64_t stride = nrows;  // chunk i + 1 is nrows partial rows further
    float mx = -INFINITY;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float sw = 0.f;
    if (mg.nparts <= kMergeBatch) {
      float l[kMergeBatch];
      f32x4 o[kMergeBatch];
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const int64_t slot = base + (int64_t)min(i, mg.nparts - 1) * stride;
        l[i] = p.part_lse[slot];
        o[i] = *(const f32x4*)(p.part_o + slot * D + 4 * d4);
      }
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i)
        if (i < mg.nparts) mx = fmaxf(mx, l[i]);
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i)
        if (i < mg.nparts) {
          const float wi = (l[i] == -INFINITY) ? 0.f : __expf(l[i] - mx);
          acc += o[i] * wi;
          sw += wi;
        }
    } else {
      for (int i = 0; i < mg.nparts; ++i) mx = fmaxf(mx, p.part_lse[base + i * stride]);
      for (int i = 0; i < mg.nparts; ++i) {
        const int64_t slot = base + i * stride;
        const float li = p.part_lse[slot];
        const float wi = (li == -INFINITY) ? 0.f : __expf(li - mx);
        const f32x4 oi = *(const f32x4*)(p.part_o + slot * D + 4 * d4);
        acc += oi * wi;
        sw += wi;
      }
    }
    const int64_t row = (int64_t)(mg.qo_start + t) * p.H_q + h;
    *(f32x4*)(p.out + row * D + 4 * d4) = acc * (1.f / sw);
    if (d4 == 0 && p.lse) p.lse[row] = mx + __logf(sw);
  }
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int dtype, hipStream_t s) {
  const int blocks = p.n_blocks;
  if (blocks == 0) return hipSuccess;
  if (dtype == 1 && p.prefill4) {
    if (p.D == 128)
      hipLaunchKernelGGL(attn_prefill4_kernel<128>, dim3(blocks), dim3(kPrefill4Threads), 0, s, p);
    else
      hipLaunchKernelGGL(attn_prefill4_kernel<64>, dim3(blocks), dim3(kPrefill4Threads), 0, s, p);
  } else if (dtype == 1) {
    if (p.D == 128)
      hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(blocks), dim3(kAttnThreads), 0, s, p);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(blocks), dim3(kAttnThreads), 0, s, p);
  } else {
    if (p.D == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(blocks), dim3(kAttnThreads), 0, s, p);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(blocks), dim3(kAttnThreads), 0, s, p);
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

}  // namespace pdk
