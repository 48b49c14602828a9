// MLA (multi-head latent attention) decode for gfx950 (MI355X, CDNA4): the
// split-KV attention of decode rows over a paged latent cache, the merge of
// its partial results, and the append of new latent rows.
//
// What is computed (Perplexity post "Disaggregated prefill and decode",
// section "DeepSeek-R1" under "Disaggregated Deployments"): MLA keeps one
// latent vector per token for all KV heads, the same on every rank.  Decode
// uses the absorbed form: each query row (token t, head h) brings a
// [latent ; rotary] vector q, and
//   S_j = scale <q, row_j>,  O = sum_j softmax(S)_j latent_j,  LSE,
// i.e. one-KV-head attention whose key is the whole cache row (576 bf16) and
// whose value is the row's first 512 entries.  Every query head of a request
// reads the same rows, so one block serves 64 query rows of a request and
// stages each 32-key step of the cache once for all of them.  (Requests of
// 128 heads use mla_wide.hip: 32 rows per wavefront, 128 per block.)
//
// Layout (see include/pd_attn.h): pool [pages][ps][576] bf16 (latent then
// rotary key), q [rows][H][576] bf16, out fp32 [rows][H][512], lse [rows][H].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "mla_common.hpp"
#include "pd_internal.hpp"

namespace pdk {
namespace {

struct MlaLanes {
  int q;        // 16-lane group
  int k_lat;    // lane part of the latent score-operand reads
  int k_rope;   // ... of the rotary score-operand reads
  int v_off;    // ... of the transposed value reads
};

// The score products of one step as a software pipeline: read r (k-step
// r / 2, keys 16 (r % 2) + (lane & 15)) is issued RING reads ahead of
// product r, which accumulates into chain r % 2.
template <int RING_>
struct MlaSPipe {
  static constexpr int NR = 2 * (kMlaWidth / 32);
  static constexpr int RING = RING_;
  template <int R>
  static constexpr int off() {  // immediate offset of read R from the lane's latent / rotary base
    return (R / 2) < 16 ? (R % 2) * (16 / Lds<128>::RPB) * Lds<128>::BLOCK + ((R / 2) / 4) * Lds<128>::bytes(32) +
                              Lds<128>::chunk_step(2 * ((R / 2) % 4))
                        : (R % 2) * (16 / Lds<64>::RPB) * Lds<64>::BLOCK + Lds<64>::chunk_step(2 * ((R / 2) - 16));
  }
};

// The value products of one step: product m (latent entries 128 (m / 8) +
// 16 (m % 8) ..) takes two transposed reads (keys 4q + e and 16 + 4q + e);
// the reads of product m + AHEAD are issued before product m waits for its
// own.  The first AHEAD products' reads are issued before the softmax.
template <int AHEAD_>
struct MlaPVPipe {
  static constexpr int N = kMlaLatent / 16;
  static constexpr int AHEAD = AHEAD_;
  static constexpr int RING = AHEAD + 1;
  template <int M, int H>
  static constexpr int off() {
    return (M / 8) * Lds<128>::bytes(32) + Lds<128>::chunk_step(M % 8) + H * (16 / Lds<128>::RPB) * Lds<128>::BLOCK;
  }
};

template <int AHEAD, int M>
__device__ __forceinline__ void mla_pv_issue(u32x2 (&va)[AHEAD + 1][2], const LDS_AS char* vp) {
  va[M % (AHEAD + 1)][0] = lds_read_tr16_asm<MlaPVPipe<AHEAD>::template off<M, 0>()>(vp);
  va[M % (AHEAD + 1)][1] = lds_read_tr16_asm<MlaPVPipe<AHEAD>::template off<M, 1>()>(vp);
}

template <int AHEAD, int M>
__device__ __forceinline__ void mla_pv_prologue(u32x2 (&va)[AHEAD + 1][2], const LDS_AS char* vp) {
  mla_pv_issue<AHEAD, M>(va, vp);
  if constexpr (M + 1 < AHEAD) mla_pv_prologue<AHEAD, M + 1>(va, vp);
}

template <int AHEAD, int M>
__device__ __forceinline__ void mla_pv_pipe(u32x2 (&va)[AHEAD + 1][2], const LDS_AS char* vp, u32x4 pb,
                                            f32x4 (&oacc)[kMlaLatent / 16]) {
  constexpr int N = MlaPVPipe<AHEAD>::N, RING = AHEAD + 1;
  if constexpr (M + AHEAD < N) mla_pv_issue<AHEAD, M + AHEAD>(va, vp);
  constexpr int LATER = 2 * ((N - 1 - M) < AHEAD ? (N - 1 - M) : AHEAD);
  static_assert(LATER < 16, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(va[M % RING][0]), "+v"(va[M % RING][1]) : "n"(LATER));
  const u32x4 a = {va[M % RING][0][0], va[M % RING][0][1], va[M % RING][1][0], va[M % RING][1][1]};
  oacc[M] = mfma16(a, pb, oacc[M]);
  if constexpr (M + 1 < N) mla_pv_pipe<AHEAD, M + 1>(va, vp, pb, oacc);
}

template <int RING, int R>
__device__ __forceinline__ void mla_s_pipe(u32x4 (&kf)[RING], f32x4 (&s)[2], const u32x4 (&qf)[kMlaWidth / 32],
                                           const LDS_AS char* kl, const LDS_AS char* kr) {
  constexpr int NR = MlaSPipe<RING>::NR;
  if constexpr (R >= RING) {
    constexpr int i = R - RING;
    lgkm_wait_for<(NR - 1 - i < RING - 1) ? NR - 1 - i : RING - 1>(kf[i % RING]);
    s[i % 2] = mfma16(kf[i % RING], qf[i / 2], s[i % 2]);
  }
  if constexpr (R < NR) kf[R % RING] = lds_read16_asm<MlaSPipe<RING>::template off<R>()>((R / 2) < 16 ? kl : kr);
  if constexpr (R + 1 < NR + RING) mla_s_pipe<RING, R + 1>(kf, s, qf, kl, kr);
}

// One 32-key step of a wavefront's 16 rows from stage `st`: S^T = K Q^T
// (K 16 bytes per lane from LDS, Q^T in registers), the speculative online
// softmax per column, then O^T += V^T P^T with V^T read transposed from the
// latent tiles.  Key order inside the step is permuted identically in P^T
// and V^T (keys 4q + e and 16 + 4q + e in lane group q).
template <int SRING, int PVAHEAD>
__device__ __forceinline__ void mla_step(const MlaParams& p, const LDS_AS char* st, int b, int lim, MlaLanes ln,
                                         const u32x4 (&qf)[MlaCfg::KS], float& m_ref, f32x4& lacc,
                                         f32x4 (&oacc)[MlaCfg::DB]) {
  const float cl = p.c_log2;
  // S^T: the two 16-key chains interleaved; operand read r feeds product r
  // (k-step r / 2, keys 16 (r % 2) ..).  With one wavefront per SIMD nothing
  // else hides the LDS latency, so the reads run RING ahead of the products.
  f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  u32x4 kf[SRING];
  mla_s_pipe<SRING, 0>(kf, s, qf, st + ln.k_lat, st + ln.k_rope);
  u32x2 va[PVAHEAD + 1][2];
  const LDS_AS char* vp = st + ln.v_off;
  mla_pv_prologue<PVAHEAD, 0>(va, vp);  // the first value reads land during the softmax
  if (b + 32 > lim) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (b + 16 * sb + 4 * ln.q + i >= lim) s[sb][i] = -INFINITY;
  }
  uint32_t pk[4];
  {
    const float mc = m_ref * cl;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        pk[2 * sb + i] = pack_bf16(fast_exp2(__builtin_fmaf(s[sb][2 * i], cl, -mc)),
                                   fast_exp2(__builtin_fmaf(s[sb][2 * i + 1], cl, -mc)));
  }
  if (wave_any(p_out_of_range(pk))) {
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = max_x16(mx);
    mx = max_x32(mx);
    const float m_new = fmaxf(m_ref, mx);
    if (m_new != -INFINITY) {  // a column with no visible key yet keeps m_ref = -inf
      const float alpha = fast_exp2((m_ref - m_new) * cl);  // m_ref = -inf -> 0
      lacc = lacc * alpha;
#pragma unroll
      for (int db = 0; db < MlaCfg::DB; ++db) oacc[db] = oacc[db] * alpha;
      m_ref = m_new;
    }
    const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * cl;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        pk[2 * sb + i] = pack_bf16(fast_exp2(__builtin_fmaf(s[sb][2 * i], cl, -mc)),
                                   fast_exp2(__builtin_fmaf(s[sb][2 * i + 1], cl, -mc)));
  }
  const u32x4 pb = {pk[0], pk[1], pk[2], pk[3]};
  lacc = mfma16(u32x4{kBf16OnesPair, kBf16OnesPair, kBf16OnesPair, kBf16OnesPair}, pb, lacc);
  // V^T[d = 16 m + (lane & 15)][keys 4q + e, 16 + 4q + e]
  mla_pv_pipe<PVAHEAD, 0>(va, vp, pb, oacc);
}

__global__ __launch_bounds__(256, 1) void mla_kernel(MlaParams p) {
  // one wavefront per SIMD: deep operand-read rings hide the LDS latency
  constexpr int SRING = 8, PVAHEAD = 7;
  __shared__ __attribute__((aligned(16))) char lds_raw[MlaCfg::LDS_BYTES];
  LDS_AS char* lds = (LDS_AS char*)lds_raw;
  const MlaItem it = ldc(p.items + blockIdx.x);
  const ReqInfo ri = ldc(p.req + it.req);
  const int lane = threadIdx.x & 63;
  const int w = uniform_i(threadIdx.x >> 6);
  const int H = p.H;
  const int n0 = 64 * it.rg + 16 * w;  // first query row of this wavefront (H is a multiple of 16)
  const bool active = n0 < ri.qo * H;
  const int t = active ? n0 / H : 0;
  const int h = n0 % H + (lane & 15);
  const int lim = min(it.k1, p.causal ? ri.kv - ri.qo + t + 1 : ri.kv);

  MlaLanes ln;
  ln.q = lane >> 4;
  // Lane group g = lane / 16 of the score operands carries entries 8 g .. +7
  // of each 32-entry k-step (chunk g of its four).
  const int kchunk = lane >> 4;
  ln.k_lat = Lds<128>::off(lane & 15, kchunk & 1) + Lds<128>::chunk_step(kchunk >> 1);
  ln.k_rope = MlaCfg::ROPE + Lds<64>::off(lane & 15, kchunk & 1) + Lds<64>::chunk_step(kchunk >> 1);
  {
    const int j = lane & 15;
    ln.v_off = Lds<128>::off(4 * ln.q + (j >> 2), (j & 3) >> 1) + 8 * (j & 1);
  }

  // Q^T fragments, loaded before any stage load, into accumulation registers
  // (a read-only MFMA operand; the architectural registers hold O^T and the
  // operand ring).  The loads are issued from inline asm: the compiler would
  // otherwise place a wait for them at their first use inside the step loop
  // (vmcnt(0), which also drains every stage load in flight, at every step).
  // They are older than all stage loads, so the loop's own wait for step 0
  // covers them.
  u32x4 qf[MlaCfg::KS];
  if (active) {
    const uint16_t* qp = (const uint16_t*)p.q + ((int64_t)(ri.qo_start + t) * H + h) * kMlaWidth + 8 * kchunk;
#pragma unroll
    for (int ks = 0; ks < MlaCfg::KS; ++ks)
      asm volatile("global_load_dwordx4 %0, %1, off" : "=a"(qf[ks]) : "v"(qp + 32 * ks) : "memory");
  } else {
#pragma unroll
    for (int ks = 0; ks < MlaCfg::KS; ++ks) qf[ks] = u32x4{0, 0, 0, 0};
  }
  f32x4 oacc[MlaCfg::DB];
#pragma unroll
  for (int db = 0; db < MlaCfg::DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;
  f32x4 lacc = {0.f, 0.f, 0.f, 0.f};  // column sums of the bf16 P (all four entries equal)

  const int nsteps = (it.k1 - it.k0 + 31) >> 5;
#pragma unroll
  for (int s = 0; s < 3; ++s)
    if (s < nsteps) {
      const int b = it.k0 + 32 * s;
      mla_issue(p, ri, b, mla_page(p, ri, b), mla_page(p, ri, b + 16), w, lane, lds + s * MlaCfg::STAGE);
    }
  int pgA = mla_page(p, ri, it.k0 + 96), pgB = mla_page(p, ri, it.k0 + 112);  // step 3
  for (int i = 0; i < nsteps; ++i) {
    mla_wait_loads<MlaCfg::LOADS_PER_WAVE>(nsteps - 1 - i);
    __syncthreads();  // step i visible to all; stage (i + 3) % 4 = (i - 1) % 4 read by all
    if (i + 3 < nsteps) {
      mla_issue(p, ri, it.k0 + 32 * (i + 3), pgA, pgB, w, lane, lds + ((i + 3) & 3) * MlaCfg::STAGE);
      pgA = mla_page(p, ri, it.k0 + 32 * (i + 4));
      pgB = mla_page(p, ri, it.k0 + 32 * (i + 4) + 16);
    }
    const int b = it.k0 + 32 * i;
    if (active && b < lim) mla_step<SRING, PVAHEAD>(p, lds + (i & 3) * MlaCfg::STAGE, b, lim, ln, qf, m_ref, lacc, oacc);
  }

  if (!active) return;
  const float l_tot = lacc[0];
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? m_ref * p.sm_scale + __logf(l_tot) : -INFINITY;
  float* po;
  if (it.part < 0) {
    const int64_t row = (int64_t)(ri.qo_start + t) * H + h;
    po = p.out + row * kMlaLatent;
    if (ln.q == 0 && p.lse) p.lse[row] = lse;
  } else {
    const int64_t slot = (int64_t)it.part * 64 + 16 * w + (lane & 15);
    po = p.part_o + slot * kMlaLatent;
    if (ln.q == 0) p.part_lse[slot] = lse;
  }
#pragma unroll
  for (int db = 0; db < MlaCfg::DB; ++db) *(f32x4*)(po + 16 * db + 4 * ln.q) = oacc[db] * inv;
}

// Log-sum-exp merge of split partial results: one wavefront per query row
// of a merge group (lanes over the 512 latent entries, 8 each), parts in
// slot order (deterministic for a fixed plan).  A group of at most
// kMlaMergeBatch parts loads every part's LSE and output at once (one round
// trip), then combines them in slot order; larger groups take two passes.
// Both orders of arithmetic are the same.
constexpr int kMlaMergeBatch = 8;

__global__ __launch_bounds__(64 * kMlaMergeWaves) void mla_merge_kernel(MlaParams p) {
  const int wg = blockIdx.x * kMlaMergeWaves + uniform_i(threadIdx.x >> 6);
  const int R = p.rows;
  const int gi = wg / R, n = wg % R;
  if (gi >= p.n_mg) return;
  const MlaMergeRec mg = ldc(p.mg + gi);
  const int rn = R * mg.rg + n;  // row of the request (token rn / H, head rn % H)
  if (rn >= mg.qo_rows) return;
  const int lane = threadIdx.x & 63;
  float mx = -INFINITY;
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  float sw = 0.f;
  if (mg.nparts <= kMlaMergeBatch) {
    float l[kMlaMergeBatch];
    f32x4 o0[kMlaMergeBatch], o1[kMlaMergeBatch];
#pragma unroll
    for (int i = 0; i < kMlaMergeBatch; ++i) {
      const int64_t slot = (int64_t)(mg.part0 + min(i, mg.nparts - 1)) * R + n;
      l[i] = ldc(p.part_lse + slot);
      const float* po = p.part_o + slot * kMlaLatent + 4 * lane;
      o0[i] = *(const f32x4*)po;
      o1[i] = *(const f32x4*)(po + 256);
    }
#pragma unroll
    for (int i = 0; i < kMlaMergeBatch; ++i)
      if (i < mg.nparts) mx = fmaxf(mx, l[i]);
#pragma unroll
    for (int i = 0; i < kMlaMergeBatch; ++i)
      if (i < mg.nparts) {
        const float wi = (l[i] == -INFINITY) ? 0.f : __expf(l[i] - mx);
        a0 += o0[i] * wi;
        a1 += o1[i] * wi;
        sw += wi;
      }
  } else {
    for (int i = 0; i < mg.nparts; ++i) mx = fmaxf(mx, ldc(p.part_lse + (int64_t)(mg.part0 + i) * R + n));
    for (int i = 0; i < mg.nparts; ++i) {
      const int64_t slot = (int64_t)(mg.part0 + i) * R + n;
      const float li = ldc(p.part_lse + slot);
      const float wi = (li == -INFINITY) ? 0.f : __expf(li - mx);
      const float* po = p.part_o + slot * kMlaLatent + 4 * lane;
      a0 += *(const f32x4*)po * wi;
      a1 += *(const f32x4*)(po + 256) * wi;
      sw += wi;
    }
  }
  const int64_t row = (int64_t)(mg.qo_start + rn / p.H) * p.H + rn % p.H;
  const float inv = 1.f / sw;
  *(f32x4*)(p.out + row * kMlaLatent + 4 * lane) = a0 * inv;
  *(f32x4*)(p.out + row * kMlaLatent + 256 + 4 * lane) = a1 * inv;
  if (lane == 0 && p.lse) p.lse[row] = mx + __logf(sw);
}

// Append: one wavefront per new token row; 72 16-byte copies of its latent
// and rotary entries into (page, slot) of position kv - qo + i.
__global__ __launch_bounds__(64) void mla_append_kernel(MlaParams p, void* pool, const void* rows_new) {
  const int row = blockIdx.x;
  int lo = 0, hi = p.B - 1;  // last request with qo_indptr[r] <= row
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ldc(p.qo_indptr + mid) <= row) lo = mid; else hi = mid - 1;
  }
  const ReqInfo ri = ldc(p.req + lo);
  const int pos = ri.kv - ri.qo + (row - ri.qo_start);
  const int page = ldc(p.page_indices + ri.page_start + (pos >> p.ps_shift));
  constexpr int RB = 2 * kMlaWidth;
  char* dst = (char*)pool + ((int64_t)page * p.ps + (pos & (p.ps - 1))) * RB;
  const char* src = (const char*)rows_new + (int64_t)row * RB;
  for (int c = threadIdx.x; c < RB / 16; c += 64) *(u32x4*)(dst + 16 * c) = *(const u32x4*)(src + 16 * c);
}

}  // namespace

hipError_t launch_mla(const MlaParams& p, hipStream_t s) {
  if (p.n_items > 0) {
    if (p.rows == 128) {
      hipError_t e = launch_mla_wide(p, s);  // 32 rows per wavefront (mla_wide.hip)
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(mla_kernel, dim3(p.n_items), dim3(256), 0, s, p);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (p.n_mg > 0)
    hipLaunchKernelGGL(mla_merge_kernel, dim3((p.n_mg * p.rows + kMlaMergeWaves - 1) / kMlaMergeWaves),
                       dim3(64 * kMlaMergeWaves), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_mla_append(const MlaParams& p, void* pool, const void* rows_new, hipStream_t s) {
  if (p.total_rows > 0) hipLaunchKernelGGL(mla_append_kernel, dim3(p.total_rows), dim3(64), 0, s, p, pool, rows_new);
  return hipGetLastError();
}

}  // namespace pdk
