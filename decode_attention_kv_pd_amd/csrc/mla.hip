// MLA (multi-head latent attention) decode for gfx950 (MI355X, CDNA4): the
// split-KV attention of decode rows over a paged latent cache, the merge of
// its partial results, and the append of new latent rows.
//
// What is computed (Perplexity post "Disaggregated prefill and decode",
// section "Sharded KV Cache Transfers", DeepSeek paragraphs): MLA keeps one
// latent vector per token for all KV heads, the same on every rank.  Decode
// uses the absorbed form: each query row (token t, head h) brings a
// [latent ; rotary] vector q, and
//   S_j = scale <q, row_j>,  O = sum_j softmax(S)_j latent_j,  LSE,
// i.e. one-KV-head attention whose key is the whole cache row (576 bf16) and
// whose value is the row's first 512 entries.  Every query head of a request
// reads the same rows, so one block serves 64 query rows of a request and
// stages each 32-key step of the cache once for all of them.
//
// Layout (see include/pd_attn.h): pool [pages][ps][576] bf16 (latent then
// rotary key), q [rows][H][576] bf16, out fp32 [rows][H][512], lse [rows][H].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "pd_internal.hpp"

namespace pdk {
namespace {

// A block: 4 wavefronts, 16 query rows each (the N index of both products),
// one key range, 32 keys per step.  A step's rows are staged in LDS as four
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
  static constexpr int LOADS_PER_WAVE = LOADS / kMlaWaves;
};
static_assert(MlaCfg::LOADS == 36 && MlaCfg::LOADS_PER_WAVE == 9, "stage loads split over the wavefronts");
static_assert(MlaCfg::LDS_BYTES <= 160 * 1024, "LDS of one block");
static_assert(Lds<128>::RPB == 4 && Lds<64>::RPB == 8, "tile geometry");

// Page id of key `key` of a request (clamped to its last key).
__device__ __forceinline__ int mla_page(const MlaParams& p, const ReqInfo& ri, int key) {
  return ldc(p.page_indices + ri.page_start + (min(key, ri.kv - 1) >> p.ps_shift));
}

// Wavefront w's share (9 of the 36 block loads) of the step at key b into
// stage `st`: latent loads i = 0..7 (tile i / 2, rows 4 (w + 4 (i % 2)) ..
// +3), then one rotary load (rows 8 w .. + 7).  pgA / pgB are the pages of
// keys b .. b + 15 and b + 16 .. b + 31 (pages hold >= 16 aligned keys).
// Keys >= kv (only in a request's last step) are read from key kv - 1
// instead: finite data, masked later, and tail slots are never read.
__device__ __forceinline__ void mla_issue(const MlaParams& p, const ReqInfo& ri, int b, int pgA, int pgB,
                                          int w, int lane, LDS_AS char* st) {
  const char* pool = (const char*)p.pool;
  const int kvm1 = ri.kv - 1;
  const int psm = p.ps - 1;
  constexpr int64_t RB = 2 * kMlaWidth;  // bytes per cache row
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

struct MlaLanes {
  int q;        // 16-lane group
  int k_lat;    // lane part of the latent score-operand reads
  int k_rope;   // ... of the rotary score-operand reads
  int v_off;    // ... of the transposed value reads
};

// One 32-key step of a wavefront's 16 rows from stage `st`: S^T = K Q^T
// (K 16 bytes per lane from LDS, Q^T in registers), the speculative online
// softmax per column, then O^T += V^T P^T with V^T read transposed from the
// latent tiles.  Key order inside the step is permuted identically in P^T
// and V^T (keys 4q + e and 16 + 4q + e in lane group q).
__device__ __forceinline__ void mla_step(const MlaParams& p, const LDS_AS char* st, int b, int lim, MlaLanes ln,
                                         const u32x4 (&qf)[MlaCfg::KS], float& m_ref, f32x4& lacc,
                                         f32x4 (&oacc)[MlaCfg::DB]) {
  const float cl = p.c_log2;
  f32x4 s[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const LDS_AS char* kp = st + ln.k_lat + sb * (16 / Lds<128>::RPB) * Lds<128>::BLOCK;
    s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      s[sb] = mfma16(lds_read16(kp + (ks / 4) * MlaCfg::QUARTER + Lds<128>::chunk_step(2 * (ks % 4))), qf[ks],
                     s[sb]);
    const LDS_AS char* rp = st + ln.k_rope + sb * (16 / Lds<64>::RPB) * Lds<64>::BLOCK;
#pragma unroll
    for (int ks = 16; ks < MlaCfg::KS; ++ks)
      s[sb] = mfma16(lds_read16(rp + Lds<64>::chunk_step(2 * (ks - 16))), qf[ks], s[sb]);
  }
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
  // V^T[d = 128 q4 + 16 db + (lane & 15)][keys 4q + e, 16 + 4q + e]
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const LDS_AS char* vp = st + q4 * MlaCfg::QUARTER + ln.v_off;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const u32x2 a1 = lds_read_tr16(vp + Lds<128>::chunk_step(db));
      const u32x2 a2 = lds_read_tr16(vp + Lds<128>::chunk_step(db) + (16 / Lds<128>::RPB) * Lds<128>::BLOCK);
      const u32x4 a = {a1[0], a1[1], a2[0], a2[1]};
      oacc[8 * q4 + db] = mfma16(a, pb, oacc[8 * q4 + db]);
    }
  }
}

// Wait until at most n of this wavefront's stage loads are in flight.
__device__ __forceinline__ void mla_wait_loads(int later_steps) {
  if (later_steps >= 2)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * MlaCfg::LOADS_PER_WAVE) : "memory");
  else if (later_steps == 1)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(MlaCfg::LOADS_PER_WAVE) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__global__ __launch_bounds__(kMlaThreads, 1) void mla_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(16))) char lds_raw[MlaCfg::LDS_BYTES];
  LDS_AS char* lds = (LDS_AS char*)lds_raw;
  const MlaItem it = ldc(p.items + blockIdx.x);
  const ReqInfo ri = ldc(p.req + it.req);
  const int lane = threadIdx.x & 63;
  const int w = uniform_i(threadIdx.x >> 6);
  const int H = p.H;
  const int n0 = kMlaRows * it.rg + 16 * w;  // first query row of this wavefront (H is a multiple of 16)
  const bool active = n0 < ri.qo * H;
  const int t = active ? n0 / H : 0;
  const int h = n0 % H + (lane & 15);
  const int lim = min(it.k1, p.causal ? ri.kv - ri.qo + t + 1 : ri.kv);

  MlaLanes ln;
  ln.q = lane >> 4;
  ln.k_lat = Lds<128>::off(lane & 15, (lane >> 4) & 1) + 32 * (lane >> 5);
  ln.k_rope = MlaCfg::ROPE + Lds<64>::off(lane & 15, (lane >> 4) & 1) + 32 * (lane >> 5);
  {
    const int j = lane & 15;
    ln.v_off = Lds<128>::off(4 * ln.q + (j >> 2), (j & 3) >> 1) + 8 * (j & 1);
  }

  u32x4 qf[MlaCfg::KS];
  {
    const uint16_t* qp = (const uint16_t*)p.q + ((int64_t)(ri.qo_start + t) * H + h) * kMlaWidth + 8 * ln.q;
#pragma unroll
    for (int ks = 0; ks < MlaCfg::KS; ++ks) qf[ks] = active ? *(const u32x4*)(qp + 32 * ks) : u32x4{0, 0, 0, 0};
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
    mla_wait_loads(nsteps - 1 - i);
    __syncthreads();  // step i visible to all; stage (i + 3) % 4 = (i - 1) % 4 read by all
    if (i + 3 < nsteps) {
      mla_issue(p, ri, it.k0 + 32 * (i + 3), pgA, pgB, w, lane, lds + ((i + 3) & 3) * MlaCfg::STAGE);
      pgA = mla_page(p, ri, it.k0 + 32 * (i + 4));
      pgB = mla_page(p, ri, it.k0 + 32 * (i + 4) + 16);
    }
    const int b = it.k0 + 32 * i;
    if (active && b < lim) mla_step(p, lds + (i & 3) * MlaCfg::STAGE, b, lim, ln, qf, m_ref, lacc, oacc);
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
    const int64_t slot = (int64_t)it.part * kMlaRows + 16 * w + (lane & 15);
    po = p.part_o + slot * kMlaLatent;
    if (ln.q == 0) p.part_lse[slot] = lse;
  }
#pragma unroll
  for (int db = 0; db < MlaCfg::DB; ++db) *(f32x4*)(po + 16 * db + 4 * ln.q) = oacc[db] * inv;
}

// Log-sum-exp merge of the partial results of one (request, row group), in
// part order (deterministic for a fixed plan).
__global__ __launch_bounds__(kMlaThreads) void mla_merge_kernel(MlaParams p) {
  const MlaMergeGroup mg = ldc(p.mg + blockIdx.x);
  const ReqInfo ri = ldc(p.req + mg.req);
  const int nrows = min(kMlaRows, ri.qo * p.H - kMlaRows * mg.rg);
  constexpr int D4 = kMlaLatent / 4;
  for (int idx = threadIdx.x; idx < nrows * D4; idx += kMlaThreads) {
    const int n = idx / D4, d4 = idx % D4;
    float mx = -INFINITY;
    for (int i = 0; i < mg.nparts; ++i) mx = fmaxf(mx, p.part_lse[(int64_t)(mg.part0 + i) * kMlaRows + n]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float sw = 0.f;
    for (int i = 0; i < mg.nparts; ++i) {
      const int64_t slot = (int64_t)(mg.part0 + i) * kMlaRows + n;
      const float li = p.part_lse[slot];
      const float wi = (li == -INFINITY) ? 0.f : __expf(li - mx);
      acc += *(const f32x4*)(p.part_o + slot * kMlaLatent + 4 * d4) * wi;
      sw += wi;
    }
    const int rn = kMlaRows * mg.rg + n;
    const int64_t row = (int64_t)(ri.qo_start + rn / p.H) * p.H + rn % p.H;
    *(f32x4*)(p.out + row * kMlaLatent + 4 * d4) = acc * (1.f / sw);
    if (d4 == 0 && p.lse) p.lse[row] = mx + __logf(sw);
  }
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
    hipLaunchKernelGGL(mla_kernel, dim3(p.n_items), dim3(kMlaThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.n_mg > 0) hipLaunchKernelGGL(mla_merge_kernel, dim3(p.n_mg), dim3(kMlaThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_mla_append(const MlaParams& p, void* pool, const void* rows_new, hipStream_t s) {
  if (p.total_rows > 0) hipLaunchKernelGGL(mla_append_kernel, dim3(p.total_rows), dim3(64), 0, s, p, pool, rows_new);
  return hipGetLastError();
}

}  // namespace pdk
