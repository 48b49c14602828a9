// MLA decode with 32 query rows per wavefront (32x32x16 bf16 products), for
// requests whose tokens bring 128 query heads.  What is computed is the same
// as in mla.hip (Perplexity post "Disaggregated prefill and decode", section
// "DeepSeek-R1" under "Disaggregated Deployments": absorbed-form attention
// with one latent KV head, key = the whole 576-entry cache row, value = its
// first 512 entries).
//
// A block is 4 wavefronts (one per SIMD) over the 128 heads of one token and
// one key chunk.  Against 16-row wavefronts, each score operand read from LDS
// serves 32 query rows instead of 16, in the 32-row lane pattern that reads
// LDS without bank conflicts, so a 32-key step reads half the LDS bytes per
// flop.  The price is registers: O^T of 32 rows x 512 entries is 256 fp32 per
// lane and Q^T 144, so one wavefront per SIMD, with O^T in the accumulation
// registers (see AccTile).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "mla_common.hpp"
#include "pd_internal.hpp"

namespace pdk {
namespace {

struct WideCfg {
  static constexpr int ROWS = 32;              // query rows per wavefront
  static constexpr int WAVES = 4;
  static constexpr int KS = kMlaWidth / 16;    // 16-entry k-steps of S^T: 32 latent + 4 rotary
  static constexpr int KS_LAT = kMlaLatent / 16;
  static constexpr int DB = kMlaLatent / 32;   // 32-entry blocks of O^T
  static constexpr int SRING = 6;              // score-operand reads in flight
  static constexpr int PVAHEAD = 3;            // value products whose reads are in flight
};
static_assert(WideCfg::ROWS * WideCfg::WAVES == 128, "one token of 128 heads per block");

// O^T lives only in the accumulation registers, outside the compiler's
// view: tile db is a[16 db .. 16 db + 15], named literally in the inline asm
// that zeroes, accumulates, scales and reads it, and listed as clobbered
// there (so the kernel's register count covers it and the compiler keeps
// nothing of its own in those registers across these statements).  Any
// O^T value held in a C++ variable lets the register allocator split the
// tiles between the register files and spill Q^T instead.
//   zero():  acc = 0 (accumulation-register writes of the constant);
//   mac():   acc += A B on a 32x32x16 bf16 product;
//   scale(): acc *= x, one register at a time through a VGPR;
//   read():  the 16 values, for the epilogue.
// The hazard recognizer does not see these dependences, so the callers
// provide the wait states: 2 after a VALU write of A or B (wide_pv_pipe), 32
// between a product and a VALU access of its accumulator (acc_settle; the
// 8-pass product needs 11), and 8 between zero() or scale() and the next
// product.  A and B are never assembled by VALU moves right before mac():
// the operand reads land in contiguous registers and P^T is written well
// before the first product (checked in the generated code).
template <int DB>
struct AccTile;

#define WIDE_RS(n) "v_accvgpr_read_b32 %0, a" #n "\n\tv_mul_f32_e32 %0, %1, %0\n\tv_accvgpr_write_b32 a" #n ", %0\n\t"
#define WIDE_Z(n) "v_accvgpr_write_b32 a" #n ", 0\n\t"
#define WIDE_RD(i, n) "v_accvgpr_read_b32 %" #i ", a" #n "\n\t"
#define WIDE_ACC_TILE(DB, REG, e0, e1, e2, e3, e4, e5, e6, e7, e8, e9, e10, e11, e12, e13, e14, e15)              \
  template <>                                                                                                    \
  struct AccTile<DB> {                                                                                           \
    static __device__ __forceinline__ void zero() {                                                              \
      asm volatile(WIDE_Z(e0) WIDE_Z(e1) WIDE_Z(e2) WIDE_Z(e3) WIDE_Z(e4) WIDE_Z(e5) WIDE_Z(e6) WIDE_Z(e7)     \
                       WIDE_Z(e8) WIDE_Z(e9) WIDE_Z(e10) WIDE_Z(e11) WIDE_Z(e12) WIDE_Z(e13) WIDE_Z(e14)         \
                           WIDE_Z(e15)                                                                           \
                   ::: "a" #e0, "a" #e1, "a" #e2, "a" #e3, "a" #e4, "a" #e5, "a" #e6, "a" #e7, "a" #e8, "a" #e9,  \
                     "a" #e10, "a" #e11, "a" #e12, "a" #e13, "a" #e14, "a" #e15);                                \
    }                                                                                                            \
    static __device__ __forceinline__ void mac(u32x4 a, u32x4 b) {                                               \
      asm volatile("v_mfma_f32_32x32x16_bf16 " REG ", %0, %1, " REG ::"v"(a), "v"(b)                             \
                   : "a" #e0, "a" #e1, "a" #e2, "a" #e3, "a" #e4, "a" #e5, "a" #e6, "a" #e7, "a" #e8, "a" #e9,    \
                     "a" #e10, "a" #e11, "a" #e12, "a" #e13, "a" #e14, "a" #e15);                                \
    }                                                                                                            \
    static __device__ __forceinline__ void scale(float x) {                                                      \
      float t;                                                                                                   \
      asm volatile(WIDE_RS(e0) WIDE_RS(e1) WIDE_RS(e2) WIDE_RS(e3) WIDE_RS(e4) WIDE_RS(e5) WIDE_RS(e6)          \
                       WIDE_RS(e7) WIDE_RS(e8) WIDE_RS(e9) WIDE_RS(e10) WIDE_RS(e11) WIDE_RS(e12) WIDE_RS(e13)   \
                           WIDE_RS(e14) WIDE_RS(e15)                                                             \
                   : "=&v"(t)                                                                                    \
                   : "v"(x)                                                                                      \
                   : "a" #e0, "a" #e1, "a" #e2, "a" #e3, "a" #e4, "a" #e5, "a" #e6, "a" #e7, "a" #e8, "a" #e9,    \
                     "a" #e10, "a" #e11, "a" #e12, "a" #e13, "a" #e14, "a" #e15);                                \
    }                                                                                                            \
    static __device__ __forceinline__ void read(float (&o)[16]) {                                                \
      asm volatile(WIDE_RD(0, e0) WIDE_RD(1, e1) WIDE_RD(2, e2) WIDE_RD(3, e3) WIDE_RD(4, e4) WIDE_RD(5, e5)     \
                       WIDE_RD(6, e6) WIDE_RD(7, e7) WIDE_RD(8, e8) WIDE_RD(9, e9) WIDE_RD(10, e10)              \
                           WIDE_RD(11, e11) WIDE_RD(12, e12) WIDE_RD(13, e13) WIDE_RD(14, e14) WIDE_RD(15, e15)  \
                   : "=v"(o[0]), "=v"(o[1]), "=v"(o[2]), "=v"(o[3]), "=v"(o[4]), "=v"(o[5]), "=v"(o[6]),         \
                     "=v"(o[7]), "=v"(o[8]), "=v"(o[9]), "=v"(o[10]), "=v"(o[11]), "=v"(o[12]), "=v"(o[13]),     \
                     "=v"(o[14]), "=v"(o[15]));                                                                  \
    }                                                                                                            \
  };
WIDE_ACC_TILE(0, "a[0:15]", 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15)
WIDE_ACC_TILE(1, "a[16:31]", 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 26, 27, 28, 29, 30, 31)
WIDE_ACC_TILE(2, "a[32:47]", 32, 33, 34, 35, 36, 37, 38, 39, 40, 41, 42, 43, 44, 45, 46, 47)
WIDE_ACC_TILE(3, "a[48:63]", 48, 49, 50, 51, 52, 53, 54, 55, 56, 57, 58, 59, 60, 61, 62, 63)
WIDE_ACC_TILE(4, "a[64:79]", 64, 65, 66, 67, 68, 69, 70, 71, 72, 73, 74, 75, 76, 77, 78, 79)
WIDE_ACC_TILE(5, "a[80:95]", 80, 81, 82, 83, 84, 85, 86, 87, 88, 89, 90, 91, 92, 93, 94, 95)
WIDE_ACC_TILE(6, "a[96:111]", 96, 97, 98, 99, 100, 101, 102, 103, 104, 105, 106, 107, 108, 109, 110, 111)
WIDE_ACC_TILE(7, "a[112:127]", 112, 113, 114, 115, 116, 117, 118, 119, 120, 121, 122, 123, 124, 125, 126, 127)
WIDE_ACC_TILE(8, "a[128:143]", 128, 129, 130, 131, 132, 133, 134, 135, 136, 137, 138, 139, 140, 141, 142, 143)
WIDE_ACC_TILE(9, "a[144:159]", 144, 145, 146, 147, 148, 149, 150, 151, 152, 153, 154, 155, 156, 157, 158, 159)
WIDE_ACC_TILE(10, "a[160:175]", 160, 161, 162, 163, 164, 165, 166, 167, 168, 169, 170, 171, 172, 173, 174, 175)
WIDE_ACC_TILE(11, "a[176:191]", 176, 177, 178, 179, 180, 181, 182, 183, 184, 185, 186, 187, 188, 189, 190, 191)
WIDE_ACC_TILE(12, "a[192:207]", 192, 193, 194, 195, 196, 197, 198, 199, 200, 201, 202, 203, 204, 205, 206, 207)
WIDE_ACC_TILE(13, "a[208:223]", 208, 209, 210, 211, 212, 213, 214, 215, 216, 217, 218, 219, 220, 221, 222, 223)
WIDE_ACC_TILE(14, "a[224:239]", 224, 225, 226, 227, 228, 229, 230, 231, 232, 233, 234, 235, 236, 237, 238, 239)
WIDE_ACC_TILE(15, "a[240:255]", 240, 241, 242, 243, 244, 245, 246, 247, 248, 249, 250, 251, 252, 253, 254, 255)
#undef WIDE_ACC_TILE
#undef WIDE_RD
#undef WIDE_Z
#undef WIDE_RS

__device__ __forceinline__ void acc_settle() { asm volatile("s_nop 15\n\ts_nop 15" ::: "memory"); }

template <int DB>
__device__ __forceinline__ void acc_zero_all() {
  AccTile<DB>::zero();
  if constexpr (DB + 1 < 16) acc_zero_all<DB + 1>();
}
template <int DB>
__device__ __forceinline__ void acc_scale_all(float x) {
  AccTile<DB>::scale(x);
  if constexpr (DB + 1 < 16) acc_scale_all<DB + 1>(x);
}

// Epilogue: O^T[32 db + 8 g + 4 h + e][row] (register 4 g + e of tile db)
// times `inv` to po[32 db + 8 g + 4 h + e].
template <int DB>
__device__ __forceinline__ void acc_store_all(float* po, int h2, float inv) {
  float o[16];
  AccTile<DB>::read(o);
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *(f32x4*)(po + 32 * DB + 8 * g + 4 * h2) = f32x4{o[4 * g], o[4 * g + 1], o[4 * g + 2], o[4 * g + 3]} * inv;
  if constexpr (DB + 1 < 16) acc_store_all<DB + 1>(po, h2, inv);
}

// Score operand read r (k-step r of S^T): lane (key i = lane % 32, half h =
// lane / 32) reads entries 16 r + 8 h .. + 7 of key i.  Offset from the
// lane's latent (r < 32) or rotary base.
template <int R>
constexpr int wide_k_off() {
  return R < WideCfg::KS_LAT ? (R / 8) * MlaCfg::QUARTER + Lds<128>::chunk_step(R % 8)
                             : Lds<64>::chunk_step(R - WideCfg::KS_LAT);
}

// LOADS: the wavefront's 9 direct loads of a later full step are issued
// between the score products (load j after product 4 j + 1) instead of all
// at once after the barrier: the products form one dependent chain, whose
// gaps take the issue, and the CU's load path moves the step's 38 KB while
// the products run.
template <int R, bool LOADS>
__device__ __forceinline__ void wide_s_pipe(u32x4 (&kf)[WideCfg::SRING], f32x16& s, const u32x4 (&qf)[WideCfg::KS],
                                            const LDS_AS char* kl, const LDS_AS char* kr, const MlaFullStep& nx,
                                            int w, int lane) {
  constexpr int NR = WideCfg::KS, RING = WideCfg::SRING;
  if constexpr (R >= RING) {
    constexpr int i = R - RING;
    lgkm_wait_for<(NR - 1 - i < RING - 1) ? NR - 1 - i : RING - 1>(kf[i % RING]);
    s = mfma32(kf[i % RING], qf[i], s);
    if constexpr (LOADS && i % 4 == 1 && i / 4 < MlaCfg::LOADS_PER_WAVE) mla_issue_full<i / 4>(nx, w, lane);
  }
  if constexpr (R < NR) kf[R % RING] = lds_read16_asm<wide_k_off<R>()>(R < WideCfg::KS_LAT ? kl : kr);
  if constexpr (R + 1 < NR + RING) wide_s_pipe<R + 1, LOADS>(kf, s, qf, kl, kr, nx, w, lane);
}
static_assert(4 * (MlaCfg::LOADS_PER_WAVE - 1) + 1 < WideCfg::KS, "every interleaved load has a product before it");

// Value product m = 16 kk + db: O^T[32 db ..][rows] += V^T[32 db ..][keys of
// k-step kk] P^T[keys of kk][rows].  Lane (entry 32 db + lane % 32, half h)
// takes keys 16 kk + 4 h + e and 16 kk + 8 + 4 h + e (e = 0..3), two
// transposed reads 8 keys apart; the score layout puts the same keys in the
// lane's P^T operand.
template <int M, int H>
constexpr int wide_v_off() {
  constexpr int kk = M / WideCfg::DB, db = M % WideCfg::DB;
  return (db / 4) * MlaCfg::QUARTER + (16 * kk / Lds<128>::RPB) * Lds<128>::BLOCK + Lds<128>::chunk_step(2 * (db % 4)) +
         H * (8 / Lds<128>::RPB) * Lds<128>::BLOCK;
}

template <int M>
__device__ __forceinline__ void wide_pv_issue(u32x2 (&va)[WideCfg::PVAHEAD + 1][2], const LDS_AS char* vp) {
  va[M % (WideCfg::PVAHEAD + 1)][0] = lds_read_tr16_asm<wide_v_off<M, 0>()>(vp);
  va[M % (WideCfg::PVAHEAD + 1)][1] = lds_read_tr16_asm<wide_v_off<M, 1>()>(vp);
}

template <int M>
__device__ __forceinline__ void wide_pv_prologue(u32x2 (&va)[WideCfg::PVAHEAD + 1][2], const LDS_AS char* vp) {
  wide_pv_issue<M>(va, vp);
  if constexpr (M + 1 < WideCfg::PVAHEAD) wide_pv_prologue<M + 1>(va, vp);
}

template <int M>
__device__ __forceinline__ void wide_pv_pipe(u32x2 (&va)[WideCfg::PVAHEAD + 1][2], const LDS_AS char* vp,
                                             const u32x4 (&pb)[2]) {
  constexpr int N = 2 * WideCfg::DB, AHEAD = WideCfg::PVAHEAD, RING = AHEAD + 1;
  if constexpr (M + AHEAD < N) wide_pv_issue<M + AHEAD>(va, vp);
  constexpr int LATER = 2 * ((N - 1 - M) < AHEAD ? (N - 1 - M) : AHEAD);
  static_assert(LATER < 16, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(va[M % RING][0]), "+v"(va[M % RING][1]) : "n"(LATER));
  const u32x4 a = {va[M % RING][0][0], va[M % RING][0][1], va[M % RING][1][0], va[M % RING][1][1]};
  if constexpr (M == 0) asm volatile("s_nop 1" ::: "memory");  // P^T was written by the VALU
  AccTile<M % WideCfg::DB>::mac(a, pb[M / WideCfg::DB]);
  if constexpr (M + 1 < N) wide_pv_pipe<M + 1>(va, vp, pb);
}

// P = exp2(s c - m c) of one step's scores, packed to bf16 in the key order
// of the value operand (pb[kk] holds keys 16 kk + 4 h + e, 16 kk + 8 + 4 h +
// e); returns this lane's sum of the rounded P (v_dot2 against bf16 ones).
// The pairs are summed from a plain array: summed from elements of the
// u32x4 vectors, this compiler reads element 0 four times.
__device__ __forceinline__ float wide_exp(const f32x16& s, float cl, float mc, u32x4 (&pb)[2]) {
  uint32_t pk[8];
  float t[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pk[i] = pack_bf16(fast_exp2(__builtin_fmaf(s[2 * i], cl, -mc)), fast_exp2(__builtin_fmaf(s[2 * i + 1], cl, -mc)));
    t[i / 4] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]),
                                               __builtin_bit_cast(bf16x2, kBf16OnesPair), t[i / 4], false);
  }
  pb[0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
  pb[1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
  return t[0] + t[1];
}

// One 32-key step of a wavefront's 32 rows from stage `st`.  S^T = K Q^T on
// one 32x32 accumulator: S^T[key 8 g + 4 h + e][row lane % 32] lands in
// s[4 g + e].  Then the speculative online softmax per row (the running
// reference max m_ref changes only when some weight would reach 2^64), and
// O^T += V^T P^T.
template <bool LOADS>
__device__ __forceinline__ void wide_step(const MlaParams& p, const LDS_AS char* st, int b, int lim, int h2,
                                          int k_lat, int k_rope, int v_off, const u32x4 (&qf)[WideCfg::KS],
                                          float& m_ref, float& lsum, const MlaFullStep& nx, int w, int lane) {
  const float cl = p.c_log2;
  f32x16 s = {};
  {
    u32x4 kf[WideCfg::SRING];
    wide_s_pipe<0, LOADS>(kf, s, qf, st + k_lat, st + k_rope, nx, w, lane);
  }
  u32x2 va[WideCfg::PVAHEAD + 1][2];
  const LDS_AS char* vp = st + v_off;
  wide_pv_prologue<0>(va, vp);  // the first value reads land during the softmax
  if (b + 32 > lim) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (b + 8 * (r >> 2) + 4 * h2 + (r & 3) >= lim) s[r] = -INFINITY;
  }
  u32x4 pb[2];
  float ts = wide_exp(s, cl, m_ref * cl, pb);
  // Some weight reached 2^64, or is inf / NaN (the first step, m_ref = -inf):
  // this lane's sum shows it.  Lanes l and l ^ 32 hold the same row.
  if (wave_any(!(ts < 0x1p64f))) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = max_x32(mx);
    const float m_new = fmaxf(m_ref, mx);
    if (m_new != -INFINITY) {  // a row with no visible key yet keeps m_ref = -inf
      if (m_ref != -INFINITY) {  // nothing accumulated before the first visible key
        const float alpha = fast_exp2((m_ref - m_new) * cl);
        lsum *= alpha;
        acc_settle();
        acc_scale_all<0>(alpha);
        asm volatile("s_nop 7" ::: "memory");  // accumulation-register writes before the next product reads them
      }
      m_ref = m_new;
    }
    const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * cl;
    ts = wide_exp(s, cl, mc, pb);
  }
  lsum += ts;
  wide_pv_pipe<0>(va, vp, pb);
}

__global__ __launch_bounds__(256, 1) void mla_wide_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(16))) char lds_raw[MlaCfg::LDS_BYTES];
  LDS_AS char* lds = (LDS_AS char*)lds_raw;
  const MlaItem it = ldc(p.items + blockIdx.x);
  const ReqInfo ri = ldc(p.req + it.req);
  const int lane = threadIdx.x & 63;
  const int w = uniform_i(threadIdx.x >> 6);
  const int H = p.H;                             // 128: row group rg is token rg
  const int t = it.rg;
  const int h = 32 * w + (lane & 31);
  const int h2 = lane >> 5;
  const int lim = min(it.k1, p.causal ? ri.kv - ri.qo + t + 1 : ri.kv);

  // Score operand: key lane % 32, entries 8 h2 .. of each 16-entry k-step.
  const int k_lat = Lds<128>::off(lane & 31, h2);
  const int k_rope = MlaCfg::ROPE + Lds<64>::off(lane & 31, h2);
  int v_off;
  {
    const int j = lane & 15, dhalf = (lane >> 4) & 1;
    v_off = Lds<128>::off(4 * h2 + (j >> 2), 2 * dhalf + ((j & 3) >> 1)) + 8 * (j & 1);
  }

  // Q^T: row h of token t, entries 16 ks + 8 h2 .. + 7 (compiler-tracked
  // loads; the explicit wait below completes them before the step loop).
  u32x4 qf[WideCfg::KS];
  {
    const uint16_t* qp = (const uint16_t*)p.q + ((int64_t)(ri.qo_start + t) * H + h) * kMlaWidth + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < WideCfg::KS; ++ks) qf[ks] = *(const u32x4*)(qp + 16 * ks);
  }
  acc_zero_all<0>();
  asm volatile("s_nop 7" ::: "memory");
  float m_ref = -INFINITY, lsum = 0.f;

  const int nsteps = (it.k1 - it.k0 + 31) >> 5;
  mla_issue(p, ri, it.k0, mla_page(p, ri, it.k0), mla_page(p, ri, it.k0 + 16), w, lane, lds);
  // vmcnt(0): Q and step 0 are in.  Written as the builtin so that the
  // compiler's wait insertion knows Q has landed and adds no wait for it
  // inside the loop (where it would drain the stage loads in flight).
  __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
  for (int s = 1; s < 3; ++s)
    if (s < nsteps) {
      const int b = it.k0 + 32 * s;
      mla_issue(p, ri, b, mla_page(p, ri, b), mla_page(p, ri, b + 16), w, lane, lds + s * MlaCfg::STAGE);
    }
  int pgA = mla_page(p, ri, it.k0 + 96), pgB = mla_page(p, ri, it.k0 + 112);  // step 3
  for (int i = 0; i < nsteps; ++i) {
    mla_wait_loads<MlaCfg::LOADS_PER_WAVE>(nsteps - 1 - i);
    __syncthreads();  // step i visible to all; stage (i + 3) % 4 = (i - 1) % 4 read by all
    const int b = it.k0 + 32 * i;
    const int b3 = b + 96;  // step i + 3, loaded during this step
    const bool compute = b < lim;
    // a full step i + 3 is loaded between this step's score products; a
    // partial one, or any step when this one computes nothing, at once
    const bool spread = compute && i + 3 < nsteps && b3 + 32 <= ri.kv;
    MlaFullStep nx{};
    if (spread) {
      nx = mla_full_step(p, b3, pgA, pgB, lds + ((i + 3) & 3) * MlaCfg::STAGE);
    } else if (i + 3 < nsteps) {
      mla_issue(p, ri, b3, pgA, pgB, w, lane, lds + ((i + 3) & 3) * MlaCfg::STAGE);
    }
    if (i + 3 < nsteps) {
      pgA = mla_page(p, ri, b3 + 32);
      pgB = mla_page(p, ri, b3 + 48);
    }
    if (spread)
      wide_step<true>(p, lds + (i & 3) * MlaCfg::STAGE, b, lim, h2, k_lat, k_rope, v_off, qf, m_ref, lsum, nx, w,
                      lane);
    else if (compute)
      wide_step<false>(p, lds + (i & 3) * MlaCfg::STAGE, b, lim, h2, k_lat, k_rope, v_off, qf, m_ref, lsum, nx, w,
                       lane);
  }

  acc_settle();
  const float l_tot = sum_x32(lsum);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? m_ref * p.sm_scale + __logf(l_tot) : -INFINITY;
  float* po;
  if (it.part < 0) {
    const int64_t row = (int64_t)(ri.qo_start + t) * H + h;
    po = p.out + row * kMlaLatent;
    if (h2 == 0 && p.lse) p.lse[row] = lse;
  } else {
    const int64_t slot = (int64_t)it.part * 128 + h;
    po = p.part_o + slot * kMlaLatent;
    if (h2 == 0) p.part_lse[slot] = lse;
  }
  acc_store_all<0>(po, h2, inv);
}

}  // namespace

hipError_t launch_mla_wide(const MlaParams& p, hipStream_t s) {
  hipLaunchKernelGGL(mla_wide_kernel, dim3(p.n_items), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pdk
