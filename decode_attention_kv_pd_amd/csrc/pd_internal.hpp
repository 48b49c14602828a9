// Internal types shared by the host runtime (api.cpp) and the HIP kernels
// (kernels.hip).  Not part of the public ABI (include/pd_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdk {

// Per-request row of the device tables.
struct ReqInfo {
  int32_t qo_start;    // first query row of the request in q / out
  int32_t qo;          // new query rows
  int32_t kv;          // cached tokens including the new ones
  int32_t page_start;  // first entry of the request in page_indices
};

// A causal query tile of a prefill request, computed by one 512-thread block
// on bf16 MFMA: tokens [q0, q0 + nq) of request `req` times the g query heads
// of KV head `hk` (row n of the tile = token q0 + n / g, head hk * g + n % g),
// over keys [0, kv_end).  Written straight to out / lse.
struct PrefillItem {
  int32_t req, hk, q0, nq, kv_end, rsv0, rsv1, rsv2;
};

// A split-KV decode unit, computed by one wavefront: query rows [c0, c0 + 16
// ncg) (clipped to qo * g <= kMaxDecodeRows) of (request, KV head) over keys
// [k0, k1); row n is token n / g, head hk * g + n % g.  Row c0 + i of the
// unit writes its partial result (normalised o and its log-sum-exp) to
// partial row part + i.  pair = 1: the unit is one half (c0 = 0 or 32) of a
// group of more than 32 rows whose two wavefronts, adjacent slots of one
// block running the same units, share their V stages.
struct DecodeItem {
  int32_t req, hk, k0, k1, part, c0, ncg, pair;
};

// What the attention kernel reads for one decode unit: the unit and its
// request's row, in one 48-byte record (one dependent load fewer).
struct DecodeUnit {
  DecodeItem it;
  ReqInfo ri;
};

// One block of the attention launch, 64 bytes, indexed by the block id (so
// that a block's first load depends on nothing else).
//   v >= 0: prefill tile v; w[0..7] = the tile, w[8..11] = its request's row.
//   v < 0:  decode block -v - 1; w[0..8] = the queue offsets of its eight
//           wavefront slots (slot k runs units [w[k], w[k + 1])), w[9] = 1
//           when its first slots hold paired queues.
struct LaunchRec {
  int32_t v;
  int32_t w[15];
};
static_assert(sizeof(PrefillItem) == 32 && sizeof(ReqInfo) == 16, "launch record layout");

// One (request, KV head) decode row group of rows = qo * g: key chunk i's
// partial result for row n sits in partial row part0 + i * rows + n; nparts
// is the number of chunks.  The merge kernel combines the chunks into
// out / lse.
struct MergeGroup {
  int32_t req, hk, part0, nparts;
};

// What the merge kernel reads for one row group, 32 bytes: its partial rows
// (chunk i's row n at part0 + i * nrows + n) and where its rows go (row n:
// token qo_start + n / g, head hk * g + n % g), so that the group's first
// loads depend on this record only.
struct MergeRec {
  int32_t part0, nparts, nrows, qo_start, hk, rsv0, rsv1, rsv2;
};

constexpr int kBlockThreads = 256;  // append, pack, merge and the fp32 kernel
constexpr int kAttnWaves = 8;       // wavefronts per block of the bf16 attention kernel
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kPrefillRows = 32 * kAttnWaves;  // query rows per prefill tile (32 per wavefront)
constexpr int kDecodeCols = 16;     // query rows of a decode column group (16x16x32 MFMA N)
constexpr int kMaxDecodeRows = 64;  // rows of a (request, KV head) the decode role takes
constexpr int kWavesPerBlock = kAttnWaves;  // decode queues per block (both attention kernels)

struct AttnParams {
  const void* q;
  const void* pool;
  float* out;
  float* lse;  // may be null
  const int32_t* qo_indptr;
  const ReqInfo* req;
  const int32_t* page_indices;
  const LaunchRec* launch;  // one record per block of the attention launch
  const DecodeUnit* du;     // decode units in queue order
  const MergeRec* mg;
  float* part_o;    // [partial rows][D]
  float* part_lse;  // [partial rows]
  int32_t n_pf, n_du, n_mg, B;
  int32_t n_blocks;  // blocks of the attention launch
  int32_t prefill4;  // prefill-only launch of 128-row tiles in 4-wavefront blocks
  int32_t H_q, H_kv, g, ps;
  int32_t ps_shift;  // log2(ps)
  int32_t D, causal;
  float sm_scale;
  float c_log2;        // sm_scale * log2(e)
  int64_t page_elems;  // elements of one page: 2 * H_kv * ps * D
};

struct AppendParams {
  void* pool;
  const void* k_new;
  const void* v_new;
  const int2* rowpos;        // [total_rows]: (page id, slot) of each new row
  int32_t total_rows, H_kv, ps, D, elt;
  int32_t rows_per_block;
};

// Page transfers between a pool (or L layer pools) and a buffer
// [L][n][2][seg_bytes]: for each listed page, the slice of seg_bytes at
// seg_off in its K half and in its V half (the whole page when seg_off = 0
// and seg_bytes = half_bytes).
struct XferParams {
  char* buf;
  void* pool0;               // the pool when layers is null (L = 1)
  void* const* layers;       // device array of L pool pointers, or null
  const int32_t* page_ids;   // device, n entries
  uint32_t* done;            // device, L per-layer block counters (zero between calls), or null
  uint32_t* progress;        // device-accessible, L per-layer completion counters, or null
  int64_t page_bytes;        // 2 * half_bytes
  int64_t half_bytes;        // H_kv * ps * D * elt
  int64_t seg_off;           // h0 * ps * D * elt
  int64_t seg_bytes;         // (h1 - h0) * ps * D * elt, a multiple of 16
  int32_t n, L;
  int32_t to_buffer;         // 1: pool -> buffer (pack), 0: buffer -> pool (unpack)
};

// ---- MLA decode over a latent cache (pool [pages][ps][kMlaWidth] bf16: per
// token the kMlaLatent latent entries, then the kMlaRope rotary-key entries).
constexpr int kMlaLatent = 512;
constexpr int kMlaRope = 64;
constexpr int kMlaWidth = kMlaLatent + kMlaRope;
// Blocks of the MLA kernels have 4 wavefronts of 16 query rows (64 rows,
// mla.hip) or 32 query rows (128 rows, requests of 128 heads, mla_wide.hip);
// a plan uses one width, MlaParams::rows.
constexpr int kMlaMergeWaves = 4;              // wavefronts per block of the merge kernel

// One block of the MLA kernel: query rows [R rg, R rg + R) of request `req`
// (R = MlaParams::rows; row n = token n / H, head n % H) over keys [k0, k1).
// part >= 0: the partial result goes to slot `part`; part < 0: straight to
// out / lse.
struct MlaItem {
  int32_t req, rg, k0, k1, part, rsv0, rsv1, rsv2;
};

// Partial results [part0, part0 + nparts) of one (request, row group).
struct MlaMergeGroup {
  int32_t req, rg, part0, nparts;
};

// What the MLA merge kernel reads for one (request, row group), 32 bytes:
// its partial slots and where the group's rows go (row R rg + n of the
// request, if below qo_rows = qo * H, is token qo_start + that row / H), so
// that its first loads depend on this record only.
struct MlaMergeRec {
  int32_t part0, nparts, rg, qo_rows, qo_start, rsv0, rsv1, rsv2;
};

struct MlaParams {
  const void* q;      // [rows][H][kMlaWidth] bf16
  const void* pool;   // [pages][ps][kMlaWidth] bf16
  float* out;         // [rows][H][kMlaLatent]
  float* lse;         // [rows][H], may be null
  const int32_t* qo_indptr;
  const ReqInfo* req;
  const int32_t* page_indices;
  const MlaItem* items;
  const MlaMergeRec* mg;
  float* part_o;      // [n_parts][rows][kMlaLatent]
  float* part_lse;    // [n_parts][rows]
  int32_t n_items, n_mg, B, total_rows;
  int32_t waves, rows;  // wavefronts per block (4); query rows per block (64, or 128 for 128 heads)
  int32_t H, ps, ps_shift, causal;
  float sm_scale;
  float c_log2;       // sm_scale * log2(e)
};

hipError_t launch_mla(const MlaParams& p, hipStream_t s);
hipError_t launch_mla_wide(const MlaParams& p, hipStream_t s);  // attention only: 128-row blocks
hipError_t launch_mla_append(const MlaParams& p, void* pool, const void* rows_new, hipStream_t s);

hipError_t launch_attention(const AttnParams& p, int dtype, hipStream_t s);
hipError_t launch_merge(const AttnParams& p, hipStream_t s);
hipError_t launch_append(const AppendParams& p, hipStream_t s);
// Single-layer transfers of at most kXferInlineIds pages take their page ids
// from host_ids in the kernel arguments (p.page_ids unused); otherwise
// p.page_ids is a device array.  Multi-layer transfers (p.done set) always
// read p.page_ids.
constexpr int kXferInlineIds = 896;
hipError_t launch_xfer(const XferParams& p, const int32_t* host_ids, hipStream_t s);

}  // namespace pdk
