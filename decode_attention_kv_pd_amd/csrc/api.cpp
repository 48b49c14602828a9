// Host runtime of libpd_attn.so: argument checks, the planner, the device
// workspace image, and the C entry points declared in include/pd_attn.h.
//
// The planner splits one step of a ragged batch (Perplexity, "Disaggregated
// prefill and decode", section "Prefill vs Decode performance": prefill and
// decode requests batched together, attention parallel over requests and
// kv_len) into
//   * prefill tiles: up to 256 query rows (tokens x the g query heads of one
//     KV head) over the tile's causal key range, one 512-thread block each,
//     ordered so that the tiles of one (request, KV head) share an XCD and
//     longest tiles start first;
//   * decode units: the <= 16 query rows of one (request, KV head) over a
//     chunk of keys, one wavefront each, the request's kv_len cut into equal
//     chunks so that the units keep every CU busy;
//   * merge groups: the chunks of one (request, KV head).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "pd_attn.h"
#include "pd_internal.hpp"
#include "host_internal.hpp"

namespace {

thread_local std::string g_last_error;

pd_status fail(pd_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

constexpr int kNumXcd = 8;  // MI355X: 8 XCDs, workgroups dispatched round robin
constexpr int32_t kMaxXferLayers = 4096;  // layers of one multi-layer transfer (grid z)

pd_status check_desc(const pd_attn_desc* d) {
  if (!d) return fail(PD_ERR_INVALID_ARG, "desc is NULL");
  if (d->num_qo_heads < 1 || d->num_kv_heads < 1)
    return fail(PD_ERR_INVALID_ARG, "head counts must be >= 1");
  if (d->num_qo_heads % d->num_kv_heads != 0)
    return fail(PD_ERR_INVALID_ARG, "num_qo_heads must be a multiple of num_kv_heads");
  if (d->num_qo_heads / d->num_kv_heads > pdk::kPrefillRows)
    return fail(PD_ERR_UNSUPPORTED, "query heads per KV head must be <= 256");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PD_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d->page_size != 16 && d->page_size != 32 && d->page_size != 64 && d->page_size != 128)
    return fail(PD_ERR_UNSUPPORTED, "page_size must be 16, 32, 64 or 128");
  if (d->dtype != PD_F32 && d->dtype != PD_BF16)
    return fail(PD_ERR_UNSUPPORTED, "dtype must be PD_F32 or PD_BF16");
  if (d->causal != 0 && d->causal != 1) return fail(PD_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!std::isfinite(d->sm_scale) || !(d->sm_scale > 0.f))
    return fail(PD_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  return PD_OK;
}

int elt_bytes(const pd_attn_desc* d) { return d->dtype == PD_F32 ? 4 : 2; }

pd_status check_mla_desc(const pd_mla_desc* d) {
  if (!d) return fail(PD_ERR_INVALID_ARG, "desc is NULL");
  if (d->kv_lora_rank != pdk::kMlaLatent || d->qk_rope_dim != pdk::kMlaRope)
    return fail(PD_ERR_UNSUPPORTED, "kv_lora_rank must be 512 and qk_rope_dim 64");
  if (d->num_qo_heads < 16 || d->num_qo_heads > 128 || d->num_qo_heads % 16 != 0)
    return fail(PD_ERR_UNSUPPORTED, "num_qo_heads must be a multiple of 16 in [16, 128]");
  if (d->page_size != 16 && d->page_size != 32 && d->page_size != 64 && d->page_size != 128)
    return fail(PD_ERR_UNSUPPORTED, "page_size must be 16, 32, 64 or 128");
  if (d->dtype != PD_BF16) return fail(PD_ERR_UNSUPPORTED, "dtype must be PD_BF16");
  if (d->causal != 0 && d->causal != 1) return fail(PD_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!std::isfinite(d->sm_scale) || !(d->sm_scale > 0.f))
    return fail(PD_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  return PD_OK;
}

int64_t mla_page_bytes_of(const pd_mla_desc* d) {
  return (int64_t)d->page_size * (d->kv_lora_rank + d->qk_rope_dim) * 2;
}

int64_t page_bytes_of(const pd_attn_desc* d) {
  return 2LL * d->num_kv_heads * d->page_size * d->head_dim * elt_bytes(d);
}

}  // namespace

struct pd_plan_s {
  pd_attn_desc desc{};
  int32_t B = 0, g = 1, total_rows = 0, chunk_keys = 0, n_parts = 0;
  std::vector<int32_t> qo_indptr;
  std::vector<pdk::ReqInfo> req;
  std::vector<int32_t> pages;
  std::vector<pdk::PrefillItem> pf;
  std::vector<pdk::DecodeItem> du;  // in queue order
  std::vector<int32_t> dq;          // wave slot s runs units [dq[s], dq[s + 1])
  std::vector<pdk::MergeGroup> mg;
  std::vector<int32_t> block_map;  // attention launch order
  bool prefill4 = false;           // 128-row tiles in 4-wavefront blocks (prefill-only launches)
  size_t off_qo = 0, off_req = 0, off_pages = 0, off_launch = 0, off_du = 0, off_mg = 0;
  size_t off_rows = 0;  // (page, slot) of each new row, for the append
  size_t meta_bytes = 0, off_part_o = 0, off_part_lse = 0, ws_bytes = 0;
  int64_t prefill_flops = 0, decode_bytes = 0;
  std::vector<char> blob;  // host image of the workspace tables
  // latent-cache (MLA) plans: pd_mla_plan fills these instead of pf / du / mg
  bool mla = false;
  pd_mla_desc mdesc{};
  int32_t mla_waves = 4, mla_rows = 64;  // MLA blocks: wavefronts, query rows
  std::vector<pdk::MlaItem> mitems;  // launch order
  std::vector<pdk::MlaMergeGroup> mmg;
  size_t off_mitems = 0, off_mmg = 0;
};

// A multi-layer transfer: the listed pages' heads [h0, h1) of L layer pools.
// Workspace image: L pool pointers, the n page ids, L block counters (zero).
struct pd_xfer_s {
  pd_attn_desc desc{};
  int32_t L = 0, n = 0, h0 = 0, h1 = 0;
  size_t off_layers = 0, off_ids = 0, off_done = 0, ws_bytes = 0;
  std::vector<uint8_t> blob;
};

namespace {

// Pinned host staging for workspace uploads, shared by all plans and reused
// across steps: a block is handed out again once the copy that last read it
// has completed (its event), so re-planning every step allocates no pinned
// memory in steady state.
struct StagingBlock {
  void* ptr = nullptr;
  size_t bytes = 0;
  hipEvent_t ev = nullptr;
  bool recorded = false;
};
std::mutex g_staging_mu;
std::vector<StagingBlock> g_staging;

pd_status hip_fail(hipError_t e, const char* what);

// Copies `n` bytes of `src` into a free pinned block and enqueues the
// host-to-device copy on `stream`.
pd_status staged_upload(void* dst, const void* src, size_t n, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_staging_mu);
  StagingBlock* blk = nullptr;
  for (auto& b : g_staging) {
    if (b.bytes < n) continue;
    if (b.recorded) {
      hipError_t q = hipEventQuery(b.ev);
      if (q == hipErrorNotReady) continue;
      if (q != hipSuccess) return hip_fail(q, "staging event query");
    }
    blk = &b;
    break;
  }
  if (!blk) {
    StagingBlock b;
    b.bytes = std::max<size_t>(n, 1 << 20);
    hipError_t e = hipHostMalloc(&b.ptr, b.bytes, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "pinned staging allocation");
    e = hipEventCreateWithFlags(&b.ev, hipEventDisableTiming);
    if (e != hipSuccess) {
      (void)hipHostFree(b.ptr);
      return hip_fail(e, "staging event creation");
    }
    g_staging.push_back(b);
    blk = &g_staging.back();
  }
  std::memcpy(blk->ptr, src, n);
  hipError_t e = hipMemcpyAsync(dst, blk->ptr, n, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "workspace upload");
  e = hipEventRecord(blk->ev, stream);
  if (e != hipSuccess) return hip_fail(e, "staging event record");
  blk->recorded = true;
  return PD_OK;
}

}  // namespace

namespace {

int64_t round_up32(int64_t x) { return (x + 31) / 32 * 32; }

constexpr int64_t kMaxParts = (int64_t)1 << 26;  // split-KV partial results of one plan

// A caller's decode_chunk_keys (> 0), rounded up to a multiple of 32 and
// clamped to the longest request (rounded up), so that no length arithmetic
// can overflow and a chunk is never longer than the keys it could cover.
int clamp_chunk_option(int32_t keys, const pd_plan_s& P) {
  int64_t max_kv = 32;
  for (const pdk::ReqInfo& ri : P.req) max_kv = std::max<int64_t>(max_kv, ri.kv);
  const int64_t c = std::min({round_up32(keys), round_up32(max_kv), (int64_t)1 << 30});
  return (int)std::max<int64_t>(c, 32);
}

// Length of each of the equal chunks (a multiple of 32 keys) that kv >= 1
// keys split into at a chunk length of about `chunk` (> 0).
int equal_chunk_len(int32_t kv, int chunk) {
  const int64_t nch = ((int64_t)kv + chunk - 1) / chunk;
  return (int)std::min<int64_t>(round_up32(((int64_t)kv + nch - 1) / nch), (int64_t)1 << 30);
}

// Length of the equal chunks of kv keys whose count is the nearest to
// kv / target (at least one), rounded up to a multiple of 32.
int nearest_chunk_len(int32_t kv, int target) {
  const int64_t nch = std::max<int64_t>(1, ((int64_t)kv + target / 2) / target);
  return (int)std::min<int64_t>(round_up32(((int64_t)kv + nch - 1) / nch), (int64_t)1 << 30);
}

// ---- decode role planning.
// A (request, KV head) whose qo * g query rows fit kMaxDecodeRows is a decode
// row group.  Rows <= 16: one wavefront with one 16-row column group; <= 32:
// one wavefront with two; <= 64: two wavefronts of one block side by side
// (rows [0, 32) and [32, 64)) on the same keys, so the second read of every
// key hits the cache.  A piece of a group over keys [k0, k1) (k0 a multiple
// of 32) is a unit; a wavefront runs a queue of units back to back.
//   * Few prefill tiles (one dispatch round): the groups of a class are laid
//     end to end (each padded to a multiple of 32 keys) and cut into equal
//     spans, one per queue, so every queue streams the same number of keys
//     and changes row group (reloading its Q) only where a span crosses a
//     group boundary.
//   * Many prefill tiles: every group is cut into chunks, each its own
//     queue, and the decode blocks interleave with the prefill tiles.  The
//     chunk is sized so that a decode block (eight chunks) lasts about as
//     long as the launch's mean prefill tile: the hardware dispatches blocks
//     in order, one XCD after the other, so blocks of very unequal length
//     leave CUs idle mid-launch and a tail at its end.  The two durations
//     are priced with the per-CU rates measured for this mix on MI355X: a
//     decode block streams 37.7-40 GB/s beside prefill tiles whatever its
//     length, a prefill tile runs 4.3 TFLOP/s.  (Long mixed workload, 2048
//     tiles of 3.8 GFLOP: 2 / 3 / 4 / 5 / 6 / 8 chunks per 32768-key group
//     ran 11.45-11.87 / 12.04 / 10.68-11.10 / 11.20 / 11.68 / 12.1 ms on the
//     same boxes, with 10 / 13 / 3 / 6.5 / - / 20 % of CU time idle.)  A
//     group's chunks are graded +-9 % about that length, longest first, and
//     the queues run longest first, so the decode blocks shorten through the
//     launch as the prefill tiles do (the same launch: 10.48-10.53 against
//     10.71-10.75 ms with equal chunks; +-6 % and +-12 % measured alike).
//     decode_chunk_keys > 0 sets the chunk instead, in equal pieces.
// Partial results: piece i of a group of `rows` rows owns the partial rows
// [part0 + i rows, part0 + (i + 1) rows).
struct DecodeGroup {
  int r, hk, rows, cls;  // cls 0: rows <= 16; 1: rows <= 32; 2: rows <= 64
  int part0;
  std::vector<std::pair<int, int>> pieces;  // key ranges, in key order
};
constexpr int kClsWidth[3] = {1, 1, 2};  // wavefronts per queue
constexpr int kClsNcg[3] = {1, 2, 2};    // 16-row column groups per wavefront
constexpr int kMinSpanKeys = 256;        // shortest span worth a queue
constexpr double kMixDecodeBytesPerCu = 38.5e9;   // B/s of one CU's decode block beside prefill tiles
constexpr double kMixPrefillFlopsPerCu = 4.3e12;  // flop/s of one CU's prefill tile in the same launch
constexpr double kStreamBytesPerS = 6.5e12;       // streaming reads of the whole chip (MI355X, measured)
constexpr double kChunkGrade = 0.09;  // spread of the planner-sized chunks of a group about their mean

pd_status build_decode(pd_plan_s& P, const pd_plan_options* opts, int num_cus, int n_prefill_tiles,
                       double mean_tile_flops, double max_tile_flops, std::vector<double>& block_cost) {
  const pd_attn_desc& d = P.desc;
  const int g = P.g, H_kv = d.num_kv_heads, D = d.head_dim, elt = elt_bytes(&d);
  std::vector<DecodeGroup> groups;
  int64_t class_keys[3] = {0, 0, 0};  // padded to multiples of 32 per group
  for (int r = 0; r < P.B; ++r) {
    const pdk::ReqInfo& ri = P.req[r];
    const int64_t rows = (int64_t)ri.qo * g;
    if (ri.qo == 0 || rows > pdk::kMaxDecodeRows) continue;
    const int cls = rows <= 16 ? 0 : rows <= 32 ? 1 : 2;
    for (int hk = 0; hk < H_kv; ++hk) groups.push_back({r, hk, (int)rows, cls, 0, {}});
    class_keys[cls] += round_up32(ri.kv) * H_kv;
    P.decode_bytes += 2LL * ri.kv * H_kv * D * elt;
  }
  P.chunk_keys = 0;
  P.dq.assign(1, 0);
  if (groups.empty()) return PD_OK;
  const int64_t wave_keys = class_keys[0] + class_keys[1] + 2 * class_keys[2];
  // queues: each a list of (group, piece) in stream order
  struct QEntry {
    int grp, piece;
  };
  std::vector<std::vector<QEntry>> queues[3];
  // One round of queues on the CUs the prefill tiles leave, unless that
  // round would outlast the longest prefill tile (its CUs would then idle
  // while the decode queues finish): then chunks interleaved with the tiles.
  bool one_round = n_prefill_tiles < num_cus && !(opts && opts->decode_chunk_keys > 0);
  if (one_round && n_prefill_tiles > 0) {
    const int free_cus = std::max(num_cus - n_prefill_tiles, num_cus / 2);
    const double round_s = (double)P.decode_bytes / std::min(free_cus * kMixDecodeBytesPerCu, kStreamBytesPerS);
    one_round = round_s <= max_tile_flops / kMixPrefillFlopsPerCu;
  }
  if (one_round) {
    const int slots =
        pdk::kWavesPerBlock * (n_prefill_tiles == 0 ? num_cus : std::max(num_cus - n_prefill_tiles, num_cus / 2));
    int lanes[3] = {0, 0, 0};
    int used = 0;
    for (int c = 0; c < 3; ++c) {
      if (!class_keys[c]) continue;
      const double share = (double)class_keys[c] * kClsWidth[c] / (double)wave_keys;
      lanes[c] = std::max(1, (int)(share * slots / kClsWidth[c]));
      lanes[c] = (int)std::min<int64_t>(lanes[c], std::max<int64_t>(1, class_keys[c] / kMinSpanKeys));
      used += lanes[c] * kClsWidth[c];
    }
    for (int c = 2; used > slots && c >= 0; --c)  // rounding overshoot: trim the widest classes
      while (used > slots && lanes[c] > 1) --lanes[c], used -= kClsWidth[c];
    for (int c = 0; c < 3; ++c) {
      if (!lanes[c]) continue;
      const int64_t steps = class_keys[c] / 32;            // 32-key steps of the class
      const int64_t per = (steps + lanes[c] - 1) / lanes[c];  // steps per queue
      queues[c].assign((size_t)((steps + per - 1) / per), {});
      int64_t pos = 0;  // first step of the current group in the class's stream
      for (size_t gi = 0; gi < groups.size(); ++gi) {
        DecodeGroup& gr = groups[gi];
        if (gr.cls != c) continue;
        const int kv = P.req[gr.r].kv;
        const int64_t gsteps = round_up32(kv) / 32;
        for (int64_t s = 0; s < gsteps;) {
          const int64_t q = (pos + s) / per;  // queue of this step
          const int64_t e = std::min(gsteps, (q + 1) * per - pos);
          gr.pieces.push_back({(int)(s * 32), (int)std::min<int64_t>(kv, e * 32)});
          queues[c][q].push_back({(int)gi, (int)gr.pieces.size() - 1});
          s = e;
        }
        pos += gsteps;
      }
    }
  } else {
    const bool forced = opts && opts->decode_chunk_keys > 0;
    int chunk;
    if (forced) {
      chunk = clamp_chunk_option(opts->decode_chunk_keys, P);
    } else {
      // keys of a chunk whose block of kWavesPerBlock chunks lasts one mean prefill tile
      const double block_bytes = mean_tile_flops / kMixPrefillFlopsPerCu * kMixDecodeBytesPerCu;
      const double c = block_bytes / pdk::kWavesPerBlock / (2.0 * D * elt);
      chunk = (int)std::min(std::max(c, 256.0), 16384.0);
    }
    P.chunk_keys = forced ? chunk : 0;  // else: the longest unit, below
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      DecodeGroup& gr = groups[gi];
      const int kv = P.req[gr.r].kv;
      const int len = forced ? equal_chunk_len(kv, chunk) : nearest_chunk_len(kv, chunk);
      const int64_t nch = ((int64_t)kv + len - 1) / len;
      int64_t k0 = 0;
      for (int64_t i = 0; k0 < kv; ++i) {
        // planner-sized chunks are graded from (1 + kChunkGrade) to (1 - kChunkGrade)
        // of the mean, so that the decode blocks, run longest first, shorten
        // through the launch as the prefill tiles (longest first) do
        int64_t k1 = k0 + len;
        if (!forced && nch > 1) {
          const double w = 1.0 + kChunkGrade * (double)(nch - 1 - 2 * i) / (double)(nch - 1);
          k1 = i + 1 >= nch ? kv : k0 + round_up32((int64_t)(w * (double)kv / (double)nch));
        }
        k1 = std::min<int64_t>(kv, k1);
        gr.pieces.push_back({(int)k0, (int)k1});
        queues[gr.cls].push_back({{(int)gi, (int)gr.pieces.size() - 1}});
        k0 = k1;
      }
    }
    for (int c = 0; c < 3; ++c)  // longest first
      std::stable_sort(queues[c].begin(), queues[c].end(), [&](const std::vector<QEntry>& x, const std::vector<QEntry>& y) {
        const auto& px = groups[x[0].grp].pieces[x[0].piece];
        const auto& py = groups[y[0].grp].pieces[y[0].piece];
        return (px.second - px.first) > (py.second - py.first);
      });
  }
  // partial rows and merge groups
  int64_t n_parts = 0;
  for (DecodeGroup& gr : groups) {
    if (gr.pieces.empty() || n_parts + (int64_t)gr.pieces.size() * gr.rows > kMaxParts)
      return fail(PD_ERR_UNSUPPORTED, "more than 2^26 split-KV partial result rows");
    gr.part0 = (int)n_parts;
    n_parts += (int64_t)gr.pieces.size() * gr.rows;
    P.mg.push_back({gr.r, gr.hk, gr.part0, (int)gr.pieces.size()});
  }
  P.n_parts = (int32_t)n_parts;
  if (!P.chunk_keys) {  // report the longest unit
    for (const DecodeGroup& gr : groups)
      for (const auto& pc : gr.pieces) P.chunk_keys = std::max(P.chunk_keys, pc.second - pc.first);
  }
  // wavefront slots: class-2 queues take an aligned pair of wavefronts of one
  // block (the two 32-row halves side by side), then the others
  std::vector<std::pair<int, int>> slot_queue;  // (class, queue) per slot; c0 of a class-2 slot by parity
  for (int q = 0; q < (int)queues[2].size(); ++q) slot_queue.push_back({2, q}), slot_queue.push_back({2, q});
  for (int c = 0; c < 2; ++c)
    for (int q = 0; q < (int)queues[c].size(); ++q) slot_queue.push_back({c, q});
  const int n_slots = (int)slot_queue.size();
  block_cost.assign((n_slots + pdk::kWavesPerBlock - 1) / pdk::kWavesPerBlock, 0.0);
  for (int s = 0; s < n_slots; ++s) {
    const int c = slot_queue[s].first, q = slot_queue[s].second;
    const int c0 = (c == 2 && (s & 1)) ? 32 : 0;
    for (const QEntry& e : queues[c][q]) {
      const DecodeGroup& gr = groups[e.grp];
      const auto& pc = gr.pieces[e.piece];
      P.du.push_back({gr.r, gr.hk, pc.first, pc.second, gr.part0 + e.piece * gr.rows + c0, c0, kClsNcg[c],
                      c == 2 ? 1 : 0});
      block_cost[s / pdk::kWavesPerBlock] += 2.0 * (pc.second - pc.first) * D * elt;
    }
    P.dq.push_back((int32_t)P.du.size());
  }
  return PD_OK;
}

pd_status build_plan(pd_plan_s& P, const pd_plan_options* opts) {
  const pd_attn_desc& d = P.desc;
  const int g = P.g;
  const int H_kv = d.num_kv_heads;
  const int64_t elt = elt_bytes(&d);
  int num_cus = (opts && opts->num_cus > 0) ? opts->num_cus : 256;

  // ---- prefill tiles: requests whose qo * g rows exceed the decode role's.
  // A launch with no decode rows whose prefill requests all have short caches
  // (at most 64 key tiles) runs 128-row tiles in 4-wavefront blocks, two per
  // CU; otherwise 256-row tiles in 8-wavefront blocks.
  {
    bool any_decode = false, any_prefill = false;
    int max_kv = 0;
    for (int r = 0; r < P.B; ++r) {
      const pdk::ReqInfo& ri = P.req[r];
      if (ri.qo == 0) continue;
      if ((int64_t)ri.qo * g <= pdk::kMaxDecodeRows) {
        any_decode = true;
      } else {
        any_prefill = true;
        max_kv = std::max(max_kv, ri.kv);
      }
    }
    const int pw = opts ? opts->prefill_block_waves : 0;
    P.prefill4 = any_prefill && !any_decode && g <= pdk::kPrefillRows / 2 &&
                 (pw == 4 || (pw == 0 && max_kv <= 64 * 64));
  }
  const int T = std::max(1, (P.prefill4 ? pdk::kPrefillRows / 2 : pdk::kPrefillRows) / g);  // tokens per tile
  std::vector<double> pf_cost;                        // flops of each tile, launch order
  struct Tile {
    pdk::PrefillItem it;
    int64_t cost;
  };
  std::vector<std::vector<Tile>> groups;  // per (request, kv head)
  for (int r = 0; r < P.B; ++r) {
    const pdk::ReqInfo& ri = P.req[r];
    if (ri.qo == 0 || (int64_t)ri.qo * g <= pdk::kMaxDecodeRows) continue;
    const int64_t pairs = (int64_t)ri.qo * (ri.kv - ri.qo) + (int64_t)ri.qo * (ri.qo + 1) / 2;
    P.prefill_flops += 4LL * d.head_dim * d.num_qo_heads * (d.causal ? pairs : (int64_t)ri.qo * ri.kv);
    for (int hk = 0; hk < H_kv; ++hk) {
      std::vector<Tile> grp;
      for (int q0 = 0; q0 < ri.qo; q0 += T) {
        const int nq = std::min(T, ri.qo - q0);
        const int kv_end = d.causal ? ri.kv - ri.qo + q0 + nq : ri.kv;
        grp.push_back({{r, hk, q0, nq, kv_end, 0, 0, 0}, (int64_t)nq * g * kv_end});
      }
      groups.push_back(std::move(grp));
    }
  }
  if (!groups.empty()) {
    // groups -> XCDs (largest group to the least loaded XCD), then tiles in
    // dispatch order: slot i runs on XCD i % 8, longest tiles first.
    std::vector<int> order(groups.size());
    std::vector<int64_t> gcost(groups.size(), 0);
    for (size_t i = 0; i < groups.size(); ++i) {
      order[i] = (int)i;
      for (auto& t : groups[i]) gcost[i] += t.cost;
    }
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return gcost[a] > gcost[b]; });
    std::vector<std::vector<Tile>> xq(kNumXcd);
    std::vector<int64_t> xload(kNumXcd, 0);
    for (int gi : order) {
      int x = (int)(std::min_element(xload.begin(), xload.end()) - xload.begin());
      xload[x] += gcost[gi];
      for (auto& t : groups[gi]) xq[x].push_back(t);
    }
    size_t total = 0;
    for (auto& q : xq) {
      std::stable_sort(q.begin(), q.end(), [](const Tile& a, const Tile& b) { return a.cost > b.cost; });
      total += q.size();
    }
    std::vector<size_t> head(kNumXcd, 0);
    P.pf.reserve(total);
    for (size_t i = 0; i < total; ++i) {
      int x = (int)(i % kNumXcd);
      if (head[x] >= xq[x].size()) {  // this XCD ran out: take from the fullest
        size_t best = 0;
        int bx = -1;
        for (int y = 0; y < kNumXcd; ++y)
          if (xq[y].size() - head[y] > best) best = xq[y].size() - head[y], bx = y;
        x = bx;
      }
      pf_cost.push_back((double)xq[x][head[x]].cost * 4.0 * d.head_dim);  // flops
      P.pf.push_back(xq[x][head[x]++].it);
    }
  }

  // ---- decode units: (request, KV head) row groups of at most kMaxDecodeRows
  // query rows, each cut into key chunks; units go to per-wavefront queues
  std::vector<double> db_cost;
  double pf_flops = 0, pf_max = 0;
  for (double c : pf_cost) pf_flops += c, pf_max = std::max(pf_max, c);
  pd_status ds = build_decode(P, opts, num_cus, (int)P.pf.size(),
                              pf_cost.empty() ? 0.0 : pf_flops / (double)pf_cost.size(), pf_max, db_cost);
  if (ds != PD_OK) return ds;
  const int n_db = (int)db_cost.size();

  // ---- launch order.  Block i is dispatched to XCD i % 8, so blocks are
  // emitted in rounds of 8: a prefill round keeps the XCD affinity of the
  // tiles built above, a decode round takes the next 8 decode blocks.  One
  // attention block fills a CU (its LDS and registers), so the two roles
  // cannot share a CU at the same time.  block_order 0 (the default)
  // interleaves the rounds so that both kinds progress at the same fraction
  // of their totals, priced at MI355X peaks (2.5 PFLOP/s, 8 TB/s): the CUs
  // that run decode blocks stream the cache from HBM while the others run
  // prefill tiles on the matrix cores (measured on the long mixed workload:
  // 7 % faster than running the roles one after the other, and insensitive
  // to the price ratio between 100 and 500 flop/B).  block_order 1 runs
  // every prefill tile first and lets the decode blocks fill the CUs that
  // the prefill tail frees.
  const int order = opts ? opts->block_order : 0;
  P.block_map.reserve(P.pf.size() + n_db);
  if (order == 1 || P.pf.empty() || n_db == 0) {
    for (size_t i = 0; i < P.pf.size(); ++i) P.block_map.push_back((int32_t)i);
    for (int i = 0; i < n_db; ++i) P.block_map.push_back(-i - 1);
  } else {
    double tot_p = 0, tot_d = 0, done_p = 0, done_d = 0;
    for (double c : pf_cost) tot_p += c / 2.5e15;
    for (double c : db_cost) tot_d += c / 8e12;
    size_t ip = 0;
    int id = 0;
    while (ip < P.pf.size() || id < n_db) {
      const bool take_p = id >= n_db || (ip < P.pf.size() && done_p / tot_p <= done_d / tot_d);
      for (int k = 0; k < kNumXcd; ++k) {
        if (take_p && ip < P.pf.size()) {
          done_p += pf_cost[ip] / 2.5e15;
          P.block_map.push_back((int32_t)ip++);
        } else if (!take_p && id < n_db) {
          done_d += db_cost[id] / 8e12;
          P.block_map.push_back(-(id++) - 1);
        }
      }
    }
  }

  // ---- workspace layout
  size_t off = 0;
  P.off_qo = off;
  off = align_up(off + sizeof(int32_t) * (P.B + 1));
  P.off_req = off;
  off = align_up(off + sizeof(pdk::ReqInfo) * P.B);
  P.off_pages = off;
  off = align_up(off + sizeof(int32_t) * P.pages.size());
  P.off_launch = off;
  off = align_up(off + sizeof(pdk::LaunchRec) * P.block_map.size());
  P.off_du = off;
  off = align_up(off + sizeof(pdk::DecodeUnit) * P.du.size());
  P.off_mg = off;
  off = align_up(off + sizeof(pdk::MergeRec) * P.mg.size());
  P.off_rows = off;
  off = align_up(off + sizeof(int32_t) * 2 * (size_t)P.total_rows);
  P.meta_bytes = off;
  P.off_part_o = off;
  off = align_up(off + sizeof(float) * (size_t)P.n_parts * d.head_dim);
  P.off_part_lse = off;
  off = align_up(off + sizeof(float) * (size_t)P.n_parts);
  P.ws_bytes = off;

  P.blob.assign(P.meta_bytes, 0);
  auto put = [&](size_t o, const void* src, size_t n) {
    if (n) std::memcpy(P.blob.data() + o, src, n);
  };
  put(P.off_qo, P.qo_indptr.data(), sizeof(int32_t) * P.qo_indptr.size());
  put(P.off_req, P.req.data(), sizeof(pdk::ReqInfo) * P.req.size());
  put(P.off_pages, P.pages.data(), sizeof(int32_t) * P.pages.size());
  {
    pdk::LaunchRec* lr = (pdk::LaunchRec*)(P.blob.data() + P.off_launch);
    const int n_slots = (int)P.dq.size() - 1;
    for (size_t i = 0; i < P.block_map.size(); ++i) {
      const int v = P.block_map[i];
      pdk::LaunchRec rec{};
      rec.v = v;
      if (v >= 0) {
        std::memcpy(rec.w, &P.pf[v], sizeof(pdk::PrefillItem));
        std::memcpy(rec.w + 8, &P.req[P.pf[v].req], sizeof(pdk::ReqInfo));
      } else {
        const int s0 = (-v - 1) * pdk::kWavesPerBlock;
        for (int k = 0; k <= pdk::kWavesPerBlock; ++k) rec.w[k] = P.dq[std::min(s0 + k, n_slots)];
        rec.w[9] = (s0 < n_slots && P.dq[s0] < P.dq[s0 + 1] && P.du[P.dq[s0]].pair) ? 1 : 0;
      }
      lr[i] = rec;
    }
    pdk::DecodeUnit* du = (pdk::DecodeUnit*)(P.blob.data() + P.off_du);
    for (size_t i = 0; i < P.du.size(); ++i) du[i] = {P.du[i], P.req[P.du[i].req]};
  }
  {
    pdk::MergeRec* mr = (pdk::MergeRec*)(P.blob.data() + P.off_mg);
    for (size_t i = 0; i < P.mg.size(); ++i) {
      const pdk::MergeGroup& m = P.mg[i];
      const pdk::ReqInfo& ri = P.req[m.req];
      mr[i] = {m.part0, m.nparts, ri.qo * P.g, ri.qo_start, m.hk, 0, 0, 0};
    }
  }
  {
    int32_t* rp = (int32_t*)(P.blob.data() + P.off_rows);
    for (int r = 0; r < P.B; ++r) {
      const pdk::ReqInfo& ri = P.req[r];
      for (int i = 0; i < ri.qo; ++i) {
        const int pos = ri.kv - ri.qo + i;
        rp[2 * (ri.qo_start + i)] = P.pages[ri.page_start + pos / d.page_size];
        rp[2 * (ri.qo_start + i) + 1] = pos % d.page_size;
      }
    }
  }
  return PD_OK;
}

// Checks a batch's lengths and page table (page size ps) and fills the
// plan's request rows and page list.
pd_status fill_requests(pd_plan_s& P, int ps, int32_t batch, const int32_t* qo_lens, const int32_t* kv_lens,
                        const int32_t* page_indptr, const int32_t* page_indices, int32_t num_pool_pages) {
  if (page_indptr[0] != 0) return fail(PD_ERR_INVALID_ARG, "page_indptr[0] must be 0");
  int64_t rows = 0;
  for (int r = 0; r < batch; ++r) {
    const int32_t qo = qo_lens[r], kv = kv_lens[r];
    if (qo < 0 || kv < 0) return fail(PD_ERR_INVALID_ARG, "request " + std::to_string(r) + ": negative length");
    if (qo > kv)
      return fail(PD_ERR_INVALID_ARG, "request " + std::to_string(r) + ": qo_len > kv_len (the new tokens are part of the cache)");
    const int64_t need = ((int64_t)kv + ps - 1) / ps;
    const int64_t have = (int64_t)page_indptr[r + 1] - page_indptr[r];
    if (have != need)
      return fail(PD_ERR_INVALID_ARG, "request " + std::to_string(r) + ": has " + std::to_string(have) +
                                          " pages, needs ceil(kv_len / page_size) = " + std::to_string(need));
    rows += qo;
  }
  if (rows > INT32_MAX) return fail(PD_ERR_INVALID_ARG, "too many query rows");
  const int64_t total_pages = page_indptr[batch];
  if (total_pages > 0 && !page_indices) return fail(PD_ERR_INVALID_ARG, "page_indices is NULL");
  {
    std::vector<uint8_t> seen((size_t)std::max(num_pool_pages, 1), 0);
    for (int64_t i = 0; i < total_pages; ++i) {
      const int32_t id = page_indices[i];
      if (id < 0 || id >= num_pool_pages)
        return fail(PD_ERR_OUT_OF_RANGE, "page id " + std::to_string(id) + " outside the pool");
      if (seen[id]) return fail(PD_ERR_INVALID_ARG, "page id " + std::to_string(id) + " appears twice");
      seen[id] = 1;
    }
  }
  P.B = batch;
  P.total_rows = (int32_t)rows;
  P.qo_indptr.resize(batch + 1);
  P.req.resize(batch);
  P.qo_indptr[0] = 0;
  for (int r = 0; r < batch; ++r) {
    P.req[r] = {P.qo_indptr[r], qo_lens[r], kv_lens[r], page_indptr[r]};
    P.qo_indptr[r + 1] = P.qo_indptr[r] + qo_lens[r];
  }
  P.pages.assign(page_indices, page_indices + total_pages);
  return PD_OK;
}

pdk::AttnParams attn_params(const pd_plan_s& P, void* d_ws) {
  char* ws = (char*)d_ws;
  pdk::AttnParams a{};
  a.qo_indptr = (const int32_t*)(ws + P.off_qo);
  a.req = (const pdk::ReqInfo*)(ws + P.off_req);
  a.page_indices = (const int32_t*)(ws + P.off_pages);
  a.launch = (const pdk::LaunchRec*)(ws + P.off_launch);
  a.du = (const pdk::DecodeUnit*)(ws + P.off_du);
  a.mg = (const pdk::MergeRec*)(ws + P.off_mg);
  a.n_blocks = (int32_t)P.block_map.size();
  a.prefill4 = P.prefill4 ? 1 : 0;
  a.part_o = (float*)(ws + P.off_part_o);
  a.part_lse = (float*)(ws + P.off_part_lse);
  a.n_pf = (int32_t)P.pf.size();
  a.n_du = (int32_t)P.du.size();
  a.n_mg = (int32_t)P.mg.size();
  a.B = P.B;
  a.H_q = P.desc.num_qo_heads;
  a.H_kv = P.desc.num_kv_heads;
  a.g = P.g;
  a.ps = P.desc.page_size;
  a.ps_shift = __builtin_ctz((unsigned)P.desc.page_size);
  a.D = P.desc.head_dim;
  a.causal = P.desc.causal;
  a.sm_scale = P.desc.sm_scale;
  a.c_log2 = P.desc.sm_scale * 1.4426950408889634f;
  a.page_elems = 2LL * P.desc.num_kv_heads * P.desc.page_size * P.desc.head_dim;
  return a;
}

// Latent-cache plan: blocks of 64 query rows of one request over a chunk of
// keys.  Each (request, row group) is cut into chunks of equal length (a
// multiple of 32 keys) so that about two blocks per CU exist; the blocks of
// one (request, chunk) read the same cache rows and are placed on one XCD,
// one dispatch round apart (block i runs on XCD i % 8), longest first.

// Chunk length for an MLA plan. A block stages the whole latent row once per
// 32-key step for all its query rows, holds one CU (its LDS ring takes most of
// the 160 KB) and writes R x 513 floats per partial, which the merge reads
// back. The cost of a candidate is the greedy (longest first) makespan of its
// blocks over one block slot per CU, each block charged its keys plus a fixed
// start-up and drain cost, plus the partial traffic spread over the chip. The
// constants are in units of one key step of one block, fitted to MI355X runs
// of 64 requests x U{1024..8192} keys at 16 and 128 heads.
int mla_pick_chunk(const pd_plan_s& P, int R, int num_cus) {
  constexpr double kBlockKeys = 96.0;    // Q load, ring fill, partial store
  const double part_keys = R / 100.0;    // R x 513 x 4 B written, then read by the merge
  int max_kv = 0;
  for (int r = 0; r < P.B; ++r)
    if (P.req[r].qo > 0) max_kv = std::max(max_kv, P.req[r].kv);
  const int top = (int)std::max<int64_t>(256, std::min<int64_t>(16384, ((int64_t)max_kv + 127) / 128 * 128));
  std::vector<int> cand;
  for (double c = 256; c < top * 1.2; c *= 1.125) {
    const int v = std::min(top, ((int)c + 127) / 128 * 128);
    if (cand.empty() || cand.back() != v) cand.push_back(v);
  }
  int best = top;
  double best_cost = -1;
  std::vector<int> blk;
  for (int chunk : cand) {
    blk.clear();
    int64_t parts = 0;
    for (int r = 0; r < P.B; ++r) {
      const pdk::ReqInfo& ri = P.req[r];
      if (ri.qo == 0) continue;
      const int ng = (int)(((int64_t)ri.qo * P.mdesc.num_qo_heads + R - 1) / R);
      const int len = equal_chunk_len(ri.kv, chunk);
      const int nch = (int)(((int64_t)ri.kv + len - 1) / len);
      if (nch > 1) parts += (int64_t)ng * nch;
      for (int c = 0; c < nch; ++c)
        for (int g = 0; g < ng; ++g)
          blk.push_back((int)(std::min<int64_t>(ri.kv, (int64_t)(c + 1) * len) - (int64_t)c * len));
    }
    if (blk.size() > (size_t)64 * num_cus && chunk != top) continue;  // far past one CU each
    std::sort(blk.begin(), blk.end(), std::greater<int>());
    std::vector<double> slot(std::min<size_t>(num_cus, blk.size()), 0.0);  // min-heap of CU finish times
    double span = 0;
    for (int k : blk) {
      std::pop_heap(slot.begin(), slot.end(), std::greater<double>());
      slot.back() += k + kBlockKeys;
      span = std::max(span, slot.back());
      std::push_heap(slot.begin(), slot.end(), std::greater<double>());
    }
    const double cost = span + parts * part_keys;
    if (best_cost < 0 || cost < best_cost) best_cost = cost, best = chunk;
  }
  return best;
}

pd_status build_mla_plan(pd_plan_s& P, const pd_plan_options* opts) {
  const pd_mla_desc& d = P.mdesc;
  const int H = d.num_qo_heads;
  const int num_cus = (opts && opts->num_cus > 0) ? opts->num_cus : 256;
  // 128 heads: one token's rows fill a block of 4 wavefronts x 32 rows, so
  // each cache step is staged once for all of them; fewer heads: 4 x 16.
  P.mla_waves = 4;
  P.mla_rows = H == 128 ? 128 : 64;  // H is a multiple of 16 in [16, 128]
  const int R = P.mla_rows;
  int64_t work = 0;  // row groups x keys
  for (int r = 0; r < P.B; ++r) {
    const pdk::ReqInfo& ri = P.req[r];
    if (ri.qo == 0) continue;
    const int ng = (int)(((int64_t)ri.qo * H + R - 1) / R);
    work += (int64_t)ng * ri.kv;
    P.decode_bytes += (int64_t)ri.kv * pdk::kMlaWidth * 2;
  }
  int chunk = 0;
  if (opts && opts->decode_chunk_keys > 0) {
    chunk = clamp_chunk_option(opts->decode_chunk_keys, P);
  } else if (work > 0) {
    chunk = mla_pick_chunk(P, R, num_cus);
  }
  P.chunk_keys = chunk;
  struct Task {  // one (request, chunk): its row groups' blocks
    int req, c, k0, k1, ng;
  };
  std::vector<Task> tasks;
  std::vector<int> base(P.B, -1), nchunks(P.B, 1);  // first partial slot of a split request, chunks
  for (int r = 0; r < P.B; ++r) {
    const pdk::ReqInfo& ri = P.req[r];
    if (ri.qo == 0) continue;
    const int ng = (int)(((int64_t)ri.qo * H + R - 1) / R);
    const int len = equal_chunk_len(ri.kv, chunk);
    const int nch = (int)(((int64_t)ri.kv + len - 1) / len);
    nchunks[r] = nch;
    if (nch < 1 || (int64_t)P.n_parts + (int64_t)ng * nch > kMaxParts)
      return fail(PD_ERR_UNSUPPORTED, "MLA plan: more than 2^26 partial results");
    if (nch > 1) {  // slots [base, base + ng * nch): row group rg's chunk c at base + rg * nch + c
      base[r] = P.n_parts;
      for (int rg = 0; rg < ng; ++rg) P.mmg.push_back({r, rg, P.n_parts + rg * nch, nch});
      P.n_parts += ng * nch;
    }
    for (int c = 0; c < nch; ++c)
      tasks.push_back({r, c, (int)((int64_t)c * len), (int)std::min<int64_t>(ri.kv, (int64_t)(c + 1) * len), ng});
  }
  std::stable_sort(tasks.begin(), tasks.end(),
                   [](const Task& a, const Task& b) { return (a.k1 - a.k0) > (b.k1 - b.k0); });
  std::vector<std::vector<pdk::MlaItem>> xq(kNumXcd);
  std::vector<int64_t> xload(kNumXcd, 0);
  for (const Task& t : tasks) {
    const int x = (int)(std::min_element(xload.begin(), xload.end()) - xload.begin());
    xload[x] += (int64_t)t.ng * (t.k1 - t.k0);
    for (int rg = 0; rg < t.ng; ++rg)
      xq[x].push_back({t.req, rg, t.k0, t.k1, base[t.req] < 0 ? -1 : base[t.req] + rg * nchunks[t.req] + t.c,
                       0, 0, 0});
  }
  size_t total = 0;
  for (auto& q : xq) total += q.size();
  std::vector<size_t> head(kNumXcd, 0);
  P.mitems.reserve(total);
  for (size_t i = 0; i < total; ++i) {
    int x = (int)(i % kNumXcd);
    if (head[x] >= xq[x].size()) {  // this XCD ran out: take from the fullest
      size_t best = 0;
      int bx = -1;
      for (int y = 0; y < kNumXcd; ++y)
        if (xq[y].size() - head[y] > best) best = xq[y].size() - head[y], bx = y;
      x = bx;
    }
    P.mitems.push_back(xq[x][head[x]++]);
  }

  size_t off = 0;
  P.off_qo = off;
  off = align_up(off + sizeof(int32_t) * (P.B + 1));
  P.off_req = off;
  off = align_up(off + sizeof(pdk::ReqInfo) * P.B);
  P.off_pages = off;
  off = align_up(off + sizeof(int32_t) * P.pages.size());
  P.off_mitems = off;
  off = align_up(off + sizeof(pdk::MlaItem) * P.mitems.size());
  P.off_mmg = off;
  off = align_up(off + sizeof(pdk::MlaMergeRec) * P.mmg.size());
  P.meta_bytes = off;
  P.off_part_o = off;
  off = align_up(off + sizeof(float) * (size_t)P.n_parts * R * pdk::kMlaLatent);
  P.off_part_lse = off;
  off = align_up(off + sizeof(float) * (size_t)P.n_parts * R);
  P.ws_bytes = off;
  P.blob.assign(P.meta_bytes, 0);
  auto put = [&](size_t o, const void* src, size_t n) {
    if (n) std::memcpy(P.blob.data() + o, src, n);
  };
  put(P.off_qo, P.qo_indptr.data(), sizeof(int32_t) * P.qo_indptr.size());
  put(P.off_req, P.req.data(), sizeof(pdk::ReqInfo) * P.req.size());
  put(P.off_pages, P.pages.data(), sizeof(int32_t) * P.pages.size());
  put(P.off_mitems, P.mitems.data(), sizeof(pdk::MlaItem) * P.mitems.size());
  {
    pdk::MlaMergeRec* mr = (pdk::MlaMergeRec*)(P.blob.data() + P.off_mmg);
    for (size_t i = 0; i < P.mmg.size(); ++i) {
      const pdk::MlaMergeGroup& m = P.mmg[i];
      const pdk::ReqInfo& ri = P.req[m.req];
      mr[i] = {m.part0, m.nparts, m.rg, ri.qo * P.mdesc.num_qo_heads, ri.qo_start, 0, 0, 0};
    }
  }
  return PD_OK;
}

pdk::MlaParams mla_params(const pd_plan_s& P, void* d_ws) {
  char* ws = (char*)d_ws;
  pdk::MlaParams a{};
  a.qo_indptr = (const int32_t*)(ws + P.off_qo);
  a.req = (const pdk::ReqInfo*)(ws + P.off_req);
  a.page_indices = (const int32_t*)(ws + P.off_pages);
  a.items = (const pdk::MlaItem*)(ws + P.off_mitems);
  a.mg = (const pdk::MlaMergeRec*)(ws + P.off_mmg);
  a.part_o = (float*)(ws + P.off_part_o);
  a.part_lse = (float*)(ws + P.off_part_lse);
  a.n_items = (int32_t)P.mitems.size();
  a.n_mg = (int32_t)P.mmg.size();
  a.B = P.B;
  a.total_rows = P.total_rows;
  a.waves = P.mla_waves;
  a.rows = P.mla_rows;
  a.H = P.mdesc.num_qo_heads;
  a.ps = P.mdesc.page_size;
  a.ps_shift = __builtin_ctz((unsigned)P.mdesc.page_size);
  a.causal = P.mdesc.causal;
  a.sm_scale = P.mdesc.sm_scale;
  a.c_log2 = P.mdesc.sm_scale * 1.4426950408889634f;
  return a;
}

pd_status hip_fail(hipError_t e, const char* what) {
  return fail(PD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Bytes of the head-[h0, h1) slice of one half (K or V) of a page.
int64_t head_seg_bytes(const pd_attn_desc* d, int32_t h0, int32_t h1) {
  return (int64_t)(h1 - h0) * d->page_size * d->head_dim * elt_bytes(d);
}

pd_status check_heads(const pd_attn_desc* d, int32_t h0, int32_t h1) {
  if (h0 < 0 || h1 > d->num_kv_heads || h0 >= h1)
    return fail(PD_ERR_INVALID_ARG, "head range [" + std::to_string(h0) + ", " + std::to_string(h1) +
                                        ") is not a non-empty range of the pool's " +
                                        std::to_string(d->num_kv_heads) + " KV heads");
  return PD_OK;
}

pd_status check_ids(int32_t num_pool_pages, const int32_t* ids, int32_t n) {
  if (num_pool_pages < 1) return fail(PD_ERR_INVALID_ARG, "num_pool_pages must be >= 1");
  std::vector<uint8_t> seen((size_t)num_pool_pages, 0);
  for (int32_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= num_pool_pages)
      return fail(PD_ERR_OUT_OF_RANGE, "page id " + std::to_string(ids[i]) + " outside the pool");
    if (seen[ids[i]]) return fail(PD_ERR_INVALID_ARG, "page id " + std::to_string(ids[i]) + " repeated");
    seen[ids[i]] = 1;
  }
  return PD_OK;
}

// Single-layer pack / unpack of heads [h0, h1) of the listed pages.
pd_status xfer_common(const pd_attn_desc* desc, const void* pool, const void* buf, int32_t num_pool_pages,
                      const int32_t* ids, int32_t n, int32_t h0, int32_t h1, size_t buf_bytes, void* scratch,
                      size_t scratch_bytes, void* stream, bool to_buffer) {
  pd_status s = check_desc(desc);
  if (s != PD_OK) return s;
  if ((s = check_heads(desc, h0, h1)) != PD_OK) return s;
  if (n < 0) return fail(PD_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return PD_OK;
  if (!ids || !pool || !buf || !scratch) return fail(PD_ERR_INVALID_ARG, "NULL pointer argument");
  if (buf_bytes < (size_t)n * 2 * (size_t)head_seg_bytes(desc, h0, h1))
    return fail(PD_ERR_WORKSPACE, "buffer smaller than the n page slices");
  if (scratch_bytes < sizeof(int32_t) * (size_t)n)
    return fail(PD_ERR_WORKSPACE, "scratch smaller than 4 * n bytes");
  if ((s = check_ids(num_pool_pages, ids, n)) != PD_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  // short id lists travel in the kernel arguments; longer ones are staged
  const bool inline_ids = n <= pdk::kXferInlineIds;
  if (!inline_ids && (s = staged_upload(scratch, ids, sizeof(int32_t) * (size_t)n, st)) != PD_OK) return s;
  pdk::XferParams p{};
  p.buf = (char*)buf;
  p.pool0 = (void*)pool;
  p.page_ids = (const int32_t*)scratch;
  p.page_bytes = page_bytes_of(desc);
  p.half_bytes = p.page_bytes / 2;
  p.seg_off = head_seg_bytes(desc, 0, h0);
  p.seg_bytes = head_seg_bytes(desc, h0, h1);
  p.n = n;
  p.L = 1;
  p.to_buffer = to_buffer ? 1 : 0;
  hipError_t e = pdk::launch_xfer(p, inline_ids ? ids : nullptr, st);
  if (e != hipSuccess) return hip_fail(e, to_buffer ? "pack launch" : "unpack launch");
  return PD_OK;
}

// Device-accessible address of a progress array: pinned host memory
// (hipHostMalloc) is translated, device memory is used as is; anything else
// is rejected.
pd_status progress_device_ptr(uint32_t* progress, uint32_t** out) {
  *out = nullptr;
  if (!progress) return PD_OK;
  hipPointerAttribute_t a{};
  hipError_t e = hipPointerGetAttributes(&a, progress);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PD_ERR_INVALID_ARG, "progress must be pinned host memory (hipHostMalloc) or device memory");
  }
  if (a.type == hipMemoryTypeHost) {
    void* d = nullptr;
    e = hipHostGetDevicePointer(&d, progress, 0);
    if (e != hipSuccess || !d) {
      (void)hipGetLastError();
      return fail(PD_ERR_INVALID_ARG, "progress host memory is not mapped into the device");
    }
    *out = (uint32_t*)d;
    return PD_OK;
  }
  if (a.type == hipMemoryTypeDevice) {
    *out = progress;
    return PD_OK;
  }
  return fail(PD_ERR_INVALID_ARG, "progress must be pinned host memory (hipHostMalloc) or device memory");
}

pd_status xfer_layers(pd_xfer_t x, void* d_ws, const void* d_buf, size_t buf_bytes, uint32_t* progress,
                      void* stream, bool to_buffer) {
  if (!x || !d_ws || !d_buf) return fail(PD_ERR_INVALID_ARG, "NULL pointer argument");
  if (buf_bytes < pd_xfer_buffer_bytes(x)) return fail(PD_ERR_WORKSPACE, "buffer smaller than pd_xfer_buffer_bytes");
  uint32_t* prog = nullptr;
  pd_status s = progress_device_ptr(progress, &prog);
  if (s != PD_OK) return s;
  if (x->n == 0) return PD_OK;
  char* ws = (char*)d_ws;
  pdk::XferParams p{};
  p.buf = (char*)d_buf;
  p.layers = (void* const*)(ws + x->off_layers);
  p.page_ids = (const int32_t*)(ws + x->off_ids);
  p.done = (uint32_t*)(ws + x->off_done);
  p.progress = prog;
  p.page_bytes = page_bytes_of(&x->desc);
  p.half_bytes = p.page_bytes / 2;
  p.seg_off = head_seg_bytes(&x->desc, 0, x->h0);
  p.seg_bytes = head_seg_bytes(&x->desc, x->h0, x->h1);
  p.n = x->n;
  p.L = x->L;
  p.to_buffer = to_buffer ? 1 : 0;
  hipError_t e = pdk::launch_xfer(p, nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, to_buffer ? "layer pack launch" : "layer unpack launch");
  return PD_OK;
}
}  // namespace

namespace pdh {

pd_status set_error(pd_status s, const char* msg) { return fail(s, msg); }

pd_status hip_error(hipError_t e, const char* what) { return hip_fail(e, what); }

PlanImage plan_image(pd_plan_t plan) {
  PlanImage im{};
  im.tables = plan->blob.data();
  im.table_bytes = plan->meta_bytes;
  im.ws_bytes = plan->ws_bytes;
  im.mla = plan->mla;
  im.total_rows = plan->total_rows;
  return im;
}

pd_status enqueue_append(pd_plan_t plan, void* d_ws, void* kv_pool, const void* k_new, const void* v_new,
                         void* stream) {
  char* ws = (char*)d_ws;
  pdk::AppendParams p{};
  p.pool = kv_pool;
  p.k_new = k_new;
  p.v_new = v_new;
  p.rowpos = (const int2*)(ws + plan->off_rows);
  p.total_rows = plan->total_rows;
  p.H_kv = plan->desc.num_kv_heads;
  p.ps = plan->desc.page_size;
  p.D = plan->desc.head_dim;
  p.elt = elt_bytes(&plan->desc);
  const int row_bytes = 2 * p.H_kv * p.D * p.elt;
  p.rows_per_block = std::max(1, 16384 / row_bytes);  // about 16 KB per block
  hipError_t e = pdk::launch_append(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return PD_OK;
}

pd_status enqueue_attention(pd_plan_t plan, void* d_ws, const void* q, const void* kv_pool, float* out, float* lse,
                            void* stream) {
  pdk::AttnParams a = attn_params(*plan, d_ws);
  a.q = q;
  a.pool = kv_pool;
  a.out = out;
  a.lse = lse;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = pdk::launch_attention(a, plan->desc.dtype, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  e = pdk::launch_merge(a, st);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return PD_OK;
}

}  // namespace pdh

extern "C" {

pd_status pd_plan(const pd_attn_desc* desc, int32_t batch, const int32_t* qo_lens, const int32_t* kv_lens,
                  const int32_t* page_indptr, const int32_t* page_indices, int32_t num_pool_pages,
                  const pd_plan_options* opts, pd_plan_t* out) {
  try {
    if (!out) return fail(PD_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    pd_status s = check_desc(desc);
    if (s != PD_OK) return s;
    if (batch < 1) return fail(PD_ERR_INVALID_ARG, "batch must be >= 1");
    if (!qo_lens || !kv_lens || !page_indptr) return fail(PD_ERR_INVALID_ARG, "NULL length or indptr array");
    if (num_pool_pages < 0) return fail(PD_ERR_INVALID_ARG, "num_pool_pages must be >= 0");
    if (opts && (opts->decode_chunk_keys < 0 || opts->num_cus < 0))
      return fail(PD_ERR_INVALID_ARG, "negative planner option");
    if (opts && opts->block_order != 0 && opts->block_order != 1)
      return fail(PD_ERR_INVALID_ARG, "block_order must be 0 or 1");
    if (opts && opts->prefill_block_waves != 0 && opts->prefill_block_waves != 4 && opts->prefill_block_waves != 8)
      return fail(PD_ERR_INVALID_ARG, "prefill_block_waves must be 0, 4 or 8");
    pd_plan_s* P = new pd_plan_s();
    s = fill_requests(*P, desc->page_size, batch, qo_lens, kv_lens, page_indptr, page_indices, num_pool_pages);
    if (s != PD_OK) {
      delete P;
      return s;
    }
    P->desc = *desc;
    P->g = desc->num_qo_heads / desc->num_kv_heads;
    s = build_plan(*P, opts);
    if (s != PD_OK) {
      delete P;
      return s;
    }
    *out = P;
    return PD_OK;
  } catch (const std::bad_alloc&) {
    return fail(PD_ERR_NO_MEMORY, "host allocation failed");
  } catch (...) {
    return fail(PD_ERR_INVALID_ARG, "unexpected error while planning");
  }
}

size_t pd_plan_workspace_bytes(pd_plan_t plan) { return plan ? plan->ws_bytes : 0; }

pd_status pd_plan_get_stats(pd_plan_t plan, pd_plan_stats* out) {
  if (!plan || !out) return fail(PD_ERR_INVALID_ARG, "NULL argument");
  out->batch = plan->B;
  out->total_q_rows = plan->total_rows;
  out->prefill_tiles = (int32_t)plan->pf.size();
  out->decode_units = (int32_t)(plan->mla ? plan->mitems.size() : plan->du.size());
  if (plan->mla) {
    int32_t groups = 0;
    for (const auto& ri : plan->req)
      groups += (int32_t)(((int64_t)ri.qo * plan->mdesc.num_qo_heads + plan->mla_rows - 1) / plan->mla_rows);
    out->decode_row_groups = groups;
  } else {
    out->decode_row_groups = (int32_t)plan->mg.size();
  }
  out->decode_chunk_keys = plan->chunk_keys;
  out->prefill_flops = plan->prefill_flops;
  out->decode_kv_bytes = plan->decode_bytes;
  out->workspace_bytes = (int64_t)plan->ws_bytes;
  return PD_OK;
}

int32_t pd_plan_work_items(pd_plan_t plan, int32_t kind, int32_t* out, int32_t max_items) {
  if (!plan) return fail(PD_ERR_INVALID_ARG, "NULL plan");
  const int32_t* src;
  size_t count, width;
  switch (kind) {
    case 0: src = (const int32_t*)plan->pf.data(); count = plan->pf.size(); width = 8; break;
    case 1:
      if (plan->mla) {
        src = (const int32_t*)plan->mitems.data(); count = plan->mitems.size();
      } else {
        src = (const int32_t*)plan->du.data(); count = plan->du.size();
      }
      width = 8;
      break;
    case 2:
      if (plan->mla) {
        src = (const int32_t*)plan->mmg.data(); count = plan->mmg.size();
      } else {
        src = (const int32_t*)plan->mg.data(); count = plan->mg.size();
      }
      width = 4;
      break;
    case 3: src = plan->block_map.data(); count = plan->block_map.size(); width = 1; break;
    case 4:
      if (plan->mla) return fail(PD_ERR_INVALID_ARG, "an MLA plan has no decode queues");
      src = plan->dq.data(); count = plan->dq.size(); width = 1;
      break;
    default: return fail(PD_ERR_INVALID_ARG, "unknown work item kind");
  }
  if (max_items > 0 && out) {
    const size_t n = std::min(count, (size_t)max_items);
    std::memcpy(out, src, n * width * sizeof(int32_t));
  }
  return (int32_t)count;
}

pd_status pd_plan_upload(pd_plan_t plan, void* d_ws, size_t ws_bytes, void* stream) {
  try {
    if (!plan || !d_ws) return fail(PD_ERR_INVALID_ARG, "NULL plan or workspace");
    if (ws_bytes < plan->ws_bytes)
      return fail(PD_ERR_WORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes, plan needs " +
                                        std::to_string(plan->ws_bytes));
    return staged_upload(d_ws, plan->blob.data(), plan->meta_bytes, (hipStream_t)stream);
  } catch (...) {
    return fail(PD_ERR_HIP, "unexpected error in upload");
  }
}

void pd_plan_free(pd_plan_t plan) { delete plan; }

pd_status pd_kv_append(pd_plan_t plan, void* d_ws, void* kv_pool, const void* k_new, const void* v_new,
                       void* stream) {
  if (!plan || !d_ws) return fail(PD_ERR_INVALID_ARG, "NULL plan or workspace");
  if (plan->mla) return fail(PD_ERR_INVALID_ARG, "an MLA plan: use pd_mla_kv_append");
  if (plan->total_rows == 0) return PD_OK;
  if (!kv_pool || !k_new || !v_new) return fail(PD_ERR_INVALID_ARG, "NULL pool or K/V pointer");
  return pdh::enqueue_append(plan, d_ws, kv_pool, k_new, v_new, stream);
}

pd_status pd_attention_run(pd_plan_t plan, void* d_ws, const void* q, const void* kv_pool, float* out,
                           float* lse, void* stream) {
  if (!plan || !d_ws) return fail(PD_ERR_INVALID_ARG, "NULL plan or workspace");
  if (plan->mla) return fail(PD_ERR_INVALID_ARG, "an MLA plan: use pd_mla_attention_run");
  if (plan->total_rows == 0) return PD_OK;
  if (!q || !kv_pool || !out) return fail(PD_ERR_INVALID_ARG, "NULL q, pool or out");
  return pdh::enqueue_attention(plan, d_ws, q, kv_pool, out, lse, stream);
}

size_t pd_kv_pack_bytes(const pd_attn_desc* desc, int32_t n_pages) {
  if (n_pages < 0 || !desc) return 0;
  if (desc->num_kv_heads < 1 || desc->page_size < 1 || desc->head_dim < 1) return 0;
  if (desc->dtype != PD_F32 && desc->dtype != PD_BF16) return 0;
  return (size_t)n_pages * (size_t)page_bytes_of(desc);
}

pd_status pd_kv_pack(const pd_attn_desc* desc, const void* kv_pool, int32_t num_pool_pages,
                     const int32_t* page_ids, int32_t n, void* d_buf, size_t buf_bytes, void* d_scratch,
                     size_t scratch_bytes, void* stream) {
  try {
    const int32_t H = desc ? desc->num_kv_heads : 0;
    return xfer_common(desc, kv_pool, d_buf, num_pool_pages, page_ids, n, 0, H, buf_bytes, d_scratch,
                       scratch_bytes, stream, true);
  } catch (...) {
    return fail(PD_ERR_NO_MEMORY, "host allocation failed");
  }
}

pd_status pd_kv_unpack(const pd_attn_desc* desc, void* kv_pool, int32_t num_pool_pages,
                       const int32_t* page_ids, int32_t n, const void* d_buf, size_t buf_bytes,
                       void* d_scratch, size_t scratch_bytes, void* stream) {
  try {
    const int32_t H = desc ? desc->num_kv_heads : 0;
    return xfer_common(desc, kv_pool, d_buf, num_pool_pages, page_ids, n, 0, H, buf_bytes, d_scratch,
                       scratch_bytes, stream, false);
  } catch (...) {
    return fail(PD_ERR_NO_MEMORY, "host allocation failed");
  }
}

size_t pd_kv_pack_heads_bytes(const pd_attn_desc* desc, int32_t n_pages, int32_t h0, int32_t h1) {
  if (n_pages < 0 || !desc) return 0;
  if (desc->num_kv_heads < 1 || desc->page_size < 1 || desc->head_dim < 1) return 0;
  if (desc->dtype != PD_F32 && desc->dtype != PD_BF16) return 0;
  if (h0 < 0 || h1 > desc->num_kv_heads || h0 >= h1) return 0;
  return (size_t)n_pages * 2 * (size_t)head_seg_bytes(desc, h0, h1);
}

pd_status pd_kv_pack_heads(const pd_attn_desc* desc, const void* kv_pool, int32_t num_pool_pages,
                           const int32_t* page_ids, int32_t n, int32_t h0, int32_t h1, void* d_buf,
                           size_t buf_bytes, void* d_scratch, size_t scratch_bytes, void* stream) {
  try {
    return xfer_common(desc, kv_pool, d_buf, num_pool_pages, page_ids, n, h0, h1, buf_bytes, d_scratch,
                       scratch_bytes, stream, true);
  } catch (...) {
    return fail(PD_ERR_NO_MEMORY, "host allocation failed");
  }
}

pd_status pd_kv_unpack_heads(const pd_attn_desc* desc, void* kv_pool, int32_t num_pool_pages,
                             const int32_t* page_ids, int32_t n, int32_t h0, int32_t h1, const void* d_buf,
                             size_t buf_bytes, void* d_scratch, size_t scratch_bytes, void* stream) {
  try {
    return xfer_common(desc, kv_pool, d_buf, num_pool_pages, page_ids, n, h0, h1, buf_bytes, d_scratch,
                       scratch_bytes, stream, false);
  } catch (...) {
    return fail(PD_ERR_NO_MEMORY, "host allocation failed");
  }
}

pd_status pd_kv_shard_transfers(int32_t num_kv_heads, int32_t src_shards, int32_t dst_shards,
                                pd_head_transfer* out, int32_t max_out, int32_t* n_out) {
  if (!n_out) return fail(PD_ERR_INVALID_ARG, "n_out is NULL");
  *n_out = 0;
  if (num_kv_heads < 1 || src_shards < 1 || dst_shards < 1)
    return fail(PD_ERR_INVALID_ARG, "head and shard counts must be >= 1");
  if (num_kv_heads % src_shards || num_kv_heads % dst_shards)
    return fail(PD_ERR_UNSUPPORTED, "both shard counts must divide num_kv_heads (replicated KV heads "
                                    "are not supported)");
  const int32_t ps = num_kv_heads / src_shards, pd = num_kv_heads / dst_shards;
  int32_t k = 0;
  // source rank s holds heads [s ps, (s + 1) ps), destination rank d holds
  // [d pd, (d + 1) pd); every overlapping pair is one transfer per page
  for (int32_t s = 0; s < src_shards; ++s)
    for (int32_t d = 0; d < dst_shards; ++d) {
      const int32_t lo = std::max(s * ps, d * pd), hi = std::min((s + 1) * ps, (d + 1) * pd);
      if (lo >= hi) continue;
      if (out && k < max_out) out[k] = {s, d, lo - s * ps, hi - s * ps, lo - d * pd, hi - d * pd};
      ++k;
    }
  *n_out = k;
  if (out && k > max_out) return fail(PD_ERR_WORKSPACE, "out holds fewer than " + std::to_string(k) + " entries");
  return PD_OK;
}

pd_status pd_xfer_plan(const pd_attn_desc* desc, int32_t num_layers, void* const* kv_pools,
                       int32_t num_pool_pages, const int32_t* page_ids, int32_t n, int32_t h0, int32_t h1,
                       pd_xfer_t* out) {
  try {
    if (!out) return fail(PD_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    pd_status s = check_desc(desc);
    if (s != PD_OK) return s;
    if ((s = check_heads(desc, h0, h1)) != PD_OK) return s;
    if (num_layers < 1 || num_layers > kMaxXferLayers)
      return fail(PD_ERR_INVALID_ARG, "num_layers must be in [1, " + std::to_string(kMaxXferLayers) + "]");
    if (n < 0) return fail(PD_ERR_INVALID_ARG, "n must be >= 0");
    if (!kv_pools || (n > 0 && !page_ids)) return fail(PD_ERR_INVALID_ARG, "NULL pointer argument");
    for (int32_t l = 0; l < num_layers; ++l)
      if (!kv_pools[l]) return fail(PD_ERR_INVALID_ARG, "pool of layer " + std::to_string(l) + " is NULL");
    if ((s = check_ids(num_pool_pages, page_ids, n)) != PD_OK) return s;
    pd_xfer_s* x = new pd_xfer_s;
    x->desc = *desc;
    x->L = num_layers;
    x->n = n;
    x->h0 = h0;
    x->h1 = h1;
    size_t off = 0;
    x->off_layers = off;
    off = align_up(off + sizeof(void*) * (size_t)num_layers);
    x->off_ids = off;
    off = align_up(off + sizeof(int32_t) * (size_t)n);
    x->off_done = off;
    off = align_up(off + sizeof(uint32_t) * (size_t)num_layers);
    x->ws_bytes = off;
    x->blob.assign(off, 0);
    std::memcpy(x->blob.data() + x->off_layers, kv_pools, sizeof(void*) * (size_t)num_layers);
    if (n) std::memcpy(x->blob.data() + x->off_ids, page_ids, sizeof(int32_t) * (size_t)n);
    *out = x;
    return PD_OK;
  } catch (...) {
    return fail(PD_ERR_NO_MEMORY, "host allocation failed");
  }
}

size_t pd_xfer_buffer_bytes(pd_xfer_t x) {
  if (!x) return 0;
  return (size_t)x->L * (size_t)x->n * 2 * (size_t)head_seg_bytes(&x->desc, x->h0, x->h1);
}

size_t pd_xfer_workspace_bytes(pd_xfer_t x) { return x ? x->ws_bytes : 0; }

pd_status pd_xfer_upload(pd_xfer_t x, void* d_ws, size_t ws_bytes, void* stream) {
  if (!x || !d_ws) return fail(PD_ERR_INVALID_ARG, "NULL pointer argument");
  if (ws_bytes < x->ws_bytes) return fail(PD_ERR_WORKSPACE, "workspace smaller than pd_xfer_workspace_bytes");
  try {
    return staged_upload(d_ws, x->blob.data(), x->ws_bytes, (hipStream_t)stream);
  } catch (...) {
    return fail(PD_ERR_HIP, "unexpected error in upload");
  }
}


pd_status pd_kv_pack_layers(pd_xfer_t x, void* d_ws, void* d_buf, size_t buf_bytes, uint32_t* progress,
                            void* stream) {
  return xfer_layers(x, d_ws, d_buf, buf_bytes, progress, stream, true);
}

pd_status pd_kv_unpack_layers(pd_xfer_t x, void* d_ws, const void* d_buf, size_t buf_bytes, uint32_t* progress,
                              void* stream) {
  return xfer_layers(x, d_ws, d_buf, buf_bytes, progress, stream, false);
}

void pd_xfer_free(pd_xfer_t x) { delete x; }

size_t pd_mla_page_bytes(const pd_mla_desc* desc) {
  if (!desc || desc->page_size < 1 || desc->kv_lora_rank < 1 || desc->qk_rope_dim < 0) return 0;
  return (size_t)mla_page_bytes_of(desc);
}

pd_status pd_mla_plan(const pd_mla_desc* desc, int32_t batch, const int32_t* qo_lens, const int32_t* kv_lens,
                      const int32_t* page_indptr, const int32_t* page_indices, int32_t num_pool_pages,
                      const pd_plan_options* opts, pd_plan_t* out) {
  try {
    if (!out) return fail(PD_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    pd_status s = check_mla_desc(desc);
    if (s != PD_OK) return s;
    if (batch < 1) return fail(PD_ERR_INVALID_ARG, "batch must be >= 1");
    if (!qo_lens || !kv_lens || !page_indptr) return fail(PD_ERR_INVALID_ARG, "NULL length or indptr array");
    if (num_pool_pages < 0) return fail(PD_ERR_INVALID_ARG, "num_pool_pages must be >= 0");
    if (opts && (opts->decode_chunk_keys < 0 || opts->num_cus < 0))
      return fail(PD_ERR_INVALID_ARG, "negative planner option");
    pd_plan_s* P = new pd_plan_s();
    s = fill_requests(*P, desc->page_size, batch, qo_lens, kv_lens, page_indptr, page_indices, num_pool_pages);
    if (s == PD_OK) {
      P->mla = true;
      P->mdesc = *desc;
      s = build_mla_plan(*P, opts);
    }
    if (s != PD_OK) {
      delete P;
      return s;
    }
    *out = P;
    return PD_OK;
  } catch (const std::bad_alloc&) {
    return fail(PD_ERR_NO_MEMORY, "host allocation failed");
  } catch (...) {
    return fail(PD_ERR_INVALID_ARG, "unexpected error while planning");
  }
}

pd_status pd_mla_kv_append(pd_plan_t plan, void* d_ws, void* kv_pool, const void* rows_new, void* stream) {
  if (!plan || !d_ws) return fail(PD_ERR_INVALID_ARG, "NULL plan or workspace");
  if (!plan->mla) return fail(PD_ERR_INVALID_ARG, "not an MLA plan: use pd_kv_append");
  if (plan->total_rows == 0) return PD_OK;
  if (!kv_pool || !rows_new) return fail(PD_ERR_INVALID_ARG, "NULL pool or rows pointer");
  pdk::MlaParams a = mla_params(*plan, d_ws);
  hipError_t e = pdk::launch_mla_append(a, kv_pool, rows_new, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "MLA append launch");
  return PD_OK;
}

pd_status pd_mla_attention_run(pd_plan_t plan, void* d_ws, const void* q, const void* kv_pool, float* out,
                               float* lse, void* stream) {
  if (!plan || !d_ws) return fail(PD_ERR_INVALID_ARG, "NULL plan or workspace");
  if (!plan->mla) return fail(PD_ERR_INVALID_ARG, "not an MLA plan: use pd_attention_run");
  if (plan->total_rows == 0) return PD_OK;
  if (!q || !kv_pool || !out) return fail(PD_ERR_INVALID_ARG, "NULL q, pool or out");
  pdk::MlaParams a = mla_params(*plan, d_ws);
  a.q = q;
  a.pool = kv_pool;
  a.out = out;
  a.lse = lse;
  hipError_t e = pdk::launch_mla(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "MLA attention launch");
  return PD_OK;
}

namespace {
pd_status mla_xfer(const pd_mla_desc* desc, const void* pool, const void* buf, int32_t num_pool_pages,
                   const int32_t* ids, int32_t n, size_t buf_bytes, void* scratch, size_t scratch_bytes,
                   void* stream, bool to_buffer) {
  pd_status s = check_mla_desc(desc);
  if (s != PD_OK) return s;
  if (n < 0) return fail(PD_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return PD_OK;
  if (!ids || !pool || !buf || !scratch) return fail(PD_ERR_INVALID_ARG, "NULL pointer argument");
  const int64_t pb = mla_page_bytes_of(desc);
  if (buf_bytes < (size_t)n * (size_t)pb) return fail(PD_ERR_WORKSPACE, "buffer smaller than the n pages");
  if (scratch_bytes < sizeof(int32_t) * (size_t)n) return fail(PD_ERR_WORKSPACE, "scratch smaller than 4 * n bytes");
  if ((s = check_ids(num_pool_pages, ids, n)) != PD_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const bool inline_ids = n <= pdk::kXferInlineIds;
  if (!inline_ids && (s = staged_upload(scratch, ids, sizeof(int32_t) * (size_t)n, st)) != PD_OK) return s;
  pdk::XferParams p{};
  p.buf = (char*)buf;
  p.pool0 = (void*)pool;
  p.page_ids = (const int32_t*)scratch;
  p.page_bytes = pb;
  p.half_bytes = pb / 2;  // a page moves as two halves of one contiguous image
  p.seg_off = 0;
  p.seg_bytes = pb / 2;
  p.n = n;
  p.L = 1;
  p.to_buffer = to_buffer ? 1 : 0;
  hipError_t e = pdk::launch_xfer(p, inline_ids ? ids : nullptr, st);
  if (e != hipSuccess) return hip_fail(e, to_buffer ? "MLA pack launch" : "MLA unpack launch");
  return PD_OK;
}
}  // namespace

pd_status pd_mla_kv_pack(const pd_mla_desc* desc, const void* kv_pool, int32_t num_pool_pages,
                         const int32_t* page_ids, int32_t n, void* d_buf, size_t buf_bytes, void* d_scratch,
                         size_t scratch_bytes, void* stream) {
  try {
    return mla_xfer(desc, kv_pool, d_buf, num_pool_pages, page_ids, n, buf_bytes, d_scratch, scratch_bytes, stream,
                    true);
  } catch (...) {
    return fail(PD_ERR_NO_MEMORY, "host allocation failed");
  }
}

pd_status pd_mla_kv_unpack(const pd_mla_desc* desc, void* kv_pool, int32_t num_pool_pages,
                           const int32_t* page_ids, int32_t n, const void* d_buf, size_t buf_bytes,
                           void* d_scratch, size_t scratch_bytes, void* stream) {
  try {
    return mla_xfer(desc, kv_pool, d_buf, num_pool_pages, page_ids, n, buf_bytes, d_scratch, scratch_bytes, stream,
                    false);
  } catch (...) {
    return fail(PD_ERR_NO_MEMORY, "host allocation failed");
  }
}

const char* pd_status_string(pd_status s) {
  switch (s) {
    case PD_OK: return "PD_OK";
    case PD_ERR_INVALID_ARG: return "PD_ERR_INVALID_ARG";
    case PD_ERR_UNSUPPORTED: return "PD_ERR_UNSUPPORTED";
    case PD_ERR_OUT_OF_RANGE: return "PD_ERR_OUT_OF_RANGE";
    case PD_ERR_WORKSPACE: return "PD_ERR_WORKSPACE";
    case PD_ERR_HIP: return "PD_ERR_HIP";
    case PD_ERR_NO_MEMORY: return "PD_ERR_NO_MEMORY";
  }
  return "unknown pd_status";
}

const char* pd_last_error(void) { return g_last_error.c_str(); }

const char* pd_version(void) { return "pd_attn 0.1.0 (gfx950)"; }

}  // extern "C"
