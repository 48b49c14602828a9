/*
 * pd_attn.h -- C ABI of the MI355X (gfx950) ragged paged-attention library
 * libpd_attn.so.
 *
 * The library runs the attention hot path behind disaggregated prefill and
 * decode on one GPU:
 *   pd_plan          split a ragged batch of requests into GPU work
 *   pd_kv_append     write each request's new K/V rows into its pages
 *   pd_attention_run causal prefill rows and decode rows in one launch, then
 *                    the merge of split-KV partial results
 *   pd_kv_pack       gather whole pages into one contiguous transfer buffer
 *   pd_kv_unpack     scatter such a buffer into (other) pages
 *   pd_kv_pack_heads, pd_kv_unpack_heads, pd_kv_shard_transfers
 *                    the same for a range of KV heads of each page, and the
 *                    head ranges that move between differently sharded ranks
 *   pd_xfer_plan, pd_kv_pack_layers, pd_kv_unpack_layers
 *                    several layers' pages in one launch, with a per-layer
 *                    completion counter a host thread can poll
 *   pd_mla_plan, pd_mla_kv_append, pd_mla_attention_run, pd_mla_kv_pack,
 *   pd_mla_kv_unpack
 *                    the same steps for a latent (MLA) KV cache: one row
 *                    per token shared by every query head
 *
 * What the operations compute follows the Perplexity post "Disaggregated
 * prefill and decode" and the kwkr.cn PD-disaggregation survey; each entry
 * point names the passage it follows.  The attention itself is standard
 * scaled-dot-product softmax attention:
 *   for request r with qo new query rows over kv cached keys, query row i sits
 *   at absolute position p = kv - qo + i and (when causal) sees keys j <= p;
 *   query head h reads KV head h / g, g = num_qo_heads / num_kv_heads;
 *   O[i,h] = sum_j softmax_j(sm_scale * <Q[i,h], K[j,h/g]>) V[j,h/g]
 *   LSE[i,h] = ln sum_j exp(sm_scale * <Q[i,h], K[j,h/g]>)   (natural log)
 *
 * Memory layouts (all row-major, C order):
 *   KV pool   [num_pool_pages][2][num_kv_heads][page_size][head_dim] elements
 *             (K half then V half of each page; "HND": heads before tokens,
 *             so a page, and each head's slice of it, is contiguous -- post,
 *             section "Sharded KV Cache Transfers").  Token t of request r is
 *             in page page_indices[page_indptr[r] + t / page_size] at slot
 *             t % page_size.
 *   q         [sum qo][num_qo_heads][head_dim], requests back to back
 *   k_new,
 *   v_new     [sum qo][num_kv_heads][head_dim], requests back to back
 *   out       [sum qo][num_qo_heads][head_dim] float32
 *   lse       [sum qo][num_qo_heads] float32
 *   element type: float32 (PD_F32) or bfloat16 (PD_BF16) for the pool, q,
 *   k_new and v_new; out and lse are always float32 (fp32 accumulation).
 *
 * Ownership: the caller allocates and owns every device buffer (pool, q,
 * k_new, v_new, out, lse, workspace, pack buffer, scratch); the library never
 * allocates or frees device memory.  The library owns the opaque plan (host
 * memory), released by pd_plan_free, and a process-wide pool of pinned host
 * staging blocks for uploads, reused across plans and never released.  A plan
 * is immutable once built; pd_plan_upload may be called again on another
 * workspace.
 *
 * Streams: every `void* stream` is a hipStream_t (NULL = the default stream);
 * all device work is enqueued on it and no call waits for the device.
 *
 * Errors: every argument is checked before anything is enqueued, so a failing
 * call has no side effect on device memory.  Calls return PD_OK or a negative
 * pd_status; pd_last_error() gives a message for the calling thread's last
 * failure.  No C++ exception crosses this interface.
 */
#ifndef PD_ATTN_H_
#define PD_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pd_status {
  PD_OK = 0,
  PD_ERR_INVALID_ARG = -1,  /* malformed lengths, page table, null pointer */
  PD_ERR_UNSUPPORTED = -2,  /* head_dim, page_size, dtype or group size the
                               kernels do not implement */
  PD_ERR_OUT_OF_RANGE = -3, /* page id outside the pool */
  PD_ERR_WORKSPACE = -4,    /* workspace / buffer / scratch too small */
  PD_ERR_HIP = -5,          /* a HIP runtime call or kernel launch failed */
  PD_ERR_NO_MEMORY = -6     /* host allocation failed */
} pd_status;

typedef enum pd_dtype { PD_F32 = 0, PD_BF16 = 1 } pd_dtype;

/* Shape of one attention layer.
 *   num_qo_heads  query heads H_q (> 0, multiple of num_kv_heads)
 *   num_kv_heads  KV heads H_kv (> 0); g = H_q / H_kv <= 256
 *   head_dim      64 or 128
 *   page_size     16, 32, 64 or 128 tokens per page
 *   dtype         pd_dtype of pool, q, k_new, v_new
 *   causal        1: end-aligned causal mask; 0: every row sees all kv keys
 *   sm_scale      softmax scale applied to <q, k> (usually 1/sqrt(head_dim)) */
typedef struct pd_attn_desc {
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t dtype;
  int32_t causal;
  float sm_scale;
} pd_attn_desc;

/* Optional planner controls (NULL = defaults).
 *   decode_chunk_keys  0 (default): when the launch has fewer prefill tiles
 *                      than compute units and one round of queues on the
 *                      CUs they leave free would end within the longest
 *                      prefill tile (priced at measured MI355X rates), the
 *                      decode row groups are laid end to end and cut into
 *                      equal spans of keys, one per wavefront queue (a
 *                      queue holds the units its span crosses); otherwise
 *                      each group is cut into equal chunks, one unit each,
 *                      sized so that a block of eight chunks lasts about
 *                      as long as the launch's mean prefill tile.
 *                      > 0: every group is cut into chunks of about this
 *                      many keys (rounded up to 32, at most the longest
 *                      cache), one unit per queue
 *   num_cus            compute units to balance over; 0 = 256 (MI355X)
 *   block_order        order of the blocks of the attention launch:
 *                      0 = interleave prefill and decode rounds by their
 *                          cost at peak rates (default: CUs running decode
 *                          blocks stream the cache while the others run
 *                          prefill tiles); 1 = all prefill tiles, then all
 *                          decode blocks
 *   prefill_block_waves 0 (default): a launch with no decode rows whose
 *                      prefill requests all have at most 4096 cached keys
 *                      (short prompts) runs 128-row query tiles in blocks of
 *                      4 wavefronts, two blocks per compute unit, so that
 *                      one block's first loads overlap the other's work;
 *                      any other launch runs 256-row tiles in blocks of 8.
 *                      4: the 4-wavefront form whenever the launch has no
 *                      decode rows (and g <= 128); 8: always 256-row tiles */
typedef struct pd_plan_options {
  int32_t decode_chunk_keys;
  int32_t num_cus;
  int32_t block_order;
  int32_t prefill_block_waves;
  int32_t reserved[4];
} pd_plan_options;

/* Plan statistics (pd_plan_get_stats). */
typedef struct pd_plan_stats {
  int32_t batch;
  int32_t total_q_rows;        /* sum qo */
  int32_t prefill_tiles;       /* MFMA query tiles (rows of prefill requests) */
  int32_t decode_units;        /* split-KV units */
  int32_t decode_row_groups;   /* (request, kv head) groups merged */
  int32_t decode_chunk_keys;   /* the decode_chunk_keys option as applied,
                                  else the longest decode unit */
  int64_t prefill_flops;       /* 4 * head_dim * H_q * visible (query, key)
                                  pairs of the prefill rows (algorithmic) */
  int64_t decode_kv_bytes;     /* K + V bytes the decode rows read */
  int64_t workspace_bytes;
} pd_plan_stats;

typedef struct pd_plan_s* pd_plan_t;

/* Build a plan for one step of a ragged batch.  Host only, synchronous; no
 * HIP call is made.
 *   batch          number of requests B (>= 1)
 *   qo_lens[B]     new query tokens of each request (>= 0; 0 = no rows)
 *   kv_lens[B]     cached tokens of each request *including* the new ones
 *                  (0 <= qo <= kv): the new rows are appended at positions
 *                  [kv - qo, kv) before attention reads [0, kv)
 *   page_indptr[B+1], page_indices[page_indptr[B]]
 *                  CSR page table; request r owns exactly ceil(kv_r /
 *                  page_size) pages, in token order; every id is in
 *                  [0, num_pool_pages) and no id appears twice
 *   opts           may be NULL
 *   out            receives the plan (release with pd_plan_free)
 * Follows the post's statement of the problem (section "Prefill vs Decode
 * performance"): each step batches prefill requests (many query tokens,
 * compute bound) with decode requests (qo_len = 1, bound by reading the
 * kv_len-long cache), and attention is spread over both the requests and
 * their kv_len to keep the device busy.  A request whose qo * g query rows
 * per KV head number at most 64 (single-token decode at g <= 64, or a
 * multi-token step such as 4 tokens at g = 8) is split over its kv_len into
 * decode units of 16 or 32 rows, one wavefront each (two side by side on the
 * same keys above 32 rows), whose partial results are merged afterwards; the
 * rows of every other request become causal MFMA query tiles of up to 256
 * rows, each over its whole causal key range.
 * Errors: PD_ERR_INVALID_ARG (null pointers, batch < 1, negative lengths,
 * qo > kv, wrong page count, duplicate page id, H_q % H_kv != 0),
 * PD_ERR_OUT_OF_RANGE (page id outside the pool), PD_ERR_UNSUPPORTED
 * (head_dim, page_size, dtype), PD_ERR_NO_MEMORY. */
pd_status pd_plan(const pd_attn_desc* desc, int32_t batch,
                  const int32_t* qo_lens, const int32_t* kv_lens,
                  const int32_t* page_indptr, const int32_t* page_indices,
                  int32_t num_pool_pages, const pd_plan_options* opts,
                  pd_plan_t* out);

/* Device workspace bytes the plan needs (page table, work lists, split-KV
 * partial results).  0 for a NULL plan. */
size_t pd_plan_workspace_bytes(pd_plan_t plan);

/* Copy the plan's tables into the caller's device workspace: the tables are
 * copied into a free pinned staging block before the call returns, and the
 * host-to-device copy is enqueued on `stream`.
 * Must precede pd_kv_append / pd_attention_run with the same d_ws.
 * Errors: PD_ERR_INVALID_ARG (null plan / d_ws), PD_ERR_WORKSPACE
 * (ws_bytes < pd_plan_workspace_bytes), PD_ERR_HIP. */
pd_status pd_plan_upload(pd_plan_t plan, void* d_ws, size_t ws_bytes,
                         void* stream);

/* Statistics of a plan (host only). */
pd_status pd_plan_get_stats(pd_plan_t plan, pd_plan_stats* out);

/* Diagnostics: copy the plan's work list (host only).
 *   kind 0: prefill tiles, 8 int32 each:
 *           {request, kv_head, first token, tokens, key end (exclusive), 0,0,0}
 *   kind 1: decode units in queue order, 8 int32 each:
 *           {request, kv_head, key begin, key end (exclusive), partial row,
 *            first row c0, 16-row column groups, paired}: rows [c0, c0 + 16 *
 *           groups) of the (request, KV head)'s qo * g rows; row c0 + i
 *           writes partial row + i; paired = 1 for groups of more than 32
 *           rows, whose two halves run in adjacent wavefronts of one block
 *           (the same units in the same order) and share their V stages
 *   kind 2: merge groups, 4 int32 each:
 *           {request, kv_head, first partial row, chunk count}; chunk i's
 *           result for row n is partial row first + i * qo g + n
 *   kind 3: the attention launch's blocks in launch order, 1 int32 each:
 *           v >= 0 is prefill tile v, v < 0 is decode block -v - 1
 *   kind 4: decode queue offsets, 1 int32 each (wavefront slots + 1
 *           entries): wavefront w of decode block b runs the units
 *           [q[8 b + w], q[8 b + w + 1]) of kind 1, one after the other
 * Writes at most max_items items to out (which may be NULL when max_items is
 * 0) and returns the total number of items of that kind, or a negative
 * pd_status (PD_ERR_INVALID_ARG for a NULL plan or an unknown kind). */
int32_t pd_plan_work_items(pd_plan_t plan, int32_t kind, int32_t* out,
                           int32_t max_items);

/* Release a plan (host memory only; uploads already enqueued are not
 * affected).  NULL is a no-op. */
void pd_plan_free(pd_plan_t plan);

/* Append the step's new K and V rows into the pool: for each request r and
 * i < qo_r, row i of its k_new / v_new block goes to token position
 * kv_r - qo_r + i.  Bit-exact copy; touches no other slot.  The post's
 * section "KV Messenger": KV entries are appended to the cache layer by
 * layer and are valid after the append and before attention.
 *   d_ws    workspace the plan was uploaded to
 *   kv_pool device pool (layout above)
 *   k_new, v_new  device [sum qo][num_kv_heads][head_dim]
 * Errors: PD_ERR_INVALID_ARG (null pointer), PD_ERR_HIP. */
pd_status pd_kv_append(pd_plan_t plan, void* d_ws, void* kv_pool,
                       const void* k_new, const void* v_new, void* stream);

/* Attention of every query row of the plan over its request's cache [0, kv).
 * Prefill tiles and decode units run in one launch; a second launch merges
 * the decode units' split-KV partial results (log-sum-exp weighted, fixed
 * order, so a fixed plan gives bitwise-reproducible output).  The post's
 * section "Prefill vs Decode performance" (prefill and decode requests
 * batched together; attention parallel over requests and kv_len) and the
 * kwkr.cn survey, section 8 (a prefill chunk attends over all earlier KV).
 *   q        device [sum qo][num_qo_heads][head_dim]
 *   kv_pool  device pool after pd_kv_append
 *   out      device float32 [sum qo][num_qo_heads][head_dim]
 *   lse      device float32 [sum qo][num_qo_heads], or NULL
 * Tail slots of a request's last page and pages outside its list are never
 * read.  Errors: PD_ERR_INVALID_ARG (null pointer), PD_ERR_HIP. */
pd_status pd_attention_run(pd_plan_t plan, void* d_ws, const void* q,
                           const void* kv_pool, float* out, float* lse,
                           void* stream);

/* Bytes of n packed pages: n * 2 * num_kv_heads * page_size * head_dim *
 * element size.  0 on a bad descriptor or n < 0. */
size_t pd_kv_pack_bytes(const pd_attn_desc* desc, int32_t n_pages);

/* Gather whole pages, in list order, into one contiguous buffer of verbatim
 * page images (bit-exact).  The post's sections "KV Messenger" and "Sharded
 * KV Cache Transfers": transfers are per page, each HND page being one
 * contiguous write, and their number is proportional to the pages moved; a
 * request's whole page list at once is the request-level transfer
 * granularity of the kwkr.cn survey, section 5.4.
 *   page_ids   HOST array of n page ids in [0, num_pool_pages), no repeats;
 *              up to 896 ids travel in the kernel arguments, longer lists
 *              are copied to d_scratch on `stream`; either way the array
 *              may be reused once the call returns
 *   d_buf      device buffer of buf_bytes >= pd_kv_pack_bytes(desc, n)
 *   d_scratch  device scratch of scratch_bytes >= 4 * n (written only when
 *              n > 896)
 * Errors: PD_ERR_INVALID_ARG, PD_ERR_OUT_OF_RANGE, PD_ERR_WORKSPACE,
 * PD_ERR_UNSUPPORTED, PD_ERR_HIP.  n == 0 is a no-op. */
pd_status pd_kv_pack(const pd_attn_desc* desc, const void* kv_pool,
                     int32_t num_pool_pages, const int32_t* page_ids,
                     int32_t n, void* d_buf, size_t buf_bytes,
                     void* d_scratch, size_t scratch_bytes, void* stream);

/* Scatter a packed buffer: buffer page i is written verbatim to pool page
 * page_ids[i].  The destination ids are the receiver's own pages and may
 * differ from the ids the buffer was packed from (post, section "KV
 * Messenger": the decoder allocates its pages before the transfer).
 * Arguments and errors as pd_kv_pack. */
pd_status pd_kv_unpack(const pd_attn_desc* desc, void* kv_pool,
                       int32_t num_pool_pages, const int32_t* page_ids,
                       int32_t n, const void* d_buf, size_t buf_bytes,
                       void* d_scratch, size_t scratch_bytes, void* stream);

/* ---- Sharded transfers (post, section "Sharded KV Cache Transfers") ----
 * When the prefiller and the decoder split the KV heads over different
 * numbers of tensor-parallel ranks, pages are split or rebuilt: each transfer
 * moves one contiguous range of KV heads of every listed page.  In an HND
 * page such a range is two contiguous runs, its K part and its V part.  The
 * pool passed here is one rank's pool (desc->num_kv_heads = that rank's
 * heads) and [h0, h1) are local head indices of it. */

/* Bytes of the head-[h0, h1) slices of n pages:
 * n * 2 * (h1 - h0) * page_size * head_dim * element size.  0 on a bad
 * descriptor, n < 0 or an empty / out-of-range head range. */
size_t pd_kv_pack_heads_bytes(const pd_attn_desc* desc, int32_t n_pages,
                              int32_t h0, int32_t h1);

/* Gather KV heads [h0, h1) of the listed pages, in list order, into a
 * contiguous buffer [n][2][h1 - h0][page_size][head_dim] (K slice then V
 * slice of each page; bit-exact).  h0 = 0, h1 = num_kv_heads is pd_kv_pack.
 *   page_ids   HOST array of n page ids in [0, num_pool_pages), no repeats;
 *              passed as in pd_kv_pack (kernel arguments up to 896 ids,
 *              else staged through pinned memory to d_scratch on `stream`)
 *   d_buf      device buffer of buf_bytes >= pd_kv_pack_heads_bytes(...)
 *   d_scratch  device scratch of scratch_bytes >= 4 * n
 * Errors: PD_ERR_INVALID_ARG (head range not within [0, num_kv_heads) or
 * empty, NULL pointer, repeated id), PD_ERR_OUT_OF_RANGE, PD_ERR_WORKSPACE,
 * PD_ERR_UNSUPPORTED, PD_ERR_HIP.  n == 0 is a no-op. */
pd_status pd_kv_pack_heads(const pd_attn_desc* desc, const void* kv_pool,
                           int32_t num_pool_pages, const int32_t* page_ids,
                           int32_t n, int32_t h0, int32_t h1, void* d_buf,
                           size_t buf_bytes, void* d_scratch,
                           size_t scratch_bytes, void* stream);

/* Scatter such a buffer into KV heads [h0, h1) of the listed (receiver's)
 * pages; the page's other heads are not touched, so a full page is rebuilt
 * from the slices of several senders.  Arguments and errors as
 * pd_kv_pack_heads. */
pd_status pd_kv_unpack_heads(const pd_attn_desc* desc, void* kv_pool,
                             int32_t num_pool_pages, const int32_t* page_ids,
                             int32_t n, int32_t h0, int32_t h1,
                             const void* d_buf, size_t buf_bytes,
                             void* d_scratch, size_t scratch_bytes,
                             void* stream);

/* One transfer of a sharded handoff: heads [src_h0, src_h1) of the source
 * rank's pool (local indices) go to heads [dst_h0, dst_h1) of the destination
 * rank's pool. */
typedef struct pd_head_transfer {
  int32_t src_rank, dst_rank;
  int32_t src_h0, src_h1;
  int32_t dst_h0, dst_h1;
} pd_head_transfer;

/* The transfers that move num_kv_heads KV heads, split evenly and in order
 * (rank r holds heads [r H / S, (r + 1) H / S)) over src_shards prefiller
 * ranks, to dst_shards decoder ranks: one entry per overlapping (source,
 * destination) pair, sources in rank order.  A destination page expects one
 * write per entry naming its rank -- the count the decoder has to know
 * (s / d "halves" when the prefiller has s = k d ranks, one write when the
 * decoder has more ranks).  Host only.
 *   out, max_out   caller array (may be NULL to query the count)
 *   n_out          number of transfers
 * Errors: PD_ERR_INVALID_ARG (counts < 1, n_out NULL), PD_ERR_UNSUPPORTED
 * (a shard count that does not divide num_kv_heads: replicated KV heads),
 * PD_ERR_WORKSPACE (max_out too small; *n_out still set). */
pd_status pd_kv_shard_transfers(int32_t num_kv_heads, int32_t src_shards,
                                int32_t dst_shards, pd_head_transfer* out,
                                int32_t max_out, int32_t* n_out);

/* ---- Multi-layer transfers with a completion counter ----
 * The post's section "KV Messenger": copies of a layer's pages start as soon
 * as that layer's KV has been appended, and a dedicated host thread polls a
 * counter to learn how far the GPU has got, which keeps the step
 * graph-capturable.  A transfer plan fixes the L layer pools, the page list
 * and the head range once (host only); its small table is uploaded to a
 * caller workspace; each pack then is ONE launch over all L layers, whose
 * blocks run layer after layer, and each layer bumps its own counter when
 * its last block has finished.
 *
 * Buffer: [L][n][2][h1 - h0][page_size][head_dim] (layer after layer, each
 * layer as pd_kv_pack_heads).  Progress: NULL, or an array of L uint32 in
 * pinned host memory (hipHostMalloc, polled by the host) or in device
 * memory.  Entry l is read and incremented by one (release store at system
 * scope) once every page of layer l has been copied and made visible; the
 * library never resets it, so values keep counting across calls and graph
 * replays (call c of a plan has finished layer l when progress[l] >=
 * start + c).  The workspace's block counters return to zero at the end of
 * each call; nothing is cleared with a memset.  Calls that share a workspace
 * must not overlap. */
typedef struct pd_xfer_s* pd_xfer_t;

/* Build a transfer plan (host only, no HIP call).
 *   kv_pools   HOST array of num_layers device pointers, one pool per layer,
 *              all [num_pool_pages][2][num_kv_heads][page_size][head_dim]
 *   page_ids   HOST array of n distinct page ids (copied into the plan)
 *   [h0, h1)   KV heads moved from every page (0, num_kv_heads: whole pages)
 * Errors: PD_ERR_INVALID_ARG (num_layers not in [1, 4096], NULL pools, bad
 * head range, repeated id), PD_ERR_OUT_OF_RANGE, PD_ERR_UNSUPPORTED,
 * PD_ERR_NO_MEMORY. */
pd_status pd_xfer_plan(const pd_attn_desc* desc, int32_t num_layers,
                       void* const* kv_pools, int32_t num_pool_pages,
                       const int32_t* page_ids, int32_t n, int32_t h0,
                       int32_t h1, pd_xfer_t* out);

/* Bytes of the plan's transfer buffer (0 for a NULL plan). */
size_t pd_xfer_buffer_bytes(pd_xfer_t xfer);

/* Bytes of device workspace the plan needs (pool pointers, ids, counters). */
size_t pd_xfer_workspace_bytes(pd_xfer_t xfer);

/* Copy the plan's table into d_ws (async on `stream`, from pinned staging
 * memory the library owns) and set its block counters to zero.  Do it once,
 * outside any graph capture, before the first pack / unpack with d_ws.
 * Errors: PD_ERR_INVALID_ARG, PD_ERR_WORKSPACE, PD_ERR_HIP. */
pd_status pd_xfer_upload(pd_xfer_t xfer, void* d_ws, size_t ws_bytes,
                         void* stream);

/* Pack every layer's page slices into d_buf: one launch, no host-to-device
 * copy, no memset (capturable into a HIP graph).  progress: see above.
 * Errors: PD_ERR_INVALID_ARG (NULL plan / workspace / buffer, progress that
 * is neither pinned host nor device memory), PD_ERR_WORKSPACE (buffer too
 * small), PD_ERR_HIP. */
pd_status pd_kv_pack_layers(pd_xfer_t xfer, void* d_ws, void* d_buf,
                            size_t buf_bytes, uint32_t* progress,
                            void* stream);

/* The inverse on a receiver: write the buffer's slices into the plan's page
 * ids of every layer pool (the receiver's own ids and pools), heads
 * [h0, h1) only.  Arguments and errors as pd_kv_pack_layers. */
pd_status pd_kv_unpack_layers(pd_xfer_t xfer, void* d_ws, const void* d_buf,
                              size_t buf_bytes, uint32_t* progress,
                              void* stream);

/* Release a transfer plan (host memory only). */
void pd_xfer_free(pd_xfer_t xfer);

/* ---- MLA decode over a latent KV cache --------------------------------
 * Perplexity, "Disaggregated prefill and decode", section "DeepSeek-R1"
 * (under "Disaggregated Deployments"): multi-head latent attention compresses
 * every KV head of a token into one latent vector, so tensor parallelism
 * cannot split the cache by heads.  Every rank holds the same latent cache,
 * and the heads are only separated after decompression.  The pages give no
 * formula.  These calls compute the absorbed decode form, the plainest reading:
 *   cache row of token j:  row_j = [ latent_j (kv_lora_rank) ;
 *                                    rotary key_j (qk_rope_dim) ]
 *   query row (token t, head h): q = [ absorbed latent query ; rotary query ]
 *   S_j = sm_scale * <q, row_j>   over the visible keys (end-aligned causal
 *                                 mask as above, or all keys)
 *   O[t,h]   = sum_j softmax_j(S) latent_j          (kv_lora_rank floats)
 *   LSE[t,h] = ln sum_j exp(S_j)
 * i.e. one-KV-head attention whose key is the whole row and whose value is
 * its latent part.  The up-projection of the values (and of the queries'
 * latent part) stays outside this step.
 *
 * Layouts (row-major):
 *   latent pool [num_pool_pages][page_size][kv_lora_rank + qk_rope_dim] bf16;
 *               token t of request r in page page_indices[page_indptr[r] +
 *               t / page_size], slot t % page_size; a page is one
 *               contiguous image, identical on every rank
 *   q           [sum qo][num_qo_heads][kv_lora_rank + qk_rope_dim] bf16
 *   rows_new    [sum qo][kv_lora_rank + qk_rope_dim] bf16
 *   out         [sum qo][num_qo_heads][kv_lora_rank] float32
 *   lse         [sum qo][num_qo_heads] float32
 * Ownership, streams and errors as for the calls above. */
typedef struct pd_mla_desc {
  int32_t num_qo_heads;  /* query heads on this rank: 16, 32, ..., 128 */
  int32_t kv_lora_rank;  /* latent entries per token: 512 */
  int32_t qk_rope_dim;   /* rotary-key entries per token: 64 */
  int32_t page_size;     /* tokens per page: 16, 32, 64 or 128 */
  int32_t dtype;         /* PD_BF16 */
  int32_t causal;        /* 1: end-aligned causal mask; 0: all kv keys */
  float sm_scale;        /* > 0 (DeepSeek: 1/sqrt(qk_nope + qk_rope dims)) */
} pd_mla_desc;

/* Bytes of one latent page: page_size * (kv_lora_rank + qk_rope_dim) * 2;
 * 0 for an invalid desc. */
size_t pd_mla_page_bytes(const pd_mla_desc* desc);

/* Plan one step of a ragged batch over a latent cache.  Arguments, checks
 * and errors as pd_plan (same page table rules); any qo <= kv is accepted
 * (qo > 1: several new tokens, e.g. multi-token prediction).  Work: blocks
 * of 4 wavefronts over one request's query rows and a chunk of its keys: 32
 * rows per wavefront (128, one token) at 128 heads, 16 (64 rows) below;
 * a request's rows are token-major (row n = token n / H, head n % H).
 * Chunks of one (request, row group) are merged afterwards; the blocks of
 * one key chunk are dispatched to the same XCD so that its L2 serves the
 * second read.  pd_plan_get_stats: decode_units = blocks, decode_row_groups
 * = (request, row group) pairs, decode_kv_bytes = latent rows read once
 * per request.  Use pd_plan_workspace_bytes / pd_plan_upload /
 * pd_plan_free / pd_plan_work_items (kind 1: blocks {request, row group,
 * key begin, key end, partial slot or -1, 0,0,0}; kind 2: merge groups
 * {request, row group, first slot, slots}).  Errors: as pd_plan;
 * PD_ERR_UNSUPPORTED for kv_lora_rank != 512, qk_rope_dim != 64, heads not
 * a multiple of 16 in [16, 128], other page sizes or dtypes. */
pd_status pd_mla_plan(const pd_mla_desc* desc, int32_t batch,
                      const int32_t* qo_lens, const int32_t* kv_lens,
                      const int32_t* page_indptr, const int32_t* page_indices,
                      int32_t num_pool_pages, const pd_plan_options* opts,
                      pd_plan_t* out);

/* Write each request's new latent rows (rows_new, token-major) at positions
 * [kv - qo, kv) of its pages (post, section "KV Messenger": cache entries
 * are appended before attention reads them).  Bit-exact copy.
 * Errors: PD_ERR_INVALID_ARG (null argument, not an MLA plan). */
pd_status pd_mla_kv_append(pd_plan_t plan, void* d_ws, void* kv_pool,
                           const void* rows_new, void* stream);

/* Attention of every query row over its request's latent cache, then the
 * merge of split chunks (fixed order: bitwise reproducible for a fixed
 * plan).  lse may be NULL.  Errors: PD_ERR_INVALID_ARG (null argument, not
 * an MLA plan), PD_ERR_HIP. */
pd_status pd_mla_attention_run(pd_plan_t plan, void* d_ws, const void* q,
                               const void* kv_pool, float* out, float* lse,
                               void* stream);

/* Copy whole latent pages (list order) into one contiguous buffer
 * [n][page bytes], and back into (other) page ids.  Every rank holds the
 * same latent pages (post, section "DeepSeek-R1"), so a page travels whole
 * from any one rank.  Arguments and errors as
 * pd_kv_pack / pd_kv_unpack (buf_bytes >= n * pd_mla_page_bytes). */
pd_status pd_mla_kv_pack(const pd_mla_desc* desc, const void* kv_pool,
                         int32_t num_pool_pages, const int32_t* page_ids,
                         int32_t n, void* d_buf, size_t buf_bytes,
                         void* d_scratch, size_t scratch_bytes, void* stream);
pd_status pd_mla_kv_unpack(const pd_mla_desc* desc, void* kv_pool,
                           int32_t num_pool_pages, const int32_t* page_ids,
                           int32_t n, const void* d_buf, size_t buf_bytes,
                           void* d_scratch, size_t scratch_bytes,
                           void* stream);

/* ---- For callers that cannot allocate --------------------------------
 * pd_attention_run_noalloc is pd_attention_run, optionally preceded by
 * pd_kv_append, for callers that cannot allocate device memory or pinned host
 * memory per step: serving loops that forbid hipMalloc, harnesses that run
 * with a fixed memory budget.  It needs no workspace argument and no
 * pd_plan_upload: the plan's tables and the split-KV partial results go to a
 * static device buffer of PD_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends.  The call allocates nothing.
 *   plan         a pd_plan (not an MLA plan) whose pd_plan_workspace_bytes
 *                is <= PD_NOALLOC_SCRATCH_BYTES
 *   q, kv_pool, out, lse   as pd_attention_run (lse may be NULL)
 *   k_new, v_new both NULL: attention only; both non-NULL: the append of
 *                pd_kv_append runs first, on the same stream
 * The tables are copied from the plan's host memory with a host-to-device
 * copy on `stream` (pageable memory: the copy has read them when the call
 * returns), so a HIP graph cannot capture this call.  Every call on one GPU
 * uses that GPU's one buffer: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be serialised by the caller;
 * calls on one stream are ordered.  Nothing in the buffer has to start at
 * zero: each call rewrites the tables and every partial result is written
 * before it is read.
 * Errors: PD_ERR_INVALID_ARG (NULL plan, an MLA plan, only one of k_new /
 * v_new, NULL q / pool / out), PD_ERR_WORKSPACE (the plan needs more than
 * PD_NOALLOC_SCRATCH_BYTES), PD_ERR_HIP; all checked before anything is
 * enqueued. */
#define PD_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
pd_status pd_attention_run_noalloc(pd_plan_t plan, const void* q, void* kv_pool,
                                   const void* k_new, const void* v_new,
                                   float* out, float* lse, void* stream);

/* Static text for a status code. */
const char* pd_status_string(pd_status s);

/* Message of the calling thread's last failed call ("" if none). */
const char* pd_last_error(void);

/* Library version string. */
const char* pd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PD_ATTN_H_ */
