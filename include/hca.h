/*
 * hca.h -- C ABI of the MI355X (gfx950) Heavily Compressed Attention library.
 *
 * The operation.  DeepSeek-V4 Heavily Compressed Attention (HCA) is
 * single-KV-head (MQA) softmax attention in which each query attends to a
 * local sliding window of raw keys plus every compressed KV entry whose
 * compression window has completed at or before the query; the pattern is
 * deterministic, with no indexer ("Add HCA Static Compilation for Splash
 * Attention [Deepseek v4]", Description).  Keys and values are one shared
 * tensor broadcast over all query heads ("[DeepSeek-V4] Implement Compressed
 * Attention Layers", review suggestions replacing the per-head repeat by an
 * einsum broadcast with k = v = kv).  Conventions fixed by this library:
 *
 *   raw key t is visible to query i       iff  i - W < t <= i, same document
 *   entry c covers raw positions [c*r, (c+1)*r) and is visible to query i
 *                                          iff  (c+1)*r <= i+1, same document
 *   document of an entry: HCA_COMPSEG_STRICT -- the document that contains
 *   the entry's whole window (no document if it straddles a boundary);
 *   HCA_COMPSEG_LAST -- the document of the window's last raw position.
 *
 * One softmax runs over the union of both key sets.  Outputs:
 *   O[b,h,i]   = sum_k P_k kv_k,   P = softmax_k(scale * <q[b,h,i], kv_k>)
 *   LSE[b,h,i] = natural log of sum_k exp(scale * <q, kv_k>)
 * A query with no visible key gets O = 0, LSE = -inf and no gradient.
 * Backward (loss gradient dO given): dQ, and one gradient for the shared raw
 * kv and one for the compressed kv, each the sum of its key-path and
 * value-path parts over all heads.
 *
 * Memory and ownership.
 *   - The caller owns every device buffer (inputs, outputs, workspace, the
 *     plan's device image) and the stream.  The library never allocates
 *     device memory; a plan owns host memory only.
 *   - All device pointers must be 16-byte aligned.  Tensors are contiguous,
 *     row-major:  q, o, dout, dq [B][H][S][D];  kv, dkv [B][S][D];
 *     kv_comp, dkv_comp [B][S_c][D];  lse [B][H][S] float32.
 *     Element type of q, kv, kv_comp, o, dout, dq, dkv, dkv_comp: the plan's
 *     dtype (float32 or bfloat16).  Accumulation is float32 throughout.
 *   - Outputs are overwritten, never accumulated into.
 *   - Work is enqueued on the given HIP stream (NULL = default stream) and is
 *     asynchronous: results are ready after the caller synchronises.  Faults
 *     inside kernels surface at that synchronisation.
 *   - One exception, inside hca_attn_bwd with stored P and dS (info.kv_keys
 *     == 64): its dQ pass runs on a second stream that the library owns (one
 *     per device, default priority, created on first use with the calling
 *     thread's current device, which must be the stream's, and kept until the
 *     process ends).  It is forked from the caller's stream and joined back
 *     into it with events before the call returns, so the call as a whole
 *     stays ordered on the caller's stream.  If that stream cannot be
 *     created, the dQ pass runs on the caller's stream instead.
 *
 * Errors.  Every entry point validates all of its arguments before it makes
 * any HIP call, and returns a status; no exception crosses the ABI.  A
 * thread-local message (hca_last_error) describes the last failure.
 */
#ifndef HCA_H_
#define HCA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hca_status {
  HCA_OK = 0,
  HCA_ERR_INVALID_ARG = 1, /* a size, pointer, layout or segment list is invalid */
  HCA_ERR_UNSUPPORTED = 2, /* valid, but outside what the GPU kernels implement  */
  HCA_ERR_WORKSPACE = 3,   /* workspace or plan buffer smaller than required     */
  HCA_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed         */
  HCA_ERR_NOMEM = 5,       /* host allocation failed                             */
  HCA_ERR_STATE = 6        /* plan used before hca_plan_upload                   */
} hca_status;

typedef enum hca_dtype { HCA_F32 = 0, HCA_BF16 = 1 } hca_dtype;

typedef enum hca_compseg_mode { HCA_COMPSEG_STRICT = 0, HCA_COMPSEG_LAST = 1 } hca_compseg_mode;

/* Tile states of the block table (one byte each). */
enum { HCA_TILE_EMPTY = 0, HCA_TILE_PARTIAL = 1, HCA_TILE_FULL = 2 };

/*
 * Tile shape of the block table: bq query positions (all heads) by bk_raw raw
 * keys, or by bk_comp compressed entries.  A zero field selects the library's
 * choice for (D, H, dtype).  Any positive shape is accepted by the planner;
 * the GPU entry points run only the shapes their kernels are built for
 * (hca_plan_info.kernel_ok).
 *
 * Three further fields shape the work items of the key-stationary backward
 * (they change the schedule, never the result beyond float summation order):
 *   kv_keys           keys per key tile of that backward; 0 = library choice.
 *                     Head dim 512, bfloat16: 64 or 128.  With 64 the dQ pass
 *                     stores P and dS (bf16, one bq * H x 32 block each per
 *                     listed (query tile, 32-key tile) pair, in the backward
 *                     workspace: hca_plan_info.ws_pds_bytes) and the key-
 *                     stationary pass reads them instead of recomputing S and
 *                     dP: faster, with a workspace of O(S (W + S / r)).  With
 *                     128 both are recomputed and the workspace is O(S).
 *                     Library choice: 64 while the store needs at most 32
 *                     GiB, else 128.  Other kernels: 32.  Any other value is
 *                     rejected.
 *   half_items_min    with 128-key items (head dim 512, bfloat16): an item whose
 *                     rows see only one 64-key half of its key tile runs over
 *                     that half alone once the plan has at least this many
 *                     items; 0 = library choice (1: always), < 0 = never.
 *   comp_item_chunks  64-position chunks of query rows per work item of a
 *                     compressed key tile; 0 = library choice (one chunk,
 *                     doubled only while the compressed tiles' partial
 *                     gradients would exceed twice the raw tiles', so the
 *                     backward workspace stays O(S)).
 */
typedef struct hca_tile_cfg {
  int32_t bq;
  int32_t bk_raw;
  int32_t bk_comp;
  int32_t half_items_min;
  int32_t comp_item_chunks;
  int32_t kv_keys;
} hca_tile_cfg;

typedef struct hca_plan hca_plan; /* opaque, host-owned */

typedef struct hca_plan_info {
  int32_t B, S, H, D, r, W, S_c;
  int32_t dtype;     /* hca_dtype */
  int32_t comp_mode; /* hca_compseg_mode */
  int32_t bq, bk_raw, bk_comp;
  int32_t nqt;       /* ceil(S / bq) query tiles per batch row */
  int32_t nkt_raw;   /* ceil(S / bk_raw) */
  int32_t nkt_comp;  /* ceil(S_c / bk_comp) */
  int32_t kernel_ok; /* 1: hca_attn_fwd / hca_attn_bwd run this plan: a kernel exists for
                        the dtype, head dim, heads and tile shape, and the sizes fit the
                        kernels' 32-bit offsets (head dim 512, bfloat16: each key tensor
                        padded to 32-key tiles times 4 D bytes below 2^31) */
  int64_t tiles_raw, tiles_comp;   /* non-empty tiles, summed over the batch */
  int64_t full_raw, full_comp;     /* of which FULL */
  int64_t pairs_raw, pairs_comp;   /* visible (query position, key) pairs, summed over the
                                      batch; multiply by H for (query row, key) pairs */
  uint64_t device_bytes;           /* size of the plan's device image */
  uint64_t ws_fwd_bytes;           /* workspace hca_attn_fwd needs (0 for float32 and for
                                      bfloat16 below head dim 512) */
  uint64_t ws_bwd_bytes;           /* workspace hca_attn_bwd needs (>= ws_fwd_bytes; the
                                      backward's layout starts with the forward's, so one
                                      buffer of ws_bwd_bytes serves both calls in turn) */
  int64_t items;                   /* work items of the key-stationary backward */
  int64_t items_half;              /* of which run over one 64-key half of their tile */
  int64_t part_blocks;             /* float32 partial-gradient blocks (kv_bk x D each) */
  int32_t comp_item_chunks;        /* 64-position chunks per compressed-tile item */
  int32_t kv_heads;                /* key/value heads G (1: MQA); see hca_block_mask_build_gqa */
  int32_t comp_masked;             /* 1: compressed visibility from a given mask (see
                                      hca_block_mask_build_masked) */
  int32_t kv_keys;                 /* keys per key tile of the key-stationary backward */
  uint64_t ws_pds_bytes;           /* of ws_bwd_bytes: the bfloat16 P and dS tiles the dQ
                                      pass stores for the key-stationary pass (64-key
                                      tiles at head dim 512; 0 otherwise) */
} hca_plan_info;

/*
 * Builds the tile-level sparsity table analytically on the host, from
 * (S, r, W, document starts) alone; no S x S mask is formed anywhere.
 * Passage: "Add HCA Static Compilation for Splash Attention [Deepseek v4]",
 * Description -- the block mask of the deterministic HCA pattern is computed
 * from coordinates on the CPU ahead of time instead of being materialised in
 * device memory; ceiling-division padding for unaligned S; segment IDs for
 * packed documents.  The compression ratio is an explicit argument (a review
 * on the same page notes it must not be inferred from S).
 *
 *   B, S, H, D    batch, sequence length, query heads, head dim (all >= 1)
 *   r             compression ratio (>= 1);  W  window (>= 0, 0 = no raw keys)
 *   S_c           number of compressed entries; must equal floor(S / r)
 *   seg_starts    document start positions of every batch row, concatenated;
 *                 per row strictly increasing, first 0, all < S.  NULL: one
 *                 document per row (seg_counts must then be NULL too)
 *   seg_counts    [B] number of documents in each row
 *   dtype, mode   element type and compressed-entry document rule
 *   tiles         NULL or a tile shape (0 fields = library choice)
 *   out           receives the plan; release it with hca_plan_destroy
 * Errors: HCA_ERR_INVALID_ARG for any violated rule above, HCA_ERR_NOMEM.
 */
hca_status hca_block_mask_build(int32_t B, int32_t S, int32_t r, int32_t W, int32_t S_c,
                                const int32_t *seg_starts, const int32_t *seg_counts,
                                int32_t H, int32_t D, hca_dtype dtype, hca_compseg_mode mode,
                                const hca_tile_cfg *tiles, hca_plan **out);

/*
 * Grouped-query variant: kv_heads = G key/value heads (G divides H), query
 * head h attending to key/value head h / (H / G).  The pages dispatch the MQA
 * kernel only when the layer has a single key/value head ("Add HCA Static
 * Compilation for Splash Attention [Deepseek v4]", Description), so layers
 * with several are served here: each (batch row, key/value head) with its
 * H / G query heads is one MQA problem of the kind above, with the batch
 * row's documents.  Layouts: q, o, dout, dq [B][H][S][D] (unchanged);
 * kv, dkv [B][G][S][D]; kv_comp, dkv_comp [B][G][S_c][D]; lse [B][H][S].
 * The plan's tables (hca_plan_export_tiles / _rows / _items) then have
 * B * G rows, row b * G + g for batch row b and key/value head g, and
 * tiles_*, full_* count over them; pairs_* stay per batch row.  G = 1 is
 * hca_block_mask_build.  Errors: as hca_block_mask_build, and
 * HCA_ERR_INVALID_ARG when G < 1, G does not divide H or B * G > 2^20.
 */
hca_status hca_block_mask_build_gqa(int32_t B, int32_t kv_heads, int32_t S, int32_t r,
                                    int32_t W, int32_t S_c, const int32_t *seg_starts,
                                    const int32_t *seg_counts, int32_t H, int32_t D,
                                    hca_dtype dtype, hca_compseg_mode mode,
                                    const hca_tile_cfg *tiles, hca_plan **out);

/*
 * Plan whose compressed-key pattern is a given dense mask instead of the HCA
 * rule: comp_mask is a host array [B][S][S_c], nonzero where query i may see
 * compressed entry c (any pattern; S_c is free, r does not enter).  This is
 * the form in which the dynamic path of "Add HCA Static Compilation for
 * Splash Attention [Deepseek v4]" (Description) hands compressed attention
 * its pattern -- a dense (B, 1, S, S_comp) mask -- kept here as the
 * comparison with the analytic plan.  The raw window keeps its rule (window
 * W, documents as in hca_block_mask_build).  The planner reads every mask
 * element (O(B S S_c) host work, against O(B S) for the analytic plan),
 * classifies tiles from it, and stores it in the plan's device image as bits
 * (ceil(S_c / 128) * 16 bytes per position), which the kernels read for the
 * compressed tiles that are PARTIAL; the caller's array is not kept.
 * hca_attn_fwd / hca_attn_bwd then run unchanged (head dim 512 bfloat16
 * kernels only; other head dims and float32 give kernel_ok = 0).
 * Errors: as hca_block_mask_build, and HCA_ERR_INVALID_ARG on a NULL mask.
 */
hca_status hca_block_mask_build_masked(int32_t B, int32_t S, int32_t W, int32_t S_c,
                                       const int32_t *seg_starts, const int32_t *seg_counts,
                                       int32_t H, int32_t D, hca_dtype dtype,
                                       const uint8_t *comp_mask, const hca_tile_cfg *tiles,
                                       hca_plan **out);

/*
 * Plan for attention over a given per-query selection of compressed entries,
 * the CSA form of the compressed path (a top-k indexer picks entries per
 * query; "Add HCA Static Compilation for Splash Attention [Deepseek v4]",
 * Description: CSA requires a top-k step): idx is a host array [B][S][K] of
 * entry indices (negative = no entry, repeats count once), shared by all
 * heads of a position, plus the raw window as above.  Same as
 * hca_block_mask_build_masked with the mask of the selection.  Errors: as
 * hca_block_mask_build_masked, and HCA_ERR_INVALID_ARG for K < 1 or an index
 * >= S_c.
 */
hca_status hca_block_mask_build_topk(int32_t B, int32_t S, int32_t W, int32_t S_c,
                                     const int32_t *seg_starts, const int32_t *seg_counts,
                                     int32_t H, int32_t D, hca_dtype dtype, const int32_t *idx,
                                     int32_t K, const hca_tile_cfg *tiles, hca_plan **out);

/* Fills *out with the plan's sizes and counts.  HCA_ERR_INVALID_ARG on NULL. */
hca_status hca_plan_get_info(const hca_plan *plan, hca_plan_info *out);

/*
 * Copies the block table to host arrays: raw_states [B][nqt][nkt_raw] and
 * comp_states [B][nqt][nkt_comp], one HCA_TILE_* byte each.  Either pointer
 * may be NULL to skip that table.  Same rule as the planner: EMPTY when no
 * in-range element is visible, FULL when every element of the nominal bq x bk
 * rectangle is in range and visible, PARTIAL otherwise.
 */
hca_status hca_plan_export_tiles(const hca_plan *plan, uint8_t *raw_states,
                                 uint8_t *comp_states);

/*
 * Copies the per-position visible intervals to a host array [B][S][3] of
 * int32: {raw_lo, comp_lo, comp_hi}.  Query i sees raw keys raw_lo..i
 * (none when raw_lo > i) and compressed entries comp_lo..comp_hi-1.
 */
hca_status hca_plan_export_rows(const hca_plan *plan, int32_t *rows);

/*
 * Key-stationary work items of the backward, for inspection.  *count
 * receives the number of items; when `items` is not NULL, min(*count,
 * capacity) rows of 8 int64 are written: batch row, kind (0 raw, 1
 * compressed), first key, keys per item, first and last listed query tile,
 * halves (bit 0 / bit 1 set when some row of the item sees a key of the lower
 * / upper half of the item's keys; 3 whenever the item runs over all of them;
 * bit 2 set when a lower-half and an upper-half item of the tile share one
 * partial block, each writing its half) and the element offset of the item's
 * float32 partial block.  The items of one key tile are consecutive and
 * their partial blocks are consecutive.  Errors:
 * HCA_ERR_INVALID_ARG on a NULL plan or count, or a negative capacity.
 */
hca_status hca_plan_export_items(const hca_plan *plan, int64_t *items, int64_t capacity,
                                 int64_t *count);

/*
 * Copies the plan's device image (schedule lists and per-position
 * intervals, info.device_bytes bytes) into the caller's device buffer with an
 * asynchronous copy on `hip_stream`, and records the buffer in the plan.  The
 * buffer must stay valid, and the plan alive, for every later call that uses
 * the plan.  HCA_ERR_WORKSPACE if bytes < info.device_bytes; HCA_ERR_HIP if
 * the copy cannot be enqueued.
 */
hca_status hca_plan_upload(hca_plan *plan, void *dev_buf, uint64_t bytes, void *hip_stream);

/* Releases the plan's host memory (not the caller's device buffer).  NULL is a no-op. */
void hca_plan_destroy(hca_plan *plan);

/*
 * Forward pass: o (plan dtype) and lse (float32).
 * Passages: the HCA pattern ("Add HCA Static Compilation for Splash Attention
 * [Deepseek v4]", Description); the shared-KV einsum form ("[DeepSeek-V4]
 * Implement Compressed Attention Layers", review suggestions).
 *   scale      logit scale (usually 1/sqrt(D)); must be finite and > 0
 *   kv_comp    may be NULL only when S_c == 0
 *   ws         device workspace of at least info.ws_fwd_bytes (may be NULL when 0)
 * Errors: HCA_ERR_INVALID_ARG (NULL or misaligned pointer, bad scale),
 * HCA_ERR_STATE (plan not uploaded), HCA_ERR_UNSUPPORTED (kernel_ok == 0),
 * HCA_ERR_WORKSPACE, HCA_ERR_HIP (launch failure).
 */
hca_status hca_attn_fwd(const hca_plan *plan, const void *q, const void *kv, const void *kv_comp,
                        float scale, void *o, float *lse, void *ws, uint64_t ws_bytes,
                        void *hip_stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory and
 * cannot hand over a workspace either: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same operation, checks,
 * kernels and results as hca_attn_fwd (bit for bit), but its workspace is a
 * scratch array the library holds in device memory: HCA_NOALLOC_SCRATCH_BYTES
 * per device, resolved once per device on the first call there (the calling
 * thread's current device must be the stream's).  The call makes no device
 * allocation and no allocating library call.  Every byte the kernels read from
 * the scratch is written earlier in the same call, so no clearing is needed.
 * All calls on one GPU share its scratch: calls that overlap in time on one
 * GPU (on different streams, or from different threads) race and must not be
 * issued; calls in sequence on one stream are fine.
 * Plans with ws_fwd_bytes == 0 (float32, bfloat16 below head dim 512) do not
 * touch the scratch.
 * Errors: as hca_attn_fwd, plus HCA_ERR_WORKSPACE (before any HIP call) when
 * the plan's ws_fwd_bytes exceeds HCA_NOALLOC_SCRATCH_BYTES, and HCA_ERR_HIP
 * when the device or the scratch address cannot be queried.
 */
#define HCA_NOALLOC_SCRATCH_BYTES (64ull << 20)
hca_status hca_attn_fwd_noalloc(const hca_plan *plan, const void *q, const void *kv,
                                const void *kv_comp, float scale, void *o, float *lse,
                                void *hip_stream);

/*
 * Backward pass: dq, dkv (raw) and dkv_comp (compressed), all in the plan
 * dtype, given the forward's o and lse and the loss gradient dout.
 *   dq[b,h,i]  = scale * sum_k dS_k kv_k
 *   dkv_k      = sum over (h, i) that see k of scale * dS_k q[b,h,i] + P_k dout[b,h,i]
 * with dS_k = P_k (<dout, kv_k> - <dout, o>).  Key K and value V are one
 * tensor, so each key's two gradient paths are summed ("[DeepSeek-V4]
 * Implement Compressed Attention Layers", review suggestions: k = kv, v = kv).
 * dQ is accumulated in registers, never through atomics to device memory;
 * the key gradients are summed from per-item partial sums in a fixed order,
 * so the same inputs and plan give bitwise the same outputs on every call.
 *   ws   device workspace of at least info.ws_bwd_bytes (its contents on
 *        return are unspecified; nothing needs to be kept between calls)
 *   dkv_comp / kv_comp may be NULL only when S_c == 0.
 * Errors as for hca_attn_fwd.
 */
hca_status hca_attn_bwd(const hca_plan *plan, const void *q, const void *kv, const void *kv_comp,
                        const void *o, const float *lse, const void *dout, float scale, void *dq,
                        void *dkv, void *dkv_comp, void *ws, uint64_t ws_bytes, void *hip_stream);

/*
 * Kernel timing (instrumentation).  While enabled, each kernel family's work
 * in a call (one launch each) is bracketed by a pair of HIP events recorded
 * on the call's stream (the dQ pass of a backward with stored P and dS: on the
 * second stream, where its span overlaps the key-stationary pass's and is no
 * exclusive time).  hca_timing_read waits for the recorded events, writes
 * per-family totals (up to `capacity` entries, *count = number of families
 * timed) and clears them.  Events that have been read are kept in a per-device
 * pool and reused, so timed calls after the first create none; a kernel whose
 * events cannot be created runs untimed.  Not thread-safe against concurrent
 * hca_attn_* calls on other threads while enabled.  Errors: HCA_ERR_INVALID_ARG
 * on NULL output pointers, HCA_ERR_HIP if a recorded event cannot be read.
 */
typedef struct hca_kernel_time {
  char name[32];    /* kernel family, e.g. "fwd", "bwd_dq", "bwd_dkv" */
  int64_t launches; /* number of timed regions (calls) since the last read */
  double total_ms;  /* summed event-to-event duration */
} hca_kernel_time;

hca_status hca_timing_enable(int32_t enable);
hca_status hca_timing_read(hca_kernel_time *out, int32_t capacity, int32_t *count);

/* Static description of a status code. */
const char *hca_status_string(hca_status s);

/* Detail message of the last failed call on this thread ("" if none). */
const char *hca_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HCA_H_ */
