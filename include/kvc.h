/*
 * kvc.h -- C ABI of libkvc, softmax-gated token-pool KV compression on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (sources: the vLLM API page "kpool_compress" for the pool-16
 * path and the SGLang page "c128_online.cuh" for the pool-128 online path):
 *
 *   pool-16   For every complete pool of 16 consecutive tokens and every
 *             channel d, take the softmax over the pool of score[i,d]+ape[i,d]
 *             and sum the keys with those weights.  Round the 128-vector to
 *             bf16, rotate it with the 128-point Walsh-Hadamard transform
 *             (Sylvester order, scaled by 1/sqrt(128)), round to bf16 again,
 *             and quantise to OCP FP8 e4m3 with one scale per vector:
 *             max(absmax, 1e-4) * fp32(1/448), optionally rounded up to a
 *             power of two.
 *   pool-128  A running fp32 (max, sum, kv) state per sequence folds tokens
 *             into the open 128-token chunk; when a chunk closes, its
 *             softmax-weighted mean (fp32) is emitted.
 *
 * Conventions shared by every entry point
 *   - head_dim is 128 everywhere; pool_size must be 16 on the pool-16 path.
 *     Other values return KVC_ERR_UNSUPPORTED.
 *   - Pointers documented as "device" are HIP device (or managed) memory;
 *     "host" pointers are ordinary CPU memory.  The caller owns every buffer;
 *     the library allocates nothing and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device entry points only enqueue work; they never synchronise.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     failed check returns a negative status and enqueues nothing;
 *     kvc_last_error() then describes it (thread-local, valid until the next
 *     call on the same thread).  A failed launch returns KVC_ERR_HIP.
 *   - Empty work (zero pools, requests, tokens or plans) returns KVC_OK and
 *     launches nothing.
 *   - Indices that live in device memory (source rows, slots, plans) cannot
 *     be checked on the host; the kernels check them and skip any item that
 *     would read or write out of bounds, leaving its outputs untouched.
 *   - bf16 arrays are passed as their raw uint16_t bit patterns.
 *   - All row starts of bf16 / fp32 vectors must be 16-byte aligned (every
 *     lane moves 128 bits); fp8 output rows 8-byte aligned.
 */
#ifndef KVC_H
#define KVC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    KVC_OK = 0,
    KVC_ERR_NULL = -1,        /* a required pointer is NULL                    */
    KVC_ERR_SHAPE = -2,       /* a size, stride or alignment is invalid         */
    KVC_ERR_UNSUPPORTED = -3, /* head_dim / pool_size other than supported      */
    KVC_ERR_PLAN = -4,        /* planner: bad lengths or capacity exceeded      */
    KVC_ERR_HIP = -5          /* the HIP runtime reported an error              */
};

/* Plan entry of the pool-128 online prefill (c128_online.cuh page,
 * OnlinePrefillPlan): one segment of consecutive extend tokens of one
 * request lying inside one 128-chunk.  ragged_id / position are the ragged
 * row and global position of the segment's LAST token; window_len (1..128)
 * is the number of tokens, so the first token is at position-window_len+1.
 * An entry whose ragged_id is 0xFFFFFFFF is padding and is skipped. */
typedef struct kvc_online_plan {
    uint32_t ragged_id;
    uint32_t batch_id;
    uint32_t position;
    uint32_t window_len;
} kvc_online_plan;

/* Work item of the single-launch pool-128 prefill: the plans one workgroup
 * runs, compress first.  Either plan may be padding (all fields 0xFFFFFFFF).
 * Both are set only when they belong to one request whose first segment
 * starts mid-chunk and closes it (reading the stored state) and whose
 * trailing segment is a write plan (replacing that state). */
typedef struct kvc_online_item {
    kvc_online_plan compress;
    kvc_online_plan write;
} kvc_online_item;

/* Library version (major*10000 + minor*100 + patch). */
int kvc_version(void);

/* Description of the last failure on this thread ("" if none). */
const char* kvc_last_error(void);

/* ------------------------------------------------------------------------
 * Host planners (pure CPU; host memory in and out).
 * ------------------------------------------------------------------------ */

/* Pool plan for a ragged prefill batch (the packing of the pool-16 prefill
 * workload): request b owns seq_lens[b] consecutive rows of the packed
 * key/score matrices, starting after the rows of requests 0..b-1.  Its
 * complete pools j = 0 .. seq_lens[b]/pool_size - 1 start at row
 * start_b + j*pool_size; tokens after the last complete pool are not
 * compressed.  Writes the first row of every pool, in request order, to
 * pool_src_row[0 .. *n_pools-1].
 *   seq_lens      host [batch], each >= 0
 *   pool_src_row  host [cap] int32 (may be NULL when cap == 0)
 *   n_pools       host, out: number of pools
 * Errors: KVC_ERR_NULL, KVC_ERR_SHAPE (negative length, rows >= 2^31),
 *         KVC_ERR_UNSUPPORTED (pool_size != 16), KVC_ERR_PLAN (cap too small;
 *         *n_pools still receives the required count). */
int kvc_plan_pool_prefill(const int64_t* seq_lens, int64_t batch, int pool_size,
                          int32_t* pool_src_row, int64_t cap, int64_t* n_pools);

/* Segment planner of the pool-128 online prefill (c128_online.cuh page,
 * plan_online_prefill_host).  Request b extends its sequence from
 * prefix = seq_lens[b] - extend_lens[b] to seq_lens[b]; its extend tokens are
 * rows counter_b .. counter_b + extend_lens[b] - 1 of the ragged input, with
 * counter_b the sum of the earlier extends.  Each extend range is cut at
 * multiples of 128.  A segment that ends on chunk position 127 becomes a
 * compress plan; the request's trailing segment that ends earlier becomes its
 * single write plan.  Plans are emitted in request order.
 *   compress_plan, write_plan  host [num_tokens] (capacity)
 *   pad_to_capacity  nonzero: fill both lists with padding entries up to
 *                    num_tokens and report num_tokens for both counts, so a
 *                    captured launch always sees the same grid.
 * Errors: KVC_ERR_NULL, KVC_ERR_PLAN (extend not in (0, seq_len], a list
 *         over capacity, or sum of extends != num_tokens), KVC_ERR_SHAPE
 *         (lengths >= 2^32). */
int kvc_c128_plan_prefill(const int64_t* seq_lens, const int64_t* extend_lens, int64_t batch,
                          int64_t num_tokens, kvc_online_plan* compress_plan,
                          kvc_online_plan* write_plan, int pad_to_capacity,
                          uint32_t* n_compress, uint32_t* n_write);

/* The plans of kvc_c128_plan_prefill, arranged as work items for
 * kvc_c128_online_prefill_fused.  Same segments, same plan entries; a
 * request's first compress plan is paired with its write plan when the
 * former starts mid-chunk (it reads the state row that the write plan
 * replaces), every other plan gets an item of its own.  Order: paired items,
 * then compress-only items, then write-only items, each in request order
 * (the longest work first).
 *   items            host [capacity]
 *   capacity         entries available in items; at least the number of
 *                    items, which never exceeds
 *                    kvc_c128_fused_capacity(num_tokens, batch)
 *   pad_to_capacity  nonzero: fill with padding items up to capacity and
 *                    report capacity, so a captured launch always sees the
 *                    same grid.  Every padding item costs an empty
 *                    workgroup, so capacity should come from
 *                    kvc_c128_fused_capacity for the largest batch the
 *                    capture serves, not from num_tokens.
 *   n_items          host, out
 * Errors: as kvc_c128_plan_prefill (KVC_ERR_PLAN when the items exceed
 *         capacity). */
int kvc_c128_plan_prefill_fused(const int64_t* seq_lens, const int64_t* extend_lens,
                                int64_t batch, int64_t num_tokens, kvc_online_item* items,
                                int64_t capacity, int pad_to_capacity, uint32_t* n_items);

/* Upper bound on the work items of any batch of at most max_batch requests
 * extending num_tokens tokens in total: a request extending E tokens touches
 * at most floor((E-1)/128) + 2 chunks, one segment each, so the items number
 * at most floor(num_tokens/128) + 2*max_batch (and never more than
 * num_tokens).  Returns 0 for negative arguments. */
int64_t kvc_c128_fused_capacity(int64_t num_tokens, int64_t max_batch);

/* ------------------------------------------------------------------------
 * Device entry points.
 * ------------------------------------------------------------------------ */

/* Pool-16 prefill compression (kpool_compress page,
 * _kpool_softmax_rotate_write_cache_kernel, packed-return mode).
 *   keys, scores    device bf16 [num_rows, *] with row strides in elements
 *                   (multiples of 8); channels 0..127 of each row are used.
 *   ape             device fp32 [16, 128], per-slot position bias.
 *   pool_src_row    device int32 [n_pools]: first row of pool p; NULL means
 *                   pool p starts at row 16*p.  A pool whose rows fall
 *                   outside [0, num_rows) is skipped.
 *   out_fp8         device uint8 [n_pools, 128] e4m3 codes.
 *   out_scale       device fp32 [n_pools].
 *   round_scale     nonzero: scale rounded up to a power of two.
 *   dbg_pooled      device fp32 [n_pools, 128] or NULL: receives the fp32
 *                   weighted mean before any rounding (for parity checks).
 * num_rows, n_pools and the row strides are at most 2^31-1.
 * Errors: KVC_ERR_NULL, KVC_ERR_SHAPE (strides, alignment, sizes),
 *         KVC_ERR_UNSUPPORTED (pool_size != 16), KVC_ERR_HIP. */
int kvc_compress_prefill(const uint16_t* keys, int64_t key_row_stride,
                         const uint16_t* scores, int64_t score_row_stride, int64_t num_rows,
                         const float* ape, int pool_size,
                         const int32_t* pool_src_row, int64_t n_pools,
                         uint8_t* out_fp8, float* out_scale, int round_scale,
                         float* dbg_pooled, void* stream);

/* Pool-16 prefill compression written into a paged indexer K cache
 * (kpool_compress page, kpool_compress_and_write_cache with write_cache and an
 * optional write_mask).  Only page_size 1 is supported: the page's token
 * order for larger pages (its preshuffled 16-token tiles) is not specified.
 * With page_size 1 the cache is [num_pages, 1, 132] bytes: page loc[p] holds
 * the 128 e4m3 codes of pool p at bytes 0..127 and its fp32 scale at bytes
 * 128..131.  Pools whose write_mask byte is 0, or whose page is outside
 * [0, num_pages), are skipped (no rows read, nothing written).
 *   keys, scores, ape, pool_src_row, n_pools, round_scale: as
 *                 kvc_compress_prefill
 *   kv_cache      device uint8 [num_pages, 132], 4-byte aligned; num_pages
 *                 at most 2^31-1
 *   loc           device int64 [n_pools]
 *   write_mask    device uint8 (bool) [n_pools] or NULL (write all)
 * Errors: KVC_ERR_NULL, KVC_ERR_SHAPE, KVC_ERR_UNSUPPORTED (pool_size != 16
 *         or page_size != 1), KVC_ERR_HIP. */
int kvc_compress_prefill_paged(const uint16_t* keys, int64_t key_row_stride,
                               const uint16_t* scores, int64_t score_row_stride, int64_t num_rows,
                               const float* ape, int pool_size, const int32_t* pool_src_row,
                               int64_t n_pools, uint8_t* kv_cache, int64_t num_pages,
                               int page_size, const int64_t* loc, const uint8_t* write_mask,
                               int round_scale, void* stream);

/* Pool-16 decode with a tail ring and ordered verify tokens (kpool_compress
 * page, _kpool_decode_update_batched_kernel).  Request r processes its tokens
 * t = 0..next_n-1 strictly in order; for entry e = r*next_n + t:
 *   blk = max(tail_slot_mapping[e], 0) / 16          (entries with
 *         blk >= num_ring_blocks are skipped entirely)
 *   if slot_mapping[e] >= 0 and positions[e] >= 0 and positions[e] % 16 == 15:
 *       the pool is ring slots 0..14 of block blk plus the current token in
 *       slot 15; its (codes, scale) go to row slot_mapping[e] of out_fp8 /
 *       out_scale (skipped if that row is >= num_out);
 *   then, if positions[e] >= 0 and tail_slot_mapping[e] >= 0, the token's key
 *       and score are stored in ring slot positions[e] % 16 of block blk.
 * A completion therefore sees the stashes of the earlier tokens of the same
 * request in the same call.  Requests must use distinct ring blocks.
 *   tail_ring        device bf16 [num_ring_blocks, 2, 16, 128] (half 0 keys,
 *                    half 1 gate scores), updated in place.
 *   key, score       device bf16, token (r, t) at r*stride_b + t*stride_t
 *                    (elements, multiples of 8).
 *   ape              device fp32 [16, 128].
 *   tail_slot_mapping, slot_mapping, positions  device int32 [num_requests,
 *                    next_n], contiguous; -1 marks padding.
 *   out_fp8, out_scale  device [num_out, 128] uint8 / [num_out] fp32.
 *   dbg_pooled       device fp32 [num_out, 128] (16-byte aligned) or NULL:
 *                    row slot_mapping[e] of every completion receives the fp32
 *                    weighted mean before any rounding (for parity checks).
 * Errors: as kvc_compress_prefill. */
int kvc_compress_decode_ring(uint16_t* tail_ring, int64_t num_ring_blocks,
                             const int32_t* tail_slot_mapping,
                             const uint16_t* key, int64_t key_stride_b, int64_t key_stride_t,
                             const uint16_t* score, int64_t score_stride_b, int64_t score_stride_t,
                             const float* ape,
                             const int32_t* slot_mapping, const int32_t* positions,
                             int64_t num_requests, int next_n, int pool_size,
                             uint8_t* out_fp8, float* out_scale, int64_t num_out,
                             int round_scale, float* dbg_pooled, void* stream);

/* Multi-layer form of kvc_compress_decode_ring: the same requests and tokens
 * (tail_slot_mapping, slot_mapping, positions are shared) in each of
 * num_layers layers, in one launch.  Layer l uses tail_ring +
 * l*ring_layer_stride, key + l*key_layer_stride, score + l*score_layer_stride
 * (bf16 elements, multiples of 8), ape + l*ape_layer_stride (floats,
 * multiple of 4), and writes out_fp8 rows / out_scale entries
 * l*num_out .. l*num_out + num_out - 1 (out_fp8 [num_layers, num_out, 128],
 * out_scale [num_layers, num_out]).  Each layer behaves exactly as a
 * separate kvc_compress_decode_ring call.  For callers that run the ring
 * decode of every layer of a model at once: one launch instead of
 * num_layers latency-bound ones.
 * Errors: as kvc_compress_decode_ring; KVC_ERR_SHAPE for num_layers > 65535
 *         or layer strides that do not step over a whole layer. */
int kvc_compress_decode_ring_layers(uint16_t* tail_ring, int64_t ring_layer_stride,
                                    int64_t num_ring_blocks, const int32_t* tail_slot_mapping,
                                    const uint16_t* key, int64_t key_layer_stride,
                                    int64_t key_stride_b, int64_t key_stride_t,
                                    const uint16_t* score, int64_t score_layer_stride,
                                    int64_t score_stride_b, int64_t score_stride_t,
                                    const float* ape, int64_t ape_layer_stride,
                                    const int32_t* slot_mapping, const int32_t* positions,
                                    int64_t num_requests, int next_n, int pool_size,
                                    uint8_t* out_fp8, float* out_scale, int64_t num_out,
                                    int64_t num_layers, int round_scale, void* stream);

/* kvc_compress_decode_ring writing completions into a page-size-1 paged cache
 * instead of packed arrays (the page's cache-write path): slot_mapping[e] is
 * the page; pages outside [0, num_pages) are skipped.  kv_cache as in
 * kvc_compress_prefill_paged.  Errors: as kvc_compress_decode_ring, plus
 * KVC_ERR_UNSUPPORTED for page_size != 1. */
int kvc_compress_decode_ring_paged(uint16_t* tail_ring, int64_t num_ring_blocks,
                                   const int32_t* tail_slot_mapping,
                                   const uint16_t* key, int64_t key_stride_b,
                                   int64_t key_stride_t, const uint16_t* score,
                                   int64_t score_stride_b, int64_t score_stride_t,
                                   const float* ape, const int32_t* slot_mapping,
                                   const int32_t* positions, int64_t num_requests, int next_n,
                                   int pool_size, uint8_t* kv_cache, int64_t num_pages,
                                   int page_size, int round_scale, void* stream);

/* Tail-ring seeding from a prefill batch (kpool_compress page,
 * _kpool_tail_seed_kernel and kpool_seed_tail_cache).  Token i carries tail
 * slot tslot[i] = block*16 + position%16, or a negative value for padding.
 * Token i is among its request's last 16 tokens exactly when the token 16
 * places ahead is past the batch, is padding, or lies in another block; its
 * key and score rows are then copied into slot tslot[i]%16 of ring block
 * tslot[i]/16 (blocks >= num_ring_blocks are skipped).  Each request's
 * tokens must be contiguous in the batch and requests must own distinct
 * blocks.
 *   tail_ring     device bf16 [num_ring_blocks, 2, 16, 128], updated in place
 *   key, score    device bf16 [n_tokens, *] with row strides in elements
 *                 (multiples of 8, >= 128)
 *   tslot         device int32 [n_tokens]
 * Errors: KVC_ERR_NULL, KVC_ERR_SHAPE, KVC_ERR_UNSUPPORTED (pool_size != 16),
 *         KVC_ERR_HIP. */
int kvc_seed_tail_ring(uint16_t* tail_ring, int64_t num_ring_blocks,
                       const uint16_t* key, int64_t key_row_stride,
                       const uint16_t* score, int64_t score_row_stride,
                       const int32_t* tslot, int64_t n_tokens, int pool_size, void* stream);

/* Pool-128 online decode (c128_online.cuh page, flash_c128_online_decode).
 * Request b appends one token at position seq_lens[b]-1; c = that position
 * mod 128 picks bias row ape[c]; s = score + ape[c].
 *   c == 0:   state := (s, 1, kv)
 *   c != 0:   state := online merge of the state with (s, 1, kv)
 *   c == 127: out[b] := merged kv (the state row is left as it was);
 *   otherwise the merged state is written back to row indices[b].
 * Rows with seq_lens[b] <= 0 or indices[b] outside [0, num_slots) are skipped.
 *   state        device fp32 [num_slots, 384] = max[128] | sum[128] | kv[128]
 *   kv_score_in  device fp32 [batch, 256] = kv[128] | score[128]
 *   out          device fp32 [batch, 128]; only emitting rows are written
 *   ape          device fp32 [128, 128]
 *   indices, seq_lens  device int32 [batch]
 * Errors: KVC_ERR_NULL, KVC_ERR_SHAPE, KVC_ERR_HIP. */
int kvc_c128_online_decode(float* state, int64_t num_slots, const float* kv_score_in,
                           float* out, const float* ape, const int32_t* indices,
                           const int32_t* seq_lens, int64_t batch, void* stream);

/* Multi-layer form of kvc_c128_online_decode: the same requests (indices,
 * seq_lens) decode one token in each of num_layers layers in one launch.
 * Layer l uses state + l*state_layer_stride, kv_score_in + l*in_layer_stride,
 * out + l*out_layer_stride and ape + l*ape_layer_stride (strides in floats,
 * multiples of 4, each covering a whole layer when num_layers > 1).  Each
 * layer behaves exactly as a separate kvc_c128_online_decode call.
 * Errors: as kvc_c128_online_decode; KVC_ERR_SHAPE for num_layers > 65535 or
 *         strides that overlap layers. */
int kvc_c128_online_decode_layers(float* state, int64_t state_layer_stride, int64_t num_slots,
                                  const float* kv_score_in, int64_t in_layer_stride, float* out,
                                  int64_t out_layer_stride, const float* ape,
                                  int64_t ape_layer_stride, const int32_t* indices,
                                  const int32_t* seq_lens, int64_t batch, int64_t num_layers,
                                  void* stream);

/* kvc_c128_online_decode with the pool-16 epilogue applied to every emitted
 * vector: bf16 round, 128-point Walsh-Hadamard / sqrt(128), bf16 round,
 * e4m3 with one scale per vector (max(absmax, 1e-4) * fp32(1/448), rounded
 * up to a power of two when round_scale).  out_fp8 device uint8 [batch, 128],
 * out_scale device fp32 [batch]; only emitting rows are written.  The state
 * update is identical to kvc_c128_online_decode. */
int kvc_c128_online_decode_quant(float* state, int64_t num_slots, const float* kv_score_in,
                                 uint8_t* out_fp8, float* out_scale, const float* ape,
                                 const int32_t* indices, const int32_t* seq_lens, int64_t batch,
                                 int round_scale, void* stream);

/* Pool-128 online ragged prefill (c128_online.cuh page,
 * flash_c128_online_prefill and run_prefill).  Two launches in stream order:
 *   1. every compress plan: the segment's softmax state, merged with state
 *      row load_indices[b] when the segment starts mid-chunk, is normalised
 *      and written to out row ragged_id.  The state buffer is only read.
 *   2. every write plan: the same, but the (max, sum, kv) state is written to
 *      row indices[b].
 * Because pass 1 finishes before pass 2 starts, every read of pass 1 sees
 * the state as it was when the call was made.  In pass 2 a write plan that
 * starts mid-chunk reads row load_indices[b] while other workgroups of the
 * same launch write rows indices[b'], so the call requires that no request
 * reads a state row another request of the call writes: the rows indices[b]
 * are distinct, and load_indices[b] is no other request's indices[b'] (true
 * when load_indices is NULL).  Otherwise the result is undefined.
 *   state          device fp32 [num_slots, 384]
 *   kv_score_in    device fp32 [num_tokens, 256]
 *   out            device fp32 [num_tokens, 128]; only chunk-closing rows
 *   ape            device fp32 [128, 128]
 *   indices        device int32 [batch]; load_indices device int32 [batch]
 *                  or NULL (= indices)
 *   compress_plan  device [n_compress]; write_plan device [n_write]; both as
 *                  produced by kvc_c128_plan_prefill for these lengths.
 *                  Malformed entries (out-of-range rows, batches or slots, or
 *                  window_len outside 1..position%128+1) are skipped.
 * Errors: KVC_ERR_NULL, KVC_ERR_SHAPE, KVC_ERR_HIP. */
int kvc_c128_online_prefill(float* state, int64_t num_slots, const float* kv_score_in,
                            float* out, int64_t num_tokens, const float* ape,
                            const int32_t* indices, const int32_t* load_indices, int64_t batch,
                            const kvc_online_plan* compress_plan, uint32_t n_compress,
                            const kvc_online_plan* write_plan, uint32_t n_write, void* stream);

/* kvc_c128_online_prefill with the rotate/quantise epilogue (as in
 * kvc_c128_online_decode_quant) on every chunk-closing vector: out_fp8
 * device uint8 [num_tokens, 128] and out_scale device fp32 [num_tokens],
 * written at row ragged_id of each compress plan.  State handling, and the
 * requirement on load_indices, are those of kvc_c128_online_prefill. */
int kvc_c128_online_prefill_quant(float* state, int64_t num_slots, const float* kv_score_in,
                                  uint8_t* out_fp8, float* out_scale, int64_t num_tokens,
                                  const float* ape, const int32_t* indices,
                                  const int32_t* load_indices, int64_t batch,
                                  const kvc_online_plan* compress_plan, uint32_t n_compress,
                                  const kvc_online_plan* write_plan, uint32_t n_write,
                                  int round_scale, void* stream);

/* Pool-128 online ragged prefill in ONE launch (c128_online.cuh page,
 * flash_c128_online_prefill; same results as kvc_c128_online_prefill).  The
 * page orders state reads before state writes with two launches; here each
 * work item from kvc_c128_plan_prefill_fused carries the only read that can
 * conflict with its write, so one workgroup does both in order and the
 * second launch (latency-bound, a few microseconds) disappears.  Requires
 * that no request reads a state row another request of the call writes: the
 * rows indices[b] are distinct, and load_indices[b] is no other request's
 * indices[b'] (true when load_indices is NULL).
 *   state, kv_score_in, num_tokens, ape, indices, load_indices, batch: as
 *                  kvc_c128_online_prefill
 *   out            device fp32 [num_tokens, 128], or NULL when out_fp8 is
 *                  given; chunk-closing rows only
 *   out_fp8, out_scale  device uint8 [num_tokens, 128] and fp32
 *                  [num_tokens] for the rotate/quantise epilogue (as
 *                  kvc_c128_online_prefill_quant), or both NULL
 *   round_scale    used with out_fp8
 *   items          device [n_items], 16-byte aligned; padding items and
 *                  malformed plans are skipped as in kvc_c128_online_prefill
 * Exactly one of out and out_fp8 (with out_scale) must be given.
 * Errors: KVC_ERR_NULL, KVC_ERR_SHAPE, KVC_ERR_HIP. */
int kvc_c128_online_prefill_fused(float* state, int64_t num_slots, const float* kv_score_in,
                                  float* out, uint8_t* out_fp8, float* out_scale,
                                  int round_scale, int64_t num_tokens, const float* ape,
                                  const int32_t* indices, const int32_t* load_indices,
                                  int64_t batch, const kvc_online_item* items, uint32_t n_items,
                                  void* stream);

/* ------------------------------------------------------------------------
 * Diagnostics.
 * ------------------------------------------------------------------------ */

/* Runs the device number-format conversions the kernels use, elementwise:
 *   bf16_out[i] = bf16 round-to-nearest-even of in[i]          (may be NULL)
 *   fp8_out[i]  = e4m3 code of clamp(in[i], -448, 448)         (may be NULL)
 * in: device fp32 [n]; n must be a multiple of 2.  For verifying the
 * hardware conversion against an independent encoder. */
int kvc_diag_convert(const float* in, uint16_t* bf16_out, uint8_t* fp8_out, int64_t n,
                     void* stream);

/* Plain streaming read, for measurement: reads `bytes` bytes at src
 * (16-byte aligned, bytes a multiple of 16) with 128-bit non-temporal loads,
 * one shot.  Workgroup w (256 threads, four waves) reads bytes
 * [w*4096*L, (w+1)*4096*L), L = loads_per_lane (2, 4, 8 or 16), every lane
 * issuing its L loads before it uses any.  With fold != 0, wave v of
 * workgroup w writes the XOR of all 32-bit words it read to sink[4w + v]
 * (zero padding past `bytes`), for checking that every word was read; with
 * fold == 0 the sink is practically never written (a lane stores only when
 * its XOR equals one fixed constant), the form for timing.  sink_words >=
 * 4*ceil(bytes / (4096*L)) either way.  It does no other work: its time over
 * a buffer is what a read-only kernel of this simple shape reaches, a
 * practical reference for the compression kernels.
 * Errors: KVC_ERR_SHAPE (size, alignment, sink too small),
 *         KVC_ERR_UNSUPPORTED (loads_per_lane), KVC_ERR_NULL, KVC_ERR_HIP. */
int kvc_diag_stream_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words,
                         int loads_per_lane, int fold, void* stream);

/* Launches a kernel that does nothing, with `workgroups` workgroups of
 * `threads` threads (1..1024), for measuring the launch and dispatch floor
 * that a kernel of that grid pays.  arg_bytes (0, 64, 112, 136 or 448) sets
 * the size of the kernel's (unused) argument block, for measuring how the
 * runtime's host-side cost of a launch depends on it.  workgroups == 0 is a
 * no-op.
 * Errors: KVC_ERR_SHAPE, KVC_ERR_UNSUPPORTED (arg_bytes), KVC_ERR_HIP. */
int kvc_diag_empty_launch(int64_t workgroups, int threads, int arg_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
