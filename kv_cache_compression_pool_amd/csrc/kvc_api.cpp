// kvc_api.cpp -- the C ABI of libkvc: argument validation, host planners and
// dispatch to the HIP launchers.  Nothing here allocates device memory or
// synchronises; every device entry point only enqueues work on `stream`.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "kvc.h"
#include "kvc_internal.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return KVC_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KVC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kHeadDim = 128;
constexpr int kPool = 16;
constexpr int64_t kMaxI32 = 0x7fffffffLL;

}  // namespace

extern "C" {

int kvc_version(void) { return 200; }

const char* kvc_last_error(void) { return g_last_error.c_str(); }

// --------------------------------------------------------------- planners
int kvc_plan_pool_prefill(const int64_t* seq_lens, int64_t batch, int pool_size,
                          int32_t* pool_src_row, int64_t cap, int64_t* n_pools) {
  if (!n_pools) return fail(KVC_ERR_NULL, "kvc_plan_pool_prefill: n_pools is NULL");
  *n_pools = 0;
  if (pool_size != kPool)
    return fail(KVC_ERR_UNSUPPORTED, "kvc_plan_pool_prefill: pool_size %d (only 16)", pool_size);
  if (batch < 0 || cap < 0) return fail(KVC_ERR_SHAPE, "kvc_plan_pool_prefill: negative size");
  if (batch > 0 && !seq_lens) return fail(KVC_ERR_NULL, "kvc_plan_pool_prefill: seq_lens is NULL");
  if (cap > 0 && !pool_src_row)
    return fail(KVC_ERR_NULL, "kvc_plan_pool_prefill: pool_src_row is NULL");
  int64_t rows = 0, need = 0;
  for (int64_t b = 0; b < batch; ++b) {
    if (seq_lens[b] < 0)
      return fail(KVC_ERR_SHAPE, "kvc_plan_pool_prefill: seq_lens[%lld] < 0", (long long)b);
    need += seq_lens[b] / pool_size;
    rows += seq_lens[b];
    if (rows > kMaxI32) return fail(KVC_ERR_SHAPE, "kvc_plan_pool_prefill: rows exceed 2^31-1");
  }
  *n_pools = need;
  if (need > cap)
    return fail(KVC_ERR_PLAN, "kvc_plan_pool_prefill: %lld pools exceed capacity %lld",
                (long long)need, (long long)cap);
  int64_t n = 0, start = 0;
  for (int64_t b = 0; b < batch; ++b) {
    const int64_t full = seq_lens[b] / pool_size;
    for (int64_t j = 0; j < full; ++j) pool_src_row[n++] = (int32_t)(start + j * pool_size);
    start += seq_lens[b];
  }
  return ok();
}

}  // extern "C"

namespace {

// Cuts every request's extend range at multiples of 128 and hands each
// segment to emit(b, plan, closes_chunk, first_of_request) in request order.
// Returns KVC_OK, the first error emit returns, or a planner error.
template <class Emit>
int walk_c128_segments(const char* fn, const int64_t* seq_lens, const int64_t* extend_lens,
                       int64_t batch, int64_t num_tokens, Emit&& emit) {
  uint64_t row = 0;
  for (int64_t b = 0; b < batch; ++b) {
    const int64_t L = seq_lens[b], E = extend_lens[b];
    if (!(E > 0 && E <= L))
      return fail(KVC_ERR_PLAN, "%s: request %lld extend %lld not in (0, %lld]", fn,
                  (long long)b, (long long)E, (long long)L);
    if (L > (int64_t)0xffffffffLL) return fail(KVC_ERR_SHAPE, "%s: seq_len exceeds 2^32-1", fn);
    const int64_t prefix = L - E;
    int64_t pos = prefix;
    while (pos < L) {
      const int64_t chunk_end = (pos / 128 + 1) * 128;          // exclusive
      const int64_t seg_end = chunk_end < L ? chunk_end : L;
      kvc_online_plan p;
      p.ragged_id = (uint32_t)(row + (uint64_t)(seg_end - 1 - prefix));
      p.batch_id = (uint32_t)b;
      p.position = (uint32_t)(seg_end - 1);
      p.window_len = (uint32_t)(seg_end - pos);
      const int rc = emit(b, p, seg_end == chunk_end, pos == prefix);
      if (rc != KVC_OK) return rc;
      pos = seg_end;
    }
    row += (uint64_t)E;
  }
  if (row != (uint64_t)num_tokens)
    return fail(KVC_ERR_PLAN, "%s: extends sum to %llu, num_tokens %lld", fn,
                (unsigned long long)row, (long long)num_tokens);
  return KVC_OK;
}

int check_plan_args(const char* fn, const int64_t* seq_lens, const int64_t* extend_lens,
                    int64_t batch, int64_t num_tokens) {
  if (batch < 0 || num_tokens < 0) return fail(KVC_ERR_SHAPE, "%s: negative size", fn);
  if (num_tokens > (int64_t)0xfffffffeLL)
    return fail(KVC_ERR_SHAPE, "%s: num_tokens exceeds 2^32-2", fn);
  if (batch > 0 && (!seq_lens || !extend_lens)) return fail(KVC_ERR_NULL, "%s: NULL lengths", fn);
  return KVC_OK;
}

constexpr kvc_online_plan kPadPlan = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};

}  // namespace

extern "C" {

int kvc_c128_plan_prefill(const int64_t* seq_lens, const int64_t* extend_lens, int64_t batch,
                          int64_t num_tokens, kvc_online_plan* compress_plan,
                          kvc_online_plan* write_plan, int pad_to_capacity,
                          uint32_t* n_compress, uint32_t* n_write) {
  const char* fn = "kvc_c128_plan_prefill";
  if (!n_compress || !n_write) return fail(KVC_ERR_NULL, "%s: NULL count", fn);
  *n_compress = *n_write = 0;
  int rc = check_plan_args(fn, seq_lens, extend_lens, batch, num_tokens);
  if (rc != KVC_OK) return rc;
  if (num_tokens > 0 && (!compress_plan || !write_plan))
    return fail(KVC_ERR_NULL, "%s: NULL plan buffer", fn);
  uint32_t nc = 0, nw = 0;
  rc = walk_c128_segments(fn, seq_lens, extend_lens, batch, num_tokens,
                          [&](int64_t, const kvc_online_plan& p, bool closes, bool) {
                            uint32_t& n = closes ? nc : nw;
                            if ((int64_t)n >= num_tokens)
                              return fail(KVC_ERR_PLAN, "%s: %s plans exceed capacity", fn,
                                          closes ? "compress" : "write");
                            (closes ? compress_plan : write_plan)[n++] = p;
                            return (int)KVC_OK;
                          });
  if (rc != KVC_OK) return rc;
  if (pad_to_capacity) {
    for (int64_t i = nc; i < num_tokens; ++i) compress_plan[i] = kPadPlan;
    for (int64_t i = nw; i < num_tokens; ++i) write_plan[i] = kPadPlan;
    nc = nw = (uint32_t)num_tokens;
  }
  *n_compress = nc;
  *n_write = nw;
  return ok();
}

int64_t kvc_c128_fused_capacity(int64_t num_tokens, int64_t max_batch) {
  if (num_tokens < 0 || max_batch < 0) return 0;
  const int64_t bound = num_tokens / 128 + 2 * max_batch;
  return bound < num_tokens ? bound : num_tokens;
}

int kvc_c128_plan_prefill_fused(const int64_t* seq_lens, const int64_t* extend_lens,
                                int64_t batch, int64_t num_tokens, kvc_online_item* items,
                                int64_t capacity, int pad_to_capacity, uint32_t* n_items) {
  const char* fn = "kvc_c128_plan_prefill_fused";
  if (!n_items) return fail(KVC_ERR_NULL, "%s: NULL count", fn);
  *n_items = 0;
  int rc = check_plan_args(fn, seq_lens, extend_lens, batch, num_tokens);
  if (rc != KVC_OK) return rc;
  if (capacity < 0 || capacity > (int64_t)0xffffffffLL)
    return fail(KVC_ERR_SHAPE, "%s: capacity out of range", fn);
  if (capacity > 0 && !items) return fail(KVC_ERR_NULL, "%s: NULL item buffer", fn);
  // A request pairs its first compress plan with its write plan when the
  // former starts mid-chunk; both conditions are fixed by its lengths.
  auto paired = [&](int64_t b) {
    const int64_t L = seq_lens[b], prefix = L - extend_lens[b];
    return prefix % 128 != 0 && (prefix / 128 + 1) * 128 < L && L % 128 != 0;
  };
  // Pass 1: validate and count each kind of item.
  uint64_t n_pair = 0, n_conly = 0, n_wonly = 0;
  rc = walk_c128_segments(fn, seq_lens, extend_lens, batch, num_tokens,
                          [&](int64_t b, const kvc_online_plan&, bool closes, bool first) {
                            const bool pr = paired(b);
                            if (closes && pr && first) ++n_pair;
                            else if (closes) ++n_conly;
                            else if (!pr) ++n_wonly;
                            return (int)KVC_OK;
                          });
  if (rc != KVC_OK) return rc;
  const uint64_t total = n_pair + n_conly + n_wonly;
  if (total > (uint64_t)capacity)
    return fail(KVC_ERR_PLAN, "%s: %llu items exceed capacity %lld", fn,
                (unsigned long long)total, (long long)capacity);
  // Pass 2: place the items.  The compress half of a paired item is written
  // when its first segment is seen, the write half when the trailing one is.
  uint64_t i_pair = 0, i_conly = n_pair, i_wonly = n_pair + n_conly;
  int64_t cur_b = -1;
  uint64_t cur_pair = 0;
  rc = walk_c128_segments(fn, seq_lens, extend_lens, batch, num_tokens,
                          [&](int64_t b, const kvc_online_plan& p, bool closes, bool first) {
                            const bool pr = paired(b);
                            if (closes && pr && first) {
                              cur_b = b;
                              cur_pair = i_pair++;
                              items[cur_pair].compress = p;
                              items[cur_pair].write = kPadPlan;
                            } else if (closes) {
                              items[i_conly].compress = p;
                              items[i_conly++].write = kPadPlan;
                            } else if (pr && cur_b == b) {
                              items[cur_pair].write = p;
                            } else {
                              items[i_wonly].compress = kPadPlan;
                              items[i_wonly++].write = p;
                            }
                            return (int)KVC_OK;
                          });
  if (rc != KVC_OK) return rc;
  uint64_t n = total;
  if (pad_to_capacity) {
    for (int64_t i = (int64_t)total; i < capacity; ++i) items[i] = {kPadPlan, kPadPlan};
    n = (uint64_t)capacity;
  }
  *n_items = (uint32_t)n;
  return ok();
}

// --------------------------------------------------------------- pool-16
namespace {

// Checks shared by the packed and paged prefill entry points; returns KVC_OK
// when the pool inputs are usable.
int check_prefill_inputs(const char* fn, const uint16_t* keys, int64_t key_row_stride,
                         const uint16_t* scores, int64_t score_row_stride, int64_t num_rows,
                         const float* ape, int pool_size, const int32_t* pool_src_row,
                         int64_t n_pools) {
  if (pool_size != kPool) return fail(KVC_ERR_UNSUPPORTED, "%s: pool_size %d (only 16)", fn, pool_size);
  if (!keys || !scores || !ape) return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if (key_row_stride < kHeadDim || score_row_stride < kHeadDim || key_row_stride % 8 ||
      score_row_stride % 8)
    return fail(KVC_ERR_SHAPE, "%s: row strides must be >= 128 and a multiple of 8", fn);
  if (!aligned(keys, 16) || !aligned(scores, 16) || !aligned(ape, 16))
    return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  if (n_pools > kMaxI32 || num_rows > kMaxI32 || key_row_stride > kMaxI32 ||
      score_row_stride > kMaxI32)
    return fail(KVC_ERR_SHAPE, "%s: sizes or strides exceed 2^31-1", fn);
  if (!pool_src_row && n_pools * kPool > num_rows)
    return fail(KVC_ERR_SHAPE, "%s: %lld pools need %lld rows, have %lld", fn, (long long)n_pools,
                (long long)(n_pools * kPool), (long long)num_rows);
  return KVC_OK;
}

int check_ring_inputs(const char* fn, const uint16_t* tail_ring, const int32_t* tail_slot_mapping,
                      const uint16_t* key, int64_t key_stride_b, int64_t key_stride_t,
                      const uint16_t* score, int64_t score_stride_b, int64_t score_stride_t,
                      const float* ape, const int32_t* slot_mapping, const int32_t* positions,
                      int64_t num_requests, int next_n) {
  if (!tail_ring || !tail_slot_mapping || !key || !score || !ape || !slot_mapping || !positions)
    return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if (key_stride_b < 0 || key_stride_t < 0 || score_stride_b < 0 || score_stride_t < 0 ||
      key_stride_b % 8 || key_stride_t % 8 || score_stride_b % 8 || score_stride_t % 8)
    return fail(KVC_ERR_SHAPE, "%s: strides must be non-negative multiples of 8", fn);
  if (!aligned(tail_ring, 16) || !aligned(key, 16) || !aligned(score, 16) || !aligned(ape, 16))
    return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  if (num_requests * (int64_t)next_n > kMaxI32)
    return fail(KVC_ERR_SHAPE, "%s: sizes exceed 2^31-1", fn);
  return KVC_OK;
}

}  // namespace

int kvc_compress_prefill(const uint16_t* keys, int64_t key_row_stride, const uint16_t* scores,
                         int64_t score_row_stride, int64_t num_rows, const float* ape,
                         int pool_size, const int32_t* pool_src_row, int64_t n_pools,
                         uint8_t* out_fp8, float* out_scale, int round_scale, float* dbg_pooled,
                         void* stream) {
  const char* fn = "kvc_compress_prefill";
  if (pool_size != kPool) return fail(KVC_ERR_UNSUPPORTED, "%s: pool_size %d (only 16)", fn, pool_size);
  if (n_pools < 0 || num_rows < 0) return fail(KVC_ERR_SHAPE, "%s: negative size", fn);
  if (n_pools == 0) return ok();
  int rc = check_prefill_inputs(fn, keys, key_row_stride, scores, score_row_stride, num_rows, ape,
                                pool_size, pool_src_row, n_pools);
  if (rc != KVC_OK) return rc;
  if (!out_fp8 || !out_scale) return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if (!aligned(out_fp8, 8) || !aligned(out_scale, 4) || (dbg_pooled && !aligned(dbg_pooled, 16)))
    return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  return hip_status(kvc::launch_pool16_prefill(keys, key_row_stride, scores, score_row_stride,
                                               num_rows, ape, pool_src_row, n_pools, out_fp8,
                                               out_scale, n_pools, false, nullptr, nullptr,
                                               round_scale != 0, dbg_pooled, (hipStream_t)stream),
                    "kvc_compress_prefill launch");
}

int kvc_compress_prefill_paged(const uint16_t* keys, int64_t key_row_stride,
                               const uint16_t* scores, int64_t score_row_stride, int64_t num_rows,
                               const float* ape, int pool_size, const int32_t* pool_src_row,
                               int64_t n_pools, uint8_t* kv_cache, int64_t num_pages,
                               int page_size, const int64_t* loc, const uint8_t* write_mask,
                               int round_scale, void* stream) {
  const char* fn = "kvc_compress_prefill_paged";
  if (pool_size != kPool) return fail(KVC_ERR_UNSUPPORTED, "%s: pool_size %d (only 16)", fn, pool_size);
  if (page_size != 1)
    return fail(KVC_ERR_UNSUPPORTED, "%s: page_size %d (only 1: the larger pages' token order is not specified)", fn, page_size);
  if (n_pools < 0 || num_rows < 0 || num_pages < 0) return fail(KVC_ERR_SHAPE, "%s: negative size", fn);
  if (num_pages > kMaxI32) return fail(KVC_ERR_SHAPE, "%s: num_pages exceeds 2^31-1", fn);
  if (n_pools == 0) return ok();
  int rc = check_prefill_inputs(fn, keys, key_row_stride, scores, score_row_stride, num_rows, ape,
                                pool_size, pool_src_row, n_pools);
  if (rc != KVC_OK) return rc;
  if (!kv_cache || !loc) return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if (!aligned(kv_cache, 4) || !aligned(loc, 8))
    return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  return hip_status(kvc::launch_pool16_prefill(keys, key_row_stride, scores, score_row_stride,
                                               num_rows, ape, pool_src_row, n_pools, kv_cache,
                                               nullptr, num_pages, true, loc, write_mask,
                                               round_scale != 0, nullptr, (hipStream_t)stream),
                    "kvc_compress_prefill_paged launch");
}

}  // extern "C"

namespace {

// Packed-output ring decode over num_layers layers (layer strides in
// elements; ignored for one layer).
int ring_decode_packed(const char* fn, uint16_t* tail_ring, int64_t ring_ls,
                       int64_t num_ring_blocks, const int32_t* tail_slot_mapping,
                       const uint16_t* key, int64_t key_ls, int64_t key_stride_b,
                       int64_t key_stride_t, const uint16_t* score, int64_t score_ls,
                       int64_t score_stride_b, int64_t score_stride_t, const float* ape,
                       int64_t ape_ls, const int32_t* slot_mapping, const int32_t* positions,
                       int64_t num_requests, int next_n, int pool_size, uint8_t* out_fp8,
                       float* out_scale, int64_t num_out, int64_t num_layers, int round_scale,
                       float* dbg_pooled, void* stream) {
  if (pool_size != kPool) return fail(KVC_ERR_UNSUPPORTED, "%s: pool_size %d (only 16)", fn, pool_size);
  if (num_requests < 0 || next_n < 0 || num_ring_blocks < 0 || num_out < 0 || num_layers < 0)
    return fail(KVC_ERR_SHAPE, "%s: negative size", fn);
  if (num_requests == 0 || next_n == 0 || num_layers == 0) return ok();
  int rc = check_ring_inputs(fn, tail_ring, tail_slot_mapping, key, key_stride_b, key_stride_t,
                             score, score_stride_b, score_stride_t, ape, slot_mapping, positions,
                             num_requests, next_n);
  if (rc != KVC_OK) return rc;
  if (num_out > 0 && (!out_fp8 || !out_scale)) return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if (num_out > 0 && (!aligned(out_fp8, 8) || !aligned(out_scale, 4)))
    return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  if (num_out > kMaxI32) return fail(KVC_ERR_SHAPE, "%s: num_out exceeds 2^31-1", fn);
  if (dbg_pooled && !aligned(dbg_pooled, 16)) return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  if (num_layers > 65535) return fail(KVC_ERR_SHAPE, "%s: num_layers exceeds 65535", fn);
  if (num_layers > 1) {
    // Each layer stride must step over a whole layer of its buffer.
    const int64_t key_extent = (num_requests - 1) * key_stride_b + (next_n - 1) * key_stride_t + 128;
    const int64_t score_extent =
        (num_requests - 1) * score_stride_b + (next_n - 1) * score_stride_t + 128;
    if (ring_ls < num_ring_blocks * 2 * kPool * kHeadDim || ring_ls % 8 || key_ls < key_extent ||
        key_ls % 8 || score_ls < score_extent || score_ls % 8 || ape_ls < kPool * kHeadDim ||
        ape_ls % 4)
      return fail(KVC_ERR_SHAPE, "%s: layer strides overlap layers or break alignment", fn);
  } else {
    ring_ls = key_ls = score_ls = ape_ls = 0;
  }
  return hip_status(kvc::launch_pool16_ring(tail_ring, num_ring_blocks, tail_slot_mapping, key,
                                            key_stride_b, key_stride_t, score, score_stride_b,
                                            score_stride_t, ape, slot_mapping, positions,
                                            num_requests, next_n, out_fp8, out_scale, num_out,
                                            false, round_scale != 0, dbg_pooled, num_layers,
                                            ring_ls, key_ls, score_ls, ape_ls,
                                            (hipStream_t)stream),
                    fn);
}

}  // namespace

extern "C" {

int kvc_compress_decode_ring(uint16_t* tail_ring, int64_t num_ring_blocks,
                             const int32_t* tail_slot_mapping, const uint16_t* key,
                             int64_t key_stride_b, int64_t key_stride_t, const uint16_t* score,
                             int64_t score_stride_b, int64_t score_stride_t, const float* ape,
                             const int32_t* slot_mapping, const int32_t* positions,
                             int64_t num_requests, int next_n, int pool_size, uint8_t* out_fp8,
                             float* out_scale, int64_t num_out, int round_scale,
                             float* dbg_pooled, void* stream) {
  return ring_decode_packed("kvc_compress_decode_ring", tail_ring, 0, num_ring_blocks,
                            tail_slot_mapping, key, 0, key_stride_b, key_stride_t, score, 0,
                            score_stride_b, score_stride_t, ape, 0, slot_mapping, positions,
                            num_requests, next_n, pool_size, out_fp8, out_scale, num_out, 1,
                            round_scale, dbg_pooled, stream);
}

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
                                    int64_t num_layers, int round_scale, void* stream) {
  return ring_decode_packed("kvc_compress_decode_ring_layers", tail_ring, ring_layer_stride,
                            num_ring_blocks, tail_slot_mapping, key, key_layer_stride,
                            key_stride_b, key_stride_t, score, score_layer_stride,
                            score_stride_b, score_stride_t, ape, ape_layer_stride, slot_mapping,
                            positions, num_requests, next_n, pool_size, out_fp8, out_scale,
                            num_out, num_layers, round_scale, nullptr, stream);
}

int kvc_compress_decode_ring_paged(uint16_t* tail_ring, int64_t num_ring_blocks,
                                   const int32_t* tail_slot_mapping, const uint16_t* key,
                                   int64_t key_stride_b, int64_t key_stride_t,
                                   const uint16_t* score, int64_t score_stride_b,
                                   int64_t score_stride_t, const float* ape,
                                   const int32_t* slot_mapping, const int32_t* positions,
                                   int64_t num_requests, int next_n, int pool_size,
                                   uint8_t* kv_cache, int64_t num_pages, int page_size,
                                   int round_scale, void* stream) {
  const char* fn = "kvc_compress_decode_ring_paged";
  if (pool_size != kPool) return fail(KVC_ERR_UNSUPPORTED, "%s: pool_size %d (only 16)", fn, pool_size);
  if (page_size != 1)
    return fail(KVC_ERR_UNSUPPORTED, "%s: page_size %d (only 1: the larger pages' token order is not specified)", fn, page_size);
  if (num_requests < 0 || next_n < 0 || num_ring_blocks < 0 || num_pages < 0)
    return fail(KVC_ERR_SHAPE, "%s: negative size", fn);
  if (num_requests == 0 || next_n == 0) return ok();
  int rc = check_ring_inputs(fn, tail_ring, tail_slot_mapping, key, key_stride_b, key_stride_t,
                             score, score_stride_b, score_stride_t, ape, slot_mapping, positions,
                             num_requests, next_n);
  if (rc != KVC_OK) return rc;
  if (num_pages > 0 && !kv_cache) return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if (num_pages > 0 && !aligned(kv_cache, 4)) return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  return hip_status(kvc::launch_pool16_ring(tail_ring, num_ring_blocks, tail_slot_mapping, key,
                                            key_stride_b, key_stride_t, score, score_stride_b,
                                            score_stride_t, ape, slot_mapping, positions,
                                            num_requests, next_n, kv_cache, nullptr, num_pages,
                                            true, round_scale != 0, nullptr, 1, 0, 0, 0, 0,
                                            (hipStream_t)stream),
                    "kvc_compress_decode_ring_paged launch");
}

int kvc_seed_tail_ring(uint16_t* tail_ring, int64_t num_ring_blocks, const uint16_t* key,
                       int64_t key_row_stride, const uint16_t* score, int64_t score_row_stride,
                       const int32_t* tslot, int64_t n_tokens, int pool_size, void* stream) {
  if (pool_size != kPool)
    return fail(KVC_ERR_UNSUPPORTED, "kvc_seed_tail_ring: pool_size %d (only 16)", pool_size);
  if (n_tokens < 0 || num_ring_blocks < 0)
    return fail(KVC_ERR_SHAPE, "kvc_seed_tail_ring: negative size");
  if (n_tokens == 0) return ok();
  if (!tail_ring || !key || !score || !tslot)
    return fail(KVC_ERR_NULL, "kvc_seed_tail_ring: NULL pointer");
  if (key_row_stride < kHeadDim || score_row_stride < kHeadDim || key_row_stride % 8 ||
      score_row_stride % 8)
    return fail(KVC_ERR_SHAPE, "kvc_seed_tail_ring: row strides must be >= 128 and a multiple of 8");
  if (!aligned(tail_ring, 16) || !aligned(key, 16) || !aligned(score, 16) || !aligned(tslot, 4))
    return fail(KVC_ERR_SHAPE, "kvc_seed_tail_ring: misaligned pointer");
  if (n_tokens > kMaxI32) return fail(KVC_ERR_SHAPE, "kvc_seed_tail_ring: n_tokens exceeds 2^31-1");
  return hip_status(kvc::launch_pool16_seed(tail_ring, num_ring_blocks, key, key_row_stride,
                                            score, score_row_stride, tslot, n_tokens,
                                            (hipStream_t)stream),
                    "kvc_seed_tail_ring launch");
}

// --------------------------------------------------------------- pool-128
namespace {

int check_decode(const char* fn, float* state, int64_t num_slots, const float* kv_score_in,
                 const float* ape, const int32_t* indices, const int32_t* seq_lens,
                 int64_t batch) {
  if (!state || !kv_score_in || !ape || !indices || !seq_lens)
    return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if (!aligned(state, 16) || !aligned(kv_score_in, 16) || !aligned(ape, 16))
    return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  if (batch > kMaxI32 || num_slots > kMaxI32) return fail(KVC_ERR_SHAPE, "%s: sizes exceed 2^31-1", fn);
  return KVC_OK;
}

int check_prefill(const char* fn, float* state, int64_t num_slots, const float* kv_score_in,
                  int64_t num_tokens, const float* ape, const int32_t* indices, int64_t batch,
                  const kvc_online_plan* compress_plan, uint32_t n_compress,
                  const kvc_online_plan* write_plan, uint32_t n_write) {
  if (!state || !kv_score_in || !ape || !indices || (n_compress && !compress_plan) ||
      (n_write && !write_plan))
    return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if (!aligned(state, 16) || !aligned(kv_score_in, 16) || !aligned(ape, 16) ||
      (compress_plan && !aligned(compress_plan, 16)) || (write_plan && !aligned(write_plan, 16)))
    return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  if (num_tokens > (int64_t)0xfffffffeLL || num_slots > kMaxI32 || batch > kMaxI32)
    return fail(KVC_ERR_SHAPE, "%s: sizes out of range", fn);
  return KVC_OK;
}

// fp32-output decode over num_layers layers (layer strides in elements;
// ignored for one layer).
int c128_decode_fp32(const char* fn, float* state, int64_t state_layer_stride, int64_t num_slots,
                     const float* kv_score_in, int64_t in_layer_stride, float* out,
                     int64_t out_layer_stride, const float* ape, int64_t ape_layer_stride,
                     const int32_t* indices, const int32_t* seq_lens, int64_t batch,
                     int64_t num_layers, void* stream) {
  if (batch < 0 || num_slots < 0 || num_layers < 0) return fail(KVC_ERR_SHAPE, "%s: negative size", fn);
  if (batch == 0 || num_layers == 0) return ok();
  int rc = check_decode(fn, state, num_slots, kv_score_in, ape, indices, seq_lens, batch);
  if (rc != KVC_OK) return rc;
  if (!out) return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if (!aligned(out, 16)) return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  if (num_layers > 65535) return fail(KVC_ERR_SHAPE, "%s: num_layers exceeds 65535", fn);
  if (num_layers > 1 &&
      (state_layer_stride < num_slots * 384 || in_layer_stride < batch * 256 ||
       out_layer_stride < batch * 128 || ape_layer_stride < 128 * 128 ||
       state_layer_stride % 4 || in_layer_stride % 4 || out_layer_stride % 4 ||
       ape_layer_stride % 4))
    return fail(KVC_ERR_SHAPE, "%s: layer strides must cover a layer and keep 16-byte rows", fn);
  if (num_layers == 1) state_layer_stride = in_layer_stride = out_layer_stride = ape_layer_stride = 0;
  return hip_status(kvc::launch_c128_decode(state, state_layer_stride, num_slots, kv_score_in,
                                            in_layer_stride, out, out_layer_stride, nullptr,
                                            nullptr, false, ape, ape_layer_stride, indices,
                                            seq_lens, batch, num_layers, (hipStream_t)stream),
                    fn);
}

}  // namespace

int kvc_c128_online_decode(float* state, int64_t num_slots, const float* kv_score_in, float* out,
                           const float* ape, const int32_t* indices, const int32_t* seq_lens,
                           int64_t batch, void* stream) {
  return c128_decode_fp32("kvc_c128_online_decode", state, 0, num_slots, kv_score_in, 0, out, 0,
                          ape, 0, indices, seq_lens, batch, 1, stream);
}

int kvc_c128_online_decode_layers(float* state, int64_t state_layer_stride, int64_t num_slots,
                                  const float* kv_score_in, int64_t in_layer_stride, float* out,
                                  int64_t out_layer_stride, const float* ape,
                                  int64_t ape_layer_stride, const int32_t* indices,
                                  const int32_t* seq_lens, int64_t batch, int64_t num_layers,
                                  void* stream) {
  return c128_decode_fp32("kvc_c128_online_decode_layers", state, state_layer_stride, num_slots,
                          kv_score_in, in_layer_stride, out, out_layer_stride, ape,
                          ape_layer_stride, indices, seq_lens, batch, num_layers, stream);
}

int kvc_c128_online_decode_quant(float* state, int64_t num_slots, const float* kv_score_in,
                                 uint8_t* out_fp8, float* out_scale, const float* ape,
                                 const int32_t* indices, const int32_t* seq_lens, int64_t batch,
                                 int round_scale, void* stream) {
  const char* fn = "kvc_c128_online_decode_quant";
  if (batch < 0 || num_slots < 0) return fail(KVC_ERR_SHAPE, "%s: negative size", fn);
  if (batch == 0) return ok();
  int rc = check_decode(fn, state, num_slots, kv_score_in, ape, indices, seq_lens, batch);
  if (rc != KVC_OK) return rc;
  if (!out_fp8 || !out_scale) return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if (!aligned(out_fp8, 4) || !aligned(out_scale, 4))
    return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  return hip_status(kvc::launch_c128_decode(state, 0, num_slots, kv_score_in, 0, nullptr, 0,
                                            out_fp8, out_scale, round_scale != 0, ape, 0, indices,
                                            seq_lens, batch, 1, (hipStream_t)stream),
                    "kvc_c128_online_decode_quant launch");
}

int kvc_c128_online_prefill(float* state, int64_t num_slots, const float* kv_score_in, float* out,
                            int64_t num_tokens, const float* ape, const int32_t* indices,
                            const int32_t* load_indices, int64_t batch,
                            const kvc_online_plan* compress_plan, uint32_t n_compress,
                            const kvc_online_plan* write_plan, uint32_t n_write, void* stream) {
  const char* fn = "kvc_c128_online_prefill";
  if (batch < 0 || num_slots < 0 || num_tokens < 0) return fail(KVC_ERR_SHAPE, "%s: negative size", fn);
  if (n_compress == 0 && n_write == 0) return ok();
  int rc = check_prefill(fn, state, num_slots, kv_score_in, num_tokens, ape, indices, batch,
                         compress_plan, n_compress, write_plan, n_write);
  if (rc != KVC_OK) return rc;
  if (n_compress && !out) return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if (out && !aligned(out, 16)) return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  return hip_status(kvc::launch_c128_prefill(state, num_slots, kv_score_in, out, nullptr, nullptr,
                                             false, num_tokens, ape, indices, load_indices, batch,
                                             compress_plan, n_compress, write_plan, n_write,
                                             (hipStream_t)stream),
                    "kvc_c128_online_prefill launch");
}

int kvc_c128_online_prefill_quant(float* state, int64_t num_slots, const float* kv_score_in,
                                  uint8_t* out_fp8, float* out_scale, int64_t num_tokens,
                                  const float* ape, const int32_t* indices,
                                  const int32_t* load_indices, int64_t batch,
                                  const kvc_online_plan* compress_plan, uint32_t n_compress,
                                  const kvc_online_plan* write_plan, uint32_t n_write,
                                  int round_scale, void* stream) {
  const char* fn = "kvc_c128_online_prefill_quant";
  if (batch < 0 || num_slots < 0 || num_tokens < 0) return fail(KVC_ERR_SHAPE, "%s: negative size", fn);
  if (n_compress == 0 && n_write == 0) return ok();
  int rc = check_prefill(fn, state, num_slots, kv_score_in, num_tokens, ape, indices, batch,
                         compress_plan, n_compress, write_plan, n_write);
  if (rc != KVC_OK) return rc;
  if (n_compress && (!out_fp8 || !out_scale)) return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if ((out_fp8 && !aligned(out_fp8, 4)) || (out_scale && !aligned(out_scale, 4)))
    return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  return hip_status(kvc::launch_c128_prefill(state, num_slots, kv_score_in, nullptr, out_fp8,
                                             out_scale, round_scale != 0, num_tokens, ape,
                                             indices, load_indices, batch, compress_plan,
                                             n_compress, write_plan, n_write,
                                             (hipStream_t)stream),
                    "kvc_c128_online_prefill_quant launch");
}

int kvc_c128_online_prefill_fused(float* state, int64_t num_slots, const float* kv_score_in,
                                  float* out, uint8_t* out_fp8, float* out_scale,
                                  int round_scale, int64_t num_tokens, const float* ape,
                                  const int32_t* indices, const int32_t* load_indices,
                                  int64_t batch, const kvc_online_item* items, uint32_t n_items,
                                  void* stream) {
  const char* fn = "kvc_c128_online_prefill_fused";
  if (batch < 0 || num_slots < 0 || num_tokens < 0) return fail(KVC_ERR_SHAPE, "%s: negative size", fn);
  if (n_items == 0) return ok();
  if (!items) return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  int rc = check_prefill(fn, state, num_slots, kv_score_in, num_tokens, ape, indices, batch,
                         nullptr, 0, nullptr, 0);
  if (rc != KVC_OK) return rc;
  if (!aligned(items, 16)) return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  const bool quant = out_fp8 != nullptr;
  if (quant ? (out != nullptr || !out_scale) : (!out || out_scale != nullptr))
    return fail(KVC_ERR_NULL, "%s: give either out or out_fp8 with out_scale", fn);
  if ((out && !aligned(out, 16)) || (out_fp8 && !aligned(out_fp8, 4)) ||
      (out_scale && !aligned(out_scale, 4)))
    return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  return hip_status(kvc::launch_c128_prefill_fused(state, num_slots, kv_score_in, out, out_fp8,
                                                   out_scale, round_scale != 0, num_tokens, ape,
                                                   indices, load_indices, batch, items, n_items,
                                                   (hipStream_t)stream),
                    "kvc_c128_online_prefill_fused launch");
}

// --------------------------------------------------------------- diagnostics
int kvc_diag_convert(const float* in, uint16_t* bf16_out, uint8_t* fp8_out, int64_t n,
                     void* stream) {
  if (n < 0 || n % 2) return fail(KVC_ERR_SHAPE, "kvc_diag_convert: n must be even and >= 0");
  if (n == 0) return ok();
  if (!in) return fail(KVC_ERR_NULL, "kvc_diag_convert: NULL input");
  return hip_status(kvc::launch_diag_convert(in, bf16_out, fp8_out, n, (hipStream_t)stream),
                    "kvc_diag_convert launch");
}

int kvc_diag_stream_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words,
                         int loads_per_lane, int fold, void* stream) {
  const char* fn = "kvc_diag_stream_read";
  if (bytes < 0 || bytes % 16) return fail(KVC_ERR_SHAPE, "%s: bytes must be a multiple of 16", fn);
  if (loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8 && loads_per_lane != 16)
    return fail(KVC_ERR_UNSUPPORTED, "%s: loads_per_lane %d (2, 4, 8 or 16)", fn, loads_per_lane);
  if (bytes == 0) return ok();
  if (!src || !sink) return fail(KVC_ERR_NULL, "%s: NULL pointer", fn);
  if (!aligned(src, 16) || !aligned(sink, 4)) return fail(KVC_ERR_SHAPE, "%s: misaligned pointer", fn);
  const int64_t per_block = 4096LL * loads_per_lane;
  const int64_t blocks = (bytes + per_block - 1) / per_block;
  if (blocks > 0x7fffffffLL) return fail(KVC_ERR_SHAPE, "%s: buffer too large", fn);
  if (sink_words < 4 * blocks)
    return fail(KVC_ERR_SHAPE, "%s: sink needs %lld words", fn, (long long)(4 * blocks));
  return hip_status(kvc::launch_diag_stream_read(src, bytes, sink, loads_per_lane, fold != 0,
                                                 (hipStream_t)stream),
                    "kvc_diag_stream_read launch");
}

int kvc_diag_empty_launch(int64_t workgroups, int threads, int arg_bytes, void* stream) {
  const char* fn = "kvc_diag_empty_launch";
  if (workgroups < 0 || workgroups > 0x7fffffffLL)
    return fail(KVC_ERR_SHAPE, "%s: workgroups out of range", fn);
  if (threads < 1 || threads > 1024) return fail(KVC_ERR_SHAPE, "%s: threads must be 1..1024", fn);
  if (arg_bytes != 0 && arg_bytes != 64 && arg_bytes != 112 && arg_bytes != 136 && arg_bytes != 448)
    return fail(KVC_ERR_UNSUPPORTED, "%s: arg_bytes %d (0, 64, 112, 136 or 448)", fn, arg_bytes);
  if (workgroups == 0) return ok();
  return hip_status(kvc::launch_diag_empty(workgroups, threads, arg_bytes, (hipStream_t)stream),
                    "kvc_diag_empty_launch launch");
}

}  // extern "C"
