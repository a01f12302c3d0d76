// kvc_internal.hpp -- launcher interface between the C-ABI layer (argument
// validation, planners) and the HIP kernel translation units.  Launchers
// assume validated arguments and only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

// out_fp8 / out_scale: packed [out_rows,128] codes and [out_rows] scales, or
// (paged) out_fp8 is a [out_rows, 132] byte cache and out_scale is unused.
// loc (optional) maps pool p to its output row; write_mask (optional) skips
// pools whose byte is 0.
hipError_t launch_pool16_prefill(const uint16_t* keys, int64_t key_stride, const uint16_t* scores,
                                 int64_t score_stride, int64_t num_rows, const float* ape,
                                 const int32_t* src_rows, int64_t n_pools, uint8_t* out_fp8,
                                 float* out_scale, int64_t out_rows, bool paged,
                                 const int64_t* loc, const uint8_t* write_mask, bool round_scale,
                                 float* dbg, hipStream_t stream);

// Ring decode over num_layers layers (blockIdx.y): layer l reads ring / key /
// score / ape at the given layer strides (elements; 0 for one layer) and
// writes output rows l*out_rows .. l*out_rows + out_rows - 1 of the sink.
hipError_t launch_pool16_ring(uint16_t* ring, int64_t num_blocks, const int32_t* tail_slot,
                              const uint16_t* key, int64_t key_sb, int64_t key_st,
                              const uint16_t* score, int64_t score_sb, int64_t score_st,
                              const float* ape, const int32_t* slot_mapping,
                              const int32_t* positions, int64_t num_requests, int next_n,
                              uint8_t* out_fp8, float* out_scale, int64_t out_rows, bool paged,
                              bool round_scale, float* dbg, int64_t num_layers,
                              int64_t ring_ls, int64_t key_ls, int64_t score_ls, int64_t ape_ls,
                              hipStream_t stream);

hipError_t launch_pool16_seed(uint16_t* ring, int64_t num_blocks, const uint16_t* key,
                              int64_t key_stride, const uint16_t* score, int64_t score_stride,
                              const int32_t* tslot, int64_t n_tokens, hipStream_t stream);

// Decode over num_layers layers (blockIdx.y); emitted vectors go to `out`
// (fp32) or, when `codes` is non-null, through the rotate/quantise epilogue
// to codes [layers][batch][128] and scales [layers][batch].
hipError_t launch_c128_decode(float* state, int64_t state_ls, int64_t num_slots, const float* in,
                              int64_t in_ls, float* out, int64_t out_ls, uint8_t* codes,
                              float* scales, bool round_scale, const float* ape, int64_t ape_ls,
                              const int32_t* indices, const int32_t* seq_lens, int64_t batch,
                              int64_t num_layers, hipStream_t stream);

// Prefill; chunk-closing vectors go to `out` (fp32 [num_tokens,128]) or,
// when `codes` is non-null, to codes [num_tokens,128] + scales [num_tokens].
hipError_t launch_c128_prefill(float* state, int64_t num_slots, const float* in, float* out,
                               uint8_t* codes, float* scales, bool round_scale,
                               int64_t num_tokens, const float* ape, const int32_t* indices,
                               const int32_t* load_indices, int64_t batch,
                               const kvc_online_plan* cplan, uint32_t n_c,
                               const kvc_online_plan* wplan, uint32_t n_w, hipStream_t stream);

// Single-launch prefill over {compress, write} work items (state rows are
// read at load_indices[b], or indices[b] when null, and written at indices[b]).
hipError_t launch_c128_prefill_fused(float* state, int64_t num_slots, const float* in, float* out,
                                     uint8_t* codes, float* scales, bool round_scale,
                                     int64_t num_tokens, const float* ape, const int32_t* indices,
                                     const int32_t* load_indices, int64_t batch,
                                     const kvc_online_item* items, uint32_t n_items,
                                     hipStream_t stream);

hipError_t launch_diag_convert(const float* in, uint16_t* bf16_out, uint8_t* fp8_out, int64_t n,
                               hipStream_t stream);

// loads_per_lane is 2, 4, 8 or 16; sink needs 4 * ceil(bytes / (4096 * loads_per_lane))
// words (one per wave).
hipError_t launch_diag_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                                   int loads_per_lane, bool fold, hipStream_t stream);
// arg_bytes: 0, 64, 112, 136 or 448 (the size of the empty kernel's argument block).
hipError_t launch_diag_empty(int64_t workgroups, int threads, int arg_bytes, hipStream_t stream);

}  // namespace kvc
