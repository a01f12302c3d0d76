// kvc_c128.hip -- pool-128 online compression kernels for gfx950.
//
// Method (SGLang page "c128_online.cuh": flash_c128_online_decode,
// flash_c128_online_prefill, c128_prefill_forward): a per-sequence fp32 state
// (max, sum, kv) holds the softmax statistics of the tokens folded into the
// open 128-token chunk; a closing chunk emits its weighted mean.
//
// Work mapping on MI355X:
//   decode   one request per half-wave (32 lanes x float4 = one 512 B state
//            row); two requests per 64-thread workgroup so even a small batch
//            spreads over many CUs.  Two round trips: slots, lengths and
//            input rows, then ape rows and states (multi-layer launches read
//            slots and lengths through scalar loads first).
//   prefill  one 512-thread workgroup per plan.  Wave w covers chunk
//            positions [16w, 16w+16); its two half-waves take even / odd
//            positions, 4 channels per lane, so every token row is read with
//            128-bit loads and each lane keeps a private two-pass softmax over
//            8 tokens in registers.  All row loads are issued branch-free
//            right after the 16-byte plan load.  Partial (max, sum, weighted sum) states
//            are merged across half-waves with a lane shuffle and across waves
//            through LDS, then merged with the stored state when the segment
//            starts mid-chunk.  Sums stay unnormalised until the end, so an
//            empty partial (max = -FLT_MAX, sums 0) merges as a no-op and never
//            produces NaN.
#include <cfloat>

#include "kvc_device.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

// ------------------------------------------------------------------ decode
// Requests (32 lanes each) per workgroup.  A single-layer call is latency-
// bound and spreads over as many CUs as possible; a multi-layer launch is
// bandwidth-bound and runs best with 256-thread workgroups (measured: 2 / 4 /
// 8 requests per workgroup give 72.7 / 74.6 / 75.1% of peak on 64 layers).
#ifndef KVC_C128_DECODE_REQ_SINGLE
#define KVC_C128_DECODE_REQ_SINGLE 2
#endif
#ifndef KVC_C128_DECODE_REQ_LAYERS
#define KVC_C128_DECODE_REQ_LAYERS 8
#endif
constexpr int kDecodeReqSingle = KVC_C128_DECODE_REQ_SINGLE;
constexpr int kDecodeReqLayers = KVC_C128_DECODE_REQ_LAYERS;

// Where emitted (chunk-closing) vectors go: fp32 rows, or e4m3 codes plus a
// per-vector scale after the bf16 / rotation / quantisation epilogue.
struct EmitSink {
  float* out;            // fp32 [rows, 128] (fp32 mode)
  uint8_t* codes;        // e4m3 [rows, 128] (quantised mode)
  float* scales;         // fp32 [rows]      (quantised mode)
  int64_t out_ls;        // per-layer strides (elements) of out / codes / scales
  int64_t codes_ls;
  int64_t scales_ls;
  bool round_scale;
};

// Emit one 128-vector held by 32 lanes (lane q: channels 4q..4q+3).  In the
// quantised mode the 32 lanes must all be active.
template <bool kQuant>
__device__ __forceinline__ void emit32(const EmitSink& o, int64_t layer, int64_t row, int q,
                                       const float (&K)[4]) {
  if constexpr (kQuant) {
    // channel 4q + t: bits 0-1 in registers, bits 2-5 in the lane of the
    // 16-lane row (q & 15), bit 6 in the row (q >> 4).
    float v[4] = {K[0], K[1], K[2], K[3]};
    float scale;
    const uint32_t code = rotate_quantise32(v, q & 15, q >> 4, o.round_scale, scale);
    reinterpret_cast<uint32_t*>(o.codes + layer * o.codes_ls + row * 128)[q] = code;
    if (q == 0) o.scales[layer * o.scales_ls + row] = scale;
  } else {
    reinterpret_cast<float4*>(o.out + layer * o.out_ls + row * 128)[q] =
        make_float4(K[0], K[1], K[2], K[3]);
  }
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 128-bit load and store of an fp32 quad: the line
// is not kept in the caches.
__device__ __forceinline__ float4 load_stream4(const float4* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream4(float4* p, float4 v) {
  __builtin_nontemporal_store((f32x4_t){v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4_t*>(p));
}

// (group, layer) of a workgroup in a multi-layer launch whose layer count is
// a multiple of 8, laid out XCD-major.  Workgroups go to the eight XCDs round
// robin in dispatch order (blockIdx.x fastest), so workgroup number n runs on
// XCD n % 8; it is given layer (n % 8) + 8 * ((n / 8) / G) and group
// (n / 8) % G (G = gridDim.x), a one-to-one map under which each XCD runs
// every group of its own layers and each layer's ape table is fetched into
// one XCD's L2 instead of all eight.
__device__ __forceinline__ void xcd_major_group_layer(uint32_t& group, uint32_t& layer) {
  const uint32_t G = gridDim.x, n = blockIdx.x + blockIdx.y * G;
  const uint32_t j = n >> 3;
  layer = (n & 7u) + 8u * (j / G);
  group = j % G;
}

// One request per 32 lanes; the workgroup handles requests group * kReq ..
// group * kReq + kReq - 1 of one layer (state, input, output and ape advance
// by their layer strides; indices and lengths are shared by all layers).
template <bool kQuant, int kReq>
__device__ __forceinline__ void c128_decode_group(
    float* __restrict__ state, int64_t state_ls, int64_t num_slots, const float* __restrict__ in,
    int64_t in_ls, const EmitSink& o, const float* __restrict__ ape, int64_t ape_ls,
    const int32_t* __restrict__ indices, const int32_t* __restrict__ seq_lens, int64_t batch,
    uint32_t group, int64_t layer) {
  static_assert(kReq == 1 || kReq % 2 == 0, "a wave holds two whole requests");
  // Single calls: take every kernel argument into SGPRs at entry.  Left to
  // itself the compiler loads arguments next to their first use, behind the
  // early exits, and one of those scalar loads (num_slots) fell between the
  // two memory round trips: 3.40-3.62 -> 3.12-3.17 us per 1024-request call.
  // A volatile asm statement counts as a memory access for alias analysis,
  // so uniform loads after it are no longer scalarised; multi-layer
  // launches, whose slots come through scalar loads, keep the compiler's
  // order.
  if constexpr (kReq <= 2)
    asm volatile("" ::"s"(state), "s"(state_ls), "s"(num_slots), "s"(in), "s"(in_ls), "s"(ape),
                 "s"(ape_ls), "s"(indices), "s"(seq_lens), "s"(batch), "s"(o.out), "s"(o.codes),
                 "s"(o.scales));
  const int64_t b = (int64_t)group * kReq + (threadIdx.x >> 5);
  const int q = threadIdx.x & 31;                       // channels 4q..4q+3
  // Two round trips.  Each issues its loads together (the empty asm
  // statements take all their values at once; without them the compiler had
  // sunk the input-row loads below the slot check and the state loads below
  // the score sum: three or four dependent round trips).
  //  * Multi-layer launches (kReq > 2): the slots and lengths of the wave's
  //    two requests are read at wave-uniform addresses, through scalar loads;
  //    then the input row, the ape row (it depends on the length) and the
  //    stored state (it depends on the slot) load together.  64 layers:
  //    75.3% -> 76.9% of HBM peak against the two vector round trips below.
  //  * Single calls: slot, length and input row, then ape row and state.  The
  //    scalar form was faster back to back (3.38 instead of 3.67 us) but no
  //    faster after an unrelated kernel (both 4.0 us) and slower under the
  //    profiler's per-dispatch tracing (4.7 us), so single calls keep this.
  constexpr bool kScalarSlots = kReq > 2;
  int32_t idx, L;
  float4 kv, sc;
  const float4* row = reinterpret_cast<const float4*>(in + layer * in_ls + b * 256);
  if constexpr (kScalarSlots) {
    // The wave's two slots and lengths at clamped indices (no branch), then
    // every other kernel argument into SGPRs: two scalar waits before the
    // vector loads instead of four (64 layers 44.32-44.40 -> 44.11-44.22 us).
    // The asm statement comes after the slot loads, which keeps them scalar.
    const int v = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t b0 = (int64_t)group * kReq + 2 * v;
    const int64_t c0 = b0 < batch ? b0 : batch - 1, c1 = b0 + 1 < batch ? b0 + 1 : batch - 1;
    int32_t i0 = indices[c0], l0 = seq_lens[c0], i1 = indices[c1], l1 = seq_lens[c1];
    asm volatile("" ::"s"(state), "s"(state_ls), "s"(num_slots), "s"(in), "s"(in_ls), "s"(ape),
                 "s"(ape_ls), "s"(o.out), "s"(o.codes), "s"(o.scales), "s"(i0), "s"(l0), "s"(i1),
                 "s"(l1));
    if (b0 >= batch) { i0 = -1; l0 = 0; }
    if (b0 + 1 >= batch) { i1 = -1; l1 = 0; }
    if (b >= batch) return;
    idx = (threadIdx.x & 32) ? i1 : i0;
    L = (threadIdx.x & 32) ? l1 : l0;
    if (L <= 0 || idx < 0 || (int64_t)idx >= num_slots) return;
    kv = row[q];
    sc = row[32 + q];
  } else {
    if (b >= batch) return;
    idx = indices[b];
    L = seq_lens[b];
    kv = row[q];
    sc = row[32 + q];
    asm volatile("" ::"v"(idx), "v"(L), "v"(kv.x), "v"(kv.y), "v"(kv.z), "v"(kv.w), "v"(sc.x),
                 "v"(sc.y), "v"(sc.z), "v"(sc.w));
    if (L <= 0 || idx < 0 || (int64_t)idx >= num_slots) return;
  }
  const int c = (L - 1) & 127;
  const float4 bias = reinterpret_cast<const float4*>(ape + layer * ape_ls + c * 128)[q];
  float4* st = reinterpret_cast<float4*>(state + layer * state_ls + (int64_t)idx * 384);
  float4 m4 = make_float4(0.f, 0.f, 0.f, 0.f), s4 = m4, k4 = m4;
  // The state row is read and rewritten through non-temporal accesses (both:
  // either one alone measured slower or no faster): 64 layers 44.8-45.0 ->
  // 42.8-43.0 us, a single 1024-request call 3.17-3.39 -> 2.97-2.99 us.
  if (c != 0) {   // the first token of a chunk does not read the state
    m4 = load_stream4(st + q);
    s4 = load_stream4(st + 32 + q);
    k4 = load_stream4(st + 64 + q);
  }
  asm volatile("" ::"v"(kv.x), "v"(kv.y), "v"(kv.z), "v"(kv.w), "v"(sc.x), "v"(sc.y), "v"(sc.z),
               "v"(sc.w), "v"(bias.x), "v"(bias.y), "v"(bias.z), "v"(bias.w), "v"(m4.x),
               "v"(m4.y), "v"(m4.z), "v"(m4.w), "v"(s4.x), "v"(s4.y), "v"(s4.z), "v"(s4.w),
               "v"(k4.x), "v"(k4.y), "v"(k4.z), "v"(k4.w));

  float s[4] = {sc.x + bias.x, sc.y + bias.y, sc.z + bias.z, sc.w + bias.w};
  float k[4] = {kv.x, kv.y, kv.z, kv.w};
  float M[4], S[4], K[4];
  if (c != 0) {
    const float om[4] = {m4.x, m4.y, m4.z, m4.w};
    const float os[4] = {s4.x, s4.y, s4.z, s4.w};
    const float ok[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mx = fmaxf(om[i], s[i]);
      const float a = os[i] * exp2_hw((om[i] - mx) * kLog2e);
      const float e = exp2_hw((s[i] - mx) * kLog2e);
      const float sum = a + e;
      M[i] = mx;
      S[i] = sum;
      K[i] = (ok[i] * a + k[i] * e) / sum;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) { M[i] = s[i]; S[i] = 1.0f; K[i] = k[i]; }
  }
  if (c == 127) {
    emit32<kQuant>(o, layer, b, q, K);
  } else {
    store_stream4(st + q, make_float4(M[0], M[1], M[2], M[3]));
    store_stream4(st + 32 + q, make_float4(S[0], S[1], S[2], S[3]));
    store_stream4(st + 64 + q, make_float4(K[0], K[1], K[2], K[3]));
  }
}

// Multi-layer launches (and single calls whose sizes exceed 32 bits): grid
// (request groups, layers).  With a multiple of 8 layers the workgroups run
// XCD-major (64 layers: 42.8 -> 40.0 us, bit-identical); otherwise workgroup
// (x, y) is group x of layer y.
template <bool kQuant, int kReq>
__global__ __launch_bounds__(32 * kReq) void c128_decode_kernel(
    float* __restrict__ state, int64_t state_ls, int64_t num_slots, const float* __restrict__ in,
    int64_t in_ls, EmitSink o, const float* __restrict__ ape, int64_t ape_ls,
    const int32_t* __restrict__ indices, const int32_t* __restrict__ seq_lens, int64_t batch) {
  uint32_t group = blockIdx.x, layer = blockIdx.y;
  if (kReq > 2 && (gridDim.y & 7u) == 0) xcd_major_group_layer(group, layer);
  c128_decode_group<kQuant, kReq>(state, state_ls, num_slots, in, in_ls, o, ape, ape_ls, indices,
                                  seq_lens, batch, group, layer);
}

// Single calls with a compact argument block (72 bytes instead of the 136 of
// the general kernel; out0 is the fp32 output or, quantised, the codes).  The
// runtime's host-side cost of a launch grows with the kernel's argument
// block, by about 1 us between 96 and 120 bytes, and this call is short
// enough on the device (about 3 us) for that to matter.
template <bool kQuant>
__global__ __launch_bounds__(32 * kDecodeReqSingle) void c128_decode_one_kernel(
    float* __restrict__ state, const float* __restrict__ in, void* __restrict__ out0,
    float* __restrict__ scales, const float* __restrict__ ape, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ seq_lens, uint32_t num_slots, uint32_t batch,
    uint32_t round_scale) {
  const EmitSink o{kQuant ? nullptr : static_cast<float*>(out0),
                   kQuant ? static_cast<uint8_t*>(out0) : nullptr, scales, 0, 0, 0,
                   round_scale != 0};
  c128_decode_group<kQuant, kDecodeReqSingle>(state, 0, num_slots, in, 0, o, ape, 0, indices,
                                              seq_lens, batch, blockIdx.x, 0);
}

// ------------------------------------------------------------------ prefill
#ifndef KVC_C128_COMPRESS_WAVES
#define KVC_C128_COMPRESS_WAVES 8
#endif
#ifndef KVC_C128_WRITE_WAVES
#define KVC_C128_WRITE_WAVES 8
#endif
// 8 waves per plan (8 chunk positions per lane) keeps every lane's row loads
// in flight at once within 128 VGPRs; measured best for both passes (the
// compress pass is bandwidth-bound, the write pass latency-bound).
constexpr int kCompressWaves = KVC_C128_COMPRESS_WAVES;
constexpr int kWriteWaves = KVC_C128_WRITE_WAVES;

// Merge partial (m2, d2, a2) into (M, D, A); d = sum of e^{s-m}, a = sum of
// k e^{s-m} (unnormalised).
__device__ __forceinline__ void merge_partial(float& M, float& D, float& A, float m2, float d2,
                                              float a2) {
  const float mx = fmaxf(M, m2);
  const float f1 = exp2_hw((M - mx) * kLog2e);
  const float f2 = exp2_hw((m2 - mx) * kLog2e);
  D = D * f1 + d2 * f2;
  A = A * f1 + a2 * f2;
  M = mx;
}

// LDS partials of one plan: (max, sum, weighted sum) per wave and channel
// (rows padded to 136 floats: the merge below reads four rows at once, which
// then fall on different banks), and the finished vector for the quantised
// epilogue.
template <int kWaves>
struct PlanLds {
  float m[kWaves][136], d[kWaves][136], a[kWaves][136];
  float k[128];
};

// One plan (16-byte entry pv) processed by the whole workgroup.  Returns
// early for padding or malformed entries (uniformly, before the barrier) and
// for the lanes that do not finish the plan (after it).  kWrite: store the
// (max, sum, kv) state to indices[b]; otherwise emit the normalised vector to
// row ragged_id.
template <bool kWrite, int kWaves, bool kQuant>
__device__ __forceinline__ void prefill_plan(
    const uint4 pv, float* __restrict__ state, int64_t num_slots, const float* __restrict__ in,
    const EmitSink& o, int64_t num_tokens, const float* __restrict__ ape,
    const int32_t* __restrict__ indices, const int32_t* __restrict__ load_indices, int64_t batch,
    PlanLds<kWaves>& lds) {
  constexpr int kTokPerLane = 128 / (2 * kWaves);   // chunk positions per lane
  const uint32_t ragged_id = pv.x, batch_id = pv.y, position = pv.z, len = pv.w;
  if (ragged_id == 0xFFFFFFFFu) return;                         // padding entry
  const uint32_t pos127 = position & 127u;
  if (len < 1u || len > pos127 + 1u || (int64_t)batch_id >= batch ||
      (int64_t)ragged_id >= num_tokens || ragged_id + 1u < len)
    return;                                                     // malformed: skip
  const uint32_t off = pos127 + 1u - len;                       // first chunk position
  const uint32_t end = pos127 + 1u;                             // one past the last
  const int64_t seg0 = (int64_t)ragged_id - (int64_t)pos127;    // row of chunk position 0

  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;                 // even / odd chunk positions
  const int q = lane & 31;                 // channels 4q..4q+3
  // After the partials meet in LDS, wave w finishes channels kChPerWave * w ..
  // kChPerWave * w + kChPerWave - 1: lane group g (kChPerWave lanes) merges
  // the partials of waves 2g and 2g + 1 for channel ch, then the groups merge
  // across lanes, and group 0 finishes the channel.
  constexpr int kChPerWave = 128 / kWaves;
  static_assert(kWaves >= 2 && kWaves <= 64 && kChPerWave * kWaves == 128,
                "two partials per lane group");
  const int ch = kChPerWave * w + lane % kChPerWave;
  const int g = lane / kChPerWave;
  const float4* in4 = reinterpret_cast<const float4*>(in);
  const float4* ape4 = reinterpret_cast<const float4*>(ape);

  // Everything below depends only on the plan, so the token rows, the slot
  // indices and (for a segment that starts mid-chunk) the stored state are
  // all requested before any of them is consumed.  The row loads carry no
  // branches: a position outside the segment re-reads the segment's last row
  // (always in bounds) and is masked out afterwards.
  float4 kv[kTokPerLane], sc[kTokPerLane], bi[kTokPerLane];
  bool valid[kTokPerLane];
#pragma unroll
  for (int i = 0; i < kTokPerLane; ++i) {
    const uint32_t j = 2u * kTokPerLane * w + 2u * i + h;
    valid[i] = j >= off && j < end;
    const uint32_t jj = valid[i] ? j : pos127;
    const int64_t r = seg0 + jj;
    kv[i] = load_stream4(in4 + r * 64 + q);
    sc[i] = load_stream4(in4 + r * 64 + 32 + q);
    bi[i] = ape4[jj * 32 + q];
  }
  int32_t load_idx = -1;
  if (off != 0u) load_idx = load_indices[batch_id];
  int32_t store_idx = -1;
  if constexpr (kWrite) store_idx = indices[batch_id];
  const bool load_ok = load_idx >= 0 && (int64_t)load_idx < num_slots;
  float m1 = 0.f, s1 = 0.f, k1 = 0.f;      // stored state of channel ch (group 0)
  if (g == 0 && off != 0u && load_ok) {
    const float* st = state + (int64_t)load_idx * 384;
    m1 = st[ch];
    s1 = st[128 + ch];
    k1 = st[256 + ch];
  }
  float4 u[kTokPerLane];
#pragma unroll
  for (int i = 0; i < kTokPerLane; ++i) {
    u[i] = valid[i] ? make_float4(sc[i].x + bi[i].x, sc[i].y + bi[i].y, sc[i].z + bi[i].z,
                                  sc[i].w + bi[i].w)
                    : make_float4(-FLT_MAX, -FLT_MAX, -FLT_MAX, -FLT_MAX);
    if (!valid[i]) kv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  float m[4] = {-FLT_MAX, -FLT_MAX, -FLT_MAX, -FLT_MAX};
#pragma unroll
  for (int i = 0; i < kTokPerLane; ++i) {
    m[0] = fmaxf(m[0], u[i].x); m[1] = fmaxf(m[1], u[i].y);
    m[2] = fmaxf(m[2], u[i].z); m[3] = fmaxf(m[3], u[i].w);
  }
  float d[4] = {0.f, 0.f, 0.f, 0.f}, a[4] = {0.f, 0.f, 0.f, 0.f};
  const float ml[4] = {m[0] * kLog2e, m[1] * kLog2e, m[2] * kLog2e, m[3] * kLog2e};
#pragma unroll
  for (int i = 0; i < kTokPerLane; ++i) {
    if (valid[i]) {
      const float uu[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
      const float kk[4] = {kv[i].x, kv[i].y, kv[i].z, kv[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float e = exp2_hw(__builtin_fmaf(uu[k], kLog2e, -ml[k]));
        d[k] += e;
        a[k] = __builtin_fmaf(kk[k], e, a[k]);
      }
    }
  }
  // half-wave merge (lane q with lane q + 32)
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float m2 = __shfl_xor(m[k], 32);
    const float d2 = __shfl_xor(d[k], 32);
    const float a2 = __shfl_xor(a[k], 32);
    merge_partial(m[k], d[k], a[k], m2, d2, a2);
  }
  if (h == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lds.m[w][4 * q + k] = m[k];
      lds.d[w][4 * q + k] = d[k];
      lds.a[w][4 * q + k] = a[k];
    }
  }
  __syncthreads();
  // A segment that needs the stored state but has no valid slot for it, or a
  // write plan without a valid destination, is malformed: skip it (the test
  // is uniform over the workgroup).
  if ((off != 0u && !load_ok) || (kWrite && (store_idx < 0 || (int64_t)store_idx >= num_slots)))
    return;

  // Every wave finishes kChPerWave channels, all its lanes working: a serial
  // merge of the kWaves partials by 32 lanes (4 channels each) had measured
  // 1.5-1.8 us of a 44 us single-launch prefill.
  float M = lds.m[2 * g][ch], D = lds.d[2 * g][ch], A = lds.a[2 * g][ch];
  merge_partial(M, D, A, lds.m[2 * g + 1][ch], lds.d[2 * g + 1][ch], lds.a[2 * g + 1][ch]);
#pragma unroll
  for (int dist = kChPerWave; dist < 64; dist *= 2) {
    const float m2 = __shfl_xor(M, dist);
    const float d2 = __shfl_xor(D, dist);
    const float a2 = __shfl_xor(A, dist);
    merge_partial(M, D, A, m2, d2, a2);
  }
  float K;
  if (off != 0u) {
    // Merge with the stored state of the open chunk: (m1, s1, k1) with k1 a
    // normalised mean, i.e. an unnormalised sum k1 * s1.
    const float mx = fmaxf(m1, M);
    const float f1 = s1 * exp2_hw((m1 - mx) * kLog2e);
    const float f2 = exp2_hw((M - mx) * kLog2e);
    const float sum = f1 + D * f2;
    K = (k1 * f1 + A * f2) / sum;
    D = sum;
    M = mx;
  } else {
    K = A / D;
  }
  if constexpr (kWrite) {
    if (g == 0) {
      float* st = state + (int64_t)store_idx * 384;
      st[ch] = M;
      st[128 + ch] = D;
      st[256 + ch] = K;
    }
  } else if constexpr (kQuant) {
    // The rotation needs the whole vector in one half-wave.
    if (g == 0) lds.k[ch] = K;
    __syncthreads();
    if (w == 0 && h == 0) {
      const float Kq[4] = {lds.k[4 * q], lds.k[4 * q + 1], lds.k[4 * q + 2], lds.k[4 * q + 3]};
      emit32<true>(o, 0, (int64_t)ragged_id, q, Kq);
    }
  } else {
    if (g == 0) o.out[(int64_t)ragged_id * 128 + ch] = K;
  }
}

// One workgroup per plan of one list (compress or write pass).
template <bool kWrite, int kWaves, bool kQuant>
__global__ __launch_bounds__(64 * kWaves) void c128_prefill_kernel(
    float* __restrict__ state, int64_t num_slots, const float* __restrict__ in,
    EmitSink o, int64_t num_tokens, const float* __restrict__ ape,
    const int32_t* __restrict__ indices, const int32_t* __restrict__ load_indices, int64_t batch,
    const kvc_online_plan* __restrict__ plans, uint32_t n_plans) {
  __shared__ PlanLds<kWaves> lds;
  // One 16-byte scalar load for the whole plan entry (the index is clamped so
  // the load needs no branch), then every kernel argument taken into SGPRs
  // before the early exits: two scalar waits before the row loads instead of
  // six (two launches 51.3-51.5 -> 50.8 us on the 32-sequence prefill).  The
  // asm statement comes after the plan load, which keeps that load scalar.
  const uint32_t pi = blockIdx.x < n_plans ? blockIdx.x : n_plans - 1;
  const uint4 pv = reinterpret_cast<const uint4*>(plans)[pi];
  asm volatile("" ::"s"(state), "s"(num_slots), "s"(in), "s"(num_tokens), "s"(ape), "s"(indices),
               "s"(load_indices), "s"(batch), "s"(pv.x), "s"(pv.y), "s"(pv.z), "s"(pv.w));
  if (blockIdx.x >= n_plans) return;
  prefill_plan<kWrite, kWaves, kQuant>(pv, state, num_slots, in, o, num_tokens, ape, indices,
                                       load_indices, batch, lds);
}

// Single-launch prefill over work items {compress plan, write plan}.  An item
// that holds both belongs to one request whose first (mid-chunk) compress
// segment reads the stored state (row load_indices[b]) that its write plan
// replaces (row indices[b]): the workgroup finishes the compress plan, whose
// state loads were consumed before the barrier, and only then stores the new
// state.  No other item of the call touches those rows (the caller guarantees
// that no request reads a row another request writes), so no ordering between
// workgroups is needed.
template <bool kQuant>
__global__ __launch_bounds__(64 * kCompressWaves) void c128_prefill_fused_kernel(
    float* __restrict__ state, int64_t num_slots, const float* __restrict__ in,
    EmitSink o, int64_t num_tokens, const float* __restrict__ ape,
    const int32_t* __restrict__ indices, const int32_t* __restrict__ load_indices, int64_t batch,
    const kvc_online_item* __restrict__ items, uint32_t n_items) {
  __shared__ PlanLds<kCompressWaves> lds;
  // Item load and kernel arguments as in c128_prefill_kernel.
  const uint32_t ii = blockIdx.x < n_items ? blockIdx.x : n_items - 1;
  const uint4* it = reinterpret_cast<const uint4*>(items) + 2 * (size_t)ii;
  const uint4 pc = it[0];
  const uint4 pw = it[1];
  asm volatile("" ::"s"(state), "s"(num_slots), "s"(in), "s"(num_tokens), "s"(ape), "s"(indices),
               "s"(load_indices), "s"(batch), "s"(pc.x), "s"(pc.y), "s"(pc.z), "s"(pc.w),
               "s"(pw.x), "s"(pw.y), "s"(pw.z), "s"(pw.w));
  if (blockIdx.x >= n_items) return;
  prefill_plan<false, kCompressWaves, kQuant>(pc, state, num_slots, in, o, num_tokens, ape,
                                              indices, load_indices, batch, lds);
  __syncthreads();   // the LDS partials are reused by the write plan
  prefill_plan<true, kCompressWaves, false>(pw, state, num_slots, in, o, num_tokens, ape, indices,
                                            load_indices, batch, lds);
}

}  // namespace

hipError_t launch_c128_decode(float* state, int64_t state_ls, int64_t num_slots, const float* in,
                              int64_t in_ls, float* out, int64_t out_ls, uint8_t* codes,
                              float* scales, bool round_scale, const float* ape, int64_t ape_ls,
                              const int32_t* indices, const int32_t* seq_lens, int64_t batch,
                              int64_t num_layers, hipStream_t stream) {
  if (batch <= 0 || num_layers <= 0) return hipSuccess;   // kernels clamp indices to batch - 1
  const EmitSink o{out, codes, scales, out_ls, batch * 128, batch, round_scale};
#define KVC_DECODE(QUANT, REQ)                                                                 \
  hipLaunchKernelGGL((c128_decode_kernel<QUANT, REQ>),                                         \
                     dim3((unsigned)((batch + (REQ) - 1) / (REQ)), (unsigned)num_layers),      \
                     dim3(32 * (REQ)), 0, stream, state, state_ls, num_slots, in, in_ls, o, ape, \
                     ape_ls, indices, seq_lens, batch)
  if (num_layers > 1) {
    if (codes) KVC_DECODE(true, kDecodeReqLayers);
    else KVC_DECODE(false, kDecodeReqLayers);
  } else if (num_slots <= 0xFFFFFFFFLL && batch <= 0xFFFFFFFFLL) {
    const dim3 grid((unsigned)((batch + kDecodeReqSingle - 1) / kDecodeReqSingle));
    if (codes)
      hipLaunchKernelGGL((c128_decode_one_kernel<true>), grid, dim3(32 * kDecodeReqSingle), 0,
                         stream, state, in, static_cast<void*>(codes), scales, ape, indices,
                         seq_lens, (uint32_t)num_slots, (uint32_t)batch, (uint32_t)round_scale);
    else
      hipLaunchKernelGGL((c128_decode_one_kernel<false>), grid, dim3(32 * kDecodeReqSingle), 0,
                         stream, state, in, static_cast<void*>(out), scales, ape, indices,
                         seq_lens, (uint32_t)num_slots, (uint32_t)batch, (uint32_t)round_scale);
  } else {
    if (codes) KVC_DECODE(true, kDecodeReqSingle);
    else KVC_DECODE(false, kDecodeReqSingle);
  }
#undef KVC_DECODE
  return hipGetLastError();
}

hipError_t launch_c128_prefill(float* state, int64_t num_slots, const float* in, float* out,
                               uint8_t* codes, float* scales, bool round_scale,
                               int64_t num_tokens, const float* ape, const int32_t* indices,
                               const int32_t* load_indices, int64_t batch,
                               const kvc_online_plan* cplan, uint32_t n_c,
                               const kvc_online_plan* wplan, uint32_t n_w, hipStream_t stream) {
  if (!load_indices) load_indices = indices;
  const EmitSink o{out, codes, scales, 0, 0, 0, round_scale};
  // Pass 1 (compress plans) only reads the state; pass 2 (write plans) writes
  // it.  Stream order puts every pass-1 read before any pass-2 write.
  if (n_c) {
    if (codes)
      hipLaunchKernelGGL((c128_prefill_kernel<false, kCompressWaves, true>), dim3(n_c),
                         dim3(64 * kCompressWaves), 0, stream, state, num_slots, in, o,
                         num_tokens, ape, indices, load_indices, batch, cplan, n_c);
    else
      hipLaunchKernelGGL((c128_prefill_kernel<false, kCompressWaves, false>), dim3(n_c),
                         dim3(64 * kCompressWaves), 0, stream, state, num_slots, in, o,
                         num_tokens, ape, indices, load_indices, batch, cplan, n_c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_w) {
    hipLaunchKernelGGL((c128_prefill_kernel<true, kWriteWaves, false>), dim3(n_w),
                       dim3(64 * kWriteWaves), 0, stream, state, num_slots, in, o, num_tokens,
                       ape, indices, load_indices, batch, wplan, n_w);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_c128_prefill_fused(float* state, int64_t num_slots, const float* in, float* out,
                                     uint8_t* codes, float* scales, bool round_scale,
                                     int64_t num_tokens, const float* ape, const int32_t* indices,
                                     const int32_t* load_indices, int64_t batch,
                                     const kvc_online_item* items, uint32_t n_items,
                                     hipStream_t stream) {
  if (n_items == 0) return hipSuccess;   // the kernel clamps its item index to n_items - 1
  if (!load_indices) load_indices = indices;
  const EmitSink o{out, codes, scales, 0, 0, 0, round_scale};
  if (codes)
    hipLaunchKernelGGL((c128_prefill_fused_kernel<true>), dim3(n_items),
                       dim3(64 * kCompressWaves), 0, stream, state, num_slots, in, o, num_tokens,
                       ape, indices, load_indices, batch, items, n_items);
  else
    hipLaunchKernelGGL((c128_prefill_fused_kernel<false>), dim3(n_items),
                       dim3(64 * kCompressWaves), 0, stream, state, num_slots, in, o, num_tokens,
                       ape, indices, load_indices, batch, items, n_items);
  return hipGetLastError();
}

}  // namespace kvc
