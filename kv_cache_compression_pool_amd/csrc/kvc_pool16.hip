// kvc_pool16.hip -- pool-16 compression kernels for gfx950.
//
// Method (vLLM API page "kpool_compress", _kpool_softmax_rotate_write_cache_kernel
// and _kpool_decode_update_batched_kernel): per channel, softmax over the 16
// pool slots of score + ape, weighted key sum, bf16 round, 128-point
// Walsh-Hadamard rotation / sqrt(128), bf16 round, per-vector fp8 e4m3 scale.
//
// Work mapping (MI355X-first, not the pages' one-program-per-pool layout):
//   * A pool is owned by one wave.  Lane 16q + c takes slots 4q..4q+3 and
//     channels 8c..8c+7, so each slot row of keys or scores is one 128-bit
//     load per lane (16 lanes x 16 B = the 256 B bf16 row) and a lane holds
//     4 x 8 values of each.  A workgroup of four waves compresses four pools.
//   * Each lane runs the two-pass softmax over its 4 slots x 8 channels in
//     fp32 registers.  The per-channel max is all-reduced over the wave's four
//     16-lane rows before the exponentials (no rescaling needed); the partial
//     sums are reduce-scattered, so each lane finishes two channels.  Row
//     exchanges are gfx950's permlane swaps (VALU, no LDS).
//   * The epilogue rotates the two channels a lane holds: channel bit 0 in a
//     register, bits 1-2 across rows, bits 3-6 across the 16 lanes of a row
//     (DPP); the absmax is a wave reduction; each lane stores 2 codes, so the
//     128-byte code vector leaves as one coalesced store.
//   * One pool per wave at every batch size: a form with two pools per wave
//     (32 lanes per pool, 120 VGPRs) measured within 2% of it, either way,
//     from 31k to 257k pools, and slower below.
//   * Slot rows are streamed with non-temporal loads, through buffer
//     resources with 32-bit offsets when keys and scores each span less than
//     4 GiB (64-bit global addresses otherwise); ape ([16,128] fp32) is
//     staged once per workgroup in LDS (measured faster than per-lane reads
//     of ape through the L1).
//   * Ring decode uses the same whole-wave layout for one request per wave.
// The path is HBM-bound (about 8.3 KB read per 132 B written); there is no
// dense contraction, so no MFMA.
#include "kvc_device.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

constexpr int kPool = 16;
constexpr int kBlock = 256;                    // 4 waves per workgroup
constexpr int kPoolsPerBlock = kBlock / 64;    // prefill, one pool per wave
constexpr int kMinWavesPerEU = 4;              // caps VGPRs at 128
constexpr int64_t kPagedBytes = 132;           // page of one token: 128 codes + fp32 scale

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Streaming 128-bit load that does not keep the line in the caches.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Streaming 128-bit store (non-temporal: the line is not kept in the caches).
__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
  __builtin_nontemporal_store((u32x4_t){v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}

// The same load through a buffer resource: the base address sits in scalar
// registers and each lane adds a 32-bit byte offset, which spares the 64-bit
// address arithmetic of the prefill's 16 row loads per lane (measured: 73.7%
// instead of 71.6% of HBM peak on the ragged prefill).  Reads at or past the
// resource's byte count return zeros.  Word 3 of the resource sets only
// DATA_FORMAT = 32 bit (value 4 in bits 15..18); untyped loads take their
// size from the instruction.  Cache-policy bit 1 is the non-temporal hint.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 load_stream(BufRsrc r, uint32_t byte_offset) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void widen8(uint4 w, float (&f)[8]) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

// Stage ape [16][128] fp32 into LDS as float4 [16][32], in two steps for a
// block of kBlock threads (2 float4 each), so the ape loads can be issued
// before the slot-row loads.
struct ApeRegs {
  float4 a, b;
};
__device__ __forceinline__ ApeRegs load_ape(const float* __restrict__ ape) {
  static_assert(kPool * 32 == 2 * kBlock, "two float4 of ape per thread");
  const float4* src = reinterpret_cast<const float4*>(ape);
  return ApeRegs{src[threadIdx.x], src[threadIdx.x + kBlock]};
}
__device__ __forceinline__ void store_ape(float4* s_ape, const ApeRegs& r) {
  s_ape[threadIdx.x] = r.a;
  s_ape[threadIdx.x + kBlock] = r.b;
  __syncthreads();
}

// Softmax-weighted mean of one pool, whole-wave layout (one pool per wave).
// Lane 16q + c holds the gate scores S[i] and keys
// K[i] of slot 4q + i, channels 8c..8c+7.  Returns x[t] = the mean of channel
// 8c + 2q + t, t = 0..1: the max is all-reduced over the four rows, the sums
// are reduce-scattered (first across the wave halves, then across row pairs),
// so each lane finishes only the two channels it rotates afterwards.
__device__ __forceinline__ void pool_mean_wave(const uint4 (&S)[4], const uint4 (&K)[4],
                                               const float4 (&A)[4][2], float (&x)[2]) {
  float u[4][8], m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) m[j] = -__builtin_huge_valf();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float s[8];
    widen8(S[i], s);
    const float4 a0 = A[i][0], a1 = A[i][1];
    const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u[i][j] = s[j] + a[j];
      m[j] = fmaxf(m[j], u[i][j]);
    }
  }
  float ml[8], den[8], acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    m[j] = max_rows32(max_rows16(m[j]));          // max over all 16 slots
    ml[j] = m[j] * kLog2e;
    den[j] = 0.0f;
    acc[j] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float k[8];
    widen8(K[i], k);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = exp2_hw(__builtin_fmaf(u[i][j], kLog2e, -ml[j]));
      den[j] += p;
      acc[j] = __builtin_fmaf(k[j], p, acc[j]);
    }
  }
  // Lower half keeps channels j = 0..3, upper half j = 4..7 (channel bit 2 =
  // q >> 1); then even rows keep j' = 0, 1 and odd rows j' = 2, 3 of those
  // (channel bit 1 = q & 1).
  float d4[4], a4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    d4[j] = sum_scatter32(den[j], den[j + 4]);
    a4[j] = sum_scatter32(acc[j], acc[j + 4]);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float d = sum_scatter16(d4[t], d4[t + 2]);
    const float a = sum_scatter16(a4[t], a4[t + 2]);
    x[t] = a * __builtin_amdgcn_rcpf(d);
  }
}

// The same mean computed over the lane's channels in two halves (8c..8c+3, then
// 8c+4..8c+7), each with its own max, exponentials and sums; ape_at(i, hf)
// returns the ape values of slot 4q + i, channels 8c + 4hf .. 8c + 4hf + 3.
// Per channel the operations and their order are those of pool_mean_wave, so
// the result is bit-identical; fewer values are live at once (92 instead of
// 102 VGPRs in the one-layer-per-wave multi-layer ring decode).
template <typename ApeAt>
__device__ __forceinline__ void pool_mean_wave_halves(const uint4 (&S)[4], const uint4 (&K)[4],
                                                      ApeAt ape_at, float (&x)[2]) {
  float den[8], acc[8];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    // Keep the halves apart: interleaved by the scheduler they need nearly as
    // many registers as the full-width form (multi-layer ring decode, four
    // tokens: 92 -> 80 VGPRs, six waves per SIMD instead of five).
    if (hf) __builtin_amdgcn_sched_barrier(0);
    float u[4][4], m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = -__builtin_huge_valf();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w0 = hf ? S[i].z : S[i].x, w1 = hf ? S[i].w : S[i].y;
      const float s[4] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
      const float4 a4 = ape_at(i, hf);
      const float a[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u[i][j] = s[j] + a[j];
        m[j] = fmaxf(m[j], u[i][j]);
      }
    }
    float ml[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ml[j] = max_rows32(max_rows16(m[j])) * kLog2e;   // max over all 16 slots
      den[4 * hf + j] = 0.0f;
      acc[4 * hf + j] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w0 = hf ? K[i].z : K[i].x, w1 = hf ? K[i].w : K[i].y;
      const float k[4] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = exp2_hw(__builtin_fmaf(u[i][j], kLog2e, -ml[j]));
        den[4 * hf + j] += p;
        acc[4 * hf + j] = __builtin_fmaf(k[j], p, acc[4 * hf + j]);
      }
    }
  }
  float d4[4], a4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    d4[j] = sum_scatter32(den[j], den[j + 4]);
    a4[j] = sum_scatter32(acc[j], acc[j + 4]);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float d = sum_scatter16(d4[t], d4[t + 2]);
    const float a = sum_scatter16(a4[t], a4[t + 2]);
    x[t] = a * __builtin_amdgcn_rcpf(d);
  }
}

// Ape values of slot 4q + i, channels 8c + 4hf .. 8c + 4hf + 3, from the
// workgroup's LDS copy (float4 [16][32]).
__device__ __forceinline__ void pool_mean_wave_lds(const uint4 (&S)[4], const uint4 (&K)[4],
                                                   const float4* __restrict__ s_ape, int c,
                                                   int q, float (&x)[2]) {
  pool_mean_wave_halves(S, K, [&](int i, int hf) { return s_ape[(4 * q + i) * 32 + 2 * c + hf]; },
                        x);
}

// Where a compressed vector goes.  Packed: codes row `row` of a [n,128]
// array and scales[row].  Paged (page size 1): page `row` of a [pages, 132]
// byte cache holding the 128 codes followed by the fp32 scale.
struct OutSink {
  uint8_t* codes;      // packed codes or the paged cache
  float* scales;       // packed scales (unused when paged)
  int64_t rows;        // rows / pages available
  bool paged;
  float* dbg;          // ring decode: fp32 [rows, 128] pre-rounding means, or null
  // The same sink advanced by `rows` rows (the next layer's outputs).
  __device__ __forceinline__ OutSink advanced(int64_t rows_by) const {
    OutSink o = *this;
    o.codes += rows_by * (paged ? kPagedBytes : 128);
    if (!paged) o.scales += rows_by;
    if (dbg) o.dbg += rows_by * 128;
    return o;
  }
  // Lane 16q + c of a wave stores the codes of channels 8c + 2q and
  // 8c + 2q + 1 (low 16 bits of code2); lane 0 also stores the scale.
  __device__ __forceinline__ void store2(int64_t row, int c, int q, uint32_t code2,
                                         float scale) const {
    uint8_t* base = codes + row * (paged ? kPagedBytes : 128);
    reinterpret_cast<uint16_t*>(base)[4 * c + q] = (uint16_t)code2;
    if (c == 0 && q == 0) {
      if (paged) *reinterpret_cast<float*>(base + 128) = scale;
      else scales[row] = scale;
    }
  }
};

// One pool per wave.
// kBuf: keys and scores each span less than 4 GiB (key_bytes / score_bytes
// from their base), so the row loads go through buffer resources with 32-bit
// offsets; otherwise through 64-bit global addresses.
// kPlan: 1 = a plan and packed output (no loc, no write mask), the common
// case; 2 = a plan and paged output (loc given, write mask optional); both
// then load their plan entry (and loc) without branches before the row loads.
// 0 = anything else.
template <bool kRoundScale, bool kDbg, bool kBuf, int kPlan>
// Arguments: 9 pointers and 8 32-bit values (104 bytes; the host checks that
// sizes and strides fit): the runtime's host-side launch cost grows by about
// 1 us once a kernel's argument block exceeds 112 bytes.
__global__ __launch_bounds__(kBlock, kMinWavesPerEU) void pool16_prefill_kernel(
    const uint16_t* __restrict__ keys, const uint16_t* __restrict__ scores,
    const float* __restrict__ ape, const int32_t* __restrict__ src_rows, uint8_t* out_codes,
    float* out_scales, const int64_t* __restrict__ loc, const uint8_t* __restrict__ write_mask,
    float* __restrict__ dbg, uint32_t key_stride, uint32_t score_stride, uint32_t num_rows,
    uint32_t n_pools, uint32_t out_rows, uint32_t paged, uint32_t key_bytes,
    uint32_t score_bytes) {
  const OutSink sink{out_codes, out_scales, (int64_t)out_rows, paged != 0u, nullptr};
  __shared__ float4 s_ape[kPool * 32];
  const int c = threadIdx.x & 15;
  const int q = (threadIdx.x >> 4) & 3;
  // The pool index is wave-uniform, so its plan entry (and, when paged, its
  // destination) comes through scalar loads, which return before the vector
  // path would: the row loads wait on them.
  const int v = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t pool = (int64_t)blockIdx.x * kPoolsPerBlock + v;
  int64_t r0 = -1, dst = pool;
  bool ok = pool < n_pools;
  if constexpr (kPlan != 0) {
    // Plan entry (and loc) first, index clamped so no branch, then every
    // kernel argument into SGPRs: one wait for the arguments and one for the
    // plan before the row loads, instead of four behind the null-pointer
    // checks (packed: 21.0-21.3 -> 20.7-20.8 us on the 64-sequence batch;
    // paged: 21.3-21.6 -> 21.2-21.3 us).  The asm statement comes after those
    // loads, which keeps them scalar; the optional mask byte is read after
    // it, through a vector load.
    const int64_t pc = ok ? pool : n_pools - 1;
    const int32_t e = src_rows[pc];
    int64_t dl = pool;
    if constexpr (kPlan == 2) dl = loc[pc];
    asm volatile("" ::"s"(keys), "s"(key_stride), "s"(scores), "s"(score_stride), "s"(num_rows),
                 "s"(ape), "s"(n_pools), "s"(sink.codes), "s"(sink.scales), "s"(sink.rows),
                 "s"(dbg), "s"(key_bytes), "s"(score_bytes), "s"(e), "s"(dl));
    if (ok) {
      r0 = e;
      dst = dl;
      if constexpr (kPlan == 2) {
        if (write_mask && !write_mask[pool]) ok = false;
      }
    }
  } else if (ok) {
    r0 = src_rows ? (int64_t)src_rows[pool] : pool * kPool;
    if (loc) dst = loc[pool];
    if (write_mask && !write_mask[pool]) ok = false;
  }
  ok = ok && r0 >= 0 && r0 + kPool <= num_rows && dst >= 0 && dst < sink.rows;

  // ape is requested first; the row loads are unconditional (a skipped pool
  // reads rows 0..15, which exist: the launcher only runs with num_rows >=
  // 16), so no branch forces the compiler to wait on them early.
  const ApeRegs ape_regs = load_ape(ape);
  uint4 S[4], K[4];
  {
    const int64_t row = (ok ? r0 : 0) + 4 * q;
    if constexpr (kBuf) {
      const BufRsrc rs = make_rsrc(scores, score_bytes), rk = make_rsrc(keys, key_bytes);
      const uint32_t so = (uint32_t)(row * score_stride * 2) + 16u * c;
      const uint32_t ko = (uint32_t)(row * key_stride * 2) + 16u * c;
      const uint32_t ss = (uint32_t)(score_stride * 2), ks = (uint32_t)(key_stride * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) S[i] = load_stream(rs, so + i * ss);
#pragma unroll
      for (int i = 0; i < 4; ++i) K[i] = load_stream(rk, ko + i * ks);
    } else {
      const uint4* sp = reinterpret_cast<const uint4*>(scores + row * score_stride) + c;
      const uint4* kp = reinterpret_cast<const uint4*>(keys + row * key_stride) + c;
      const int64_t ss = score_stride >> 3, ks = key_stride >> 3;
#pragma unroll
      for (int i = 0; i < 4; ++i) S[i] = load_stream(sp + i * ss);
#pragma unroll
      for (int i = 0; i < 4; ++i) K[i] = load_stream(kp + i * ks);
    }
  }
  store_ape(s_ape, ape_regs);
  if (!ok) return;   // uniform over the wave: the row exchanges below stay complete

  float4 A[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    A[i][0] = s_ape[(4 * q + i) * 32 + 2 * c];
    A[i][1] = s_ape[(4 * q + i) * 32 + 2 * c + 1];
  }
  float x[2];
  pool_mean_wave(S, K, A, x);
  if constexpr (kDbg)   // channels 8c + 2q + t
    reinterpret_cast<float2*>(dbg + pool * 128)[4 * c + q] = make_float2(x[0], x[1]);
  float scale;
  const uint32_t codes = rotate_quantise64(x, c, q, kRoundScale, scale);
  sink.store2(dst, c, q, codes, scale);
}

// Per-layer strides of a multi-layer ring decode (blockIdx.y = layer): ring,
// key and score in bf16 elements, ape in floats, outputs in rows.  All zero
// for a single layer.
struct RingLayers {
  int64_t ring, key, score, ape, out_rows;
};

// Tail-ring decode with one request per wave.  Request r processes its
// tokens strictly in order (the page's semantics): a token at position p with
// p % 16 == 15 and an output row completes the pool (ring slots 0..14 plus
// itself), then every valid token stashes its key / score rows in ring slot
// p % 16.
//  * Tokens run in windows of kMaxN (one window unless next_n > kMaxN); a
//    window's maps and key / score rows are requested in one round trip.
//  * The loop runs over completions, not tokens.  Before completion t* reads
//    its ring block, the stashes of the tokens before t* are stored from the
//    lanes that read those slots back (row q of the wave owns slots
//    4q..4q+3), so same-lane program order orders them.
//  * A whole wave per request halves each lane's share of the softmax and
//    rotation (4 slots x 8 channels, then 2 channels) compared with the
//    32-lane layout: in this latency-bound call the dependent arithmetic of
//    one completion, not bandwidth, sets the time.
//  * ape: single calls load each completing lane's 32 ape values with the
//    ring rows, so waves that only stash never read it and no barrier sits in
//    the chain; multi-layer launches stage ape in LDS once per workgroup,
//    because those registers would cost occupancy there.
//  * Multi-layer launches (kParkTokens with kMaxN <= 8) store the stashes and
//    read the ring rows with non-temporal accesses: 64 layers of 256 x 4
//    19.8-19.9 -> 18.3-18.4 us, bit-identical.  Single calls keep cached
//    accesses (non-temporal ones made 256 x 4 4.21 -> 4.38 us per call).
//  * kParkTokens (multi-layer launches, and windows of more than 8 tokens):
//    the token rows are parked in LDS after loading (the wave's four rows
//    share the loads) instead of staying in registers through the completion
//    path: about 30 fewer VGPRs, for an LDS round trip on the critical path.
//  * The workgroup handles requests group * 4 .. group * 4 + 3 of one layer;
//    the kernels below choose the group and offset the pointers to the layer.
template <bool kRoundScale, int kMaxN, bool kParkTokens>
__device__ __forceinline__ void ring_decode_group(
    uint16_t* ring, int64_t num_blocks, const int32_t* __restrict__ tail_slot,
    const uint16_t* __restrict__ key, int64_t key_sb, int64_t key_st,
    const uint16_t* __restrict__ score, int64_t score_sb, int64_t score_st,
    const float* __restrict__ ape, const int32_t* __restrict__ slot_mapping,
    const int32_t* __restrict__ positions, int64_t num_requests, int next_n, OutSink sink,
    int64_t group) {
  static_assert(kMaxN <= 32, "completion mask is 32 bits");
  constexpr int kReqPerBlock = kBlock / 64;
  constexpr bool kStreamRing = kParkTokens && kMaxN <= 8;   // multi-layer launches
  const int c = threadIdx.x & 15;
  const int q = (threadIdx.x >> 4) & 3;
  // The request index is made wave-uniform for the 4- and 8-token instances:
  // the token maps then come through scalar loads into SGPRs and the row
  // addresses take a scalar base, which frees 22-46 VGPRs and shortens the
  // first round trip (256 x 4: 4.27 -> 4.12 us; 256 x 8: 5.58 -> 5.28 us;
  // 64 layers 27.1 -> 26.7 us).  The 16-token instance keeps vector loads:
  // 48 scalar map loads measured 25-30% slower there.
  const int wave_in_block = kMaxN <= 8 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6))
                                       : (int)(threadIdx.x >> 6);
  const int64_t r = group * kReqPerBlock + wave_in_block;
  const int64_t rr = r < num_requests ? r : 0;   // waves past the batch read request 0, stop below

  __shared__ uint4 s_tok[kParkTokens ? kReqPerBlock : 1][kParkTokens ? kMaxN : 1][2][16];
  __shared__ float4 s_ape[kParkTokens ? kPool * 32 : 1];
  const int w = threadIdx.x >> 6;
  // Multi-layer launches stage ape once per workgroup in LDS (its registers
  // would cost occupancy); single calls load each completing lane's ape
  // values with the ring rows instead, which keeps the barrier and the ape
  // load off the chain of waves that only stash.
  ApeRegs ape_regs;
  if constexpr (kParkTokens) ape_regs = load_ape(ape);
  // Tokens are processed in windows of kMaxN (one window unless next_n >
  // kMaxN): window tokens t = 0..kMaxN-1 are request tokens base + t.
  int32_t loc[kMaxN], pos[kMaxN], ts[kMaxN];
  // Without parking every row of the wave loads every token's key and score
  // chunk c (the rows need them in registers); with parking the wave's four
  // rows share the 2*kMaxN row loads, kMaxN/2 each.
  constexpr int kTokRegs = kParkTokens ? 1 : kMaxN;
  constexpr int kParkLoads = (2 * kMaxN + 3) / 4;
  uint4 kv[kTokRegs], sv[kTokRegs];
  // Token t's key / score chunk c, from registers or from the parked copy.
  auto tok_key = [&](int t) -> uint4 {
    if constexpr (kParkTokens) return s_tok[w][t][0][c];
    else return kv[t];
  };
  auto tok_score = [&](int t) -> uint4 {
    if constexpr (kParkTokens) return s_tok[w][t][1][c];
    else return sv[t];
  };
  for (int base = 0;;) {   // windows; uniform over the wave and the workgroup
    uint4 pk[kParkTokens ? kParkLoads : 1];
#pragma unroll
    for (int t = 0; t < kMaxN; ++t) {
      const int tt = base + t < next_n ? base + t : next_n - 1;   // in bounds; unused if clamped
      const int64_t e = rr * next_n + tt;
      loc[t] = slot_mapping[e];
      pos[t] = positions[e];
      ts[t] = tail_slot[e];
      if constexpr (!kParkTokens) {
        kv[t] = reinterpret_cast<const uint4*>(key + rr * key_sb + tt * key_st)[c];
        sv[t] = reinterpret_cast<const uint4*>(score + rr * score_sb + tt * score_st)[c];
      }
    }
    if constexpr (kParkTokens) {
#pragma unroll
      for (int j = 0; j < kParkLoads; ++j) {
        const int g = 4 * j + q;                     // row g: token g / 2, key (0) or score (1)
        const int gg = g < 2 * kMaxN ? g : 2 * kMaxN - 1;
        const int t = base + (gg >> 1);
        const int tt = t < next_n ? t : next_n - 1;
        const uint16_t* src = (gg & 1) ? score + rr * score_sb + tt * score_st
                                       : key + rr * key_sb + tt * key_st;
        pk[j] = reinterpret_cast<const uint4*>(src)[c];
      }
    }
    // Issue every token load in this one round trip (the compiler would
    // otherwise sink some of them next to their first use).
#pragma unroll
    for (int t = 0; t < kMaxN; ++t)
      asm volatile("" ::"v"(loc[t]), "v"(pos[t]), "v"(ts[t]));
#pragma unroll
    for (int t = 0; t < kTokRegs; ++t)
      asm volatile("" ::"v"(kv[t].x), "v"(kv[t].y), "v"(kv[t].z), "v"(kv[t].w), "v"(sv[t].x),
                   "v"(sv[t].y), "v"(sv[t].z), "v"(sv[t].w));
    if constexpr (kParkTokens) {
      // Park the rows in LDS for the whole wave.  The hardware runs one
      // wave's LDS accesses in order, so the earlier window's reads precede
      // these writes and the writes precede the reads that follow; the empty
      // asm statements keep the compiler from moving accesses across them.
      asm volatile("" ::: "memory");
#pragma unroll
      for (int j = 0; j < kParkLoads; ++j) {
        asm volatile("" ::"v"(pk[j].x), "v"(pk[j].y), "v"(pk[j].z), "v"(pk[j].w));
        const int g = 4 * j + q;
        if (g < 2 * kMaxN) s_tok[w][g >> 1][g & 1][c] = pk[j];
      }
      asm volatile("" ::: "memory");
    }
    if (base == 0) {
      if constexpr (kParkTokens) store_ape(s_ape, ape_regs);
      if (r >= num_requests) return;   // whole waves: the row exchanges below stay complete
    }
    int32_t blk[kMaxN];
    uint32_t completes = 0, stashes = 0;
#pragma unroll
    for (int t = 0; t < kMaxN; ++t) {
      const int64_t b = (int64_t)(ts[t] > 0 ? ts[t] : 0) / kPool;
      blk[t] = (int32_t)b;   // ts is int32, so the block index fits
      if (base + t >= next_n || b >= num_blocks) continue;
      if (loc[t] >= 0 && pos[t] >= 0 && (pos[t] & (kPool - 1)) == kPool - 1) completes |= 1u << t;
      if (pos[t] >= 0 && ts[t] >= 0 && ((pos[t] & (kPool - 1)) >> 2) == q) stashes |= 1u << t;
    }

    auto stash_range = [&](uint32_t mask) {
#pragma unroll
      for (int t = 0; t < kMaxN; ++t) {
        if (mask & (1u << t)) {
          uint16_t* ring_k = ring + (int64_t)blk[t] * (2 * kPool * 128);
          const int slot = pos[t] & (kPool - 1);
          uint4* dk = reinterpret_cast<uint4*>(ring_k + slot * 128) + c;
          uint4* ds = reinterpret_cast<uint4*>(ring_k + kPool * 128 + slot * 128) + c;
          if constexpr (kStreamRing) {
            store_stream(dk, tok_key(t));
            store_stream(ds, tok_score(t));
          } else {
            *dk = tok_key(t);
            *ds = tok_score(t);
          }
        }
      }
    };

    uint32_t done = 0;   // tokens whose stash has been stored: bits below the cursor
    while (completes) {  // uniform over the wave: one request per wave
      const int t1 = __builtin_ctz(completes);
      completes &= completes - 1;
      const uint32_t before = (1u << t1) - 1;
      stash_range(stashes & before & ~done);
      done = before;
      int32_t b1 = 0, l1 = 0;
      uint4 k1 = make_uint4(0, 0, 0, 0), s1 = k1;
#pragma unroll
      for (int t = 0; t < kMaxN; ++t) {
        if (t == t1) {
          b1 = blk[t];
          l1 = loc[t];
          if constexpr (!kParkTokens) {
            k1 = kv[t];
            s1 = sv[t];
          }
        }
      }
      if constexpr (kParkTokens) {
        k1 = tok_key(t1);
        s1 = tok_score(t1);
      }
      const uint16_t* ring_k = ring + (int64_t)b1 * (2 * kPool * 128);
      const uint16_t* ring_s = ring_k + kPool * 128;
      // The ring rows of the pool (and, for single calls, the lane's ape
      // values: slots 4q..4q+3, channels 8c..8c+7) in one round trip.
      uint4 S[4], K[4];
      float4 A[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = 4 * q + i;
        const uint4* rs = reinterpret_cast<const uint4*>(ring_s + slot * 128) + c;
        const uint4* rk = reinterpret_cast<const uint4*>(ring_k + slot * 128) + c;
        S[i] = kStreamRing ? load_stream(rs) : *rs;
        K[i] = kStreamRing ? load_stream(rk) : *rk;
        if constexpr (!kParkTokens) {
          const float4* ap = reinterpret_cast<const float4*>(ape) + slot * 32 + 2 * c;
          A[i][0] = ap[0];
          A[i][1] = ap[1];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        asm volatile("" ::"v"(S[i].x), "v"(S[i].y), "v"(S[i].z), "v"(S[i].w), "v"(K[i].x),
                     "v"(K[i].y), "v"(K[i].z), "v"(K[i].w));
      // Multi-layer instances take the ape values from LDS inside the mean
      // (pool_mean_wave_lds); the 16-token single-call instance reads them
      // here (0.07 us faster on 256 x 16 than the halves).
      if constexpr (kParkTokens && kMaxN > 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          A[i][0] = s_ape[(4 * q + i) * 32 + 2 * c];
          A[i][1] = s_ape[(4 * q + i) * 32 + 2 * c + 1];
        }
      }
      // Slot 15 is the completing token itself: row 3 replaces what it read
      // there (a load kept unconditional so the row loads stay branch-free).
      if (q == 3) {
        S[3] = s1;
        K[3] = k1;
      }
      float x[2];
      if constexpr (kParkTokens && kMaxN <= 8) pool_mean_wave_lds(S, K, s_ape, c, q, x);
      else pool_mean_wave(S, K, A, x);
      if (sink.dbg && l1 < sink.rows)   // channels 8c + 2q + t
        reinterpret_cast<float2*>(sink.dbg + (int64_t)l1 * 128)[4 * c + q] =
            make_float2(x[0], x[1]);
      float scale;
      const uint32_t codes = rotate_quantise64(x, c, q, kRoundScale, scale);
      if (l1 < sink.rows) sink.store2(l1, c, q, codes, scale);
    }
    stash_range(stashes & ~done);
    // Launches pick kMaxN >= next_n except for the 16-token instance, which is
    // also the one that walks longer verify batches window by window.
    if constexpr (kMaxN < 16) break;
    base += kMaxN;
    if (base >= next_n) break;
  }
}

// Multi-layer launches (blockIdx.y = layer), and single calls whose sizes do
// not fit the compact form below.  Workgroup x of layer y takes request group
// (x + y) mod gridDim.x.  Workgroups go to the eight XCDs round robin in
// launch order, and the token maps are shared by all layers, so without the
// rotation the XCD that holds a group's completing requests would get them
// again in every layer, and the busiest XCD would set the launch time (64
// layers of 256 x 4: 24.9 us without, 20.4 us with, bit-identical).
template <bool kRoundScale, int kMaxN, bool kParkTokens>
__global__ __launch_bounds__(kBlock) void pool16_ring_wave_kernel(
    uint16_t* ring, int64_t num_blocks, const int32_t* __restrict__ tail_slot,
    const uint16_t* __restrict__ key, int64_t key_sb, int64_t key_st,
    const uint16_t* __restrict__ score, int64_t score_sb, int64_t score_st,
    const float* __restrict__ ape, const int32_t* __restrict__ slot_mapping,
    const int32_t* __restrict__ positions, int64_t num_requests, int next_n, OutSink sink,
    RingLayers ls) {
  const int64_t layer = blockIdx.y;
  ring_decode_group<kRoundScale, kMaxN, kParkTokens>(
      ring + layer * ls.ring, num_blocks, tail_slot, key + layer * ls.key, key_sb, key_st,
      score + layer * ls.score, score_sb, score_st, ape + layer * ls.ape, slot_mapping, positions,
      num_requests, next_n, sink.advanced(layer * ls.out_rows),
      ((int64_t)blockIdx.x + blockIdx.y) % gridDim.x);
}

// Single calls with a compact argument block: 112 bytes (32-bit sizes and
// strides; the paged flag in bit 31 of next_n_paged) instead of 448 (the
// general kernel's 192 plus the runtime's hidden arguments, which its use of
// gridDim brings in).  The runtime's host-side cost of a launch grows with
// the argument block, by about 1 us above 112 bytes and 1.5 us at 448, and a
// single call takes about 4 us on the device.
template <bool kRoundScale, int kMaxN, bool kParkTokens>
__global__ __launch_bounds__(kBlock) void pool16_ring_one_kernel(
    uint16_t* ring, const int32_t* __restrict__ tail_slot, const uint16_t* __restrict__ key,
    const uint16_t* __restrict__ score, const float* __restrict__ ape,
    const int32_t* __restrict__ slot_mapping, const int32_t* __restrict__ positions,
    uint8_t* codes, float* scales, float* dbg, uint32_t num_blocks, uint32_t num_requests,
    uint32_t next_n_paged, uint32_t rows, uint32_t key_sb, uint32_t key_st, uint32_t score_sb,
    uint32_t score_st) {
  const OutSink sink{codes, scales, (int64_t)rows, (next_n_paged >> 31) != 0u, dbg};
  ring_decode_group<kRoundScale, kMaxN, kParkTokens>(
      ring, num_blocks, tail_slot, key, key_sb, key_st, score, score_sb, score_st, ape,
      slot_mapping, positions, num_requests, (int)(next_n_paged & 0x7FFFFFFFu), sink,
      blockIdx.x);
}

// Tail-ring seeding.  Each lane decides for one token whether it is among its
// request's last 16 (no token 16 positions later maps to the same ring
// block); the wave then copies its few seeded tokens together, two per step,
// one 16-lane row per 256 B key or score row.  Seeded tokens are rare (at
// most 16 per request), so a wave mostly just reads 64 slot-map entries.
__global__ __launch_bounds__(256) void pool16_seed_kernel(uint16_t* __restrict__ ring,
                                                          int64_t num_blocks,
                                                          const uint16_t* __restrict__ key,
                                                          int64_t key_stride,
                                                          const uint16_t* __restrict__ score,
                                                          int64_t score_stride,
                                                          const int32_t* __restrict__ tslot,
                                                          int64_t n_tokens) {
  // Every kernel argument into SGPRs at entry, so no argument load waits
  // between the map loads and the row copies (3.26-3.28 -> 3.22 us on the
  // 64-sequence batch); the kernel's own loads are vector loads either way.
  asm volatile("" ::"s"(ring), "s"(num_blocks), "s"(key), "s"(key_stride), "s"(score),
               "s"(score_stride), "s"(tslot), "s"(n_tokens));
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x & 63;
  int32_t t = -1;
  bool seed = false;
  if (i < n_tokens) {
    t = tslot[i];
    const int32_t ahead = (i + kPool < n_tokens) ? tslot[i + kPool] : -1;
    seed = t >= 0 && (int64_t)(t / kPool) < num_blocks && !(ahead >= 0 && ahead / kPool == t / kPool);
  }
  uint64_t mask = __ballot(seed);
  const int64_t wave_base = i - lane;
  const int half = lane >> 5;                 // which of the step's two tokens
  const int which = (lane >> 4) & 1;          // 0: key row, 1: score row
  const int c = lane & 15;                    // 16-byte chunk of the row
  while (mask) {                              // uniform over the wave
    const int j0 = __builtin_ctzll(mask);
    mask &= mask - 1;
    int j1 = -1;
    if (mask) {
      j1 = __builtin_ctzll(mask);
      mask &= mask - 1;
    }
    const int j = half ? j1 : j0;
    const int32_t tj = __shfl(t, j >= 0 ? j : j0);
    if (j >= 0) {
      const int64_t tok = wave_base + j;
      const uint16_t* src = which ? score + tok * score_stride : key + tok * key_stride;
      uint16_t* dst = ring + (int64_t)(tj / kPool) * (2 * kPool * 128) +
                      (which * kPool + tj % kPool) * 128;
      reinterpret_cast<uint4*>(dst)[c] = reinterpret_cast<const uint4*>(src)[c];
    }
  }
}

}  // namespace

hipError_t launch_pool16_prefill(const uint16_t* keys, int64_t key_stride, const uint16_t* scores,
                                 int64_t score_stride, int64_t num_rows, const float* ape,
                                 const int32_t* src_rows, int64_t n_pools, uint8_t* out_fp8,
                                 float* out_scale, int64_t out_rows, bool paged,
                                 const int64_t* loc, const uint8_t* write_mask, bool round_scale,
                                 float* dbg, hipStream_t stream) {
  if (num_rows < kPool || n_pools <= 0) return hipSuccess;   // no pool can be complete
  // n_pools >= 1 here, so the kernels' clamped plan index is valid
  const int plan_mode = !src_rows ? 0 : (!loc && !write_mask) ? 1 : loc ? 2 : 0;
  const dim3 grid((unsigned)((n_pools + kPoolsPerBlock - 1) / kPoolsPerBlock));
  const dim3 block(kBlock);
  // The kernel takes sizes and strides as 32-bit values.
  constexpr int64_t kU32 = 0xFFFFFFFFLL;
  if (key_stride > kU32 || score_stride > kU32 || num_rows > kU32 || n_pools > kU32 ||
      out_rows > kU32)
    return hipErrorInvalidValue;
  // Bytes from each base to the end of its last row: buffer loads when both
  // fit in 32-bit offsets.
  const int64_t key_bytes = (num_rows - 1) * key_stride * 2 + 256;
  const int64_t score_bytes = (num_rows - 1) * score_stride * 2 + 256;
  const bool buf = key_bytes < (1LL << 32) && score_bytes < (1LL << 32);
  const uint32_t kb = buf ? (uint32_t)key_bytes : 0u, sb = buf ? (uint32_t)score_bytes : 0u;
#define KVC_ARGS                                                                               \
  keys, scores, ape, src_rows, out_fp8, out_scale, loc, write_mask, dbg, (uint32_t)key_stride,   \
      (uint32_t)score_stride, (uint32_t)num_rows, (uint32_t)n_pools, (uint32_t)out_rows,         \
      (uint32_t)(paged ? 1 : 0), kb, sb
#define KVC_LAUNCH(RS, DBG, BUF)                                                              \
  do {                                                                                        \
    if (plan_mode == 1)                                                                       \
      hipLaunchKernelGGL((pool16_prefill_kernel<RS, DBG, BUF, 1>), grid, block, 0, stream,    \
                         KVC_ARGS);                                                           \
    else if (plan_mode == 2)                                                                  \
      hipLaunchKernelGGL((pool16_prefill_kernel<RS, DBG, BUF, 2>), grid, block, 0, stream,    \
                         KVC_ARGS);                                                           \
    else                                                                                      \
      hipLaunchKernelGGL((pool16_prefill_kernel<RS, DBG, BUF, 0>), grid, block, 0, stream,    \
                         KVC_ARGS);                                                           \
  } while (0)
  if (buf) {
    if (round_scale) {
      if (dbg) KVC_LAUNCH(true, true, true); else KVC_LAUNCH(true, false, true);
    } else {
      if (dbg) KVC_LAUNCH(false, true, true); else KVC_LAUNCH(false, false, true);
    }
  } else {
    if (round_scale) {
      if (dbg) KVC_LAUNCH(true, true, false); else KVC_LAUNCH(true, false, false);
    } else {
      if (dbg) KVC_LAUNCH(false, true, false); else KVC_LAUNCH(false, false, false);
    }
  }
#undef KVC_LAUNCH
#undef KVC_ARGS
  return hipGetLastError();
}

hipError_t launch_pool16_ring(uint16_t* ring, int64_t num_blocks, const int32_t* tail_slot,
                              const uint16_t* key, int64_t key_sb, int64_t key_st,
                              const uint16_t* score, int64_t score_sb, int64_t score_st,
                              const float* ape, const int32_t* slot_mapping,
                              const int32_t* positions, int64_t num_requests, int next_n,
                              uint8_t* out_fp8, float* out_scale, int64_t out_rows, bool paged,
                              bool round_scale, float* dbg, int64_t num_layers,
                              int64_t ring_ls, int64_t key_ls, int64_t score_ls, int64_t ape_ls,
                              hipStream_t stream) {
  const dim3 block(kBlock);
  const OutSink sink{out_fp8, out_scale, out_rows, paged, dbg};
  const RingLayers ls{ring_ls, key_ls, score_ls, ape_ls, out_rows};
  constexpr int kWaveReq = kBlock / 64;
  dim3 grid((unsigned)((num_requests + kWaveReq - 1) / kWaveReq), (unsigned)num_layers);
  constexpr int64_t kU32 = 0xFFFFFFFFLL;
  const bool one = num_layers == 1 && num_blocks <= kU32 && num_requests <= kU32 &&
                   out_rows <= kU32 && key_sb <= kU32 && key_st <= kU32 && score_sb <= kU32 &&
                   score_st <= kU32;
  const uint32_t next_n_paged = (uint32_t)next_n | (paged ? 0x80000000u : 0u);
  // The kernel instance (round_scale, window, parking) and its argument form
  // (the parked 4- and 8-token instances serve multi-layer launches only).
#define KVC_RING(RS, N, PARK)                                                                  \
  do {                                                                                         \
    if constexpr (!PARK || N > 8) {                                                            \
      if (one) {                                                                               \
        hipLaunchKernelGGL((pool16_ring_one_kernel<RS, N, PARK>), grid, block, 0, stream, ring,  \
                           tail_slot, key, score, ape, slot_mapping, positions, out_fp8,         \
                           out_scale, dbg, (uint32_t)num_blocks, (uint32_t)num_requests,         \
                           next_n_paged, (uint32_t)out_rows, (uint32_t)key_sb,                   \
                           (uint32_t)key_st, (uint32_t)score_sb, (uint32_t)score_st);            \
        break;                                                                                 \
      }                                                                                        \
    }                                                                                          \
    hipLaunchKernelGGL((pool16_ring_wave_kernel<RS, N, PARK>), grid, block, 0, stream, ring,     \
                       num_blocks, tail_slot, key, key_sb, key_st, score, score_sb, score_st,    \
                       ape, slot_mapping, positions, num_requests, next_n, sink, ls);           \
  } while (0)
  const bool park = num_layers > 1;
  if (next_n <= 4) {
    if (round_scale) {
      if (park) KVC_RING(true, 4, true);
      else KVC_RING(true, 4, false);
    } else {
      if (park) KVC_RING(false, 4, true);
      else KVC_RING(false, 4, false);
    }
  } else if (next_n <= 8) {
    if (round_scale) {
      if (park) KVC_RING(true, 8, true);
      else KVC_RING(true, 8, false);
    } else {
      if (park) KVC_RING(false, 8, true);
      else KVC_RING(false, 8, false);
    }
  } else {
    // 16 tokens' rows do not fit in registers: parked in LDS, and longer
    // verify batches run in windows of 16 tokens
    if (round_scale) KVC_RING(true, 16, true);
    else KVC_RING(false, 16, true);
  }
#undef KVC_RING
  return hipGetLastError();
}

hipError_t launch_pool16_seed(uint16_t* ring, int64_t num_blocks, const uint16_t* key,
                              int64_t key_stride, const uint16_t* score, int64_t score_stride,
                              const int32_t* tslot, int64_t n_tokens, hipStream_t stream) {
  const dim3 grid((unsigned)((n_tokens + 255) / 256));
  hipLaunchKernelGGL(pool16_seed_kernel, grid, dim3(256), 0, stream, ring, num_blocks, key,
                     key_stride, score, score_stride, tslot, n_tokens);
  return hipGetLastError();
}

}  // namespace kvc
