// kvc_pool16.hip -- pool-16 compression kernels for gfx950.
//
// Method (vLLM API page "kpool_compress", _kpool_softmax_rotate_write_cache_kernel
// and _kpool_decode_update_batched_kernel): per channel, softmax over the 16
// pool slots of score + ape, weighted key sum, bf16 round, 128-point
// Walsh-Hadamard rotation / sqrt(128), bf16 round, per-vector fp8 e4m3 scale.
//
// Work mapping (MI355X-first, not the pages' one-program-per-pool layout):
//   * A pool is owned by one 16-lane DPP row of a wave64, so a wave compresses
//     four pools.  Lane c of the row owns channels 8c..8c+7: one 128-bit load
//     per token row and per tensor, 16 lanes x 16 B = one 256 B bf16 row.
//   * Each lane runs the two-pass softmax over all 16 slots of its 8 channels
//     in fp32 registers (no cross-lane reduction on the hot loop; exp on the
//     hardware exp2 unit).
//   * The rotation keeps channel bits 0-2 in registers and bits 3-6 across
//     the row's lanes (DPP quad_perm / row_half_mirror / row_ror exchanges);
//     the absmax is a 4-step DPP row reduction; the 8 codes of a lane leave as
//     one 8-byte store, so a row writes its 128-byte code vector coalesced.
//   * ape ([16,128] fp32) is staged once per workgroup in LDS.
// The path is HBM-bound (about 8.3 KB read per 132 B written); there is no
// dense contraction, so no MFMA.
#include "kvc_device.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

constexpr int kPool = 16;
constexpr int kRowsPerBlock = 16;                 // pools (16-lane rows) per block
constexpr int kBlock = kRowsPerBlock * 16;        // 256 threads = 4 waves

__device__ __forceinline__ void widen8(uint4 w, float (&f)[8]) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

// Stage ape [16][128] fp32 into LDS as float4 [16][32].
__device__ __forceinline__ void stage_ape(float4* s_ape, const float* __restrict__ ape) {
  const float4* src = reinterpret_cast<const float4*>(ape);
  for (int i = threadIdx.x; i < kPool * 32; i += blockDim.x) s_ape[i] = src[i];
  __syncthreads();
}

// Softmax-weighted mean of one pool for the 8 channels of lane c.
// S[i], K[i]: slot i's gate scores / keys for channels 8c..8c+7 (bf16 x 8).
__device__ __forceinline__ void pool_mean8(const uint4 (&S)[kPool], const uint4 (&K)[kPool],
                                           const float4* __restrict__ s_ape, int c,
                                           float (&x)[8]) {
  float u[kPool][8];
  float m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) m[j] = -__builtin_huge_valf();
#pragma unroll
  for (int i = 0; i < kPool; ++i) {
    float s[8];
    widen8(S[i], s);
    const float4 a0 = s_ape[i * 32 + 2 * c];
    const float4 a1 = s_ape[i * 32 + 2 * c + 1];
    u[i][0] = s[0] + a0.x; u[i][1] = s[1] + a0.y; u[i][2] = s[2] + a0.z; u[i][3] = s[3] + a0.w;
    u[i][4] = s[4] + a1.x; u[i][5] = s[5] + a1.y; u[i][6] = s[6] + a1.z; u[i][7] = s[7] + a1.w;
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = fmaxf(m[j], u[i][j]);
  }
  float ml[8], den[8], acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { ml[j] = m[j] * kLog2e; den[j] = 0.0f; acc[j] = 0.0f; }
#pragma unroll
  for (int i = 0; i < kPool; ++i) {
    float k[8];
    widen8(K[i], k);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = exp2_hw(__builtin_fmaf(u[i][j], kLog2e, -ml[j]));
      den[j] += p;
      acc[j] = __builtin_fmaf(k[j], p, acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = acc[j] * __builtin_amdgcn_rcpf(den[j]);
}

// bf16 round -> rotate -> bf16 round -> scale -> e4m3 codes for the row.
// Returns the 8 codes of lane c packed little-endian (channel 8c in byte 0).
__device__ __forceinline__ uint2 pool_epilogue(const float (&x)[8], int c, bool round_scale,
                                               float& scale_out) {
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = round_bf16(x[j]);
  wht128_row(v, c);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] = round_bf16(v[j] * kInvSqrt128);
    amax = fmaxf(amax, fabsf(v[j]));
  }
  amax = row_max16(amax);
  const float scale = fp8_scale(amax, round_scale);
  float q[8];
  if (round_scale) {
    const float inv = pow2_recip(scale);   // exact: scale is a power of two
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = clamp_fp8(v[j] * inv);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = clamp_fp8(v[j] / scale);   // IEEE division
  }
  scale_out = scale;
  return make_uint2(pack_e4m3x4(q[0], q[1], q[2], q[3]), pack_e4m3x4(q[4], q[5], q[6], q[7]));
}

template <bool kRoundScale, bool kDbg>
__global__ __launch_bounds__(kBlock) void pool16_prefill_kernel(
    const uint16_t* __restrict__ keys, int64_t key_stride, const uint16_t* __restrict__ scores,
    int64_t score_stride, int64_t num_rows, const float* __restrict__ ape,
    const int32_t* __restrict__ src_rows, int64_t n_pools, uint8_t* __restrict__ out_fp8,
    float* __restrict__ out_scale, float* __restrict__ dbg) {
  __shared__ float4 s_ape[kPool * 32];
  stage_ape(s_ape, ape);

  const int c = threadIdx.x & 15;
  const int64_t pool = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  if (pool >= n_pools) return;
  const int64_t r0 = src_rows ? (int64_t)src_rows[pool] : pool * kPool;
  if (r0 < 0 || r0 + kPool > num_rows) return;     // whole row leaves together

  const uint4* kp = reinterpret_cast<const uint4*>(keys + r0 * key_stride) + c;
  const uint4* sp = reinterpret_cast<const uint4*>(scores + r0 * score_stride) + c;
  const int64_t ks = key_stride >> 3, ss = score_stride >> 3;
  uint4 S[kPool], K[kPool];
#pragma unroll
  for (int i = 0; i < kPool; ++i) S[i] = sp[i * ss];
#pragma unroll
  for (int i = 0; i < kPool; ++i) K[i] = kp[i * ks];

  float x[8];
  pool_mean8(S, K, s_ape, c, x);
  if constexpr (kDbg) {
    float4* d = reinterpret_cast<float4*>(dbg + pool * 128 + 8 * c);
    d[0] = make_float4(x[0], x[1], x[2], x[3]);
    d[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
  float scale;
  const uint2 codes = pool_epilogue(x, c, kRoundScale, scale);
  reinterpret_cast<uint2*>(out_fp8 + pool * 128)[c] = codes;
  if (c == 0) out_scale[pool] = scale;
}

// Tail-ring decode: one 16-lane row per request, tokens in order.
template <bool kRoundScale>
__global__ __launch_bounds__(kBlock) void pool16_ring_kernel(
    uint16_t* ring, int64_t num_blocks, const int32_t* __restrict__ tail_slot,
    const uint16_t* __restrict__ key, int64_t key_sb, int64_t key_st,
    const uint16_t* __restrict__ score, int64_t score_sb, int64_t score_st,
    const float* __restrict__ ape, const int32_t* __restrict__ slot_mapping,
    const int32_t* __restrict__ positions, int64_t num_requests, int next_n,
    uint8_t* __restrict__ out_fp8, float* __restrict__ out_scale, int64_t num_out) {
  __shared__ float4 s_ape[kPool * 32];
  stage_ape(s_ape, ape);

  const int c = threadIdx.x & 15;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  if (r >= num_requests) return;

  for (int t = 0; t < next_n; ++t) {
    const int64_t e = r * next_n + t;
    const int32_t loc = slot_mapping[e];
    const int32_t pos = positions[e];
    const int32_t ts = tail_slot[e];
    const int64_t blk = (int64_t)(ts > 0 ? ts : 0) / kPool;
    if (blk >= num_blocks) continue;
    const bool complete = loc >= 0 && pos >= 0 && (pos & (kPool - 1)) == kPool - 1;
    const bool stash = pos >= 0 && ts >= 0;
    if (!complete && !stash) continue;

    uint16_t* ring_k = ring + blk * (2 * kPool * 128);
    uint16_t* ring_s = ring_k + kPool * 128;
    const uint4 kv = reinterpret_cast<const uint4*>(key + r * key_sb + t * key_st)[c];
    const uint4 sv = reinterpret_cast<const uint4*>(score + r * score_sb + t * score_st)[c];

    if (complete) {
      // Slots 0..14 come from the ring (including stashes made earlier in
      // this call by the same lanes); slot 15 is the current token.
      uint4 S[kPool], K[kPool];
#pragma unroll
      for (int i = 0; i < kPool - 1; ++i) {
        S[i] = reinterpret_cast<const uint4*>(ring_s + i * 128)[c];
        K[i] = reinterpret_cast<const uint4*>(ring_k + i * 128)[c];
      }
      S[kPool - 1] = sv;
      K[kPool - 1] = kv;
      float x[8];
      pool_mean8(S, K, s_ape, c, x);
      float scale;
      const uint2 codes = pool_epilogue(x, c, kRoundScale, scale);
      if (loc < num_out) {
        reinterpret_cast<uint2*>(out_fp8 + (int64_t)loc * 128)[c] = codes;
        if (c == 0) out_scale[loc] = scale;
      }
    }
    if (stash) {
      const int slot = pos & (kPool - 1);
      reinterpret_cast<uint4*>(ring_k + slot * 128)[c] = kv;
      reinterpret_cast<uint4*>(ring_s + slot * 128)[c] = sv;
    }
  }
}

__global__ __launch_bounds__(256) void diag_convert_kernel(const float* __restrict__ in,
                                                           uint16_t* __restrict__ bf16_out,
                                                           uint8_t* __restrict__ fp8_out,
                                                           int64_t n) {
  const int64_t i = 2 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= n) return;
  const float a = in[i], b = in[i + 1];
  if (bf16_out) {
    bf16_out[i] = bf16_bits(a);
    bf16_out[i + 1] = bf16_bits(b);
  }
  if (fp8_out) {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_fp8(a), clamp_fp8(b), 0, false);
    fp8_out[i] = (uint8_t)(w & 0xff);
    fp8_out[i + 1] = (uint8_t)((w >> 8) & 0xff);
  }
}

}  // namespace

hipError_t launch_pool16_prefill(const uint16_t* keys, int64_t key_stride, const uint16_t* scores,
                                 int64_t score_stride, int64_t num_rows, const float* ape,
                                 const int32_t* src_rows, int64_t n_pools, uint8_t* out_fp8,
                                 float* out_scale, bool round_scale, float* dbg,
                                 hipStream_t stream) {
  const dim3 grid((unsigned)((n_pools + kRowsPerBlock - 1) / kRowsPerBlock));
  const dim3 block(kBlock);
#define KVC_LAUNCH(RS, DBG)                                                                   \
  hipLaunchKernelGGL((pool16_prefill_kernel<RS, DBG>), grid, block, 0, stream, keys,          \
                     key_stride, scores, score_stride, num_rows, ape, src_rows, n_pools,     \
                     out_fp8, out_scale, dbg)
  if (round_scale) {
    if (dbg) KVC_LAUNCH(true, true); else KVC_LAUNCH(true, false);
  } else {
    if (dbg) KVC_LAUNCH(false, true); else KVC_LAUNCH(false, false);
  }
#undef KVC_LAUNCH
  return hipGetLastError();
}

hipError_t launch_pool16_ring(uint16_t* ring, int64_t num_blocks, const int32_t* tail_slot,
                              const uint16_t* key, int64_t key_sb, int64_t key_st,
                              const uint16_t* score, int64_t score_sb, int64_t score_st,
                              const float* ape, const int32_t* slot_mapping,
                              const int32_t* positions, int64_t num_requests, int next_n,
                              uint8_t* out_fp8, float* out_scale, int64_t num_out,
                              bool round_scale, hipStream_t stream) {
  const dim3 grid((unsigned)((num_requests + kRowsPerBlock - 1) / kRowsPerBlock));
  const dim3 block(kBlock);
  if (round_scale)
    hipLaunchKernelGGL((pool16_ring_kernel<true>), grid, block, 0, stream, ring, num_blocks,
                       tail_slot, key, key_sb, key_st, score, score_sb, score_st, ape,
                       slot_mapping, positions, num_requests, next_n, out_fp8, out_scale,
                       num_out);
  else
    hipLaunchKernelGGL((pool16_ring_kernel<false>), grid, block, 0, stream, ring, num_blocks,
                       tail_slot, key, key_sb, key_st, score, score_sb, score_st, ape,
                       slot_mapping, positions, num_requests, next_n, out_fp8, out_scale,
                       num_out);
  return hipGetLastError();
}

hipError_t launch_diag_convert(const float* in, uint16_t* bf16_out, uint8_t* fp8_out, int64_t n,
                               hipStream_t stream) {
  const int64_t pairs = n / 2;
  const dim3 grid((unsigned)((pairs + 255) / 256));
  hipLaunchKernelGGL(diag_convert_kernel, grid, dim3(256), 0, stream, in, bf16_out, fp8_out, n);
  return hipGetLastError();
}

}  // namespace kvc
