// kvc_device.hpp -- gfx950 device building blocks shared by the kernels:
// bf16 widening / rounding, base-2 exponentials, DPP lane exchanges inside a
// 16-lane row, swizzles between two rows, permlane swaps between the four
// rows of a wave, the 128-point Walsh-Hadamard butterfly over 32 or 64 lanes,
// and the e4m3 quantiser.  Everything here is wave64 code for CDNA4; no other
// target.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr float kLog2e = 1.4426950408889634f;
// fp32 nearest to 1/sqrt(128); the rotation's normalisation factor.
constexpr float kInvSqrt128 = 0.088388347648318440550f;
constexpr float kFp8Max = 448.0f;
// fp32(1/448): the scale multiplies the absmax by this constant.
constexpr float kInvFp8Max = (float)(1.0 / 448.0);
constexpr float kScaleFloor = 1e-4f;

// ---- bf16 ---------------------------------------------------------------
// A 32-bit word holds two bf16 values: channel 2j in the low half, 2j+1 in
// the high half.  Widening is a shift / mask (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to bf16 (nearest-even, v_cvt_pk_bf16_f32 on gfx950) and widen back.
__device__ __forceinline__ float round_bf16(float x) { return (float)(__bf16)x; }
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// ---- exponentials ---------------------------------------------------------
// e^x evaluated as 2^(x*log2 e) on the hardware exp2 unit (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- DPP lane exchanges inside one 16-lane row ----------------------------
// Lane l of a row receives the value of lane l ^ m.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xf, 0xf, true));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kQuadRev = 0x1B;        // quad_perm [3,2,1,0]  (l ^ 3)
constexpr int kRowHalfMirror = 0x141; // l -> 7 - l within each 8 lanes (l ^ 7)
constexpr int kRowRor8 = 0x128;       // rotate the 16-lane row by 8 (l ^ 8)

template <int kMask>
__device__ __forceinline__ float row_xor(float v) {
  if constexpr (kMask == 1) return dpp<kQuadXor1>(v);
  else if constexpr (kMask == 2) return dpp<kQuadXor2>(v);
  else if constexpr (kMask == 4) return dpp<kQuadRev>(dpp<kRowHalfMirror>(v));
  else return dpp<kRowRor8>(v);
}

// Lane l receives the value of lane l ^ 16: swaps the two 16-lane rows of
// each 32-lane half (ds_swizzle bit-mask mode: and 0x1f, or 0, xor 0x10).
__device__ __forceinline__ float swap_rows16(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}

// Max over the 16 lanes of a row (every lane receives the result).
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<kQuadXor1>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  v = fmaxf(v, dpp<kRowHalfMirror>(v));   // quad max with the mirrored quad
  v = fmaxf(v, dpp<kRowRor8>(v));
  return v;
}

// ---- exchanges between the four 16-lane rows of a wave -------------------
// gfx950's v_permlane16_swap / v_permlane32_swap move whole rows between two
// registers on the VALU (no LDS).  Called with (a, b) they return
//   permlane16: d = (odd row)    ? b[l-16] : a[l],  s = (even row)   ? a[l+16] : b[l]
//   permlane32: d = (upper half) ? b[l-32] : a[l],  s = (lower half) ? a[l+32] : b[l]
struct LanePair {
  float d, s;
};
__device__ __forceinline__ LanePair permlane16_swap(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return LanePair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair permlane32_swap(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return LanePair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Value of lane l ^ 16 (odd: this lane is in an odd row).
__device__ __forceinline__ float xor_rows16(float v, bool odd) {
  const LanePair p = permlane16_swap(v, v);
  return odd ? p.d : p.s;
}
// Value of lane l ^ 32 (upper: this lane is in the upper half).
__device__ __forceinline__ float xor_rows32(float v, bool upper) {
  const LanePair p = permlane32_swap(v, v);
  return upper ? p.d : p.s;
}
// Max with lane l ^ 16 / l ^ 32 (every lane receives it).
__device__ __forceinline__ float max_rows16(float v) {
  const LanePair p = permlane16_swap(v, v);
  return fmaxf(p.d, p.s);
}
__device__ __forceinline__ float max_rows32(float v) {
  const LanePair p = permlane32_swap(v, v);
  return fmaxf(p.d, p.s);
}
// Reduce-scatter of two values with lane l ^ 16: even rows receive
// a[l] + a[l ^ 16], odd rows b[l] + b[l ^ 16].
__device__ __forceinline__ float sum_scatter16(float a, float b) {
  const LanePair p = permlane16_swap(a, b);
  return p.d + p.s;
}
// The same with lane l ^ 32: the lower half receives the a sums, the upper
// half the b sums.
__device__ __forceinline__ float sum_scatter32(float a, float b) {
  const LanePair p = permlane32_swap(a, b);
  return p.d + p.s;
}

// ---- Walsh-Hadamard over a 32-lane-distributed 128-vector ----------------
// A 128-vector is spread over two 16-lane rows: lane c of row h holds the
// channels 8c + 4h + t, t = 0..3, in v[0..3].  Channel index bits 0-1 live in
// the register index, bit 2 in the row index, bits 3-6 in the lane index.
// Every stage maps the pair (a, b) at channel indices (i, i + 2^k) to
// (a + b, a - b), giving the unnormalised Sylvester-ordered transform H v.
template <int kMask, int N>
__device__ __forceinline__ void wht_lane_stage(float (&v)[N], int c) {
  const float sgn = (c & kMask) ? -1.0f : 1.0f;
#pragma unroll
  for (int t = 0; t < N; ++t) {
    const float p = row_xor<kMask>(v[t]);
    v[t] = __builtin_fmaf(v[t], sgn, p);   // lane bit clear: v + p; set: p - v
  }
}

__device__ __forceinline__ void wht128_split(float (&v)[4], int c, int h) {
#pragma unroll
  for (int k = 1; k < 4; k <<= 1) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (!(t & k)) {
        const float a = v[t], b = v[t + k];
        v[t] = a + b;
        v[t + k] = a - b;
      }
    }
  }
  {
    const float sgn = h ? -1.0f : 1.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = __builtin_fmaf(v[t], sgn, swap_rows16(v[t]));
  }
  wht_lane_stage<1>(v, c);
  wht_lane_stage<2>(v, c);
  wht_lane_stage<4>(v, c);
  wht_lane_stage<8>(v, c);
}

// ---- scale + e4m3 -----------------------------------------------------------
// Smallest power of two >= t for a positive normal t (bit-exact).
__device__ __forceinline__ float pow2_ceil(float t) {
  uint32_t u = __float_as_uint(t);
  if ((u & 0x007fffffu) == 0u) return t;
  return __uint_as_float(((u >> 23) + 1u) << 23);
}

// Reciprocal of a power of two 2^k (exact as long as 2^-k is normal).
__device__ __forceinline__ float pow2_recip(float p) {
  uint32_t e = __float_as_uint(p) >> 23;
  return __uint_as_float((254u - e) << 23);
}

// Pack four fp32 values (already clamped to +-448) into four e4m3 codes,
// nearest-even, byte i = code of value i (v_cvt_pk_fp8_f32, OCP e4m3 on gfx950).
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float clamp_fp8(float q) {
  return __builtin_amdgcn_fmed3f(q, -kFp8Max, kFp8Max);
}

// Per-vector scale from the row's absmax (the pages' formula, fp32).
__device__ __forceinline__ float fp8_scale(float absmax, bool round_scale) {
  float a = fmaxf(absmax, kScaleFloor);
  float t = a * kInvFp8Max;
  return round_scale ? pow2_ceil(t) : t;
}

// ---- rotate + quantise one 128-vector held by 32 lanes --------------------
// v[0..3]: fp32 values of 4 channels per lane, spread as wht128_split
// expects (2 channel bits in registers, 4 in the row's lanes, 1 across the
// two rows).  The Walsh-Hadamard matrix is a tensor product over the index
// bits, so any such assignment of channel bits gives the same transform as
// long as input and output use it.  Steps: bf16 round, rotate, scale by
// 1/sqrt(128), bf16 round, per-vector scale, clamp, e4m3.  Returns the 4 codes
// (little-endian) and the vector's scale (same in all 32 lanes).
__device__ __forceinline__ uint32_t rotate_quantise32(float (&v)[4], int c, int h,
                                                      bool round_scale, float& scale_out) {
#pragma unroll
  for (int t = 0; t < 4; ++t) v[t] = round_bf16(v[t]);
  wht128_split(v, c, h);
  float amax = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v[t] = round_bf16(v[t] * kInvSqrt128);
    amax = fmaxf(amax, fabsf(v[t]));
  }
  amax = row_max16(amax);
  amax = fmaxf(amax, swap_rows16(amax));
  const float scale = fp8_scale(amax, round_scale);
  float q[4];
  if (round_scale) {
    const float inv = pow2_recip(scale);   // exact: scale is a power of two
#pragma unroll
    for (int t = 0; t < 4; ++t) q[t] = clamp_fp8(v[t] * inv);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) q[t] = clamp_fp8(v[t] / scale);   // IEEE division
  }
  scale_out = scale;
  return pack_e4m3x4(q[0], q[1], q[2], q[3]);
}

// ---- rotate + quantise one 128-vector held by a whole wave -----------------
// Lane l = 16q + c holds channels 8c + 2q + t, t = 0..1, in v[0..1]: channel
// bit 0 in the register index, bit 1 in the row parity (q & 1), bit 2 in the
// wave half (q >> 1), bits 3-6 in the lane of the row.  Same steps and result
// as rotate_quantise32.  Returns the 2 codes in the low 16 bits and the
// vector's scale (same in all 64 lanes).
__device__ __forceinline__ uint32_t rotate_quantise64(float (&v)[2], int c, int q,
                                                      bool round_scale, float& scale_out) {
  const bool odd = q & 1, upper = q >> 1;
#pragma unroll
  for (int t = 0; t < 2; ++t) v[t] = round_bf16(v[t]);
  {
    const float a = v[0], b = v[1];
    v[0] = a + b;
    v[1] = a - b;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) v[t] = __builtin_fmaf(v[t], odd ? -1.0f : 1.0f, xor_rows16(v[t], odd));
#pragma unroll
  for (int t = 0; t < 2; ++t)
    v[t] = __builtin_fmaf(v[t], upper ? -1.0f : 1.0f, xor_rows32(v[t], upper));
  wht_lane_stage<1>(v, c);
  wht_lane_stage<2>(v, c);
  wht_lane_stage<4>(v, c);
  wht_lane_stage<8>(v, c);
  float amax = 0.0f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    v[t] = round_bf16(v[t] * kInvSqrt128);
    amax = fmaxf(amax, fabsf(v[t]));
  }
  amax = row_max16(amax);
  amax = max_rows16(amax);
  amax = max_rows32(amax);
  const float scale = fp8_scale(amax, round_scale);
  float qv[2];
  if (round_scale) {
    const float inv = pow2_recip(scale);   // exact: scale is a power of two
#pragma unroll
    for (int t = 0; t < 2; ++t) qv[t] = clamp_fp8(v[t] * inv);
  } else {
#pragma unroll
    for (int t = 0; t < 2; ++t) qv[t] = clamp_fp8(v[t] / scale);   // IEEE division
  }
  scale_out = scale;
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(qv[0], qv[1], 0, false) & 0xffffu;
}

}  // namespace kvc
