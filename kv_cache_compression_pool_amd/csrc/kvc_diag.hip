// kvc_diag.hip -- verification and measurement helpers (not part of the
// compression path): the device number-format conversions the kernels use,
// exposed elementwise, and a plain streaming-read reference kernel.
#include "kvc_device.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

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

// Plain streaming read: 4 independent 128-bit loads in flight per lane,
// grid-stride over the buffer.
__global__ __launch_bounds__(256) void diag_stream_read_kernel(const u32x4_t* __restrict__ p,
                                                               int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (int64_t base = tid; base < n16; base += 4 * stride) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + u * stride;
      v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : (u32x4_t){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[tid] = acc;
}

}  // namespace

hipError_t launch_diag_convert(const float* in, uint16_t* bf16_out, uint8_t* fp8_out, int64_t n,
                               hipStream_t stream) {
  const int64_t pairs = n / 2;
  const dim3 grid((unsigned)((pairs + 255) / 256));
  hipLaunchKernelGGL(diag_convert_kernel, grid, dim3(256), 0, stream, in, bf16_out, fp8_out, n);
  return hipGetLastError();
}

hipError_t launch_diag_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(diag_stream_read_kernel, dim3(kStreamBlocks), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4_t*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace kvc
