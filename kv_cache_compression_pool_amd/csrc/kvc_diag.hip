// kvc_diag.hip -- verification and measurement helpers (not part of the
// compression path): the device number-format conversions the kernels use,
// exposed elementwise, a plain streaming-read kernel and an empty kernel
// (launch floor).
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

// Plain streaming read, one shot: workgroup w reads the 16-byte words
// [w*256*L, (w+1)*256*L), load u of thread i taking word w*256*L + u*256 + i,
// so each wave-wide load covers 1 KB of consecutive bytes and every lane
// issues its L non-temporal loads before it uses any of them.  The words are
// XOR-folded over the workgroup and the result is written to sink[w]; the
// fold keeps the loads alive and lets a test check that every word was read.
template <int L>
__global__ __launch_bounds__(256) void diag_stream_read_kernel(const u32x4_t* __restrict__ p,
                                                               int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * (256 * L) + threadIdx.x;
  u32x4_t v[L];
#pragma unroll
  for (int u = 0; u < L; ++u) {
    const int64_t i = base + u * 256;
    v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : (u32x4_t){0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < L; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
  __shared__ uint32_t s_fold[4];
  if ((threadIdx.x & 63) == 0) s_fold[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_fold[0] ^ s_fold[1] ^ s_fold[2] ^ s_fold[3];
}

// A kernel that does nothing: its launch-to-launch time with a given grid is
// the dispatch floor that any kernel of that grid pays.
__global__ __launch_bounds__(1024) void diag_empty_kernel() {}

}  // namespace

hipError_t launch_diag_convert(const float* in, uint16_t* bf16_out, uint8_t* fp8_out, int64_t n,
                               hipStream_t stream) {
  const int64_t pairs = n / 2;
  const dim3 grid((unsigned)((pairs + 255) / 256));
  hipLaunchKernelGGL(diag_convert_kernel, grid, dim3(256), 0, stream, in, bf16_out, fp8_out, n);
  return hipGetLastError();
}

hipError_t launch_diag_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                                   int loads_per_lane, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t per_block = 256LL * loads_per_lane;
  const dim3 grid((unsigned)((n16 + per_block - 1) / per_block));
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(src);
  switch (loads_per_lane) {
    case 4:
      hipLaunchKernelGGL(diag_stream_read_kernel<4>, grid, dim3(256), 0, stream, p, n16, sink);
      break;
    case 8:
      hipLaunchKernelGGL(diag_stream_read_kernel<8>, grid, dim3(256), 0, stream, p, n16, sink);
      break;
    default:
      hipLaunchKernelGGL(diag_stream_read_kernel<16>, grid, dim3(256), 0, stream, p, n16, sink);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_diag_empty(int64_t workgroups, int threads, hipStream_t stream) {
  hipLaunchKernelGGL(diag_empty_kernel, dim3((unsigned)workgroups), dim3(threads), 0, stream);
  return hipGetLastError();
}

}  // namespace kvc
