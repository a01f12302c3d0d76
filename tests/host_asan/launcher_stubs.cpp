// Launcher stubs for the host-only AddressSanitizer build of the C ABI layer:
// every launcher succeeds without touching a device, so the planners and the
// argument validation run on the CPU alone.
#include <hip/hip_runtime.h>
#include "kvc_internal.hpp"
namespace kvc {
hipError_t launch_pool16_prefill(const uint16_t*, int64_t, const uint16_t*, int64_t, int64_t, const float*, const int32_t*, int64_t, uint8_t*, float*, int64_t, bool, const int64_t*, const uint8_t*, bool, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_pool16_ring(uint16_t*, int64_t, const int32_t*, const uint16_t*, int64_t, int64_t, const uint16_t*, int64_t, int64_t, const float*, const int32_t*, const int32_t*, int64_t, int, uint8_t*, float*, int64_t, bool, bool, float*, int64_t, int64_t, int64_t, int64_t, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_pool16_seed(uint16_t*, int64_t, const uint16_t*, int64_t, const uint16_t*, int64_t, const int32_t*, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_c128_decode(float*, int64_t, int64_t, const float*, int64_t, float*, int64_t, uint8_t*, float*, bool, const float*, int64_t, const int32_t*, const int32_t*, int64_t, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_c128_prefill(float*, int64_t, const float*, float*, uint8_t*, float*, bool, int64_t, const float*, const int32_t*, const int32_t*, int64_t, const kvc_online_plan*, uint32_t, const kvc_online_plan*, uint32_t, hipStream_t) { return hipSuccess; }
hipError_t launch_c128_prefill_fused(float*, int64_t, const float*, float*, uint8_t*, float*, bool, int64_t, const float*, const int32_t*, const int32_t*, int64_t, const kvc_online_item*, uint32_t, hipStream_t) { return hipSuccess; }
hipError_t launch_diag_convert(const float*, uint16_t*, uint8_t*, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_diag_stream_read(const void*, int64_t, uint32_t*, int, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_diag_empty(int64_t, int, int, hipStream_t) { return hipSuccess; }
}
