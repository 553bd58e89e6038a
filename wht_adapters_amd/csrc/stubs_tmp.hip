#include <hip/hip_runtime.h>
#include <stdint.h>
namespace whtq {
hipError_t launch_qwha(const void*, int64_t, int64_t, const int32_t*, const int32_t*, const void*, int, int64_t, void*, int64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_harp(const void*, void*, int, int64_t, int64_t, int64_t, const uint32_t*, int, const float*, hipStream_t) { return hipErrorNotSupported; }
}
