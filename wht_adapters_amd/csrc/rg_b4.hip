// Instances of the online-RHT low-bit product for 4-bit codes.
#include "rht_gemv.hpp"

namespace whtq {
template hipError_t launch_rht_gemv_bits<4>(int, int, const void*, int64_t, int64_t, const uint8_t*,
                                            const uint16_t*, int64_t, const uint32_t*, void*, int64_t,
                                            hipStream_t);
}  // namespace whtq
