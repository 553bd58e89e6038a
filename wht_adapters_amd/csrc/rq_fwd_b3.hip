// Instances of the RHT + RTN quantiser for 3-bit codes.
#include "rht_quant_mx.hpp"

namespace whtq {
template hipError_t launch_rht_quant_bits<3>(int, int, int, const void*, int64_t, int64_t, const uint32_t*,
                                             uint8_t*, uint16_t*, hipStream_t);
}  // namespace whtq
