// Instances of the dequantise + inverse RHT kernels for 3-bit codes.
#include "rht_quant.hpp"

namespace whtq {
template hipError_t launch_rht_dequant_bits<3>(int, int, int, const uint8_t*, const uint16_t*, int64_t,
                                               const uint32_t*, void*, int64_t, hipStream_t);
}  // namespace whtq
