// Dispatch of rht_quantize_rtn / rht_dequantize_inverse / rht_lowbit_gemv over
// the code width; the kernels live in rht_quant.hpp (instantiated per width in
// rq_*_b*.hip) and rht_gemv.hpp (rg_b*.hip).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace whtq {

template <int BITS>
hipError_t launch_rht_quant_bits(int logn, int din, int logg, const void* w, int64_t rows, int64_t ldw,
                                 const uint32_t* sb, uint8_t* codes, uint16_t* scales, hipStream_t s);
template <int BITS>
hipError_t launch_rht_dequant_bits(int logn, int dout, int logg, const uint8_t* codes, const uint16_t* scales,
                                   int64_t rows, const uint32_t* sb, void* out, int64_t ldo, hipStream_t s);

extern template hipError_t launch_rht_quant_bits<2>(int, int, int, const void*, int64_t, int64_t, const uint32_t*, uint8_t*, uint16_t*, hipStream_t);
extern template hipError_t launch_rht_quant_bits<3>(int, int, int, const void*, int64_t, int64_t, const uint32_t*, uint8_t*, uint16_t*, hipStream_t);
extern template hipError_t launch_rht_quant_bits<4>(int, int, int, const void*, int64_t, int64_t, const uint32_t*, uint8_t*, uint16_t*, hipStream_t);
extern template hipError_t launch_rht_dequant_bits<2>(int, int, int, const uint8_t*, const uint16_t*, int64_t, const uint32_t*, void*, int64_t, hipStream_t);
extern template hipError_t launch_rht_dequant_bits<3>(int, int, int, const uint8_t*, const uint16_t*, int64_t, const uint32_t*, void*, int64_t, hipStream_t);
extern template hipError_t launch_rht_dequant_bits<4>(int, int, int, const uint8_t*, const uint16_t*, int64_t, const uint32_t*, void*, int64_t, hipStream_t);

template <int BITS>
hipError_t launch_rht_gemv_bits(int logn, int logg, const void* x, int64_t tokens, int64_t ldx,
                                const uint8_t* codes, const uint16_t* scales, int64_t rows, const uint32_t* sb,
                                void* y, int64_t ldy, hipStream_t s);
extern template hipError_t launch_rht_gemv_bits<2>(int, int, const void*, int64_t, int64_t, const uint8_t*, const uint16_t*, int64_t, const uint32_t*, void*, int64_t, hipStream_t);
extern template hipError_t launch_rht_gemv_bits<4>(int, int, const void*, int64_t, int64_t, const uint8_t*, const uint16_t*, int64_t, const uint32_t*, void*, int64_t, hipStream_t);

hipError_t launch_rht_quant(int logn, int din, int bits, int logg, const void* w, int64_t rows,
                            int64_t ldw, const uint32_t* sb, uint8_t* codes, uint16_t* scales,
                            hipStream_t s) {
  switch (bits) {
    case 2: return launch_rht_quant_bits<2>(logn, din, logg, w, rows, ldw, sb, codes, scales, s);
    case 3: return launch_rht_quant_bits<3>(logn, din, logg, w, rows, ldw, sb, codes, scales, s);
    case 4: return launch_rht_quant_bits<4>(logn, din, logg, w, rows, ldw, sb, codes, scales, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_rht_dequant(int logn, int dout, int bits, int logg, const uint8_t* codes,
                              const uint16_t* scales, int64_t rows, const uint32_t* sb, void* out,
                              int64_t ldo, hipStream_t s) {
  switch (bits) {
    case 2: return launch_rht_dequant_bits<2>(logn, dout, logg, codes, scales, rows, sb, out, ldo, s);
    case 3: return launch_rht_dequant_bits<3>(logn, dout, logg, codes, scales, rows, sb, out, ldo, s);
    case 4: return launch_rht_dequant_bits<4>(logn, dout, logg, codes, scales, rows, sb, out, ldo, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_rht_gemv(int logn, int bits, int logg, const void* x, int64_t tokens, int64_t ldx,
                           const uint8_t* codes, const uint16_t* scales, int64_t rows, const uint32_t* sb,
                           void* y, int64_t ldy, hipStream_t s) {
  switch (bits) {
    case 2: return launch_rht_gemv_bits<2>(logn, logg, x, tokens, ldx, codes, scales, rows, sb, y, ldy, s);
    case 4: return launch_rht_gemv_bits<4>(logn, logg, x, tokens, ldx, codes, scales, rows, sb, y, ldy, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace whtq
