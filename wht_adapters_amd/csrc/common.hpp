// Device helpers shared by the gfx950 kernels of libwhtq.
//
// Butterfly notation: the Sylvester WHT of length n = 2^L is the product of L
// radix-2 butterflies, one per index bit; they commute, so every kernel is
// free to visit the bits in whatever order its data layout makes cheap
// (QWHA explainer, 2.1: the +-1 kernel is computed recursively with
// additions and subtractions only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace whtq {

typedef float    f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16   bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16   bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

// Largest magnitude among 16-bit floats (bf16 or fp16), exactly and with no
// floating-point arithmetic: for non-NaN values |a| <= |b| exactly when the
// bit patterns with the sign cleared compare the same way as integers.  acc
// holds two running maxima (one per 16-bit half of the words folded in).
__device__ __forceinline__ u16x2 absmax16(u16x2 acc, uint32_t w) {
  const uint32_t m = w & 0x7fff7fffu;
  return __builtin_elementwise_max(acc, u16x2{(uint16_t)(m & 0xffffu), (uint16_t)(m >> 16)});
}
__device__ __forceinline__ uint32_t absmax16(u16x2 acc) { return acc.x > acc.y ? acc.x : acc.y; }

// The maximum of a non-negative value over the 64 lanes, returned as a
// wave-uniform value: an inclusive max-scan (row_shr 1, 2, 4, 8 within rows
// of 16 lanes, row_bcast 15 / 31 across rows; lanes without a source read 0,
// the identity), then lane 63's result.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t x) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xf, false);
  return o > x ? o : x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = dpp_max_step<0x111, 0xf>(x);
  x = dpp_max_step<0x112, 0xf>(x);
  x = dpp_max_step<0x114, 0xf>(x);
  x = dpp_max_step<0x118, 0xf>(x);
  x = dpp_max_step<0x142, 0xa>(x);
  x = dpp_max_step<0x143, 0xc>(x);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// For the magnitude bits b of a bf16 value (sign cleared): an exponent E with
// |value| < 2^E (E = biased exponent - 126; subnormals get the normal range's
// bound, -126); 0 for b = 0.
__device__ __forceinline__ int bf16_mag_exp(uint32_t b) { return b ? (int)(b >> 7) - 126 : 0; }

constexpr int popc_c(unsigned x) { return x ? (int)(x & 1u) + popc_c(x >> 1) : 0; }

// In-register radix-2 butterfly: (a, b) -> (a + b, a - b).
__device__ __forceinline__ void bfly(float& a, float& b) {
  float s = a + b;
  b = a - b;
  a = s;
}

// Cross-lane radix-2 butterfly over lane bit 0 or 1 of a quad, one VALU op
// per value: x <- x + c * x[partner] with c = +1 on the lower lane and -1 on
// the upper lane.  The upper lane therefore ends up holding the negated
// difference; callers track that sign (rho) and fold it into a later scale.
// The leading s_nop covers the VALU-write -> DPP-read hazard of the first
// values of the batch; later values were written long before.
#define WHTQ_DPP_Q0 "quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
#define WHTQ_DPP_Q1 "quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"

#define WHTQ_DPP8(CTRL)                                   \
  asm volatile("s_nop 1\n\t"                              \
               "v_fmac_f32_dpp %0, %0, %8 " CTRL "\n\t"   \
               "v_fmac_f32_dpp %1, %1, %8 " CTRL "\n\t"   \
               "v_fmac_f32_dpp %2, %2, %8 " CTRL "\n\t"   \
               "v_fmac_f32_dpp %3, %3, %8 " CTRL "\n\t"   \
               "v_fmac_f32_dpp %4, %4, %8 " CTRL "\n\t"   \
               "v_fmac_f32_dpp %5, %5, %8 " CTRL "\n\t"   \
               "v_fmac_f32_dpp %6, %6, %8 " CTRL "\n\t"   \
               "v_fmac_f32_dpp %7, %7, %8 " CTRL           \
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), \
                 "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])  \
               : "v"(k))

template <int LANEBIT>
__device__ __forceinline__ void dpp_bfly8(float* v, float k) {
  if constexpr (LANEBIT == 0) WHTQ_DPP8(WHTQ_DPP_Q0);
  else WHTQ_DPP8(WHTQ_DPP_Q1);
}

template <int LANEBIT>
__device__ __forceinline__ void dpp_bfly4(float& a, float& b, float& c, float& d, float k) {
  if constexpr (LANEBIT == 0) {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %4 " WHTQ_DPP_Q0 "\n\t"
        "v_fmac_f32_dpp %1, %1, %4 " WHTQ_DPP_Q0 "\n\t"
        "v_fmac_f32_dpp %2, %2, %4 " WHTQ_DPP_Q0 "\n\t"
        "v_fmac_f32_dpp %3, %3, %4 " WHTQ_DPP_Q0
        : "+v"(a), "+v"(b), "+v"(c), "+v"(d)
        : "v"(k));
  } else {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %4 " WHTQ_DPP_Q1 "\n\t"
        "v_fmac_f32_dpp %1, %1, %4 " WHTQ_DPP_Q1 "\n\t"
        "v_fmac_f32_dpp %2, %2, %4 " WHTQ_DPP_Q1 "\n\t"
        "v_fmac_f32_dpp %3, %3, %4 " WHTQ_DPP_Q1
        : "+v"(a), "+v"(b), "+v"(c), "+v"(d)
        : "v"(k));
  }
}

// max over the 2 or 4 lanes of a quad (lane bits 0 / 0..1).
__device__ __forceinline__ float quad_max(float x, int lanes) {
  if (lanes >= 2)
    x = fmaxf(x, as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0xB1, 0xF, 0xF, true)));
  if (lanes >= 4)
    x = fmaxf(x, as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0x4E, 0xF, 0xF, true)));
  return x;
}

// acc <- max(acc, |a|, |b|) in one v_max3_f32 with abs source modifiers
// (the compiler otherwise splits it into two or three v_max_f32).
__device__ __forceinline__ float max3abs(float acc, float a, float b) {
  asm("v_max3_f32 %0, |%1|, |%2|, %0" : "+v"(acc) : "v"(a), "v"(b));
  return acc;
}

// bf16 pair <-> fp32 (exact widening; the pair's low half is the lower index).
__device__ __forceinline__ float bf16lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return as_f(w & 0xffff0000u); }

// fp32 -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f16x2_t p = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// Eight 16-bit values (packed words x0 = (v0, v1), x1 = (v2, v3), x2, x3)
// to fp32 with the butterflies on index bits 0 and 1 applied, per quad:
//   y0 = v0+v1+v2+v3, y1 = v0-v1+v2-v3, y2 = v0+v1-v2-v3, y3 = v0-v1-v2+v3.
// VOP3P v_dot2_f32_{bf16,f16} with a +-1 pair k (low half = lower index):
// d = x.lo * k.lo + x.hi * k.hi + acc; the products with +-1 are exact.
// gfx950 does not interlock a dot2 result against its next readers, so the
// block spaces dependent dot2s by at least three instructions and ends with
// three wait states before anything else may read its outputs.
template <bool BF16> struct PM {
  static constexpr uint32_t PP = BF16 ? 0x3f803f80u : 0x3c003c00u;  // (+1, +1)
  static constexpr uint32_t PN = BF16 ? 0xbf803f80u : 0xbc003c00u;  // (+1, -1)
  static constexpr uint32_t NN = BF16 ? 0xbf80bf80u : 0xbc00bc00u;  // (-1, -1)
  static constexpr uint32_t NP = BF16 ? 0x3f80bf80u : 0x3c00bc00u;  // (-1, +1)
};

#define WHTQ_QUAD8(OP)                                                        \
  asm(OP " %8, %12, %16, 0\n\t"   /* s0 = x0 . (+,+)            */          \
      OP " %9, %12, %17, 0\n\t"   /* d0 = x0 . (+,-)            */          \
      OP " %10, %14, %16, 0\n\t"  /* s1 = x2 . (+,+)            */          \
      OP " %11, %14, %17, 0\n\t"  /* d1 = x2 . (+,-)            */          \
      "s_nop 0\n\t"                                                           \
      OP " %0, %13, %16, %8\n\t"  /* y0 = s0 + x1 . (+,+)       */          \
      OP " %2, %13, %18, %8\n\t"  /* y2 = s0 + x1 . (-,-)       */          \
      OP " %1, %13, %17, %9\n\t"  /* y1 = d0 + x1 . (+,-)       */          \
      OP " %3, %13, %19, %9\n\t"  /* y3 = d0 + x1 . (-,+)       */          \
      OP " %4, %15, %16, %10\n\t"                                             \
      OP " %6, %15, %18, %10\n\t"                                             \
      OP " %5, %15, %17, %11\n\t"                                             \
      OP " %7, %15, %19, %11\n\t"                                             \
      "s_nop 2"                                                               \
      : "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3]),                   \
        "=&v"(y[4]), "=&v"(y[5]), "=&v"(y[6]), "=&v"(y[7]),                   \
        "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)                            \
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]),                           \
        "s"(PM<BF16>::PP), "s"(PM<BF16>::PN), "s"(PM<BF16>::NN), "s"(PM<BF16>::NP))

template <bool BF16>
__device__ __forceinline__ void oct_bfly16(const uint32_t* x, float* y) {
  float t0, t1, t2, t3;
  if constexpr (BF16) WHTQ_QUAD8("v_dot2_f32_bf16");
  else WHTQ_QUAD8("v_dot2_f32_f16");
}

// The same butterflies with a +-1 sign per input folded into the products:
// k[q] is the pair (s_2q, s_2q+1) of +-1 (low half = lower index) for word
// x[q], and the VOP3P neg_lo / neg_hi modifiers on the coefficient operand
// give the other three sign patterns, so no separate sign flip is needed.
#define WHTQ_QUAD8K(OP)                                                       \
  asm(OP " %8, %12, %16, 0\n\t"                         /* s0 = x0 . k0      */ \
      OP " %9, %12, %16, 0 neg_hi:[0,1,0]\n\t"          /* d0 = x0 . k0(+,-) */ \
      OP " %10, %14, %18, 0\n\t"                                               \
      OP " %11, %14, %18, 0 neg_hi:[0,1,0]\n\t"                                \
      "s_nop 0\n\t"                                                            \
      OP " %0, %13, %17, %8\n\t"                        /* y0 = s0 + x1 . k1 */ \
      OP " %2, %13, %17, %8 neg_lo:[0,1,0] neg_hi:[0,1,0]\n\t" /* y2 = s0 - x1 . k1 */ \
      OP " %1, %13, %17, %9 neg_hi:[0,1,0]\n\t"         /* y1 = d0 + x1 . k1(+,-) */ \
      OP " %3, %13, %17, %9 neg_lo:[0,1,0]\n\t"         /* y3 = d0 + x1 . k1(-,+) */ \
      OP " %4, %15, %19, %10\n\t"                                              \
      OP " %6, %15, %19, %10 neg_lo:[0,1,0] neg_hi:[0,1,0]\n\t"                \
      OP " %5, %15, %19, %11 neg_hi:[0,1,0]\n\t"                               \
      OP " %7, %15, %19, %11 neg_lo:[0,1,0]\n\t"                               \
      "s_nop 2"                                                               \
      : "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3]),                   \
        "=&v"(y[4]), "=&v"(y[5]), "=&v"(y[6]), "=&v"(y[7]),                   \
        "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)                            \
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]),                           \
        "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]))

template <bool BF16>
__device__ __forceinline__ void oct_bfly16_signed(const uint32_t* x, const uint32_t* k, float* y) {
  float t0, t1, t2, t3;
  if constexpr (BF16) WHTQ_QUAD8K("v_dot2_f32_bf16");
  else WHTQ_QUAD8K("v_dot2_f32_f16");
}

// +-1 coefficient pair of oct_bfly16_signed from two sign bits (bit 0: the
// lower index; a set bit means -1)
template <bool BF16>
__device__ __forceinline__ uint32_t sign_coef16(uint32_t b2) {
  return PM<BF16>::PP ^ (((b2 & 1u) << 15) | ((b2 & 2u) << 30));
}

// acc += a * h (h an fp16 value in the low / high half of `w`), one
// v_fma_mix_f32 with the fp16 operand widened exactly inside the FMA.
__device__ __forceinline__ void fma_mix_lo(float& acc, float a, uint32_t w) {
  asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[0,1,0]" : "+v"(acc) : "v"(a), "v"(w));
}
__device__ __forceinline__ void fma_mix_hi(float& acc, float a, uint32_t w) {
  asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(acc) : "v"(a), "v"(w));
}

// s * h for the fp16 value h in the low / high half of `w` (exact widening
// inside the mixed-precision FMA, one rounding of the product).
__device__ __forceinline__ float f16_mul_lo(float s, uint32_t w) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(d) : "v"(s), "v"(w));
  return d;
}
__device__ __forceinline__ float f16_mul_hi(float s, uint32_t w) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(d) : "v"(s), "v"(w));
  return d;
}
// (lo, hi) -> (lo + hi, lo - hi) on an fp16 pair, one packed add.
__device__ __forceinline__ f16x2_t f16_pair_bfly(f16x2_t a) {
  f16x2_t d;
  asm("v_pk_add_f16 %0, %1, %1 op_sel:[0,1] op_sel_hi:[0,1] neg_hi:[0,1]" : "=v"(d) : "v"(a));
  return d;
}

// Load from a pointer known to be in global memory, whatever the compiler can
// still infer about it (keeps global_load rather than flat_load, whose
// completion also counts against the LDS wait counter).
template <typename V>
__device__ __forceinline__ V ldg_global(const void* p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) V*>(reinterpret_cast<uintptr_t>(p));
}

// Global loads / stores with explicit widths.
template <typename V>
__device__ __forceinline__ V ldg(const void* p) { return *reinterpret_cast<const V*>(p); }
template <typename V>
__device__ __forceinline__ void stg(void* p, V v) { *reinterpret_cast<V*>(p) = v; }

}  // namespace whtq
