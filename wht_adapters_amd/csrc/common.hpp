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
typedef __bf16   bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16   bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

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

// |a| max over three values in one v_max3_f32.
__device__ __forceinline__ float max3abs(float acc, float a, float b) {
  return __builtin_fmaxf(acc, __builtin_fmaxf(__builtin_fabsf(a), __builtin_fabsf(b)));
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

// Sum and difference of a bf16 / fp16 pair straight into fp32: the products
// with +-1 are exact, so each result is the correctly rounded lo +- hi.
__device__ __forceinline__ void pair_sumdiff_bf16(uint32_t w, float& s, float& d) {
  const bf16x2_t x = __builtin_bit_cast(bf16x2_t, w);
  s = __builtin_amdgcn_fdot2_f32_bf16(x, __builtin_bit_cast(bf16x2_t, 0x3f803f80u), 0.0f, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(x, __builtin_bit_cast(bf16x2_t, 0xbf803f80u), 0.0f, false);
}
__device__ __forceinline__ void pair_sumdiff_f16(uint32_t w, float& s, float& d) {
  const f16x2_t x = __builtin_bit_cast(f16x2_t, w);
  s = __builtin_amdgcn_fdot2(x, __builtin_bit_cast(f16x2_t, 0x3c003c00u), 0.0f, false);
  d = __builtin_amdgcn_fdot2(x, __builtin_bit_cast(f16x2_t, 0xbc003c00u), 0.0f, false);
}

// Global loads / stores with explicit widths.
template <typename V>
__device__ __forceinline__ V ldg(const void* p) { return *reinterpret_cast<const V*>(p); }
template <typename V>
__device__ __forceinline__ void stg(void* p, V v) { *reinterpret_cast<V*>(p) = v; }

}  // namespace whtq
