// Row loads / stores between HBM and the engine's register layouts.
#pragma once

#include "engine.hpp"

namespace whtq {

enum Dt : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

template <int DT> struct DtInfo;
template <> struct DtInfo<DT_F32>  { static constexpr int BYTES = 4; };
template <> struct DtInfo<DT_BF16> { static constexpr int BYTES = 2; };
template <> struct DtInfo<DT_F16>  { static constexpr int BYTES = 2; };

__device__ __forceinline__ float widen16(uint32_t w, bool hi, int dt) {
  if (dt == DT_BF16) return hi ? bf16hi(w) : bf16lo(w);
  f16x2_t h = __builtin_bit_cast(f16x2_t, w);
  return hi ? (float)h[1] : (float)h[0];
}

// Raw bytes of 8 contiguous values (one 16-byte vector for 16-bit types, two
// for fp32), fetched ahead of use so that the next row's loads overlap the
// current row's arithmetic.
struct Raw8 {
  u32x4 a, b;
};

template <int DT>
__device__ __forceinline__ void fetch8(const void* rowp, int i, Raw8& r) {
  if constexpr (DT == DT_F32) {
    const float* p = reinterpret_cast<const float*>(rowp) + i;
    r.a = ldg<u32x4>(p);
    r.b = ldg<u32x4>(p + 4);
  } else {
    r.a = ldg<u32x4>(reinterpret_cast<const uint16_t*>(rowp) + i);
  }
}

// Widen fetched raw values into v[0..7].  16-bit inputs come out with the
// butterflies on index bits 0 and 1 already applied (oct_bfly16); fp32
// inputs come out raw.  Signs: for 16-bit inputs `m` holds the four +-1
// coefficient pairs (sign_coef16) the butterflies fold the signs into, for
// fp32 `sb` holds the sign byte.
template <int DT> struct Fused { static constexpr int LO = DT == DT_F32 ? 0 : 2; };

template <int DT, bool SIGNS>
__device__ __forceinline__ void widen8(const Raw8& r, float* v, const uint32_t* m, uint32_t sb) {
  if constexpr (DT == DT_F32) {
    uint32_t u[8] = {r.a[0], r.a[1], r.a[2], r.a[3], r.b[0], r.b[1], r.b[2], r.b[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (SIGNS) u[e] ^= ((sb >> e) & 1u) << 31;
      v[e] = as_f(u[e]);
    }
  } else {
    const uint32_t x[4] = {r.a[0], r.a[1], r.a[2], r.a[3]};
    if constexpr (SIGNS) oct_bfly16_signed<DT == DT_BF16>(x, m, v);
    else oct_bfly16<DT == DT_BF16>(x, v);
  }
}

template <int DT, bool SIGNS>
__device__ __forceinline__ void load8(const void* rowp, int i, float* v, const uint32_t* m, uint32_t sb) {
  Raw8 r;
  fetch8<DT>(rowp, i, r);
  widen8<DT, SIGNS>(r, v, m, sb);
}

// Store 8 contiguous fp32 values at element `i` of `row` in dtype DT.
template <int DT>
__device__ __forceinline__ void store8(void* rowp, int i, const float* v) {
  if constexpr (DT == DT_F32) {
    float* p = reinterpret_cast<float*>(rowp) + i;
    stg<f32x4>(p, f32x4{v[0], v[1], v[2], v[3]});
    stg<f32x4>(p + 4, f32x4{v[4], v[5], v[6], v[7]});
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(rowp) + i;
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = DT == DT_BF16 ? pack_bf16(v[2 * q], v[2 * q + 1]) : pack_f16(v[2 * q], v[2 * q + 1]);
    stg<u32x4>(p, w);
  }
}

// Generic (possibly short, n < 8) contiguous load / store of K values.
template <int DT, int K>
__device__ __forceinline__ void loadK(const void* rowp, int i, float* v) {
  if constexpr (DT == DT_F32) {
    const float* p = reinterpret_cast<const float*>(rowp) + i;
#pragma unroll
    for (int e = 0; e < K; ++e) v[e] = p[e];
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(rowp) + i;
#pragma unroll
    for (int e = 0; e < K; ++e) v[e] = widen16((uint32_t)p[e], false, DT);
  }
}
template <int DT, int K>
__device__ __forceinline__ void storeK(void* rowp, int i, const float* v) {
  if constexpr (DT == DT_F32) {
    float* p = reinterpret_cast<float*>(rowp) + i;
#pragma unroll
    for (int e = 0; e < K; ++e) p[e] = v[e];
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(rowp) + i;
#pragma unroll
    for (int e = 0; e < K; ++e) {
      uint32_t w = DT == DT_BF16 ? pack_bf16(v[e], 0.f) : pack_f16(v[e], 0.f);
      p[e] = (uint16_t)(w & 0xffffu);
    }
  }
}

}  // namespace whtq
