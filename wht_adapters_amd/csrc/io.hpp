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

// Load 8 contiguous values starting at element `i` of `row` into v[0..7].
// 16-bit inputs come in with the index-bit-0 butterfly already applied
// (v[2p] = x[2p] + x[2p+1], v[2p+1] = x[2p] - x[2p+1]); fp32 inputs come in
// raw.  `m` holds per-pair sign-flip masks (16-bit) or is ignored (fp32; the
// caller passes the sign byte in `sb` instead).
template <int DT, bool SIGNS>
__device__ __forceinline__ void load8(const void* rowp, int i, float* v, const uint32_t* m, uint32_t sb) {
  if constexpr (DT == DT_F32) {
    const float* p = reinterpret_cast<const float*>(rowp) + i;
    f32x4 a = ldg<f32x4>(p), b = ldg<f32x4>(p + 4);
    uint32_t u[8] = {as_u(a[0]), as_u(a[1]), as_u(a[2]), as_u(a[3]),
                     as_u(b[0]), as_u(b[1]), as_u(b[2]), as_u(b[3])};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (SIGNS) u[e] ^= ((sb >> e) & 1u) << 31;
      v[e] = as_f(u[e]);
    }
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(rowp) + i;
    u32x4 w = ldg<u32x4>(p);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t x = w[q];
      if constexpr (SIGNS) x ^= m[q];
      if constexpr (DT == DT_BF16) pair_sumdiff_bf16(x, v[2 * q], v[2 * q + 1]);
      else pair_sumdiff_f16(x, v[2 * q], v[2 * q + 1]);
    }
  }
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
