// Register / LDS engine for a batched Sylvester FWHT of rows of n = 2^L
// values (2 <= n <= 8192), one row per T = n / R cooperating lanes, each
// lane holding R = min(64, n) fp32 values in VGPRs.
//
// A row's L butterflies are split over at most two register layouts:
//
//   layout B ("natural"):   index = t * R + r.  A lane owns R contiguous
//       values; register bits are index bits 0..5 and the two low lane bits
//       (a quad) carry index bits 6 and 7, reached with DPP.
//   layout A (n >= 512):    register bits 0..2 are index bits 0..2 (16-byte
//       vector loads of 8 values), register bits 3..5 the top three index
//       bits; the quad bits carry index bits L-5 and L-4, the remaining lane
//       bits index bits 3..L-6.
//
// Layout A covers index bit 0 and every index bit >= 8, layout B the bits
// 0..7, so one LDS transpose between them completes the transform (13 bits
// at n = 8192: 5 in A, 8 in B).  The LDS image of a row is padded by 4 floats
// per 64 so that the 16-byte reads of layout B are bank-conflict free.
//
// DPP butterflies leave the upper lane of each pair holding the negated
// result; the sign accumulated by an element is (-1)^popcount(i & RHO_MASK)
// (`rho`), and every kernel folds it into a scale or sign it applies anyway.
#pragma once

#include "common.hpp"

namespace whtq {

template <int LOGN_>
struct Geo {
  static constexpr int LOGN = LOGN_;
  static constexpr int N = 1 << LOGN;
  static constexpr int LOGR = LOGN < 6 ? LOGN : 6;
  static constexpr int R = 1 << LOGR;
  static constexpr int LOGT = LOGN - LOGR;
  static constexpr int T = 1 << LOGT;
  static constexpr bool TWO = LOGT >= 3;
  static constexpr int LDS_ROW = TWO ? N + N / 16 : 0;  // floats per row slot

  // index bits whose butterfly runs over DPP (so carry the rho sign)
  static constexpr unsigned RHO_MASK =
      (LOGN > 6 ? 1u << 6 : 0u) | (LOGN > 7 ? 1u << 7 : 0u) |
      ((TWO && LOGN - 5 >= 8) ? 1u << (LOGN - 5) : 0u) |
      ((TWO && LOGN - 4 >= 8) ? 1u << (LOGN - 4) : 0u);

  // layout A: element index of (lane t, register r)
  __device__ static __forceinline__ int idxA(int t, int r) {
    return (r & 7) | ((r >> 3) << (LOGN - 3)) | ((t & 3) << (LOGN - 5)) | ((t >> 2) << 3);
  }
  static constexpr int idxA_reg(int r) { return (r & 7) | ((r >> 3) << (LOGN - 3)); }
  __device__ static __forceinline__ int idxA_lane(int t) {
    return ((t & 3) << (LOGN - 5)) | ((t >> 2) << 3);
  }
  // layout B
  __device__ static __forceinline__ int idxB(int t, int r) { return t * R + r; }

  __device__ static __forceinline__ int phys(int i) { return i + ((i >> 6) << 2); }
};

// ---------------------------------------------------------------- butterflies

template <int R, int K>
__device__ __forceinline__ void reg_stage(float (&v)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (!(r & (1 << K))) bfly(v[r], v[r | (1 << K)]);
}

template <int R, int K>
__device__ __forceinline__ void lane_stage(float (&v)[R], int t) {
  const float c = ((t >> K) & 1) ? -1.0f : 1.0f;
#pragma unroll
  for (int r = 0; r < R; r += 4) dpp_bfly4<K>(v[r], v[r + 1], v[r + 2], v[r + 3], c);
}

// Layout B stages on index bits [lo, 8) (register bits lo..5, quad bits 6, 7).
template <int LOGN, int LO>
__device__ __forceinline__ void stages_B(float (&v)[Geo<LOGN>::R], int t) {
  using G = Geo<LOGN>;
  constexpr int R = G::R;
  if constexpr (LO <= 0 && G::LOGR > 0) reg_stage<R, 0>(v);
  if constexpr (LO <= 1 && G::LOGR > 1) reg_stage<R, 1>(v);
  if constexpr (LO <= 2 && G::LOGR > 2) reg_stage<R, 2>(v);
  if constexpr (LO <= 3 && G::LOGR > 3) reg_stage<R, 3>(v);
  if constexpr (LO <= 4 && G::LOGR > 4) reg_stage<R, 4>(v);
  if constexpr (LO <= 5 && G::LOGR > 5) reg_stage<R, 5>(v);
  if constexpr (G::LOGT >= 1) lane_stage<R, 0>(v, t);
  if constexpr (G::LOGT >= 2) lane_stage<R, 1>(v, t);
}

// Layout A stages on index bits >= 8 (and bit 0 when WITH_BIT0).
template <int LOGN, bool WITH_BIT0>
__device__ __forceinline__ void stages_A(float (&v)[64], int t) {
  static_assert(Geo<LOGN>::TWO, "layout A only exists for n >= 512");
  if constexpr (WITH_BIT0) reg_stage<64, 0>(v);
  if constexpr (LOGN - 3 >= 8) reg_stage<64, 3>(v);
  if constexpr (LOGN - 2 >= 8) reg_stage<64, 4>(v);
  if constexpr (LOGN - 1 >= 8) reg_stage<64, 5>(v);
  if constexpr (LOGN - 5 >= 8) lane_stage<64, 0>(v, t);
  if constexpr (LOGN - 4 >= 8) lane_stage<64, 1>(v, t);
}

// ------------------------------------------------------------- LDS transposes

template <int LOGN>
__device__ __forceinline__ void lds_write_A(float* row, const float (&v)[64], int t) {
  using G = Geo<LOGN>;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float* p = row + G::phys(G::idxA(t, c * 8));
    *reinterpret_cast<f32x4*>(p) = f32x4{v[c * 8 + 0], v[c * 8 + 1], v[c * 8 + 2], v[c * 8 + 3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[c * 8 + 4], v[c * 8 + 5], v[c * 8 + 6], v[c * 8 + 7]};
  }
}

template <int LOGN>
__device__ __forceinline__ void lds_read_A(const float* row, float (&v)[64], int t) {
  using G = Geo<LOGN>;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float* p = row + G::phys(G::idxA(t, c * 8));
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    v[c * 8 + 0] = a[0]; v[c * 8 + 1] = a[1]; v[c * 8 + 2] = a[2]; v[c * 8 + 3] = a[3];
    v[c * 8 + 4] = b[0]; v[c * 8 + 5] = b[1]; v[c * 8 + 6] = b[2]; v[c * 8 + 7] = b[3];
  }
}

template <int LOGN>
__device__ __forceinline__ void lds_write_B(float* row, const float (&v)[64], int t) {
  float* p = row + t * 68;
#pragma unroll
  for (int q = 0; q < 16; ++q)
    *reinterpret_cast<f32x4*>(p + 4 * q) = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
}

template <int LOGN>
__device__ __forceinline__ void lds_read_B(const float* row, float (&v)[64], int t) {
  const float* p = row + t * 68;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * q);
    v[4 * q] = a[0]; v[4 * q + 1] = a[1]; v[4 * q + 2] = a[2]; v[4 * q + 3] = a[3];
  }
}

// rho sign of lane t in layout B (register bits never carry DPP bits there).
template <int LOGN>
__device__ __forceinline__ bool rho_B(int t) {
  using G = Geo<LOGN>;
  return __builtin_popcount((unsigned)(t * G::R) & G::RHO_MASK) & 1;
}

// rho sign of (lane t, register r) in layout A, split into lane and register parts.
template <int LOGN>
__device__ __forceinline__ bool rho_A_lane(int t) {
  using G = Geo<LOGN>;
  return __builtin_popcount((unsigned)G::idxA_lane(t) & G::RHO_MASK) & 1;
}
template <int LOGN>
constexpr bool rho_A_reg(int r) {
  return popc_c((unsigned)Geo<LOGN>::idxA_reg(r) & Geo<LOGN>::RHO_MASK) & 1;
}

// Sign byte covering index bits [base, base + 8) of a uint32 bitmask (base % 8 == 0).
__device__ __forceinline__ uint32_t sign_byte(const uint32_t* bits, int base) {
  return (bits[base >> 5] >> (base & 31)) & 0xffu;
}
// XOR mask flipping the sign bits of a 16-bit pair from two sign bits.
__device__ __forceinline__ uint32_t pair_mask16(uint32_t b2) {
  return ((b2 & 1u) << 15) | ((b2 & 2u) << 30);
}

}  // namespace whtq
