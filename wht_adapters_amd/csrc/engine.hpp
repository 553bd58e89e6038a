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
// at n = 8192: 5 in A, 8 in B).
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
  static constexpr int LDS_ROW = TWO ? N / 2 + N / 16 : 0;  // floats per row slot (half row, padded)

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

  // Work-group shape: one wave per block while a row fits in a wave
  // (rows never straddle waves, so the LDS hand-off needs no block
  // barrier), else one row per block.
  static constexpr int THREADS = T >= 64 ? T : 64;
  static constexpr int RPB = THREADS / T;  // rows per block
};

// Hand-off point of the LDS transpose.  Within one wave the LDS executes a
// wave's instructions in issue order, so waiting for its own LDS traffic is
// enough; a multi-wave block needs the barrier.
template <int THREADS>
__device__ __forceinline__ void row_sync() {
  if constexpr (THREADS == 64) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  } else {
    __syncthreads();
  }
}

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
  if constexpr (R % 8 == 0) {
#pragma unroll
    for (int r = 0; r < R; r += 8) dpp_bfly8<K>(v + r, c);
  } else {
#pragma unroll
    for (int r = 0; r < R; r += 4) dpp_bfly4<K>(v[r], v[r + 1], v[r + 2], v[r + 3], c);
  }
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

// Layout A stages on index bits >= 8 (and bits 0, 1 when WITH_LOW01).
template <int LOGN, bool WITH_LOW01>
__device__ __forceinline__ void stages_A(float (&v)[64], int t) {
  static_assert(Geo<LOGN>::TWO, "layout A only exists for n >= 512");
  if constexpr (WITH_LOW01) {
    reg_stage<64, 0>(v);
    reg_stage<64, 1>(v);
  }
  if constexpr (LOGN - 3 >= 8) reg_stage<64, 3>(v);
  if constexpr (LOGN - 2 >= 8) reg_stage<64, 4>(v);
  if constexpr (LOGN - 1 >= 8) reg_stage<64, 5>(v);
  if constexpr (LOGN - 5 >= 8) lane_stage<64, 0>(v, t);
  if constexpr (LOGN - 4 >= 8) lane_stage<64, 1>(v, t);
}

// ------------------------------------------------------------- LDS transposes
//
// The A <-> B exchange runs in two halves split on index bit 2, which is a
// register bit in both layouts: each half moves one 16-byte float4 out of
// every 8-value chunk, so the LDS image holds half a row (index bit 2
// removed: c(i) = (i & 3) | ((i >> 3) << 2)) and the registers a half reads
// into are exactly those its write has just freed.
//
// Padding: 4 floats per 32.  Measured on gfx950 with the bank-conflict
// counter: 16-byte LDS writes are served 8 consecutive lanes at a time over
// 32 four-byte banks, 16-byte reads 16 lanes at a time over 64 banks.  With
// this padding the layout-B side (lane t at 32 t + 4 k) is conflict-free both
// ways; the layout-A side is conflict-free for n = 4096 writes and n = 8192
// reads and 2-way for n = 8192 writes and n = 4096 reads.  A search over
// paddings that add multiples of 4 floats per power-of-two block found none
// better over both directions; the kernels that pay it are VALU-bound.

template <int LOGN>
__device__ __forceinline__ int hphys(int ci) { return ci + ((ci >> 5) << 2); }

template <int LOGN, int THREADS>
__device__ __forceinline__ void transpose_AB(float* row, float (&v)[64], int t) {
  using G = Geo<LOGN>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int ci = G::idxA(t, c * 8) >> 1;
      *reinterpret_cast<f32x4*>(row + hphys<LOGN>(ci)) =
          f32x4{v[c * 8 + 4 * h], v[c * 8 + 4 * h + 1], v[c * 8 + 4 * h + 2], v[c * 8 + 4 * h + 3]};
    }
    row_sync<THREADS>();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int q = 2 * k + h;
      const f32x4 a = *reinterpret_cast<const f32x4*>(row + hphys<LOGN>(t * 32 + 4 * k));
      v[4 * q] = a[0]; v[4 * q + 1] = a[1]; v[4 * q + 2] = a[2]; v[4 * q + 3] = a[3];
    }
    row_sync<THREADS>();
  }
}

template <int LOGN, int THREADS>
__device__ __forceinline__ void transpose_BA(float* row, float (&v)[64], int t) {
  using G = Geo<LOGN>;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int q = 2 * k + h;
      *reinterpret_cast<f32x4*>(row + hphys<LOGN>(t * 32 + 4 * k)) =
          f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    }
    row_sync<THREADS>();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int ci = G::idxA(t, c * 8) >> 1;
      const f32x4 a = *reinterpret_cast<const f32x4*>(row + hphys<LOGN>(ci));
      v[c * 8 + 4 * h] = a[0]; v[c * 8 + 4 * h + 1] = a[1];
      v[c * 8 + 4 * h + 2] = a[2]; v[c * 8 + 4 * h + 3] = a[3];
    }
    row_sync<THREADS>();
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
// All +1 signs for the largest row (8192 bits): read in place of a sign
// vector when none applies, so that sign loads need no branch.
__device__ uint32_t kNoSigns[256];  // zero-initialised, never written

// Sign bytes at bases base[0..NC) (multiples of 8) of a uint32 bitmask, or
// zeros when `on` is false (`on` must be uniform).  The loads are
// unconditional (kNoSigns stands in), so they go out back to back and the
// compiler can put independent loads ahead of their first use.
// sign_words issues the loads, sign_bytes_of extracts the bytes (split so a
// caller can put other loads between the two).
template <int NC>
__device__ __forceinline__ void sign_words(const uint32_t* bits, bool on, const int* base, uint32_t* wv) {
  const uint32_t* p = on ? bits : kNoSigns;
#pragma unroll
  for (int c = 0; c < NC; ++c) wv[c] = p[base[c] >> 5];
}
template <int NC>
__device__ __forceinline__ void sign_bytes_of(const uint32_t* wv, const int* base, uint32_t* sb) {
#pragma unroll
  for (int c = 0; c < NC; ++c) sb[c] = (wv[c] >> (base[c] & 31)) & 0xffu;
}
template <int NC>
__device__ __forceinline__ void sign_bytes(const uint32_t* bits, bool on, const int* base, uint32_t* sb) {
  uint32_t wv[NC];
  sign_words<NC>(bits, on, base, wv);
  sign_bytes_of<NC>(wv, base, sb);
}
// XOR mask flipping the sign bits of a 16-bit pair from two sign bits.
__device__ __forceinline__ uint32_t pair_mask16(uint32_t b2) {
  return ((b2 & 1u) << 15) | ((b2 & 2u) << 30);
}

}  // namespace whtq
