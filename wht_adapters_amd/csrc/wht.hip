// wht_batched: y = Hn(S x), Hn(x) or S Hn(x) along the rows of x.
//
// Orthonormal Sylvester WHT (HARP explainer, 2.2: normalised Sylvester
// Hadamard; section 1: the randomized Hadamard transform is a fixed sign
// diagonal followed by the Hadamard transform, O(d log d)).  One fp32
// register row per T lanes, persistent over row groups; see engine.hpp for
// the layouts.
#include "io.hpp"
#include "launch.hpp"

namespace whtq {

enum SignMode : int { SIGN_NONE = 0, SIGN_BEFORE = 1, SIGN_AFTER = 2 };

template <int LOGN, int DIN, int DOUT>
__global__ __launch_bounds__(256) void k_wht(const uint8_t* x, uint8_t* y,
                                             int64_t rows, int64_t ldx_b, int64_t ldy_b,
                                             const uint32_t* __restrict__ sbits, int sign_mode,
                                             float scale) {
  using G = Geo<LOGN>;
  constexpr int T = G::T, R = G::R, RPW = 256 / T;
  const int tid = threadIdx.x, slot = tid / T, t = tid % T;
  const int64_t ngroups = (rows + RPW - 1) / RPW;

  if constexpr (G::TWO) {
    __shared__ float lds[RPW * G::LDS_ROW];
    float* myrow = lds + slot * G::LDS_ROW;
    uint32_t sb[8], m[8][4];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      sb[c] = sign_mode == SIGN_BEFORE ? sign_byte(sbits, G::idxA(t, c * 8)) : 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) m[c][q] = pair_mask16(sb[c] >> (2 * q));
    }
    uint32_t sa0 = 0, sa1 = 0;
    if (sign_mode == SIGN_AFTER) { sa0 = sbits[2 * t]; sa1 = sbits[2 * t + 1]; }
    const float cs = rho_B<LOGN>(t) ? -scale : scale;

    for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
      const int64_t row = g * RPW + slot;
      const bool valid = row < rows;
      float v[64];
      if (valid) {
        const uint8_t* xr = x + row * ldx_b;
        if (sign_mode == SIGN_BEFORE) {
#pragma unroll
          for (int c = 0; c < 8; ++c) load8<DIN, true>(xr, G::idxA(t, c * 8), v + 8 * c, m[c], sb[c]);
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) load8<DIN, false>(xr, G::idxA(t, c * 8), v + 8 * c, m[c], 0u);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 64; ++r) v[r] = 0.f;
      }
      stages_A<LOGN, DIN == DT_F32>(v, t);
      lds_write_A<LOGN>(myrow, v, t);
      __syncthreads();
      lds_read_B<LOGN>(myrow, v, t);
      __syncthreads();
      stages_B<LOGN, 1>(v, t);
#pragma unroll
      for (int r = 0; r < 64; ++r) v[r] *= cs;
      if (sign_mode == SIGN_AFTER) {
#pragma unroll
        for (int r = 0; r < 64; ++r)
          v[r] = as_f(as_u(v[r]) ^ ((((r < 32 ? sa0 >> r : sa1 >> (r - 32))) & 1u) << 31));
      }
      if (valid) {
        uint8_t* yr = y + row * ldy_b;
#pragma unroll
        for (int q = 0; q < 8; ++q) store8<DOUT>(yr, t * 64 + 8 * q, v + 8 * q);
      }
    }
  } else {
    // Single layout (n <= 256): R contiguous values per lane, T <= 4 lanes per row.
    const float cs = rho_B<LOGN>(t) ? -scale : scale;
    for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
      const int64_t row = g * RPW + slot;
      const bool valid = row < rows;
      const int base = t * R;
      float v[R];
      constexpr bool FUSED = (R >= 8) && (DIN != DT_F32);
      if (valid) {
        const uint8_t* xr = x + row * ldx_b;
        if constexpr (R >= 8) {
#pragma unroll
          for (int q = 0; q < R / 8; ++q) {
            const int i = base + 8 * q;
            uint32_t s8 = sign_mode == SIGN_BEFORE ? sign_byte(sbits, i) : 0u;
            uint32_t mm[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) mm[p] = pair_mask16(s8 >> (2 * p));
            load8<DIN, true>(xr, i, v + 8 * q, mm, s8);
          }
        } else {
          loadK<DIN, R>(xr, base, v);
          if (sign_mode == SIGN_BEFORE) {
#pragma unroll
            for (int e = 0; e < R; ++e)
              if ((sbits[(base + e) >> 5] >> ((base + e) & 31)) & 1u) v[e] = -v[e];
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) v[r] = 0.f;
      }
      stages_B<LOGN, FUSED ? 1 : 0>(v, t);
#pragma unroll
      for (int r = 0; r < R; ++r) v[r] *= cs;
      if (sign_mode == SIGN_AFTER) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          if ((sbits[(base + r) >> 5] >> ((base + r) & 31)) & 1u) v[r] = -v[r];
      }
      if (valid) {
        uint8_t* yr = y + row * ldy_b;
        if constexpr (R >= 8) {
#pragma unroll
          for (int q = 0; q < R / 8; ++q) store8<DOUT>(yr, base + 8 * q, v + 8 * q);
        } else {
          storeK<DOUT, R>(yr, base, v);
        }
      }
    }
  }
}

template <int LOGN, int DIN, int DOUT>
static hipError_t run_wht(const void* x, void* y, int64_t rows, int64_t ldx, int64_t ldy,
                          const uint32_t* sbits, int sign_mode, float scale, hipStream_t s) {
  using G = Geo<LOGN>;
  constexpr int RPW = 256 / G::T;
  const int64_t groups = (rows + RPW - 1) / RPW;
  auto k = k_wht<LOGN, DIN, DOUT>;
  const unsigned grid = persistent_grid(k, groups, 256, 0);
  hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, s, (const uint8_t*)x, (uint8_t*)y, rows,
                     ldx * DtInfo<DIN>::BYTES, ldy * DtInfo<DOUT>::BYTES, sbits, sign_mode, scale);
  return hipGetLastError();
}

template <int DIN, int DOUT>
static hipError_t dispatch_n(int logn, const void* x, void* y, int64_t rows, int64_t ldx, int64_t ldy,
                             const uint32_t* sbits, int sign_mode, float scale, hipStream_t s) {
  switch (logn) {
#define WHTQ_CASE(L) case L: return run_wht<L, DIN, DOUT>(x, y, rows, ldx, ldy, sbits, sign_mode, scale, s);
    WHTQ_CASE(1) WHTQ_CASE(2) WHTQ_CASE(3) WHTQ_CASE(4) WHTQ_CASE(5) WHTQ_CASE(6) WHTQ_CASE(7)
    WHTQ_CASE(8) WHTQ_CASE(9) WHTQ_CASE(10) WHTQ_CASE(11) WHTQ_CASE(12) WHTQ_CASE(13)
#undef WHTQ_CASE
    default: return hipErrorInvalidValue;
  }
}

// Entry from the C ABI; arguments already validated.
hipError_t launch_wht(int logn, int din, int dout, const void* x, void* y, int64_t rows, int64_t ldx,
                      int64_t ldy, const uint32_t* sbits, int sign_mode, float scale, hipStream_t s) {
  if (din == DT_F32 && dout == DT_F32) return dispatch_n<DT_F32, DT_F32>(logn, x, y, rows, ldx, ldy, sbits, sign_mode, scale, s);
  if (din == DT_BF16 && dout == DT_BF16) return dispatch_n<DT_BF16, DT_BF16>(logn, x, y, rows, ldx, ldy, sbits, sign_mode, scale, s);
  if (din == DT_F16 && dout == DT_F16) return dispatch_n<DT_F16, DT_F16>(logn, x, y, rows, ldx, ldy, sbits, sign_mode, scale, s);
  if (din == DT_BF16 && dout == DT_F32) return dispatch_n<DT_BF16, DT_F32>(logn, x, y, rows, ldx, ldy, sbits, sign_mode, scale, s);
  if (din == DT_F16 && dout == DT_F32) return dispatch_n<DT_F16, DT_F32>(logn, x, y, rows, ldx, ldy, sbits, sign_mode, scale, s);
  return hipErrorInvalidValue;
}

}  // namespace whtq
