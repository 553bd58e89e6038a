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
__global__ __launch_bounds__(Geo<LOGN>::THREADS) void k_wht(const uint8_t* x, uint8_t* y, int64_t rows,
                                                           int64_t ldx_b, int64_t ldy_b,
                                                           const uint32_t* __restrict__ sbits,
                                                           int sign_mode, float scale) {
  using G = Geo<LOGN>;
  constexpr int T = G::T, R = G::R, RPB = G::RPB;
  const int tid = threadIdx.x, slot = tid / T, t = tid % T;
  const int64_t ngroups = (rows + RPB - 1) / RPB;
  const float cs = rho_B<LOGN>(t) ? -scale : scale;

  if constexpr (G::TWO) {
    __shared__ float lds[RPB * G::LDS_ROW];
    float* myrow = lds + slot * G::LDS_ROW;
    int col[8];
    uint32_t sb[8], m[8][4];
#pragma unroll
    for (int c = 0; c < 8; ++c) col[c] = G::idxA(t, c * 8);
    sign_bytes<8>(sbits, sign_mode == SIGN_BEFORE, col, sb);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) m[c][q] = sign_coef16<DIN == DT_BF16>(sb[c] >> (2 * q));
    uint32_t sa0 = 0, sa1 = 0;
    if (sign_mode == SIGN_AFTER) { sa0 = sbits[2 * t]; sa1 = sbits[2 * t + 1]; }

    for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
      const int64_t row = g * RPB + slot;
      const bool valid = row < rows;
      // rows past the end (last block only) transform a copy of the last row
      // and store nothing
      const uint8_t* xr = x + (valid ? row : rows - 1) * ldx_b;
      float v[64];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        Raw8 raw;
        fetch8<DIN>(xr, col[c], raw);
        widen8<DIN, true>(raw, v + 8 * c, m[c], sb[c]);   // (coefficients are +1 unless SIGN_BEFORE)
      }
      stages_A<LOGN, DIN == DT_F32>(v, t);
      transpose_AB<LOGN, G::THREADS>(myrow, v, t);
      stages_B<LOGN, 2>(v, t);
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
    constexpr int NSB = R >= 8 ? R / 8 : 1;
    uint32_t s8v[NSB];
    {
      int sbase[NSB];
#pragma unroll
      for (int q = 0; q < NSB; ++q) sbase[q] = t * R + 8 * q;
      sign_bytes<NSB>(sbits, R >= 8 && sign_mode == SIGN_BEFORE, sbase, s8v);
    }
    for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
      const int64_t row = g * RPB + slot;
      const bool valid = row < rows;
      const int base = t * R;
      float v[R];
      constexpr int LO = R >= 8 ? Fused<DIN>::LO : 0;
      {
        const uint8_t* xr = x + (valid ? row : rows - 1) * ldx_b;
        if constexpr (R >= 8) {
#pragma unroll
          for (int q = 0; q < R / 8; ++q) {
            const int i = base + 8 * q;
            const uint32_t s8 = s8v[q];
            uint32_t mm[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) mm[p] = sign_coef16<DIN == DT_BF16>(s8 >> (2 * p));
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
      }
      stages_B<LOGN, LO>(v, t);
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


// ---------------------------------------------------------------------------
// Small batches (fewer rows than the chip has SIMDs to give one wave each):
// one block of N/E threads per row, E = 16 values per thread (32 at n = 8192),
// so a row is spread over up to four waves.  The log2 n butterfly stages run
// in three register phases; between phases the row passes through LDS in
// place (each thread reads back exactly the values its next phase needs).
// Phase p holds the E values whose index bits [a_p, a_p + e) vary (a_0 = 0,
// a_1 = e, a_2 = L - e) and applies the stages on bits [b_p, b_p+1) with
// b = (0, e, 2e, L); the other index bits are the thread id in order.
namespace wsm {
template <int LOGN> struct Cfg {
  static constexpr int N = 1 << LOGN;
  static constexpr int LOGE = LOGN >= 13 ? 5 : 4;
  static constexpr int E = 1 << LOGE;
  static constexpr int THREADS = N / E;
  static constexpr int A[3] = {0, LOGE, LOGN - LOGE};
  static constexpr int B[4] = {0, LOGE, 2 * LOGE, LOGN};
  static_assert(3 * LOGE >= LOGN && LOGN >= 2 * LOGE, "three phases cover the index");
};
// index of value r of thread t in phase p (r's bits at [a, a + LOGE))
template <int LOGE>
__device__ __forceinline__ int at(int t, int r, int a) {
  return (t & ((1 << a) - 1)) | (r << a) | ((t >> a) << (a + LOGE));
}
__device__ __forceinline__ int pad(int i) { return i + (i >> 4); }  // one float per 16: spreads banks
// eight consecutive values widened to fp32, nothing else applied
template <int DT>
__device__ __forceinline__ void load8_plain(const uint8_t* rowp, int i, float* v) {
  if constexpr (DT == DT_F32) {
    const f32x4 a = ldg<f32x4>(reinterpret_cast<const float*>(rowp) + i);
    const f32x4 b = ldg<f32x4>(reinterpret_cast<const float*>(rowp) + i + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = a[q];
      v[4 + q] = b[q];
    }
  } else {
    const u32x4 w = ldg<u32x4>(reinterpret_cast<const uint16_t*>(rowp) + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = widen16(w[q], false, DT);
      v[2 * q + 1] = widen16(w[q], true, DT);
    }
  }
}
}  // namespace wsm

template <int LOGN, int DIN, int DOUT>
__global__ __launch_bounds__(wsm::Cfg<LOGN>::THREADS) void k_wht_blk(const uint8_t* x, uint8_t* y, int64_t rows,
                                                                   int64_t ldx_b, int64_t ldy_b,
                                                                   const uint32_t* __restrict__ sbits,
                                                                   int sign_mode, float scale) {
  using C = wsm::Cfg<LOGN>;
  constexpr int E = C::E, LE = C::LOGE;
  __shared__ float lds[C::N + C::N / 16];
  const int t = threadIdx.x;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    float v[E];
    // ---- phase 0: E contiguous values, sign before, stages on bits [0, e)
    {
      const uint8_t* xr = x + row * ldx_b;
      const int i0 = t * E;
#pragma unroll
      for (int q = 0; q < E / 8; ++q) wsm::load8_plain<DIN>(xr, i0 + 8 * q, v + 8 * q);
      if (sign_mode == SIGN_BEFORE) {
        const uint32_t sw = sbits[i0 >> 5] >> (i0 & 31);
#pragma unroll
        for (int r = 0; r < E; ++r) v[r] = as_f(as_u(v[r]) ^ (((sw >> r) & 1u) << 31));
      }
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      if (p > 0) {
        __syncthreads();  // the previous phase's values are all in LDS
#pragma unroll
        for (int r = 0; r < E; ++r) v[r] = lds[wsm::pad(wsm::at<LE>(t, r, C::A[p]))];
      }
#pragma unroll
      for (int bit = C::B[p]; bit < C::B[p + 1]; ++bit) {
        const int m = 1 << (bit - C::A[p]);
#pragma unroll
        for (int r = 0; r < E; ++r)
          if (!(r & m)) {
            const float a = v[r], b = v[r | m];
            v[r] = a + b;
            v[r | m] = a - b;
          }
      }
      if (p < 2) {
        if (p > 0) __syncthreads();  // everyone has read this phase's values
#pragma unroll
        for (int r = 0; r < E; ++r) lds[wsm::pad(wsm::at<LE>(t, r, C::A[p]))] = v[r];
      }
    }
    // ---- scale, sign after, store (lane-consecutive indices: coalesced)
    uint8_t* yr = y + row * ldy_b;
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const int i = wsm::at<LE>(t, r, C::A[2]);
      float o = v[r] * scale;
      if (sign_mode == SIGN_AFTER) o = as_f(as_u(o) ^ (((sbits[i >> 5] >> (i & 31)) & 1u) << 31));
      if constexpr (DOUT == DT_F32) reinterpret_cast<float*>(yr)[i] = o;
      else if constexpr (DOUT == DT_BF16) reinterpret_cast<uint16_t*>(yr)[i] = (uint16_t)(pack_bf16(o, 0.f) & 0xffffu);
      else reinterpret_cast<uint16_t*>(yr)[i] = (uint16_t)(pack_f16(o, 0.f) & 0xffffu);
    }
    __syncthreads();  // the next row reuses LDS
  }
}

// Rows below this use the block-per-row kernel (n >= 1024): with one wave
// per row they would leave most of the chip's 1024 SIMDs idle.
constexpr int64_t SMALL_BATCH_ROWS = 1024;

template <int LOGN, int DIN, int DOUT>
static hipError_t run_wht(const void* x, void* y, int64_t rows, int64_t ldx, int64_t ldy,
                          const uint32_t* sbits, int sign_mode, float scale, hipStream_t s) {
  if constexpr (LOGN >= 10) {
    if (rows < SMALL_BATCH_ROWS) {
      using C = wsm::Cfg<LOGN>;
      auto kb = k_wht_blk<LOGN, DIN, DOUT>;
      static const int nbb = blocks_per_cu(kb, C::THREADS, 0);
      hipLaunchKernelGGL(kb, dim3(persistent_grid(rows, nbb)), dim3(C::THREADS), 0, s, (const uint8_t*)x,
                         (uint8_t*)y, rows, ldx * DtInfo<DIN>::BYTES, ldy * DtInfo<DOUT>::BYTES, sbits, sign_mode,
                         scale);
      return hipGetLastError();
    }
  }
  using G = Geo<LOGN>;
  const int64_t groups = (rows + G::RPB - 1) / G::RPB;
  auto k = k_wht<LOGN, DIN, DOUT>;
  static const int nb = blocks_per_cu(k, G::THREADS, 0);
  const unsigned grid = persistent_grid(groups, nb);
  hipLaunchKernelGGL(k, dim3(grid), dim3(G::THREADS), 0, s, (const uint8_t*)x, (uint8_t*)y, rows,
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
