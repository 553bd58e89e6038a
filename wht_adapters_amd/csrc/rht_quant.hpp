// rht_quantize_rtn / rht_dequantize_inverse.
//
// Forward: y = Hn(S w) (randomized Hadamard transform, HARP explainer
// section 1: fixed random sign diagonal then Hadamard, exactly orthogonal),
// then per group of g consecutive transformed coordinates a symmetric absmax
// scale, stored as fp16 (round to nearest even), and signed b-bit codes
// q = rint(y / s) in [-qmax, qmax], qmax = 2^(b-1) - 1, packed LSB-first
// into a little-endian bit stream (the pages leave the quantiser to other
// systems; these are this library's fixed conventions).
//
// Inverse: unpack, y_hat = q * s, x_hat = S Hn(y_hat): both factors are
// involutions, so the inverse exists and is the same transform.
//
// Quantiser epilogue, per element:
//   f = fma(y_raw, m_g, 1.5*2^23),  m_g = rho * n^-1/2 / s16_g
// The fma rounds the exact product once, to an integer (the ulp at 2^23 is
// 1, round half to even), and |q| <= 2^(b-1) keeps f in [2^23, 2^24), so the
// low b bits of f are q in two's complement.  Codes are packed with a
// funnel shift (v_alignbit_b32) that moves just those bits into the word.
#pragma once

#include <type_traits>

#include "io.hpp"
#include "launch.hpp"


namespace whtq {

template <int BITS>
struct QPack {
  static constexpr int QMAX = (1 << (BITS - 1)) - 1;
  static constexpr float MAGIC = 12582912.0f;  // 1.5 * 2^23
  static constexpr int PER_WORD = 32 / BITS;   // BITS 2 or 4
};

// ------------------------------------------------------------------ forward

template <int LOGN, int DIN, int BITS, int LOGG>
__global__ __launch_bounds__(Geo<LOGN>::THREADS) void k_rht_quant(
    const uint8_t* __restrict__ w, int64_t rows, int64_t ldw_b, const uint32_t* __restrict__ sbits,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales, float inv_sqrt_n) {
  using G = Geo<LOGN>;
  static_assert(G::R == 64, "quantiser needs n >= 64");
  constexpr int T = G::T, RPB = G::RPB;
  constexpr int GS = 1 << LOGG;
  constexpr int GL = GS <= 64 ? GS : 64;           // group length inside one lane
  constexpr int NG = 64 / GL;                      // groups per lane
  constexpr int SPAN = GS <= 64 ? 1 : GS / 64;     // lanes per group
  constexpr int ROW_CODE_B = (G::N * BITS) / 8;
  constexpr int LANE_CODE_B = 8 * BITS;            // 64 codes
  constexpr int NSC = G::N / GS;                   // scales per row
  constexpr float QM = (float)QPack<BITS>::QMAX;
  using QP = QPack<BITS>;

  const int tid = threadIdx.x, slot = tid / T, t = tid % T;
  const int64_t ngroups = (rows + RPB - 1) / RPB;
  const bool rho = rho_B<LOGN>(t);

  __shared__ float lds[G::TWO ? RPB * G::LDS_ROW : 1];
  float* myrow = lds + slot * G::LDS_ROW;

  // per-lane sign bytes for the load layout (A when two-phase, else B)
  int col[8];
  uint32_t sw[8], sb[8], m[8][4];
#pragma unroll
  for (int c = 0; c < 8; ++c) col[c] = G::TWO ? G::idxA(t, c * 8) : t * 64 + c * 8;
  // slots past the end (last block only) transform a copy of the last row
  // and store the same bytes there, so every lane runs the same code
  // without branches
  auto row_ptr = [&](int64_t g) {
    const int64_t row = g * RPB + slot;
    return w + (row < rows ? row : rows - 1) * ldw_b;
  };
  sign_words<8>(sbits, sbits != nullptr, col, sw);
  sign_bytes_of<8>(sw, col, sb);
  // 16-bit rows: the signs ride on the +-1 coefficients of the first
  // butterflies (fp32 rows flip sign bits with sb instead)
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) m[c][q] = sign_coef16<DIN == DT_BF16>(sb[c] >> (2 * q));

  auto do_row = [&](Raw8 (&raw)[8], int64_t g) {
    const int64_t row = g * RPB + slot;
    const bool valid = row < rows;
    float v[64];
#pragma unroll
    for (int c = 0; c < 8; ++c) widen8<DIN, true>(raw[c], v + 8 * c, m[c], sb[c]);
    // 16-bit loads arrive with the index-bit 0 and 1 butterflies applied
    if constexpr (G::TWO) {
      stages_A<LOGN, DIN == DT_F32>(v, t);
      transpose_AB<LOGN, G::THREADS>(myrow, v, t);
      stages_B<LOGN, 2>(v, t);
    } else {
      stages_B<LOGN, Fused<DIN>::LO>(v, t);
    }

    // ---- epilogue: group absmax -> fp16 scale -> codes
    float mult[NG];
    uint16_t s16b[NG];
    bool ovf = false;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      // four independent max3 chains, then combined (short dependency chains)
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e + 1 < GL; e += 2) a4[(e >> 1) & 3] = max3abs(a4[(e >> 1) & 3], v[k * GL + e], v[k * GL + e + 1]);
      float a = __builtin_fmaxf(__builtin_fmaxf(a4[0], a4[1]), __builtin_fmaxf(a4[2], a4[3]));
      a = quad_max(a, SPAN);
      const float s_pre = (a * inv_sqrt_n) / QM;
      const _Float16 h = (_Float16)s_pre;
      const float sf = (float)h;
      // an fp16 scale > 0 is >= 2^-24, so the max() only changes the
      // all-zero group, whose multiplier is 0; no branch around the divide
      const float dv = inv_sqrt_n / __builtin_fmaxf(sf, 1.17549435e-38f);
      const float mm = sf > 0.f ? dv : 0.f;
      mult[k] = rho ? -mm : mm;
      s16b[k] = __builtin_bit_cast(uint16_t, h);
      // fp16 rounding can shrink the scale enough (only where it is
      // subnormal) that the group maximum lands past qmax + 1/2: then q
      // must be clipped to +-qmax
      ovf |= a * mm > QM + 0.25f;
    }
    uint32_t cw[LANE_CODE_B / 4];
    auto codes_of = [&](auto clip) {
      auto q_of = [&](int r) {
        float f = __builtin_fmaf(v[r], mult[r / GL], QP::MAGIC);
        if constexpr (decltype(clip)::value) f = __builtin_amdgcn_fmed3f(f, QP::MAGIC - QM, QP::MAGIC + QM);
        return as_u(f);
      };
      if constexpr (BITS == 3) {
#pragma unroll
        for (int j = 0; j < 6; ++j) cw[j] = 0u;
#pragma unroll
        for (int r = 0; r < 64; ++r) {
          const uint32_t c = q_of(r) & 7u;
          const int bit = 3 * r, wi = bit >> 5, off = bit & 31;
          cw[wi] |= c << off;
          if (off > 29) cw[wi + 1] |= c >> (32 - off);
        }
      } else {
#pragma unroll
        for (int j = 0; j < LANE_CODE_B / 4; ++j) {
          // each step shifts the word down by BITS and puts the next code's
          // bits on top: the first code ends in the lowest field
          uint32_t acc = 0;
#pragma unroll
          for (int k = 0; k < QP::PER_WORD; ++k) acc = __builtin_amdgcn_alignbit(q_of(j * QP::PER_WORD + k), acc, BITS);
          cw[j] = acc;
        }
      }
    };
    // the clipping copy runs only for a wave that needs it
    if (__builtin_amdgcn_ballot_w64(ovf)) codes_of(std::true_type{});
    else codes_of(std::false_type{});
    // Stores are unconditional (no branch, so no conservative wait at a
    // join): a slot past the last row has recomputed the last row and writes
    // the same bytes there.  Lanes sharing a group write the same scale.
    const int64_t srow = valid ? row : rows - 1;
    uint8_t* cr = codes + srow * (int64_t)ROW_CODE_B + t * LANE_CODE_B;
    if constexpr (BITS == 4) {
      stg<u32x4>(cr, u32x4{cw[0], cw[1], cw[2], cw[3]});
      stg<u32x4>(cr + 16, u32x4{cw[4], cw[5], cw[6], cw[7]});
    } else if constexpr (BITS == 2) {
      stg<u32x4>(cr, u32x4{cw[0], cw[1], cw[2], cw[3]});
    } else {
      stg<u32x2>(cr, u32x2{cw[0], cw[1]});
      stg<u32x2>(cr + 8, u32x2{cw[2], cw[3]});
      stg<u32x2>(cr + 16, u32x2{cw[4], cw[5]});
    }
    uint16_t* sr = scales + srow * (int64_t)NSC;
    if constexpr (SPAN == 1) {
#pragma unroll
      for (int k = 0; k < NG; ++k) sr[t * NG + k] = s16b[k];
    } else {
      sr[t / SPAN] = s16b[0];
    }
  };
  auto fetch_row = [&](Raw8 (&raw)[8], int64_t g) {
#pragma unroll
    for (int c = 0; c < 8; ++c) fetch8<DIN>(row_ptr(g), col[c], raw[c]);
  };
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    Raw8 ra[8];
    fetch_row(ra, g);
    do_row(ra, g);
  }
}

// ------------------------------------------------------------------ inverse

template <int BITS>
__device__ __forceinline__ int code_at(const uint32_t* cw, int r) {
  if constexpr (BITS == 3) {
    const int bit = 3 * r, wi = bit >> 5, off = bit & 31;
    uint32_t u = cw[wi] >> off;
    if (off > 29) u |= cw[wi + 1] << (32 - off);
    return ((int)(u << 29)) >> 29;
  } else {
    constexpr int PW = 32 / BITS;
    return __builtin_amdgcn_sbfe((int)cw[r / PW], (r % PW) * BITS, BITS);
  }
}

// Dequantise a lane's 64 codes (BITS 2 or 4, one scale for all of them) and
// apply the butterflies on index bits 0..5 (the lane's own) on the way.
// Those six stages only add and subtract codes, so they run on the exact
// integers in packed fp16 (|sum| <= 64 * 2^(b-1) <= 512, exact there): two
// values per VALU op instead of one.  A register pair holds codes k and
// k + CPW/2 of a 32-bit code word, which sit 16 bits apart, so one shift
// and one and-or turn a word into fp16 pairs 1024 + q + 2^(b-1) (offset
// binary after flipping the code's sign bit; 0x6400 is 1024.0, whose ulp
// is 1).  Each result is then widened and scaled in one mixed FMA:
// v = s * (H_64 q), one rounding instead of a rounding per stage.
template <int BITS>
__device__ __forceinline__ void dequant_lane_h64(const uint32_t* cw, float s, float* v) {
  static_assert(BITS == 2 || BITS == 4, "codes must tile 16-bit halves");
  constexpr int CPW = 32 / BITS, HALF = CPW / 2, NW = 64 / CPW;
  constexpr uint32_t FIELD = (1u << BITS) - 1, MASK = FIELD | (FIELD << 16);
  constexpr uint32_t FLIP = BITS == 2 ? 0xaaaaaaaau : 0x88888888u;
  constexpr _Float16 BIAS = (_Float16)(1024 + (1 << (BITS - 1)));
  // the magic in a VGPR: with the mask in an SGPR the and-or is one VOP3
  // (gfx9 reads one scalar operand per VALU instruction)
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));
  f16x2_t R[NW][HALF];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t u = cw[w] ^ FLIP;
#pragma unroll
    for (int k = 0; k < HALF; ++k) {
      const uint32_t b = ((u >> (BITS * k)) & MASK) | magic;
      R[w][k] = __builtin_bit_cast(f16x2_t, b) - f16x2_t{BIAS, BIAS};
    }
  }
  // element index r = CPW w + HALF h + k: the pair bit h is a stage inside
  // each register, the bits of k and w pair registers
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int k = 0; k < HALF; ++k) R[w][k] = f16_pair_bfly(R[w][k]);
#pragma unroll
  for (int kb = 1; kb < HALF; kb <<= 1)
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int k = 0; k < HALF; ++k)
        if (!(k & kb)) {
          const f16x2_t a = R[w][k], b = R[w][k | kb];
          R[w][k] = a + b;
          R[w][k | kb] = a - b;
        }
#pragma unroll
  for (int wb = 1; wb < NW; wb <<= 1)
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (!(w & wb))
#pragma unroll
        for (int k = 0; k < HALF; ++k) {
          const f16x2_t a = R[w][k], b = R[w | wb][k];
          R[w][k] = a + b;
          R[w | wb][k] = a - b;
        }
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int k = 0; k < HALF; ++k) {
      const uint32_t b = __builtin_bit_cast(uint32_t, R[w][k]);
      v[CPW * w + k] = f16_mul_lo(s, b);
      v[CPW * w + HALF + k] = f16_mul_hi(s, b);
    }
}

// The 64 codes (8*BITS bytes) of one lane.
// The inverse streams codes in and rows out once each: non-temporal accesses
// (11.4 vs 14.3 us at 4096 x 4096 INT4 on MI355X).
template <typename V>
__device__ __forceinline__ V ldg_dq(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
}
template <typename V>
__device__ __forceinline__ void stg_dq(void* p, V v) {
  __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
}

template <int BITS>
__device__ __forceinline__ void fetch_codes(const uint8_t* cr, uint32_t* cw) {
  if constexpr (BITS == 4) {
    u32x4 a = ldg_dq<u32x4>(cr), b = ldg_dq<u32x4>(cr + 16);
    cw[0] = a[0]; cw[1] = a[1]; cw[2] = a[2]; cw[3] = a[3];
    cw[4] = b[0]; cw[5] = b[1]; cw[6] = b[2]; cw[7] = b[3];
  } else if constexpr (BITS == 2) {
    u32x4 a = ldg_dq<u32x4>(cr);
    cw[0] = a[0]; cw[1] = a[1]; cw[2] = a[2]; cw[3] = a[3];
  } else {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      u32x2 a = ldg<u32x2>(cr + 8 * j);
      cw[2 * j] = a[0]; cw[2 * j + 1] = a[1];
    }
  }
}

template <int LOGN, int BITS, int LOGG, int DOUT>
__global__ __launch_bounds__(Geo<LOGN>::THREADS) void k_rht_dequant(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int64_t rows,
    const uint32_t* __restrict__ sbits, uint8_t* __restrict__ out, int64_t ldo_b, float inv_sqrt_n) {
  using G = Geo<LOGN>;
  static_assert(G::R == 64, "dequantiser needs n >= 64");
  constexpr int T = G::T, RPB = G::RPB;
  constexpr int GS = 1 << LOGG;
  constexpr int GL = GS <= 64 ? GS : 64;
  constexpr int NG = 64 / GL;
  constexpr int SPAN = GS <= 64 ? 1 : GS / 64;
  constexpr int ROW_CODE_B = (G::N * BITS) / 8;
  constexpr int LANE_CODE_B = 8 * BITS;
  constexpr int NSC = G::N / GS;

  const int tid = threadIdx.x, slot = tid / T, t = tid % T;
  const int64_t ngroups = (rows + RPB - 1) / RPB;

  __shared__ float lds[G::TWO ? RPB * G::LDS_ROW : 1];
  float* myrow = lds + slot * G::LDS_ROW;

  // A row's inputs: its codes and the raw fp16 scales of this lane's groups.
  struct In {
    uint32_t cw[LANE_CODE_B / 4];
    uint16_t hb[NG];
  };
  // rows past the end (last block only) recompute the last row
  auto fetch_row = [&](In& in, int64_t g) {
    const int64_t row = g * RPB + slot;
    const int64_t rl = row < rows ? row : rows - 1;
    fetch_codes<BITS>(codes + rl * (int64_t)ROW_CODE_B + t * LANE_CODE_B, in.cw);
    const uint16_t* sr = scales + rl * (int64_t)NSC;
#pragma unroll
    for (int k = 0; k < NG; ++k) in.hb[k] = SPAN == 1 ? sr[t * NG + k] : sr[t / SPAN];
  };
  // the first row's codes are in flight while the sign masks are built
  In ia;
  if (blockIdx.x < ngroups) fetch_row(ia, blockIdx.x);
  // output sign masks (S and the rho of the DPP butterflies) for the store layout
  uint32_t sw[8], sb[8], m[8];
  int obase[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) obase[c] = G::TWO ? G::idxA(t, c * 8) : t * 64 + c * 8;
  sign_words<8>(sbits, sbits != nullptr, obase, sw);

  sign_bytes_of<8>(sw, obase, sb);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if constexpr (G::TWO) {
      const bool rl = rho_A_lane<LOGN>(t);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (rl ^ rho_A_reg<LOGN>(c * 8 + e)) sb[c] ^= 1u << e;
    } else {
      if (rho_B<LOGN>(t)) sb[c] ^= 0xffu;
    }
    // one word per chunk: the signs of elements 2q and 2q + 1 on bits
    // 15 - q and 31 - q, so (x << q) & 0x80008000 is pair q's mask (8
    // registers instead of 32, room for the next row's codes)
    uint32_t x = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      x |= ((sb[c] >> (2 * q)) & 1u) << (15 - q) | ((sb[c] >> (2 * q + 1)) & 1u) << (31 - q);
    m[c] = x;
  }

  auto do_row = [&](const In& in, int64_t g) {
    const int64_t row = g * RPB + slot;
    float ms[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) ms[k] = (float)__builtin_bit_cast(_Float16, in.hb[k]) * inv_sqrt_n;
    float v[64];
    if constexpr (BITS != 3 && NG == 1) {
      dequant_lane_h64<BITS>(in.cw, ms[0], v);  // index bits 0..5 done
      stages_B<LOGN, 6>(v, t);
    } else {
#pragma unroll
      for (int r = 0; r < 64; ++r) v[r] = (float)code_at<BITS>(in.cw, r) * ms[r / GL];
      stages_B<LOGN, 0>(v, t);
    }
    if constexpr (G::TWO) {
      transpose_BA<LOGN, G::THREADS>(myrow, v, t);
      stages_A<LOGN, false>(v, t);
    }
    // unconditional stores: a slot past the last row writes the last row's
    // bytes again
    uint8_t* orow = out + (row < rows ? row : rows - 1) * ldo_b;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int i = G::TWO ? G::idxA(t, c * 8) : t * 64 + c * 8;
      if constexpr (DOUT == DT_F32) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = as_f(as_u(v[c * 8 + e]) ^ (((sb[c] >> e) & 1u) << 31));
        store8<DT_F32>(orow, i, o);
      } else {
        u32x4 wv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t p = DOUT == DT_BF16 ? pack_bf16(v[c * 8 + 2 * q], v[c * 8 + 2 * q + 1])
                                             : pack_f16(v[c * 8 + 2 * q], v[c * 8 + 2 * q + 1]);
          wv[q] = p ^ ((m[c] << q) & 0x80008000u);
        }
        stg_dq<u32x4>(reinterpret_cast<uint16_t*>(orow) + i, wv);
      }
    }
  };
  // the next row's codes are requested before this row's arithmetic (at
  // n = 8192 they cost the fourth wave per SIMD, and still measured 4 %
  // faster at 28672 rows: the code loads' latency was exposed every row)
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    In ib;
    if (g + gridDim.x < ngroups) fetch_row(ib, g + gridDim.x);
    do_row(ia, g);
    ia = ib;
  }
}

// ------------------------------------------------------------------ dispatch

// 16-bit rows of n = 4096 or 8192 take the matrix-core kernel (rht_quant_mx.hpp).
template <int LOGN, int DIN, int BITS, int LOGG>
static hipError_t run_q_mx(const void* w, int64_t rows, int64_t ldw, const uint32_t* sb, uint8_t* codes,
                           uint16_t* scales, hipStream_t s);

template <int LOGN, int DIN, int BITS, int LOGG>
static hipError_t run_q(const void* w, int64_t rows, int64_t ldw, const uint32_t* sb, uint8_t* codes,
                        uint16_t* scales, hipStream_t s) {
  if constexpr ((LOGN == 12 || LOGN == 13) && DIN != DT_F32)
    return run_q_mx<LOGN, DIN, BITS, LOGG>(w, rows, ldw, sb, codes, scales, s);
  using G = Geo<LOGN>;
  auto k = k_rht_quant<LOGN, DIN, BITS, LOGG>;
  static const int nb = blocks_per_cu(k, G::THREADS, 0);
  const unsigned grid = persistent_grid((rows + G::RPB - 1) / G::RPB, nb);
  hipLaunchKernelGGL(k, dim3(grid), dim3(G::THREADS), 0, s, (const uint8_t*)w, rows,
                     ldw * DtInfo<DIN>::BYTES, sb, codes, scales, (float)(1.0 / __builtin_sqrt((double)(1 << LOGN))));
  return hipGetLastError();
}

template <int LOGN, int BITS, int LOGG, int DOUT>
static hipError_t run_dq(const uint8_t* codes, const uint16_t* scales, int64_t rows, const uint32_t* sb,
                         void* out, int64_t ldo, hipStream_t s) {
  using G = Geo<LOGN>;
  auto k = k_rht_dequant<LOGN, BITS, LOGG, DOUT>;
  static const int nb = blocks_per_cu(k, G::THREADS, 0);
  const unsigned grid = persistent_grid((rows + G::RPB - 1) / G::RPB, nb);
  hipLaunchKernelGGL(k, dim3(grid), dim3(G::THREADS), 0, s, codes, scales, rows, sb, (uint8_t*)out,
                     ldo * DtInfo<DOUT>::BYTES, (float)(1.0 / __builtin_sqrt((double)(1 << LOGN))));
  return hipGetLastError();
}

// Supported instances: n = 2^6 .. 2^13, bits 2/3/4, g = 2^3 .. 2^8 (g <= n).
#define WHTQ_G_CASES(MACRO, L, ...) \
  switch (logg) {                   \
    case 3: MACRO(L, 3, __VA_ARGS__) \
    case 4: MACRO(L, 4, __VA_ARGS__) \
    case 5: MACRO(L, 5, __VA_ARGS__) \
    case 6: MACRO(L, 6, __VA_ARGS__) \
    case 7: if constexpr (L >= 7) { MACRO(L, 7, __VA_ARGS__) } break; \
    case 8: if constexpr (L >= 8) { MACRO(L, 8, __VA_ARGS__) } break; \
    default: break;                 \
  }

template <int L, int DIN, int BITS>
static hipError_t q_logg(int logg, const void* w, int64_t rows, int64_t ldw, const uint32_t* sb,
                         uint8_t* codes, uint16_t* scales, hipStream_t s) {
#define Q_CALL(LL, GG, ...) return run_q<LL, DIN, BITS, GG>(w, rows, ldw, sb, codes, scales, s);
  WHTQ_G_CASES(Q_CALL, L, 0)
#undef Q_CALL
  return hipErrorInvalidValue;
}

template <int L, int DOUT, int BITS>
static hipError_t dq_logg(int logg, const uint8_t* codes, const uint16_t* scales, int64_t rows,
                          const uint32_t* sb, void* out, int64_t ldo, hipStream_t s) {
#define DQ_CALL(LL, GG, ...) return run_dq<LL, BITS, GG, DOUT>(codes, scales, rows, sb, out, ldo, s);
  WHTQ_G_CASES(DQ_CALL, L, 0)
#undef DQ_CALL
  return hipErrorInvalidValue;
}

template <int BITS, int DIN>
static hipError_t q_n(int logn, int logg, const void* w, int64_t rows, int64_t ldw,
                      const uint32_t* sb, uint8_t* codes, uint16_t* scales, hipStream_t s) {
  switch (logn) {
#define QN(L) case L: return q_logg<L, DIN, BITS>(logg, w, rows, ldw, sb, codes, scales, s);
    QN(6) QN(7) QN(8) QN(9) QN(10) QN(11) QN(12) QN(13)
#undef QN
  }
  return hipErrorInvalidValue;
}

template <int BITS, int DOUT>
static hipError_t dq_n(int logn, int logg, const uint8_t* codes, const uint16_t* scales,
                       int64_t rows, const uint32_t* sb, void* out, int64_t ldo, hipStream_t s) {
  switch (logn) {
#define DQN(L) case L: return dq_logg<L, DOUT, BITS>(logg, codes, scales, rows, sb, out, ldo, s);
    DQN(6) DQN(7) DQN(8) DQN(9) DQN(10) DQN(11) DQN(12) DQN(13)
#undef DQN
  }
  return hipErrorInvalidValue;
}

// One translation unit per (direction, bits) instantiates these.
template <int BITS>
hipError_t launch_rht_quant_bits(int logn, int din, int logg, const void* w, int64_t rows, int64_t ldw,
                                 const uint32_t* sb, uint8_t* codes, uint16_t* scales, hipStream_t s) {
  if (din == DT_BF16) return q_n<BITS, DT_BF16>(logn, logg, w, rows, ldw, sb, codes, scales, s);
  if (din == DT_F32) return q_n<BITS, DT_F32>(logn, logg, w, rows, ldw, sb, codes, scales, s);
  if (din == DT_F16) return q_n<BITS, DT_F16>(logn, logg, w, rows, ldw, sb, codes, scales, s);
  return hipErrorInvalidValue;
}

template <int BITS>
hipError_t launch_rht_dequant_bits(int logn, int dout, int logg, const uint8_t* codes, const uint16_t* scales,
                                   int64_t rows, const uint32_t* sb, void* out, int64_t ldo, hipStream_t s) {
  if (dout == DT_BF16) return dq_n<BITS, DT_BF16>(logn, logg, codes, scales, rows, sb, out, ldo, s);
  if (dout == DT_F32) return dq_n<BITS, DT_F32>(logn, logg, codes, scales, rows, sb, out, ldo, s);
  if (dout == DT_F16) return dq_n<BITS, DT_F16>(logn, logg, codes, scales, rows, sb, out, ldo, s);
  return hipErrorInvalidValue;
}

}  // namespace whtq
