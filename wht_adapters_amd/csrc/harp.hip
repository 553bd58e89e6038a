// harp_rotate: y = Stage_2( Stage_1( Stage_0( P x ) ) ), d = 4096 = 16^3.
//
// HARP explainer, 2.1: a mixed-radix schedule with prod b_t = d, each stage a
// block-diagonal orthogonal matrix acting on coordinate groups separated by a
// stride permutation; 2.2: blocks B_{t,c} = Q_{t,c} G (G the normalised
// Sylvester Hadamard), with Theta = 0 (Q = I) giving back the fixed
// randomized Hadamard transform P = Hn S; 2.4: the stages cost O(d log d) and
// are applied by fused kernels without materialising the permutations.
//
// Digit convention: index i = i0 + 16 i1 + 256 i2; stage t acts on digit t;
// its block c is i with digit t removed (remaining digits in increasing
// significance); out_sub[k] = sum_j B[k][j] in_sub[j].
//
// The preconditioning is itself three radix-16 stages: the Sylvester matrix
// factors over the digits, Hn = (G (x) G (x) G) with G = H16 / 4, so P x is
// G applied along each digit after the sign flips.  Every radix-16 stage,
// fixed (G) or learned (B_{t,c}), runs the same way: one 16 x 16 x 16 MFMA
// per block and per tile of 16 tokens, D[k][tok] = sum_j Blk[k][j] X[tok][j].
//
// One workgroup (8 waves) per CU, looping over tiles of 16 tokens kept in
// LDS as fp16 (140 KB with padding):
//   load   each wave takes two token rows: sign flips, and an exact power-of-
//          two scale that puts 64 max |x_i|, a bound on the row's L2 norm, in
//          [2^13, 2^14) (every later value is bounded by that norm, all
//          stages being orthogonal); the
//          rows stay bf16 in the tile and the first G pass (bf16 MFMA) applies
//          the scale to its fp32 result before rounding to fp16; the next
//          tile's rows are fetched meanwhile;
//   passes G along digit 1, G along digit 2, G then B_0 along digit 0
//          (chained MFMAs, G and B_0 act on the same digit), B_1 along digit
//          1, B_2 along digit 2, each reading and writing the tile in place
//          with 8-byte LDS accesses; the last pass unscales and rounds to bf16;
//   store  each wave writes its two rows with 16-byte stores.
// Without preconditioning the G passes and the sign flips are skipped.
#include "io.hpp"
#include "launch.hpp"

namespace whtq {

namespace hp {
constexpr int N = 4096;
constexpr int TT = 16;        // tokens per tile = MFMA N
constexpr int NW = 8;         // waves per workgroup; wave w owns tile rows 2w, 2w+1 for load / store
constexpr int THREADS = NW * 64;
constexpr int RS = 4492;      // row stride in halfwords: >= lay(4095) + 1, RS / 2 = 2 (mod 4)
constexpr int TILE_BYTES = TT * RS * 2;
constexpr int LDS_BYTES = TILE_BYTES + TT * 4;  // + per-token exponents
static_assert(LDS_BYTES <= 160 * 1024, "tile must fit in LDS");
static_assert(TT == 2 * NW, "two rows per wave");
static_assert(RS >= 4096 + 4 * 64 + 4 * 4 && (RS / 2) % 4 == 2, "row stride");
}  // namespace hp

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

// Power-of-two exponent e of a row whose largest magnitude has bf16 bits
// `mb` (wave-uniform): ||x|| <= sqrt(4096) max |x_i| < 2^e, so every value of
// every later stage (all stages are orthogonal) stays below 2^e.  The exact
// maximum cannot overflow or underflow the way a sum of squares in fp32
// would.  e >= -112 keeps the scale 2^(14-e) and its inverse normal fp32
// numbers (a row with max |x_i| < 2^-118 is staged with a smaller scale
// than this bound would allow).
__device__ __forceinline__ int row_exponent(uint32_t mb) {
  const int e = bf16_mag_exp(mb) + 6;
  return mb ? (e > -112 ? e : -112) : 0;
}

// Tile layout (halfwords): row n at n * RS; element i at lay(i), which pads
// 4 halfwords (8 bytes) after every 64 elements and 4 more after every 1024.
// Units of 4 consecutive elements stay contiguous, and lay() is additive over
// disjoint bit fields (lay(a | b) = lay(a) + lay(b) when a & b == 0), so an
// address splits into a lane part and a compile-time group part.  LDS serves
// an 8-byte access 16 lanes at a time over 32 four-byte banks (measured with
// the bank-conflict counter): the 16 lanes of an MFMA operand access are the
// 16 token rows, and RS / 2 = 2 (mod 4) banks per row puts them on distinct
// bank pairs; in the row-contiguous load / store accesses the padding after
// every 64 elements does the same for lanes 8 apart.
__device__ __forceinline__ constexpr int lay(int i) { return i + 4 * (i >> 6) + 4 * (i >> 10); }

__device__ __forceinline__ u32x2 lds_rd8(const uint16_t* tile, int off) {
  return *reinterpret_cast<const u32x2*>(tile + off);
}
__device__ __forceinline__ void lds_wr8(uint16_t* tile, int off, u32x2 v) {
  *reinterpret_cast<u32x2*>(tile + off) = v;
}

__device__ __forceinline__ f16x4_t as_h4(u32x2 v) { return __builtin_bit_cast(f16x4_t, v); }
__device__ __forceinline__ f16x4_t f4_to_h4(f32x4_t a) {
  return f16x4_t{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3]};
}
__device__ __forceinline__ u32x2 h4_bits(f32x4_t d) {
  return u32x2{pack_f16(d[0], d[1]), pack_f16(d[2], d[3])};
}

__device__ __forceinline__ f32x4_t mfma16(f16x4_t a, f16x4_t b) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t mfma16_bf16(u32x2 a, u32x2 b) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                   f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// 4 x 4 transpose of 16-bit values held as four 8-byte rows r[j] = (v[j][0..3]):
// o[a] = (v[0][a], v[1][a], v[2][a], v[3][a]).
__device__ __forceinline__ void tr4x4(const u32x2* r, u32x2* o) {
  constexpr uint32_t LO = 0x05040100u, HI = 0x07060302u;  // v_perm selectors: low / high halves of (s1, s0)
  o[0] = u32x2{__builtin_amdgcn_perm(r[1].x, r[0].x, LO), __builtin_amdgcn_perm(r[3].x, r[2].x, LO)};
  o[1] = u32x2{__builtin_amdgcn_perm(r[1].x, r[0].x, HI), __builtin_amdgcn_perm(r[3].x, r[2].x, HI)};
  o[2] = u32x2{__builtin_amdgcn_perm(r[1].y, r[0].y, LO), __builtin_amdgcn_perm(r[3].y, r[2].y, LO)};
  o[3] = u32x2{__builtin_amdgcn_perm(r[1].y, r[0].y, HI), __builtin_amdgcn_perm(r[3].y, r[2].y, HI)};
}

// A operand of block c of one stage: Blk[m = lane % 16][k = 4 kg .. 4 kg + 3],
// from fp32 blocks (rounded to fp16 here) or fp16 blocks (used as stored).
template <bool F16B> struct Blk;
template <> struct Blk<false> {
  typedef f32x4_t raw;
  static constexpr int STAGE = 65536 * 4;  // bytes per stage
  static __device__ __forceinline__ raw load(const uint8_t* stage, int c, int n, int kg) {
    return ldg_global<f32x4_t>(reinterpret_cast<const float*>(stage) + c * 256 + n * 16 + 4 * kg);
  }
  static __device__ __forceinline__ f16x4_t op(raw r) { return f4_to_h4(r); }
};
template <> struct Blk<true> {
  typedef u32x2 raw;
  static constexpr int STAGE = 65536 * 2;
  static __device__ __forceinline__ raw load(const uint8_t* stage, int c, int n, int kg) {
    return ldg_global<u32x2>(reinterpret_cast<const uint16_t*>(stage) + c * 256 + n * 16 + 4 * kg);
  }
  static __device__ __forceinline__ f16x4_t op(raw r) { return as_h4(r); }
};

// A_G_IN: G on the tile's raw bf16 input (bf16 MFMA, exact operands), the
// row scale applied to the fp32 result before rounding to fp16; A_G: G on the
// fp16 tile; A_BLK: the stage's blocks; A_BLK_LAST: blocks, then unscale and
// round to bf16 for the output.
enum PassA : int { A_G_IN = 0, A_G = 1, A_BLK = 2, A_BLK_LAST = 3 };

// Stage along digit D (1 or 2), in place.  Block c = i0 + 16 v, v the other
// digit; a group is 4 blocks with consecutive i0 = 4e .. 4e + 3, so the
// operand reads are 8-byte rows along i0 transposed in registers.  Wave w
// takes groups 8w .. 8w + 7.
template <int D, int MODE, bool F16B>
__device__ __forceinline__ void pass_dd(uint16_t* tile, const uint8_t* stage, f16x4_t g, u32x2 gb, float us, int w,
                                        int n, int kg) {
  using B = Blk<F16B>;
  constexpr int ST = D == 1 ? 16 : 256;  // stride of the stage's digit
  constexpr int SV = D == 1 ? 256 : 16;  // stride of the other digit
  // element index = ST (4 kg + j) + 4 e + SV v with v = 2w + gi / 4, e = gi % 4;
  // lane part ST 4 kg and wave part SV 2w occupy bit fields disjoint from the rest
  const int wb = n * hp::RS + lay(ST * 4 * kg) + lay(SV * 2 * w);
  typename B::raw an[4];
  if constexpr (MODE >= A_BLK) {
#pragma unroll
    for (int a = 0; a < 4; ++a) an[a] = B::load(stage, a + 32 * w, n, kg);
  }
  // group gi's four 8-byte rows; the next group's rows are read before this
  // group's MFMAs (groups touch disjoint addresses)
  auto off = [&](int gi, int j) { return wb + lay(4 * (gi & 3) + SV * (gi >> 2) + ST * j); };
  u32x2 rn[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) rn[j] = lds_rd8(tile, off(0, j));
#pragma unroll
  for (int gi = 0; gi < 8; ++gi) {
    const int grp = 8 * w + gi;
    typename B::raw ac[4];
    if constexpr (MODE >= A_BLK) {
#pragma unroll
      for (int a = 0; a < 4; ++a) ac[a] = an[a];
      if (gi + 1 < 8) {
        const int g2 = grp + 1;
#pragma unroll
        for (int a = 0; a < 4; ++a) an[a] = B::load(stage, 4 * (g2 & 3) + a + 16 * (g2 >> 2), n, kg);
      }
    }
    u32x2 r[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = rn[j];
    if (gi + 1 < 8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) rn[j] = lds_rd8(tile, off(gi + 1, j));
    }
    tr4x4(r, b);
    u32x2 o[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4_t d;
      if constexpr (MODE == A_G_IN) {
        d = mfma16_bf16(gb, b[a]);
        o[a] = h4_bits(f32x4_t{d[0] * us, d[1] * us, d[2] * us, d[3] * us});
        continue;
      } else {
        d = mfma16(MODE == A_G ? g : B::op(ac[a]), as_h4(b[a]));
      }
      if constexpr (MODE == A_BLK_LAST)
        o[a] = u32x2{pack_bf16(d[0] * us, d[1] * us), pack_bf16(d[2] * us, d[3] * us)};
      else
        o[a] = h4_bits(d);
    }
    tr4x4(o, r);
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_wr8(tile, off(gi, j), r[j]);
  }
}

// Stage along digit 0, in place: block c = i1 + 16 i2 reads one 8-byte row
// per lane.  CHAIN applies G first (the last preconditioning factor) and then
// the stage's block, both along digit 0.  Wave w takes blocks 32w .. 32w + 31.
template <bool CHAIN, bool F16B>
__device__ __forceinline__ void pass_d0(uint16_t* tile, const uint8_t* stage, f16x4_t g, int w, int n, int kg) {
  using B = Blk<F16B>;
  // element index = 4 kg + 16 c with c = 32 w + 4 gi + a: lane, wave and group bit fields are disjoint
  const int wb = n * hp::RS + lay(4 * kg) + lay(512 * w);
  typename B::raw an[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) an[a] = B::load(stage, 32 * w + a, n, kg);
  auto off = [&](int gi, int a) { return wb + lay(64 * gi + 16 * a); };
  u32x2 rn[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) rn[a] = lds_rd8(tile, off(0, a));
#pragma unroll
  for (int gi = 0; gi < 8; ++gi) {
    const int c0 = 32 * w + 4 * gi;
    typename B::raw ac[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) ac[a] = an[a];
    if (gi + 1 < 8) {
#pragma unroll
      for (int a = 0; a < 4; ++a) an[a] = B::load(stage, c0 + 4 + a, n, kg);
    }
    u32x2 r[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) r[a] = rn[a];
    if (gi + 1 < 8) {
#pragma unroll
      for (int a = 0; a < 4; ++a) rn[a] = lds_rd8(tile, off(gi + 1, a));
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f16x4_t bx = as_h4(r[a]);
      if constexpr (CHAIN) bx = f4_to_h4(mfma16(g, bx));
      r[a] = h4_bits(mfma16(B::op(ac[a]), bx));
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) lds_wr8(tile, off(gi, a), r[a]);
  }
}

template <bool F16B>
__global__ __launch_bounds__(hp::THREADS) void k_harp(const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                      int64_t tokens, int64_t ldx, int64_t ldy,
                                                      const uint32_t* __restrict__ sbits, int precondition,
                                                      const uint8_t* __restrict__ blocks) {
  constexpr int SB = Blk<F16B>::STAGE;
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);
  int* texp = reinterpret_cast<int*>(smem + hp::TILE_BYTES);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int64_t ntiles = (tokens + hp::TT - 1) / hp::TT;
  const bool pre = precondition != 0;

  // sign-flip masks for the lane's load columns 8 (lane + 64 r) .. + 7
  uint32_t msk[8][4], sb[8];
  int sbase[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) sbase[r] = 8 * (lane + 64 * r);
  sign_bytes<8>(sbits, pre && sbits != nullptr, sbase, sb);
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) msk[r][q] = pair_mask16(sb[r] >> (2 * q));
  // G = H16 / 4 as the A operand: G[m = n][k = 4 kg + i]
  f16x4_t g;
  uint32_t gbh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool neg = __builtin_popcount(n & (4 * kg + i)) & 1;
    g[i] = neg ? (_Float16)-0.25f : (_Float16)0.25f;
    gbh[i] = neg ? 0xbe80u : 0x3e80u;  // +-0.25 in bf16
  }
  const u32x2 gb = {gbh[0] | (gbh[1] << 16), gbh[2] | (gbh[3] << 16)};

  u32x4 raw[2][8];
  auto fetch = [&](int64_t tl) {
    const int64_t t0 = tl * hp::TT;
    const int nt = (int)min<int64_t>(hp::TT, tokens - t0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint16_t* xr = x + (t0 + min(2 * w + s, nt - 1)) * ldx;
#pragma unroll
      for (int r = 0; r < 8; ++r) raw[s][r] = ldg<u32x4>(xr + 8 * (lane + 64 * r));
    }
  };
  if ((int64_t)blockIdx.x < ntiles) fetch(blockIdx.x);

  for (int64_t tl = blockIdx.x; tl < ntiles; tl += gridDim.x) {
    const int64_t tok0 = tl * hp::TT;
    const int ntok = (int)min<int64_t>(hp::TT, tokens - tok0);

    // ---- load: signs, per-row power-of-two scale, fp16 into the tile
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int row = 2 * w + s;
      u16x2 am{0, 0};
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        u32x4 v = raw[s][r];
        v.x ^= msk[r][0];
        v.y ^= msk[r][1];
        v.z ^= msk[r][2];
        v.w ^= msk[r][3];
        raw[s][r] = v;
        am = absmax16(absmax16(absmax16(absmax16(am, v.x), v.y), v.z), v.w);
      }
      const int e = row_exponent(wave_max_u32(absmax16(am)));
      if (lane == 0) texp[row] = e;
      if (pre) {
        // raw (sign-flipped) bf16: the first G pass reads it with a bf16 MFMA and scales its result
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const u32x4 v = raw[s][r];
          const int o = row * hp::RS + lay(8 * lane) + lay(512 * r);
          lds_wr8(tile, o, u32x2{v.x, v.y});
          lds_wr8(tile, o + 4, u32x2{v.z, v.w});
        }
      } else {
        const float sc = ldexpf(1.0f, 14 - e);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const u32x4 v = raw[s][r];
          const int o = row * hp::RS + lay(8 * lane) + lay(512 * r);
          lds_wr8(tile, o, u32x2{pack_f16(bf16lo(v.x) * sc, bf16hi(v.x) * sc),
                                 pack_f16(bf16lo(v.y) * sc, bf16hi(v.y) * sc)});
          lds_wr8(tile, o + 4, u32x2{pack_f16(bf16lo(v.z) * sc, bf16hi(v.z) * sc),
                                     pack_f16(bf16lo(v.w) * sc, bf16hi(v.w) * sc)});
        }
      }
    }
    if (tl + gridDim.x < ntiles) fetch(tl + gridDim.x);
    __syncthreads();

    // ---- radix-16 stages on MFMA
    // the block operands are re-read from L2 per tile; an opaque copy of the
    // pointer keeps the compiler from hoisting (and spilling) them across tiles
    const uint8_t* bl = blocks;
    asm volatile("" : "+s"(bl));
    if (pre) {
      pass_dd<1, A_G_IN, F16B>(tile, nullptr, g, gb, ldexpf(1.0f, 14 - texp[n]), w, n, kg);
      __syncthreads();
      pass_dd<2, A_G, F16B>(tile, nullptr, g, gb, 1.f, w, n, kg);
      __syncthreads();
      pass_d0<true, F16B>(tile, bl, g, w, n, kg);
    } else {
      pass_d0<false, F16B>(tile, bl, g, w, n, kg);
    }
    __syncthreads();
    pass_dd<1, A_BLK, F16B>(tile, bl + SB, g, gb, 1.f, w, n, kg);
    __syncthreads();
    const float us = ldexpf(1.0f, texp[n] - 14);
    pass_dd<2, A_BLK_LAST, F16B>(tile, bl + 2 * SB, g, gb, us, w, n, kg);
    __syncthreads();

    // ---- store: bf16 rows 2w, 2w + 1
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int row = 2 * w + s;
      if (row < ntok) {
        uint16_t* yr = y + (tok0 + row) * ldy;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int o = row * hp::RS + lay(8 * lane) + lay(512 * r);
          const u32x2 lo = lds_rd8(tile, o), hi = lds_rd8(tile, o + 4);
          stg(yr + 8 * (lane + 64 * r), u32x4{lo.x, lo.y, hi.x, hi.y});
        }
      }
    }
    // the next tile's load writes only rows 2w, 2w + 1, which this wave alone reads here
  }
}

template <bool F16B>
static hipError_t run_harp(const void* x, void* y, int64_t tokens, int64_t ldx, int64_t ldy, const uint32_t* sbits,
                           int precondition, const void* blocks, hipStream_t s) {
  static const bool attr = hipFuncSetAttribute((const void*)k_harp<F16B>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, hp::LDS_BYTES) == hipSuccess;
  (void)attr;
  const int64_t ntiles = (tokens + hp::TT - 1) / hp::TT;
  const unsigned grid = persistent_grid(ntiles, 1);
  hipLaunchKernelGGL(k_harp<F16B>, dim3(grid), dim3(hp::THREADS), hp::LDS_BYTES, s, (const uint16_t*)x,
                     (uint16_t*)y, tokens, ldx, ldy, sbits, precondition, (const uint8_t*)blocks);
  return hipGetLastError();
}

hipError_t launch_harp(const void* x, void* y, int dt, int64_t tokens, int64_t ldx, int64_t ldy,
                       const uint32_t* sbits, int precondition, const void* blocks, int bdt, hipStream_t s) {
  if (dt != DT_BF16) return hipErrorInvalidValue;
  if (bdt == DT_F16) return run_harp<true>(x, y, tokens, ldx, ldy, sbits, precondition, blocks, s);
  if (bdt == DT_F32) return run_harp<false>(x, y, tokens, ldx, ldy, sbits, precondition, blocks, s);
  return hipErrorInvalidValue;
}

}  // namespace whtq
