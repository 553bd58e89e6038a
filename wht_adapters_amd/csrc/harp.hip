// harp_rotate: y = Stage_2( Stage_1( Stage_0( P x ) ) ), d = 4096 = 16^3.
//
// HARP explainer, 2.1: a mixed-radix schedule with prod b_t = d, each stage a
// block-diagonal orthogonal matrix acting on coordinate groups separated by a
// stride permutation; 2.2: blocks B_{t,c} = Q_{t,c} G (G the normalised
// Sylvester Hadamard), and the random-sign Hadamard preconditioning P = Hn S
// in front; 2.4: the stages cost O(d log d) and are applied by fused kernels
// without materialising the permutations.
//
// Digit convention: index i = i0 + 16 i1 + 256 i2; stage t acts on digit t;
// its block c is i with digit t removed (remaining digits in increasing
// significance); out_sub[k] = sum_j B[k][j] in_sub[j].
//
// One block per tile of 15 tokens, all of it kept on chip:
//   1. P x: each wave transforms one token row at a time with the fp32
//      register / LDS FWHT engine; the row is scaled by an exact power of two
//      that puts its L2 norm in [2^13, 2^14) (every later value is bounded by
//      that norm, the stages being orthogonal) and stored to the fp16 tile;
//   2. each stage: for every 16 x 16 block, one MFMA
//      D[n][tok] = sum_k B[n][k] X[tok][idx(c, k)] (fp16 operands, fp32
//      accumulation), read from and written back to the tile in place;
//   3. the tile is unscaled, rounded to bf16 and written with 16-byte stores.
#include "io.hpp"
#include "launch.hpp"

namespace whtq {

namespace hp {
constexpr int LOGN = 12;
constexpr int N = 1 << LOGN;
constexpr int TT = 15;        // tokens per tile (the 16th MFMA column is a duplicate)
constexpr int THREADS = 512;  // 8 waves (4 run the preconditioning transforms)
constexpr int FWAVES = 4;
constexpr int TILE_BYTES = TT * N * 2;
constexpr int SCRATCH_BYTES = 4 * Geo<LOGN>::LDS_ROW * 4;
constexpr int LDS_BYTES = TILE_BYTES + SCRATCH_BYTES + 4 * 16;  // + per-token exponents
static_assert(LDS_BYTES <= 160 * 1024, "tile + scratch must fit in LDS");
}  // namespace hp

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

// power-of-two scale for a row with squared norm `ss` (wave-uniform)
__device__ __forceinline__ int row_exponent(float ss) {
  int e = 0;
  if (ss > 0.f) (void)frexpf(__builtin_sqrtf(ss), &e);  // ||z|| = m 2^e, m in [0.5, 1)
  return e;
}

__device__ __forceinline__ float wave_sum(float a) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) a += __shfl_xor(a, s);
  return a;
}

// Tile layout: token row r at r * 4096 halves, element i stored at
// i ^ (r << 3): whole 16-byte chunks are permuted per row, so row-contiguous
// 16-byte accesses stay contiguous while the 64 lanes of a stage access
// (16 tokens x 4 digit groups, same offset in every row) spread over the LDS
// banks instead of all hitting one.
__device__ __forceinline__ int tsw(int row, int i) { return i ^ (row << 3); }

// element index of digit value k in block c of stage t (stride 16^t)
__device__ __forceinline__ int harp_idx(int t, int c, int k) {
  const int st = 1 << (4 * t);
  return (c & (st - 1)) + k * st + (c >> (4 * t)) * (st << 4);
}

__global__ __launch_bounds__(hp::THREADS) void k_harp(const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                      int64_t tokens, int64_t ldx, int64_t ldy,
                                                      const uint32_t* __restrict__ sbits, int precondition,
                                                      const float* __restrict__ blocks) {
  using G = Geo<hp::LOGN>;
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);
  float* scratch = reinterpret_cast<float*>(smem + hp::TILE_BYTES);
  int* texp = reinterpret_cast<int*>(smem + hp::TILE_BYTES + hp::SCRATCH_BYTES);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t ntiles = (tokens + hp::TT - 1) / hp::TT;

  // per-lane sign masks for the engine's load layout
  int col[8];
  uint32_t sb[8], m[8][4];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    col[c] = G::idxA(lane, c * 8);
    sb[c] = sbits ? sign_byte(sbits, col[c]) : 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) m[c][q] = pair_mask16(sb[c] >> (2 * q));
  }
  const float cs = rho_B<hp::LOGN>(lane) ? -1.0f / 64.0f : 1.0f / 64.0f;
  float* myscr = scratch + wave * G::LDS_ROW;

  for (int64_t tl = blockIdx.x; tl < ntiles; tl += gridDim.x) {
    const int64_t tok0 = tl * hp::TT;
    const int ntok = (int)min<int64_t>(hp::TT, tokens - tok0);

    // ---- 1. preconditioning (or plain copy) into the fp16 tile
    for (int k = wave; wave < hp::FWAVES && k < hp::TT; k += hp::FWAVES) {
      const uint16_t* xr = x + (tok0 + min(k, ntok - 1)) * ldx;
      uint16_t* trow = tile + k * hp::N;
      float v[64];
      if (precondition) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          Raw8 raw;
          fetch8<DT_BF16>(xr, col[c], raw);
          widen8<DT_BF16, true>(raw, v + 8 * c, m[c], sb[c]);
        }
        stages_A<hp::LOGN, false>(v, lane);
        transpose_AB<hp::LOGN, 64>(myscr, v, lane);
        stages_B<hp::LOGN, 2>(v, lane);
#pragma unroll
        for (int r = 0; r < 64; ++r) v[r] *= cs;
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(xr + lane * 64 + 8 * q);
          const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            v[8 * q + 2 * p] = bf16lo(wv[p]);
            v[8 * q + 2 * p + 1] = bf16hi(wv[p]);
          }
        }
      }
      float ss = 0.f;
#pragma unroll
      for (int r = 0; r < 64; ++r) ss = __builtin_fmaf(v[r], v[r], ss);
      const int e = row_exponent(wave_sum(ss));
      const float sc = ldexpf(1.0f, 14 - e);
      if (lane == 0) texp[k] = e;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) w[p] = pack_f16(v[8 * q + 2 * p] * sc, v[8 * q + 2 * p + 1] * sc);
        *reinterpret_cast<u32x4*>(trow + tsw(k, lane * 64 + 8 * q)) = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
    __syncthreads();

    // ---- 2. three radix-16 stages on MFMA
    // lane l: token l % 16 (column 15 duplicates row 14), k-group l / 16
    const int tcol = lane & 15, kg = lane >> 4;
    const int rrd = min(tcol, hp::TT - 1);
    const uint16_t* trd = tile + rrd * hp::N;
    uint16_t* twr = tile + tcol * hp::N;
    constexpr int NW = hp::THREADS / 64;
    for (int t = 0; t < 3; ++t) {
      const float* bt = blocks + (size_t)t * 256 * 256 + tcol * 16 + 4 * kg;
      // A operand of block c: B_{t,c}[n = l % 16][k = 4 kg .. 4 kg + 3], fetched one block ahead
      float bw[4];
      __builtin_memcpy(bw, bt + wave * 256, 16);
      for (int c = wave; c < 256; c += NW) {
        const f16x4_t a = {(_Float16)bw[0], (_Float16)bw[1], (_Float16)bw[2], (_Float16)bw[3]};
        if (c + NW < 256) __builtin_memcpy(bw, bt + (c + NW) * 256, 16);
        // B operand: X[tok][idx(c, k)], k = 4 kg .. 4 kg + 3
        uint16_t bh[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bh[i] = trd[tsw(rrd, harp_idx(t, c, 4 * kg + i))];
        f16x4_t b;
        __builtin_memcpy(&b, bh, 8);
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
        d = __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, d, 0, 0, 0);
        float dd[4];
        __builtin_memcpy(dd, &d, 16);
        // D[n = 4 kg + i][tok = l % 16]
        if (tcol < hp::TT) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            twr[tsw(tcol, harp_idx(t, c, 4 * kg + i))] = (uint16_t)(pack_f16(dd[i], 0.f) & 0xffffu);
        }
      }
      __syncthreads();
    }

    // ---- 3. unscale, round to bf16, write the tile
    for (int i = tid; i < ntok * (hp::N / 8); i += hp::THREADS) {
      const int k = i / (hp::N / 8), q = i - k * (hp::N / 8);
      const float us = ldexpf(1.0f, texp[k] - 14);
      uint32_t w[4];
      __builtin_memcpy(w, tile + k * hp::N + tsw(k, 8 * q), 16);
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const f16x2_t h = __builtin_bit_cast(f16x2_t, w[p]);
        o[p] = pack_bf16((float)h[0] * us, (float)h[1] * us);
      }
      *reinterpret_cast<u32x4*>(y + (tok0 + k) * ldy + 8 * q) = u32x4{o[0], o[1], o[2], o[3]};
    }
    __syncthreads();
  }
}

hipError_t launch_harp(const void* x, void* y, int dt, int64_t tokens, int64_t ldx, int64_t ldy,
                       const uint32_t* sbits, int precondition, const float* blocks, hipStream_t s) {
  if (dt != DT_BF16) return hipErrorInvalidValue;
  static const bool attr = hipFuncSetAttribute((const void*)k_harp, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               hp::LDS_BYTES) == hipSuccess;
  (void)attr;
  const int64_t ntiles = (tokens + hp::TT - 1) / hp::TT;
  int dev = 0;
  (void)hipGetDevice(&dev);
  const unsigned grid = (unsigned)std::min<int64_t>(ntiles, (int64_t)device_cu_count(dev));
  hipLaunchKernelGGL(k_harp, dim3(grid), dim3(hp::THREADS), hp::LDS_BYTES, s, (const uint16_t*)x,
                     (uint16_t*)y, tokens, ldx, ldy, sbits, precondition, blocks);
  return hipGetLastError();
}

}  // namespace whtq
