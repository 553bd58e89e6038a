// qwha_adapter_forward: y = (x Hn) F^T with F sparse (CSR), d_in = 4096.
//
// QWHA explainer, 2.1: the adapter is Delta W = F H^-1, one Walsh-Hadamard
// transform on the input side and a sparse coefficient matrix F built from a
// value vector and an index list; with the orthonormal Hn this is
// y = x Delta W^T = (x Hn) F^T.
//
// One block per tile of 8 tokens:
//   1. each wave transforms one token row at a time with the register / LDS
//      FWHT engine (fp32); the row is scaled by an exact power of two so its
//      largest entry sits near 2^14, rounded to fp16 and staged token-major;
//   2. the staged tile is re-laid out to Z[k][8 tokens] (16 bytes per
//      column), so one ds_read_b128 returns a column for all 8 tokens;
//   3. rows of F are bucketed by their nnz (ceil(nnz / 8)) so that the 8 rows
//      a wave handles together need about the same number of iterations;
//   4. CSR gather SpMM: 8 lanes per row, one nonzero per lane per iteration,
//      8 fp32 accumulators per lane (v_fma_mix with the fp16 column), a DPP
//      reduction over the 8 lanes, and the bf16 result staged in LDS;
//   5. the 8 x d_out tile is written with 16-byte stores.
#include "io.hpp"
#include "launch.hpp"

namespace whtq {

namespace qw {
constexpr int LOGN = 12;
constexpr int N = 1 << LOGN;
constexpr int TT = 8;                     // tokens per block
constexpr int THREADS = 256;              // 4 waves
constexpr int NBKT = 512;                 // nnz buckets: ceil(nnz / 8), capped
}  // namespace qw

// LDS map (bytes):
//   [0, 64K)        Z[k][tok] fp16, 16 B per column      (FWHT scratch before step 2)
//   [64K, 128K)     staging Zt[tok][k] fp16 in steps 1-2, then Y[tok][o] bf16
//   [128K, +8K)     sorted row ids (uint16)
//   [+8K, +2K)      bucket counters (uint32)
//   [+2K, +32)      per-token exponent
constexpr int QW_LDS_Z = 0;
constexpr int QW_LDS_Y = 65536;
constexpr int QW_LDS_ORDER = 131072;
constexpr int QW_LDS_BKT = QW_LDS_ORDER + 8192;
constexpr int QW_LDS_EXP = QW_LDS_BKT + 4 * qw::NBKT;
constexpr int QW_LDS_BYTES = QW_LDS_EXP + 4 * qw::TT;

__device__ __forceinline__ float dpp_sum8(float x) {
  // sum over the 8 lanes of an aligned lane octet; every lane gets the total
  x += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0xB1, 0xF, 0xF, true));   // ^1
  x += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0x4E, 0xF, 0xF, true));   // ^2
  x += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
  return x;
}

template <int VALDT>
__global__ __launch_bounds__(qw::THREADS) void k_qwha(const uint16_t* __restrict__ x, int64_t tokens,
                                                      int64_t ldx, const int32_t* __restrict__ row_ptr,
                                                      const int32_t* __restrict__ col_idx,
                                                      const void* __restrict__ vals, int d_out,
                                                      uint16_t* __restrict__ y, int64_t ldy) {
  using G = Geo<qw::LOGN>;
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tok0 = (int64_t)blockIdx.x * qw::TT;
  const int ntok = (int)min<int64_t>(qw::TT, tokens - tok0);

  uint16_t* order = reinterpret_cast<uint16_t*>(smem + QW_LDS_ORDER);
  uint32_t* bkt = reinterpret_cast<uint32_t*>(smem + QW_LDS_BKT);
  int* texp = reinterpret_cast<int*>(smem + QW_LDS_EXP);

  // ---- 3a. bucket histogram of row lengths (overlaps with the transforms)
  for (int i = tid; i < qw::NBKT; i += qw::THREADS) bkt[i] = 0;
  __syncthreads();
  for (int o = tid; o < d_out; o += qw::THREADS) {
    const int len = row_ptr[o + 1] - row_ptr[o];
    const int b = min((len + 7) >> 3, qw::NBKT - 1);
    atomicAdd(&bkt[qw::NBKT - 1 - b], 1u);  // longest rows first
  }

  // ---- 1. FWHT of the token rows, staged as fp16 token-major
  {
    float* scratch = reinterpret_cast<float*>(smem + QW_LDS_Z) + wave * G::LDS_ROW;
    uint16_t* zt = reinterpret_cast<uint16_t*>(smem + QW_LDS_Y);
    const int t = lane;
    const bool rho = rho_B<qw::LOGN>(t);
    int col[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) col[c] = G::idxA(t, c * 8);
    const uint32_t nomask[4] = {0u, 0u, 0u, 0u};
    for (int k = wave; k < qw::TT; k += qw::THREADS / 64) {
      const int64_t tok = tok0 + min(k, ntok - 1);  // tail tokens recompute the last one
      const uint16_t* xr = x + tok * ldx;
      float v[64];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        Raw8 raw;
        fetch8<DT_BF16>(xr, col[c], raw);
        widen8<DT_BF16, false>(raw, v + 8 * c, nomask, 0u);
      }
      stages_A<qw::LOGN, false>(v, t);
      transpose_AB<qw::LOGN, 64>(scratch, v, t);
      stages_B<qw::LOGN, 2>(v, t);
      // exact power-of-two scale putting max |z| in [2^13, 2^14)
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 64; r += 2) a4[(r >> 1) & 3] = max3abs(a4[(r >> 1) & 3], v[r], v[r + 1]);
      float a = fmaxf(fmaxf(a4[0], a4[1]), fmaxf(a4[2], a4[3]));
#pragma unroll
      for (int s = 1; s < 64; s <<= 1) a = fmaxf(a, __shfl_xor(a, s));
      int e = 0;
      if (a > 0.f) (void)frexpf(a, &e);       // a = m 2^e, m in [0.5, 1)
      const float mult = ldexpf(rho ? -1.0f : 1.0f, 14 - e);
      if (lane == 0) texp[k] = e;
      uint16_t* zrow = zt + k * qw::N + t * 64;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        u32x4 w;
#pragma unroll
        for (int p = 0; p < 4; ++p) w[p] = pack_f16(v[8 * q + 2 * p] * mult, v[8 * q + 2 * p + 1] * mult);
        *reinterpret_cast<u32x4*>(zrow + 8 * q) = w;
      }
    }
  }
  __syncthreads();

  // ---- 2. Zt[tok][k] -> Z[k][tok]
  {
    const uint16_t* zt = reinterpret_cast<const uint16_t*>(smem + QW_LDS_Y);
    u32x4* z = reinterpret_cast<u32x4*>(smem + QW_LDS_Z);
    for (int kk = tid; kk < qw::N; kk += qw::THREADS) {
      uint32_t h[qw::TT];
#pragma unroll
      for (int k = 0; k < qw::TT; ++k) h[k] = zt[k * qw::N + kk];
      z[kk] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
  }
  // ---- 3b. bucket offsets (one wave), then scatter row ids
  if (wave == 0) {
    uint32_t run = 0;
    for (int base = 0; base < qw::NBKT; base += 64) {
      const uint32_t c = bkt[base + lane];
      uint32_t incl = c;
#pragma unroll
      for (int s = 1; s < 64; s <<= 1) {
        const uint32_t o = __shfl_up(incl, s);
        if (lane >= s) incl += o;
      }
      bkt[base + lane] = run + incl - c;
      run += __shfl(incl, 63);
    }
  }
  __syncthreads();
  for (int o = tid; o < d_out; o += qw::THREADS) {
    const int len = row_ptr[o + 1] - row_ptr[o];
    const int b = min((len + 7) >> 3, qw::NBKT - 1);
    const uint32_t pos = atomicAdd(&bkt[qw::NBKT - 1 - b], 1u);
    order[pos] = (uint16_t)o;
  }
  __syncthreads();

  // ---- 4. gather SpMM: lane octet j of a wave handles row order[8*grp + j]
  {
    const u32x4* z = reinterpret_cast<const u32x4*>(smem + QW_LDS_Z);
    uint16_t* yl = reinterpret_cast<uint16_t*>(smem + QW_LDS_Y);
    const int oct = lane >> 3, slot = lane & 7;
    float osc[qw::TT];
#pragma unroll
    for (int k = 0; k < qw::TT; ++k) osc[k] = ldexpf(1.0f, texp[k] - 20);  // 2^(e-14) / 64
    const int ngrp = (d_out + 7) >> 3;
    for (int grp = wave; grp < ngrp; grp += qw::THREADS / 64) {
      const int oi = grp * 8 + oct;
      const bool live = oi < d_out;
      const int o = live ? order[oi] : 0;
      const int beg = live ? row_ptr[o] : 0;
      const int end = live ? row_ptr[o + 1] : 0;
      float acc[qw::TT];
#pragma unroll
      for (int k = 0; k < qw::TT; ++k) acc[k] = 0.f;
      for (int j = beg + slot; __builtin_amdgcn_ballot_w64(j < end); j += 8) {
        if (j < end) {
          const int c = col_idx[j];
          float fv;
          if constexpr (VALDT == DT_BF16) fv = bf16lo((uint32_t)reinterpret_cast<const uint16_t*>(vals)[j]);
          else fv = reinterpret_cast<const float*>(vals)[j];
          // (copied out as words: subscripting the loaded vector with the
          // unrolled loop index was miscompiled into a single 4-byte read)
          uint32_t zc[4];
          __builtin_memcpy(zc, &z[c], 16);
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            fma_mix_lo(acc[2 * p], fv, zc[p]);
            fma_mix_hi(acc[2 * p + 1], fv, zc[p]);
          }
        }
      }
      float mine = 0.f;
#pragma unroll
      for (int k = 0; k < qw::TT; ++k) {
        const float s = dpp_sum8(acc[k]);
        mine = slot == k ? s : mine;
      }
      if (live && slot < ntok) {
        const float yv = mine * osc[slot];
        yl[slot * qw::N + o] = (uint16_t)(pack_bf16(yv, 0.f) & 0xffffu);
      }
    }
  }
  __syncthreads();

  // ---- 5. write the tile
  {
    const uint16_t* yl = reinterpret_cast<const uint16_t*>(smem + QW_LDS_Y);
    const int per_row = d_out >> 3;  // 16-byte chunks per token row (d_out % 8 == 0)
    for (int i = tid; i < ntok * per_row; i += qw::THREADS) {
      const int k = i / per_row, q = i - k * per_row;
      *reinterpret_cast<u32x4*>(y + (tok0 + k) * ldy + 8 * q) =
          *reinterpret_cast<const u32x4*>(yl + k * qw::N + 8 * q);
    }
  }
}

hipError_t launch_qwha(const void* x, int64_t tokens, int64_t ldx, const int32_t* row_ptr,
                       const int32_t* col_idx, const void* vals, int val_dt, int64_t d_out, void* y,
                       int64_t ldy, hipStream_t s) {
  const unsigned grid = (unsigned)((tokens + qw::TT - 1) / qw::TT);
  if (val_dt == DT_BF16) {
    static const bool attr = hipFuncSetAttribute((const void*)k_qwha<DT_BF16>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 QW_LDS_BYTES) == hipSuccess;
    (void)attr;
    hipLaunchKernelGGL(k_qwha<DT_BF16>, dim3(grid), dim3(qw::THREADS), QW_LDS_BYTES, s,
                       (const uint16_t*)x, tokens, ldx, row_ptr, col_idx, vals, (int)d_out,
                       (uint16_t*)y, ldy);
  } else {
    static const bool attr = hipFuncSetAttribute((const void*)k_qwha<DT_F32>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 QW_LDS_BYTES) == hipSuccess;
    (void)attr;
    hipLaunchKernelGGL(k_qwha<DT_F32>, dim3(grid), dim3(qw::THREADS), QW_LDS_BYTES, s,
                       (const uint16_t*)x, tokens, ldx, row_ptr, col_idx, vals, (int)d_out,
                       (uint16_t*)y, ldy);
  }
  return hipGetLastError();
}

}  // namespace whtq
