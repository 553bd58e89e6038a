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
//   4. CSR gather SpMM: 8 lanes per row, up to 8 nonzeros per lane per step
//      with the next row group's first step fetched ahead, 8 fp32
//      accumulators per lane (v_fma_mix with the fp16 column), a DPP
//      reduction over the 8 lanes; each lane stores one token's bf16 output.
#include "io.hpp"
#include "launch.hpp"

namespace whtq {

namespace qw {
constexpr int LOGN = 12;
constexpr int N = 1 << LOGN;
constexpr int TT = 8;                     // tokens per block
constexpr int THREADS = 1024;             // 16 waves (4 transform token rows)
constexpr int NBKT = 512;                 // nnz buckets: ceil(nnz / 8), capped
constexpr int FWAVES = 4;                 // waves that run the token transforms
constexpr int UNROLL = 8;                 // nonzeros per lane per step
}  // namespace qw

// LDS map (bytes):
//   [0, 64K)        Z[k][tok] fp16, 16 B per column      (FWHT scratch before step 2)
//   [64K, 128K)     staging Zt[tok][k] fp16 in steps 1-2; afterwards the
//                   length-sorted row list: id (u16), start (i32), length (u16)
//   [128K, +2K)     bucket counters (uint32)
//   [+2K, +32)      per-token exponent
constexpr int QW_LDS_Z = 0;
constexpr int QW_LDS_Y = 65536;
constexpr int QW_LDS_RID = QW_LDS_Y;
constexpr int QW_LDS_RBEG = QW_LDS_Y + 8192;
constexpr int QW_LDS_RLEN = QW_LDS_Y + 8192 + 16384;
constexpr int QW_LDS_BKT = 131072;
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

  uint16_t* rid = reinterpret_cast<uint16_t*>(smem + QW_LDS_RID);
  int* rbeg = reinterpret_cast<int*>(smem + QW_LDS_RBEG);
  uint16_t* rlen = reinterpret_cast<uint16_t*>(smem + QW_LDS_RLEN);
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
  if (wave < qw::FWAVES) {
    float* scratch = reinterpret_cast<float*>(smem + QW_LDS_Z) + wave * G::LDS_ROW;
    uint16_t* zt = reinterpret_cast<uint16_t*>(smem + QW_LDS_Y);
    const int t = lane;
    const bool rho = rho_B<qw::LOGN>(t);
    int col[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) col[c] = G::idxA(t, c * 8);
    const uint32_t nomask[4] = {0u, 0u, 0u, 0u};
    for (int k = wave; k < qw::TT; k += qw::FWAVES) {
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
    const int beg = row_ptr[o];
    const int len = row_ptr[o + 1] - beg;
    const int b = min((len + 7) >> 3, qw::NBKT - 1);
    const uint32_t pos = atomicAdd(&bkt[qw::NBKT - 1 - b], 1u);
    rid[pos] = (uint16_t)o;
    rbeg[pos] = beg;
    rlen[pos] = (uint16_t)min(len, 65535);
  }
  __syncthreads();

  // ---- 4. gather SpMM: lane octet j of a wave handles sorted row 8*grp + j
  {
    const u32x4* z = reinterpret_cast<const u32x4*>(smem + QW_LDS_Z);
    const int oct = lane >> 3, slot = lane & 7;
    const float osc = ldexpf(1.0f, texp[min(slot, qw::TT - 1)] - 20);  // 2^(e-14) / 64 of token `slot`
    constexpr int NW = qw::THREADS / 64;
    const int ngrp = d_out >> 3;

    // one step = up to UNROLL nonzeros per lane: j = start + slot + 8 u
    struct Step { int c[qw::UNROLL]; float fv[qw::UNROLL]; };
    auto fetch = [&](Step& st, int start, int end) {
#pragma unroll
      for (int u = 0; u < qw::UNROLL; ++u) {
        const int j = start + slot + 8 * u;
        const bool ok = j < end;
        st.c[u] = ok ? col_idx[j] : -1;
        if constexpr (VALDT == DT_BF16)
          st.fv[u] = ok ? bf16lo((uint32_t)reinterpret_cast<const uint16_t*>(vals)[j]) : 0.f;
        else
          st.fv[u] = ok ? reinterpret_cast<const float*>(vals)[j] : 0.f;
      }
    };
    auto consume = [&](const Step& st, float* acc) {
#pragma unroll
      for (int u = 0; u < qw::UNROLL; ++u) {
        if (st.c[u] >= 0) {
          // (copied out as words: subscripting the loaded vector with the
          // unrolled loop index was miscompiled into a single 4-byte read)
          uint32_t zc[4];
          __builtin_memcpy(zc, &z[st.c[u]], 16);
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            fma_mix_lo(acc[2 * p], st.fv[u], zc[p]);
            fma_mix_hi(acc[2 * p + 1], st.fv[u], zc[p]);
          }
        }
      }
    };

    Step cur, nxt;
    int g = wave;
    int pos = g * 8 + oct;
    int beg = g < ngrp ? rbeg[pos] : 0;
    int end = g < ngrp ? beg + rlen[pos] : 0;
    fetch(cur, beg, end);
    for (; g < ngrp; g += NW) {
      const int o = rid[pos];
      // fetch the next group's first step before working on this one
      const int gn = g + NW;
      const int posn = gn * 8 + oct;
      const int begn = gn < ngrp ? rbeg[posn] : 0;
      const int endn = gn < ngrp ? begn + rlen[posn] : 0;
      fetch(nxt, begn, endn);
      float acc[qw::TT];
#pragma unroll
      for (int k = 0; k < qw::TT; ++k) acc[k] = 0.f;
      consume(cur, acc);
      // rows longer than 8 * UNROLL (few after sorting) take more steps
      for (int j0 = beg + 8 * qw::UNROLL; __builtin_amdgcn_ballot_w64(j0 < end); j0 += 8 * qw::UNROLL) {
        Step more;
        fetch(more, j0, end);
        consume(more, acc);
      }
      float mine = 0.f;
#pragma unroll
      for (int k = 0; k < qw::TT; ++k) {
        const float sum = dpp_sum8(acc[k]);
        mine = slot == k ? sum : mine;
      }
      if (slot < ntok)
        y[(tok0 + slot) * ldy + o] = (uint16_t)(pack_bf16(mine * osc, 0.f) & 0xffffu);
      cur = nxt;
      pos = posn;
      beg = begn;
      end = endn;
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
