// rht_lowbit_gemv: y = x W_hat^T for weights stored as the codes and fp16
// scales of rht_quantize_rtn, with the rotation applied to the activations.
//
// HARP explainer, 1 and 2.4: low-bit weights live in the Hadamard-rotated
// basis and the rotation moves onto the activations at inference, in fused
// kernels of O(d log d) cost per token.  With W_hat[o] = S Hn (q[o] s[o]) and
// Hn symmetric,
//     y[t][o] = sum_k q[o][k] s[o][k / g] xr_t[k],   xr_t = Hn (S x_t),
// so the weights are read once, as codes, and never rotated back.
//
// One persistent block of eight waves per CU:
//  1. every wave issues the loads of its first weight row;
//  2. xr_t by a 256-thread FWHT per token (V = n / 256 values per lane:
//     register and quad-DPP butterflies, one LDS transpose, another round of
//     register and DPP butterflies); the DPP butterflies leave a sign on
//     known index bits (RHO), folded in at step 3;
//  3. a power-of-two sigma_t puts max |H S x_t| in [2^14, 2^15) (the 1/sqrt(n)
//     of Hn is applied to the fp32 result); the values
//     are rounded to fp16, each divided by 2^(bits pos) (step 4), and stored
//     in LDS in the order the lanes consume them; every wave copies them into
//     registers (n / 128 per token) and forms its per-group constants;
//  4. weight rows: lane l takes the 16-byte chunks l, l + 64, ... of a row.
//     A code word with its sign bits flipped holds u = q + 2^(bits-1); one
//     and-or onto 0x6400 (fp16 1024.0, ulp 1) turns two fields that sit at
//     mantissa bit bits * pos into the fp16 pair 1024 + u 2^(bits pos), and
//     v_dot2_f32_f16 multiplies it by the stored pair xr 2^-(bits pos): two
//     codes per dot2 and no conversion instruction per code.  The dot's
//     constant part, sum_k h_k (1024 + 2^(bits-1) 2^(bits pos_k)), depends on
//     the lane only and is subtracted once per scale group:
//     y = sum_groups s (acc - corr), summed over the wave by DPP, / sigma.
#pragma once

#include "io.hpp"
#include "launch.hpp"

namespace whtq {

namespace gv {
constexpr int WAVES = 8;
constexpr int THREADS = 64 * WAVES;
constexpr int GT = 256;    // threads of one token's FWHT
constexpr int NGRP = THREADS / GT;
}  // namespace gv

template <int LOGN>
struct GvGeo {
  static constexpr int N = 1 << LOGN;
  static constexpr int LOGV = LOGN - 8;        // FWHT values per thread: 2^4 or 2^5
  static constexpr int V = 1 << LOGV;
  static constexpr int B1 = LOGV + 2;          // index bits of round 1 (registers + quad)
  static constexpr int R2 = LOGN - B1 - LOGV;  // lane bits of round 2 (1 or 2)
  // index bits whose butterflies ran over DPP (upper lane negated)
  static constexpr unsigned RHO = (3u << LOGV) | (((1u << R2) - 1u) << (B1 + LOGV));
  // LDS slot of index i: 4 floats per 32 keep the 16-byte round-1 writes
  // conflict-free, a shift of 64 / 2^R2 banks per round-2 lane block the
  // round-2 reads
  __host__ __device__ static constexpr int pos(int i) {
    return i + ((i >> 5) << 2) + ((i >> (LOGN - R2)) << (6 - R2));
  }
  static constexpr int SCR = (pos(N - 1) + 4) & ~3;  // floats per token slot
  static constexpr int NV = N / 128;                 // fp16-pair registers per token
};

template <int BITS>
struct GvCode {
  static constexpr int CPW = 32 / BITS;     // codes per 32-bit word
  static constexpr int HALF = CPW / 2;      // pairs per word: fields (p, p + HALF)
  static constexpr int CC = 4 * CPW;        // codes per 16-byte chunk
  static constexpr int POSMAX = 10 / BITS;  // fields that fit the fp16 mantissa
  static constexpr int SHIFT = POSMAX * BITS;
  static constexpr uint32_t FIELD = (1u << BITS) - 1u;
  static constexpr uint32_t FLIP = BITS == 2 ? 0xaaaaaaaau : 0x88888888u;
  static constexpr int OFF = 1 << (BITS - 1);
  __host__ __device__ static constexpr int pos_of(int p) { return p < POSMAX ? p : p - POSMAX; }
};

// Sum over the 64 lanes; the result is read from lane 63.
__device__ __forceinline__ float gv_wave_sum(float v) {
  v += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), 0xB1, 0xF, 0xF, true));   // xor 1
  v += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), 0x4E, 0xF, 0xF, true));   // xor 2
  v += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), 0x141, 0xF, 0xF, true));  // half-row mirror
  v += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), 0x140, 0xF, 0xF, true));  // row mirror
  v += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), 0x142, 0xA, 0xF, false)); // row bcast 15
  v += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(v), 0x143, 0xC, 0xF, false)); // row bcast 31
  return as_f((uint32_t)__builtin_amdgcn_readlane((int)as_u(v), 63));
}

__device__ __forceinline__ float gv_wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// x [tn][ldx] bf16 (tn <= TT tokens of this pass), codes [rows][n bits / 8],
// scales [rows][n / g] fp16 bits, y [tn][ldy] bf16.
template <int LOGN, int BITS, int GPC, int TT>
__global__ __launch_bounds__(gv::THREADS) void k_rht_gemv(const uint16_t* __restrict__ x, int tn, int64_t ldx,
                                                          const uint8_t* __restrict__ codes,
                                                          const uint16_t* __restrict__ scales, int64_t rows,
                                                          int logg, const uint32_t* __restrict__ sbits,
                                                          uint16_t* __restrict__ y, int64_t ldy) {
  using G = GvGeo<LOGN>;
  using C = GvCode<BITS>;
  constexpr int N = G::N, V = G::V, NV = G::NV;
  constexpr int CPL = N * BITS / 8192;  // 16-byte chunks per lane per row
  constexpr int RB = N * BITS / 8;      // bytes per code row
  constexpr float RSQRTN = LOGN == 12 ? 0.015625f : 0.011048543456039806f;  // 1 / sqrt(n)
  static_assert(CPL >= 1 && NV == CPL * 4 * C::HALF, "lane layout");
  static_assert(GPC == 1 || GPC == 2 || GPC == 4, "scale groups per chunk");

  __shared__ __align__(16) float scr[gv::NGRP][G::SCR];
  __shared__ __align__(16) uint32_t hl[TT][NV / 4][64][4];
  __shared__ float red[gv::NGRP][4];
  __shared__ float sig_inv[TT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ng = (int)(N >> logg);  // scale groups per row

  // ---- 1. first weight row in flight
  struct Row {
    u32x4 cw[CPL];
    uint32_t sc[CPL][GPC == 4 ? 2 : 1];
  };
  auto fetch = [&](Row& r, int64_t o) {
    const uint8_t* cr = codes + o * RB;
    const uint16_t* sr = scales + o * ng;
#pragma unroll
    for (int j = 0; j < CPL; ++j) r.cw[j] = ldg<u32x4>(cr + (j * 64 + lane) * 16);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int first = ((j * 64 + lane) * C::CC) >> logg;
      if constexpr (GPC == 1) r.sc[j][0] = sr[first];
      else if constexpr (GPC == 2) r.sc[j][0] = ldg<uint32_t>(sr + first);
      else {
        const u32x2 w2 = ldg<u32x2>(sr + first);
        r.sc[j][0] = w2[0];
        r.sc[j][1] = w2[1];
      }
    }
  };
  const int64_t tw = (int64_t)gridDim.x * gv::WAVES;
  int64_t o = (int64_t)blockIdx.x * gv::WAVES + wave;
  Row cur;
  fetch(cur, o < rows ? o : rows - 1);

  // ---- 2./3. rotated activations
  const int grp = tid / gv::GT, g = tid % gv::GT;
#pragma unroll
  for (int tb = 0; tb < TT; tb += gv::NGRP) {
    const int ts = tb + grp;
    const bool act = ts < TT;  // uniform per wave
    float v[V];
    float* sc = scr[grp];
    if (act) {
      if (ts < tn) {
        const uint16_t* xr = x + ts * ldx + g * V;
#pragma unroll
        for (int q = 0; q < V / 8; ++q) {
          const u32x4 w = ldg<u32x4>(xr + 8 * q);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[8 * q + 2 * e] = bf16lo(w[e]);
            v[8 * q + 2 * e + 1] = bf16hi(w[e]);
          }
        }
        if (sbits) {
          const uint32_t sw = V == 32 ? sbits[g] : sbits[g >> 1] >> (16 * (g & 1));
#pragma unroll
          for (int r = 0; r < V; ++r) v[r] = as_f(as_u(v[r]) ^ (((sw >> r) & 1u) << 31));
        }
      } else {
#pragma unroll
        for (int r = 0; r < V; ++r) v[r] = 0.f;
      }
      if constexpr (G::LOGV > 0) reg_stage<V, 0>(v);
      if constexpr (G::LOGV > 1) reg_stage<V, 1>(v);
      if constexpr (G::LOGV > 2) reg_stage<V, 2>(v);
      if constexpr (G::LOGV > 3) reg_stage<V, 3>(v);
      if constexpr (G::LOGV > 4) reg_stage<V, 4>(v);
      lane_stage<V, 0>(v, g);
      lane_stage<V, 1>(v, g);
#pragma unroll
      for (int r = 0; r < V; r += 4)
        *reinterpret_cast<f32x4*>(sc + G::pos(g * V + r)) = f32x4{v[r], v[r + 1], v[r + 2], v[r + 3]};
    }
    __syncthreads();
    auto idx2 = [&](int r) {
      return (g >> G::R2) | (r << G::B1) | ((g & ((1 << G::R2) - 1)) << (G::B1 + G::LOGV));
    };
    if (act) {
#pragma unroll
      for (int r = 0; r < V; ++r) v[r] = sc[G::pos(idx2(r))];
      if constexpr (G::LOGV > 0) reg_stage<V, 0>(v);
      if constexpr (G::LOGV > 1) reg_stage<V, 1>(v);
      if constexpr (G::LOGV > 2) reg_stage<V, 2>(v);
      if constexpr (G::LOGV > 3) reg_stage<V, 3>(v);
      if constexpr (G::LOGV > 4) reg_stage<V, 4>(v);
      lane_stage<V, 0>(v, g);
      if constexpr (G::R2 == 2) lane_stage<V, 1>(v, g);
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < V; ++r) m = fmaxf(m, fabsf(v[r]));
      m = gv_wave_max(m);
      if (lane == 0) red[grp][(g >> 6)] = m;
    }
    __syncthreads();
    if (act) {
      const float mx = fmaxf(fmaxf(red[grp][0], red[grp][1]), fmaxf(red[grp][2], red[grp][3]));
      // sigma = 2^(14 - e) with max = f 2^e, f in [1, 2); 1 for an all-zero
      // or non-finite token
      // (at most 2^126, so that 1 / sigma stays a normal fp32 number)
      int e = 0;
      const bool fin = mx > 0.f && __builtin_isfinite(mx);
      if (fin) e = ((int)((as_u(mx) >> 23) & 0xffu)) - 127;
      const int se = fin ? (14 - e < 126 ? 14 - e : 126) : 0;
      uint16_t* hh = reinterpret_cast<uint16_t*>(&hl[ts][0][0][0]);
#pragma unroll
      for (int r = 0; r < V; ++r) {
        const int i = idx2(r);
        const int c = i / C::CC, rem = i % C::CC;
        const int l = c & 63, j = c >> 6;
        const int w = rem / C::CPW, f = rem % C::CPW;
        const int half = f / C::HALF, p = f % C::HALF;
        const int vr = (j * 4 + w) * C::HALF + p;
        const int pp = p < C::POSMAX ? p : p - C::POSMAX;
        const float sgn = (__builtin_popcount((unsigned)i & G::RHO) & 1) ? -1.f : 1.f;
        const float hv = ldexpf(v[r] * sgn, se - BITS * pp);
        hh[(((vr >> 2) * 64 + l) * 4 + (vr & 3)) * 2 + half] = __builtin_bit_cast(uint16_t, (_Float16)hv);
      }
      if (g == 0) sig_inv[ts] = ldexpf(1.f, -se);
    }
    __syncthreads();
  }

  // every wave's copy of the rotated activations, and its constants
  uint32_t h[TT][NV];
  float corr[TT][CPL][GPC];
  float sinv[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    sinv[t] = sig_inv[t];
#pragma unroll
    for (int q = 0; q < NV / 4; ++q) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(&hl[t][q][lane][0]);
      h[t][4 * q] = w[0];
      h[t][4 * q + 1] = w[1];
      h[t][4 * q + 2] = w[2];
      h[t][4 * q + 3] = w[3];
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int gp = 0; gp < GPC; ++gp) {
        float a = 0.f;
#pragma unroll
        for (int w = gp * 4 / GPC; w < (gp + 1) * 4 / GPC; ++w)
#pragma unroll
          for (int p = 0; p < C::HALF; ++p) {
            const f16x2_t hp = __builtin_bit_cast(f16x2_t, h[t][(j * 4 + w) * C::HALF + p]);
            const float k = (float)(1024 + C::OFF * (1 << (BITS * C::pos_of(p))));
            a = fmaf((float)hp[0], k, a);
            a = fmaf((float)hp[1], k, a);
          }
        corr[t][j][gp] = a;
      }
  }

  // ---- 4. weight rows
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));
  for (; o < rows; o += tw) {
    Row nxt;
    const int64_t on = o + tw;
    fetch(nxt, on < rows ? on : rows - 1);
    float ya[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) ya[t] = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float acc[TT][GPC];
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int gp = 0; gp < GPC; ++gp) acc[t][gp] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int gp = w * GPC / 4;
        const uint32_t u = cur.cw[j][w] ^ C::FLIP;
        const uint32_t u2 = u >> C::SHIFT;
#pragma unroll
        for (int p = 0; p < C::HALF; ++p) {
          const uint32_t mask = (C::FIELD << (BITS * C::pos_of(p))) * 0x10001u;
          const uint32_t b = ((p < C::POSMAX ? u : u2) & mask) | magic;
#pragma unroll
          for (int t = 0; t < TT; ++t)
            acc[t][gp] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, b),
                                                __builtin_bit_cast(f16x2_t, h[t][(j * 4 + w) * C::HALF + p]),
                                                acc[t][gp], false);
        }
      }
#pragma unroll
      for (int gp = 0; gp < GPC; ++gp) {
        const uint32_t sw = GPC == 1 ? cur.sc[j][0] : cur.sc[j][gp >> 1] >> (16 * (gp & 1));
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(sw & 0xffffu));
#pragma unroll
        for (int t = 0; t < TT; ++t) ya[t] = fmaf(s, acc[t][gp] - corr[t][j][gp], ya[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float tot = gv_wave_sum(ya[t]) * RSQRTN * sinv[t];
      if (t < tn && lane == 0) y[t * ldy + o] = __builtin_bit_cast(uint16_t, (__bf16)tot);
    }
    cur = nxt;
  }
}

template <int LOGN, int BITS, int GPC, int TT>
static hipError_t run_gemv(const void* x, int tn, int64_t ldx, const uint8_t* codes, const uint16_t* scales,
                           int64_t rows, int logg, const uint32_t* sb, void* y, int64_t ldy, hipStream_t s) {
  auto k = k_rht_gemv<LOGN, BITS, GPC, TT>;
  // one block per CU: every block rotates the activations itself
  const unsigned grid = persistent_grid((rows + gv::WAVES - 1) / gv::WAVES, 1);
  hipLaunchKernelGGL(k, dim3(grid), dim3(gv::THREADS), 0, s, (const uint16_t*)x, tn, ldx, codes, scales, rows,
                     logg, sb, (uint16_t*)y, ldy);
  return hipGetLastError();
}

template <int LOGN, int BITS, int TT>
static hipError_t gemv_gpc(const void* x, int tn, int64_t ldx, const uint8_t* codes, const uint16_t* scales,
                           int64_t rows, int logg, const uint32_t* sb, void* y, int64_t ldy, hipStream_t s) {
  constexpr int LOGCC = BITS == 2 ? 6 : 5;  // log2 codes per 16-byte chunk
  const int gpc_log = logg >= LOGCC ? 0 : LOGCC - logg;
  switch (gpc_log) {
    case 0: return run_gemv<LOGN, BITS, 1, TT>(x, tn, ldx, codes, scales, rows, logg, sb, y, ldy, s);
    case 1: return run_gemv<LOGN, BITS, 2, TT>(x, tn, ldx, codes, scales, rows, logg, sb, y, ldy, s);
    case 2: return run_gemv<LOGN, BITS, 4, TT>(x, tn, ldx, codes, scales, rows, logg, sb, y, ldy, s);
  }
  return hipErrorInvalidValue;
}

// Tokens go in passes of up to 4 (n = 4096) or 2 (n = 8192): each pass holds
// its rotated activations in registers (n / 128 per token) and reads the
// weights once.
template <int BITS>
hipError_t launch_rht_gemv_bits(int logn, int logg, const void* x, int64_t tokens, int64_t ldx,
                                const uint8_t* codes, const uint16_t* scales, int64_t rows, const uint32_t* sb,
                                void* y, int64_t ldy, hipStream_t s) {
  const int ttmax = logn == 12 ? 4 : 2;
  for (int64_t t0 = 0; t0 < tokens; t0 += ttmax) {
    const int tn = (int)std::min<int64_t>(ttmax, tokens - t0);
    const uint16_t* xp = (const uint16_t*)x + t0 * ldx;
    uint16_t* yp = (uint16_t*)y + t0 * ldy;
    hipError_t e = hipErrorInvalidValue;
    if (logn == 12) {
      if (tn == 1) e = gemv_gpc<12, BITS, 1>(xp, tn, ldx, codes, scales, rows, logg, sb, yp, ldy, s);
      else if (tn == 2) e = gemv_gpc<12, BITS, 2>(xp, tn, ldx, codes, scales, rows, logg, sb, yp, ldy, s);
      else e = gemv_gpc<12, BITS, 4>(xp, tn, ldx, codes, scales, rows, logg, sb, yp, ldy, s);
    } else if (logn == 13) {
      if (tn == 1) e = gemv_gpc<13, BITS, 1>(xp, tn, ldx, codes, scales, rows, logg, sb, yp, ldy, s);
      else e = gemv_gpc<13, BITS, 2>(xp, tn, ldx, codes, scales, rows, logg, sb, yp, ldy, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace whtq
