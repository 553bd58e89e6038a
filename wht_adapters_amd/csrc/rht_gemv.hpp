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
// One persistent block per CU:
//  1. the token rows are requested first, then every wave puts its first
//     weight row in flight (a CU returns vector loads in order, so the
//     transform below does not wait for the weights);
//  2. H S x_t by 4096-point jobs of 256 threads (16 values per lane:
//     register and quad-DPP butterflies, one LDS transpose, another round);
//     n = 8192 splits a token on its top index bit into the jobs lo + hi
//     and lo - hi.  The DPP butterflies leave a sign on known index bits
//     (RHO), folded in when the values go to LDS with the token's maximum;
//  3. fixed point: a power-of-two sigma_t puts max |H S x_t| sigma_t in
//     [2^13, 2^14) and X = rint(H S x_t sigma_t) is written as four signed
//     base-16 digits, X = d0 + 16 d1 + 256 d2 + 4096 d3 (d in [-8, 7]:
//     the nibbles of ((X + 0x8888) xor 0x8888)).  Digit p of eight codes'
//     X makes one 32-bit "limb word"; the limb words go to LDS in the order
//     the lanes consume them and every wave copies them into registers
//     (n / 128 per token).  The 1/sqrt(n) of Hn and 1/sigma are applied to
//     the fp32 result;
//  4. weight rows: lane l takes the 16-byte chunks l, l + 64, ... of a row.
//     v_dot8_i32_i4 multiplies eight signed nibbles by eight signed nibbles:
//     4-bit codes are such nibbles as stored; a word of sixteen 2-bit codes,
//     its sign bits flipped to offset binary u = q + 2, splits into the even
//     and odd codes' nibbles with two masks.  One dot8 per limb and eight
//     codes, exact int32 sums per scale group, acc = sum_p 16^p acc_p minus
//     2 sum X for the offset, then y += s (float) acc; summed over the wave
//     by DPP and scaled by 1 / (sigma sqrt(n)).
#pragma once

#include "io.hpp"
#include "launch.hpp"

namespace whtq {

namespace gv {
constexpr int GT = 256;  // threads of one 4096-point transform job
constexpr int PF = 1;    // weight rows in flight per wave while one is consumed
// LDS slot of transform index i: 4 floats per 32 keep the 16-byte round-1
// writes conflict-free, 16 more per 1024 the round-2 reads
__host__ __device__ constexpr int pos(int i) { return i + ((i >> 5) << 2) + ((i >> 10) << 4); }
}  // namespace gv

// A 4096-point transform job: 256 threads x 16 values.
struct GvJob {
  static constexpr int LOGN = 12, N = 4096;
  static constexpr int LOGV = 4, V = 16;
  static constexpr int B1 = 6;  // index bits of round 1 (4 registers + 2 quad)
  static constexpr int R2 = 2;  // lane bits of round 2
  // index bits whose butterflies ran over DPP (upper lane negated)
  static constexpr unsigned RHO = (3u << 4) | (3u << 10);
  __host__ __device__ static constexpr int pos(int i) { return gv::pos(i); }
  static constexpr int SCR = (gv::pos(N - 1) + 4) & ~3;
  // round-2 index of (thread g, register r)
  __device__ static int idx2(int g, int r) { return (g >> 2) | (r << 6) | ((g & 3) << 10); }
};

template <int BITS>
struct GvCode {
  static constexpr int CPW = 32 / BITS;    // codes per 32-bit code word
  static constexpr int CC = 4 * CPW;       // codes per 16-byte chunk
  static constexpr int SETS = BITS == 2 ? 2 : 1;  // nibble words per code word (even / odd codes)
  static constexpr int RPW = 4 * SETS;     // limb registers per code word
};

// LDS slot of code position k in the fixed-point staging rows: 4 floats per
// 64 and 16 per 1024 keep both the transform's writes and the limb builder's
// 16-byte reads free of bank conflicts
__host__ __device__ constexpr int gv_xpos(int k) { return k + ((k >> 6) << 2) + ((k >> 10) << 4); }

template <int LOGN, int BITS, int TT>
struct GvShape {
  static constexpr int N = 1 << LOGN;
  static constexpr int NV = N / 128;            // fp16-pair registers per token
  static constexpr int CPL = N * BITS / 8192;   // 16-byte code chunks per lane per row
  static constexpr int HALVES = N / 4096;
  static constexpr int JOBS = TT * HALVES;
  // 16 waves (4 per SIMD, at most 128 VGPRs) for one token with at most two
  // chunks per lane; more tokens or chunks take the registers of 8 waves
  static constexpr int WAVES = TT == 1 && CPL <= 2 ? 16 : 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int NGRP = THREADS / gv::GT;  // jobs at a time
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

// Block barrier for LDS hand-offs only.  __syncthreads() also orders global
// memory, which makes it wait for every load in flight, the rows streaming
// into LDS among them; this one waits for the wave's LDS operations alone.
__device__ __forceinline__ void gv_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float gv_wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// x [tn][ldx] bf16 (tn <= TT tokens of this pass), codes [rows][n bits / 8],
// scales [rows][n / g] fp16 bits, y [tn][ldy] bf16.
template <int LOGN, int BITS, int GPC, int TT>
__global__ __launch_bounds__((GvShape<LOGN, BITS, TT>::THREADS)) void k_rht_gemv(
    const uint16_t* __restrict__ x, int tn, int64_t ldx, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, int64_t rows, int logg, const uint32_t* __restrict__ sbits,
    uint16_t* __restrict__ y, int64_t ldy, int64_t lastq, int64_t lastr) {
  using J = GvJob;
  using C = GvCode<BITS>;
  using S = GvShape<LOGN, BITS, TT>;
  constexpr int N = S::N, NV = S::NV, V = J::V, WAVES = S::WAVES, NGRP = S::NGRP;
  constexpr int PF = gv::PF;
  constexpr int CPL = S::CPL;
  constexpr int RB = N * BITS / 8;                 // bytes per code row
  constexpr float RSQRTN = LOGN == 12 ? 0.015625f : 0.011048543456039806f;  // 1 / sqrt(n)
  static_assert(CPL >= 1 && NV == CPL * 4 * C::RPW, "lane layout");
  static_assert(GPC == 1 || GPC == 2 || GPC == 4, "scale groups per chunk");
  static_assert(NGRP % S::HALVES == 0, "a token's jobs run in one round");
  constexpr int XT = (gv_xpos(N - 1) + 4) & ~3;  // floats per token staging row
  constexpr int ITEMS = TT * (N / C::CPW);      // limb builder items: one code word of one token

  constexpr int SLOTS = NGRP < S::JOBS ? NGRP : S::JOBS;  // transform jobs per round
  __shared__ __align__(16) float scr0[SLOTS * J::SCR];  // [SLOTS][SCR] transform scratch
  __shared__ __align__(16) float xt[TT][XT];
  __shared__ __align__(16) uint32_t hl[TT][NV / 4][64][4];
  __shared__ int corl[TT][CPL][GPC][64];  // sum of X over a lane's group part (2-bit codes)
  __shared__ uint32_t tmax[TT];           // max |H S x_t| as float bits

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ng = (int)(N >> logg);  // scale groups per row
  const int grp = wave / (gv::GT / 64), g = tid % gv::GT;

  for (int i = tid; i < TT * CPL * GPC * 64; i += S::THREADS) (&corl[0][0][0][0])[i] = 0;
  if (tid < TT) tmax[tid] = 0u;

  // ---- 1. token rows, then the first weight rows
  float v[V];
  struct XRaw {
    u32x4 a[V / 8], b[V / 8];
    uint32_t sa, sb;
  };
  // loads of a job's inputs (issued ahead of the weight rows) ...
  auto load_job = [&](int round, XRaw& xr) {
    const int jb = round * NGRP + grp, ts = jb / S::HALVES;
    if (jb >= S::JOBS || ts >= tn) return;
    const uint16_t* xp = x + ts * ldx + g * V;
#pragma unroll
    for (int q = 0; q < V / 8; ++q) xr.a[q] = ldg<u32x4>(xp + 8 * q);
    if constexpr (S::HALVES == 2) {
#pragma unroll
      for (int q = 0; q < V / 8; ++q) xr.b[q] = ldg<u32x4>(xp + 4096 + 8 * q);
    }
    // raw sign words, unconditional (kNoSigns stands in for no signs)
    const uint32_t* sp = sbits ? sbits : kNoSigns;
    xr.sa = sp[g >> 1];
    if constexpr (S::HALVES == 2) xr.sb = sp[128 + (g >> 1)];
  };
  // ... and the job's first values: signs, then lo + hi or lo - hi
  auto start_job = [&](int round, const XRaw& xr) {
    const int jb = round * NGRP + grp, ts = jb / S::HALVES, half = jb % S::HALVES;
    if (jb >= S::JOBS) return;
    if (ts >= tn) {
#pragma unroll
      for (int r = 0; r < V; ++r) v[r] = 0.f;
      return;
    }
    const uint32_t sa = xr.sa >> (16 * (g & 1));
    const uint32_t sb = S::HALVES == 2 ? xr.sb >> (16 * (g & 1)) : 0u;
#pragma unroll
    for (int r = 0; r < V; ++r) {
      const uint32_t wa = xr.a[r / 8][(r % 8) / 2];
      const float xa = as_f(((r & 1) ? (wa & 0xffff0000u) : (wa << 16)) ^ (((sa >> r) & 1u) << 31));
      if constexpr (S::HALVES == 2) {
        const uint32_t wb = xr.b[r / 8][(r % 8) / 2];
        const float xb = as_f(((r & 1) ? (wb & 0xffff0000u) : (wb << 16)) ^ (((sb >> r) & 1u) << 31));
        v[r] = half ? xa - xb : xa + xb;
      } else {
        v[r] = xa;
      }
    }
  };
  XRaw xr0;
  load_job(0, xr0);

  struct Row {
    u32x4 cw[CPL];
    uint32_t sc[CPL][GPC == 4 ? 2 : 1];
  };
  const uint32_t loff = (uint32_t)lane * 16u;
  auto fetch_sc = [&](uint32_t (&sc)[CPL][GPC == 4 ? 2 : 1], int64_t o) {
    const uint16_t* sr = scales + o * ng;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int first = ((j * 64 + lane) * C::CC) >> logg;
      if constexpr (GPC == 1) sc[j][0] = sr[first];
      else if constexpr (GPC == 2) sc[j][0] = ldg<uint32_t>(sr + first);
      else {
        const u32x2 w2 = ldg<u32x2>(sr + first);
        sc[j][0] = w2[0];
        sc[j][1] = w2[1];
      }
    }
  };
  auto fetch = [&](Row& r, int64_t o) {
    const uint8_t* cr = codes + o * RB;
#pragma unroll
    for (int j = 0; j < CPL; ++j) r.cw[j] = ldg<u32x4>(cr + j * 1024 + loff);
    fetch_sc(r.sc, o);
  };
  const int64_t tw = (int64_t)gridDim.x * WAVES;
  int64_t o = (int64_t)blockIdx.x * WAVES + wave;
  constexpr int NS = PF + 1;  // ring slots: PF rows in flight while one is consumed
  Row buf[NS];                // slot k % NS holds row o + k tw
  // Look-ahead loads past the end re-read the wave's own last row (an L2
  // hit, different for every wave): unconditional loads keep the in-order
  // wait counts exact, and clamping to one shared row would make every wave
  // hit the same addresses.
  // last = the largest row below rows that is o mod tw (host: lastq = (rows - 1) / tw * tw,
  // lastr = (rows - 1) % tw)
  const int64_t last = o >= rows ? rows - 1 : o + (o <= lastr ? lastq : lastq - tw);
#pragma unroll
  for (int k = 0; k < PF; ++k) fetch(buf[k], o + k * tw < rows ? o + k * tw : last);
  start_job(0, xr0);

  // ---- 2. rotated tokens into the staging rows, with each token's maximum
#pragma unroll
  for (int round = 0; round * NGRP < S::JOBS; ++round) {
    const int jb = round * NGRP + grp, ts = jb / S::HALVES, half = jb % S::HALVES;
    const bool act = jb < S::JOBS;  // uniform per wave
    float* sc = scr0 + (grp < SLOTS ? grp : 0) * J::SCR;
    if (round > 0) {
      XRaw xr;
      load_job(round, xr);
      start_job(round, xr);
    }
    if (act) {
      reg_stage<V, 0>(v);
      reg_stage<V, 1>(v);
      reg_stage<V, 2>(v);
      reg_stage<V, 3>(v);
      lane_stage<V, 0>(v, g);
      lane_stage<V, 1>(v, g);
      // the slots are affine in r: one base address, immediate offsets
      float* w1 = sc + J::pos(g * V);  // pos(16 g + r) = pos(16 g) + r for r < 16
#pragma unroll
      for (int r = 0; r < V; r += 4)
        *reinterpret_cast<f32x4*>(w1 + r) = f32x4{v[r], v[r + 1], v[r + 2], v[r + 3]};
    }
    gv_barrier();
    if (act) {
      const float* r2 = sc + J::pos(J::idx2(g, 0));  // + 72 r: r << 6 adds 64 r + 4 (2 r)
#pragma unroll
      for (int r = 0; r < V; ++r) v[r] = r2[72 * r];
      reg_stage<V, 0>(v);
      reg_stage<V, 1>(v);
      reg_stage<V, 2>(v);
      reg_stage<V, 3>(v);
      lane_stage<V, 0>(v, g);
      lane_stage<V, 1>(v, g);
      // RHO's bits (4, 5, 10, 11) come from g alone, so the sign is the thread's;
      // staging slots are xpos(k0) + 68 r (r << 6 adds 64 r + 4 r, never a 1024 carry)
      const uint32_t sneg = (__builtin_popcount((unsigned)J::idx2(g, 0) & J::RHO) & 1) << 31;
      float* w3 = &xt[ts][gv_xpos(half * 4096 + J::idx2(g, 0))];
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < V; ++r) {
        w3[68 * r] = as_f(as_u(v[r]) ^ sneg);
        m = fmaxf(m, fabsf(v[r]));
      }
      m = gv_wave_max(m);
      if (lane == 0) atomicMax(&tmax[ts], as_u(m));  // non-negative floats order as their bits
    }
    gv_barrier();
  }

  // ---- 3. limb words: item = one code word (8 or 16 codes) of one token
  for (int it = tid; it < ITEMS; it += S::THREADS) {
    const int t = it / (N / C::CPW), k0 = (it % (N / C::CPW)) * C::CPW;
    const int c = k0 / C::CC, l = c & 63, j = c >> 6, w = (k0 % C::CC) / C::CPW;
    // sigma = 2^(13 - e) with max = f 2^e, f in [1, 2), at most 2^126 so
    // that 1 / sigma stays a normal fp32 number; 1 for an all-zero or
    // non-finite token
    const float mx = as_f(tmax[t]);
    int e = 0;
    const bool fin = mx > 0.f && __builtin_isfinite(mx);
    if (fin) e = ((int)((as_u(mx) >> 23) & 0xffu)) - 127;
    const int se = fin ? (13 - e < 126 ? 13 - e : 126) : 0;
    const float sig = ldexpf(1.f, se);
    uint32_t z[C::CPW];
    int xsum = 0;
#pragma unroll
    for (int q = 0; q < C::CPW / 4; ++q) {
      const f32x4 f = *reinterpret_cast<const f32x4*>(&xt[t][gv_xpos(k0 + 4 * q)]);
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int X = (int)__builtin_rintf(f[e4] * sig);
        xsum += X;
        z[4 * q + e4] = (uint32_t)((X + 0x8888) ^ 0x8888);  // nibble p = digit p (two's complement)
      }
    }
    uint32_t lw[C::SETS][4];
#pragma unroll
    for (int st = 0; st < C::SETS; ++st)
#pragma unroll
      for (int pl = 0; pl < 4; ++pl) {
        uint32_t acc = 0;
#pragma unroll
        for (int m = 0; m < 8; ++m) acc |= ((z[C::SETS * m + st] >> (4 * pl)) & 15u) << (4 * m);
        lw[st][pl] = acc;
      }
#pragma unroll
    for (int st = 0; st < C::SETS; ++st)
      *reinterpret_cast<u32x4*>(&hl[t][(j * 4 + w) * C::SETS + st][l][0]) =
          u32x4{lw[st][0], lw[st][1], lw[st][2], lw[st][3]};
    if constexpr (BITS == 2) atomicAdd(&corl[t][j][w * GPC / 4][l], xsum);
  }
  gv_barrier();

  // every wave's copy of the limb words, and its constants
  uint32_t h[TT][NV];
  int corr[TT][CPL][GPC];
  float sinv[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float mx = as_f(tmax[t]);
    int e = 0;
    const bool fin = mx > 0.f && __builtin_isfinite(mx);
    if (fin) e = ((int)((as_u(mx) >> 23) & 0xffu)) - 127;
    const int se = fin ? (13 - e < 126 ? 13 - e : 126) : 0;
    sinv[t] = ldexpf(1.f, -se);
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
      for (int gp = 0; gp < GPC; ++gp) corr[t][j][gp] = BITS == 2 ? 2 * corl[t][j][gp][lane] : 0;
  }

  // ---- 4. weight rows, PF of each wave in flight
  auto row_dot = [&](const Row& r, int64_t orow) {
    float ya[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) ya[t] = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      int acc[TT][GPC][4];
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int gp = 0; gp < GPC; ++gp)
#pragma unroll
          for (int pl = 0; pl < 4; ++pl) acc[t][gp][pl] = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int gp = w * GPC / 4;
        uint32_t nw[C::SETS];
        if constexpr (BITS == 2) {
          const uint32_t u = r.cw[j][w] ^ 0xaaaaaaaau;  // offset binary: u = q + 2
          nw[0] = u & 0x33333333u;
          nw[1] = (u >> 2) & 0x33333333u;
        } else {
          nw[0] = r.cw[j][w];
        }
#pragma unroll
        for (int st = 0; st < C::SETS; ++st)
#pragma unroll
          for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int pl = 0; pl < 4; ++pl)
              acc[t][gp][pl] = __builtin_amdgcn_sdot8((int)nw[st], (int)h[t][((j * 4 + w) * C::SETS + st) * 4 + pl],
                                                      acc[t][gp][pl], false);
      }
#pragma unroll
      for (int gp = 0; gp < GPC; ++gp) {
        const uint32_t sw = GPC == 1 ? r.sc[j][0] : r.sc[j][gp >> 1] >> (16 * (gp & 1));
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(sw & 0xffffu));
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const int a = acc[t][gp][0] + acc[t][gp][1] * 16 + acc[t][gp][2] * 256 + acc[t][gp][3] * 4096 -
                        corr[t][j][gp];
          ya[t] = fmaf(s, (float)a, ya[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float tot = gv_wave_sum(ya[t]) * RSQRTN * sinv[t];
      if (t < tn && lane == 0) y[t * ldy + orow] = __builtin_bit_cast(uint16_t, (__bf16)tot);
    }
  };
  // the row PF tw further on goes out before each row is consumed
  for (; o < rows; o += NS * tw) {
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int64_t ok = o + k * tw, onext = ok + PF * tw;
      fetch(buf[(k + PF) % NS], onext < rows ? onext : last);
      if (ok < rows) row_dot(buf[k], ok);
    }
  }
}

template <int LOGN, int BITS, int GPC, int TT>
static hipError_t run_gemv(const void* x, int tn, int64_t ldx, const uint8_t* codes, const uint16_t* scales,
                           int64_t rows, int logg, const uint32_t* sb, void* y, int64_t ldy, hipStream_t s) {
  using S = GvShape<LOGN, BITS, TT>;
  auto k = k_rht_gemv<LOGN, BITS, GPC, TT>;
  // one block per CU: every block rotates the tokens itself
  const unsigned grid = persistent_grid((rows + S::WAVES - 1) / S::WAVES, 1);
  const int64_t tw = (int64_t)grid * S::WAVES;
  hipLaunchKernelGGL(k, dim3(grid), dim3(S::THREADS), 0, s, (const uint16_t*)x, tn, ldx, codes, scales, rows,
                     logg, sb, (uint16_t*)y, ldy, (rows - 1) / tw * tw, (rows - 1) % tw);
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
// its rotated tokens in registers (n / 128 per token) and reads the weights
// once.
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
