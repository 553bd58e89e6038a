// qwha_adapter_forward: y = (x Hn) F^T with F sparse (CSR), d_in a power of
// two in [64, 8192].
//
// QWHA explainer, 2.1: the adapter is Delta W = F H^-1, one Walsh-Hadamard
// transform on the input side and a sparse coefficient matrix F built from a
// value vector and an index list; with the orthonormal Hn this is
// y = x Delta W^T = (x Hn) F^T.
//
// One block per tile of 8 tokens:
//   1. each of 4 waves transforms token rows with the register / LDS FWHT
//      engine (fp32); a row is scaled by an exact power of two so its largest
//      entry sits in [2^13, 2^14), rounded to fp16 and staged token-major;
//   2. the staged tile is re-laid out to Z[k][8 tokens] (16 bytes per
//      column), so one ds_read_b128 returns a column for all 8 tokens;
//   3. the rows of F are taken in chunks of 2048 consecutive rows; within a
//      chunk they are bucketed by the number of 16-entry steps they need
//      (longest first), so the 16 rows a wave handles together finish at
//      about the same time;
//   4. CSR gather SpMM: a quad of lanes per row, each lane taking 4
//      consecutive entries per step with 16-byte index loads (the quad reads
//      64 contiguous bytes of col_idx), 8 fp32 accumulators per lane
//      (v_fma_mix with the fp16 column), a quad DPP reduction per row; the
//      results go to a token-major bf16 buffer in LDS;
//   5. the chunk's outputs leave with 16-byte row-contiguous stores.
//
// The same kernel computes the adapter's gradient with respect to its input,
// dx = dy Delta W = (dy F) Hn (Hn is symmetric): the tile is dy as it is (no
// transform in step 1), the CSR is that of F^T, the gathered rows (dy F)
// stay on chip in bf16 for all d_in columns, and step 6 transforms them.
//
// Other widths, from two exact identities of the Sylvester matrix:
//   d_in < 4096: (H_4096 [x; 0])[k] = (H_d x)[k] for k < d, so x is
//     zero-extended to 4096 on load and the result scaled by 64 / sqrt(d);
//   d_in = 8192 (WIDE): H_8192 = H_2 (x) H_4096 over the top index bit, so
//     the half h of H_8192 x is H_4096 (x_lo +- x_hi): one wave per
//     (token, half) runs the 4096-point engine on x_lo + x_hi or x_lo - x_hi.
//     The tile holds 4 tokens (8-byte columns), and each token's fp16 scale
//     comes from ||x||_2, a bound on every |z_k| that both of its waves
//     compute identically.
#include <cmath>

#include "io.hpp"
#include "launch.hpp"

namespace whtq {

namespace qw {
constexpr int THREADS = 1024;  // 16 waves (4 transform token rows)
constexpr int NW = THREADS / 64;
constexpr int FWAVES = 4;      // waves that run the token transforms
constexpr int CHUNK = 2048;    // rows per output chunk
constexpr int NBKT = 256;      // buckets: 16-entry steps per row, capped
}  // namespace qw

// Tile geometry: WIDE (d_in = 8192) keeps 4 tokens, else 8; the forward tile
// spans the (extended) transform width, the backward's spans dy (<= 4096).
template <bool BWD, bool WIDE>
struct QwGeo {
  static constexpr int TT = WIDE ? 4 : 8;              // tokens per block
  static constexpr int NT = WIDE ? 8192 : 4096;        // transform width
  static constexpr int ZW = BWD ? 4096 : NT;           // tile columns
  static constexpr int CB = 2 * TT;                    // bytes per tile column
  static constexpr int CSH = WIDE ? 3 : 4;             // log2(CB)
};

// LDS map (bytes):
//   [0, ZB)       Z[k][tok] fp16, CB bytes per column (FWHT scratch before
//                 step 2, and in the backward before step 6)
//   [ZB, ...)     staging Zt[tok][k] fp16 in steps 1-2; afterwards, per chunk,
//                 the sorted row list (row u16, start i32, end i32) and the
//                 output buffer O[tok][row] bf16 (the backward keeps all NT
//                 rows of it: [tok][NT])
//   then          bucket counters (uint32), per-token exponent
template <bool BWD, bool WIDE>
struct QwLds {
  using Q = QwGeo<BWD, WIDE>;
  static constexpr int Z = 0;
  static constexpr int ZB = 65536;
  static constexpr int ZT = ZB;
  static constexpr int RID = ZB;
  static constexpr int RBEG = RID + 2 * qw::CHUNK;
  static constexpr int REND = RBEG + 4 * qw::CHUNK;
  static constexpr int OUT = REND + 4 * qw::CHUNK;
  static constexpr int OSTRIDE = BWD ? Q::NT : qw::CHUNK;  // output buffer row stride (elements)
  static constexpr int OUT_END = OUT + 2 * Q::TT * OSTRIDE;
  static constexpr int BKT = OUT_END > ZT + Q::ZW * Q::CB ? OUT_END : ZT + Q::ZW * Q::CB;
  static constexpr int EXP = BKT + 4 * qw::NBKT;
  static constexpr int BYTES = EXP + 4 * Q::TT;
  static_assert(Q::ZW * Q::CB <= ZB && OUT % 16 == 0 && BYTES <= 160 * 1024, "LDS map");
};

// 16-entry steps of a row [beg, end) whose steps start at beg rounded down to a multiple of 4
__device__ __forceinline__ int qw_steps(int beg, int end) { return end > beg ? (end - (beg & ~3) + 15) >> 4 : 0; }

// four consecutive values of F, from an index that is a multiple of 4
template <int VALDT> struct ValQuad;
template <> struct ValQuad<DT_BF16> {  // 8 bytes
  typedef u32x2 raw;
  static __device__ __forceinline__ raw load(const void* v, int j) {
    return ldg<u32x2>(reinterpret_cast<const uint8_t*>(v) + 2u * (uint32_t)j);
  }
  static __device__ __forceinline__ float get(const raw& r, int q) {
    const uint32_t w = q < 2 ? r.x : r.y;
    return (q & 1) ? bf16hi(w) : bf16lo(w);
  }
};
template <> struct ValQuad<DT_F32> {  // 16 bytes
  typedef f32x4 raw;
  static __device__ __forceinline__ raw load(const void* v, int j) {
    return ldg<f32x4>(reinterpret_cast<const uint8_t*>(v) + 4u * (uint32_t)j);
  }
  static __device__ __forceinline__ float get(const raw& r, int q) { return r[q]; }
};

// Forward (BWD = false): x = activations, CSR of F (d_out rows), y = outputs.
// Backward to the input (BWD = true): x = dy [tokens][in_cols], CSR of F^T
// (d_in = 4096 rows, entries indexing columns of dy), y = dx [tokens][4096].
template <int VALDT, bool BWD, bool WIDE>
__global__ __launch_bounds__(qw::THREADS) void k_qwha(const uint16_t* __restrict__ x, int64_t tokens,
                                                      int64_t ldx, int in_cols, const int32_t* __restrict__ row_ptr,
                                                      const int32_t* __restrict__ col_idx,
                                                      const void* __restrict__ vals, int d_out, int nnz,
                                                      uint16_t* __restrict__ y, int64_t ldy, int vec, int out_cols,
                                                      float wscale, float pscale) {
  using G = Geo<12>;
  using V = ValQuad<VALDT>;
  using Q = QwGeo<BWD, WIDE>;
  using L = QwLds<BWD, WIDE>;
  constexpr int TT = Q::TT;
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tok0 = (int64_t)blockIdx.x * TT;
  const int ntok = (int)min<int64_t>(TT, tokens - tok0);

  uint16_t* rid = reinterpret_cast<uint16_t*>(smem + L::RID);
  int* rbeg = reinterpret_cast<int*>(smem + L::RBEG);
  int* rend = reinterpret_cast<int*>(smem + L::REND);
  uint16_t* obuf = reinterpret_cast<uint16_t*>(smem + L::OUT);
  uint32_t* bkt = reinterpret_cast<uint32_t*>(smem + L::BKT);
  int* texp = reinterpret_cast<int*>(smem + L::EXP);

  auto histogram = [&](int base, int cn) {
    for (int r = tid; r < cn; r += qw::THREADS) {
      const int st = qw_steps(row_ptr[base + r], row_ptr[base + r + 1]);
      atomicAdd(&bkt[qw::NBKT - 1 - min(st, qw::NBKT - 1)], 1u);  // longest rows first
    }
  };

  // ---- bucket histogram of the first chunk (overlaps with the transforms)
  for (int i = tid; i < qw::NBKT; i += qw::THREADS) bkt[i] = 0;
  __syncthreads();
  histogram(0, min(qw::CHUNK, d_out));

  // ---- 1. FWHT of the token rows (backward: the dy rows as they are),
  // staged as fp16 token-major; the wide forward runs one job per (token, half)
  if (wave < qw::FWAVES) {
    float* scratch = reinterpret_cast<float*>(smem + L::Z) + wave * G::LDS_ROW;
    uint16_t* zt = reinterpret_cast<uint16_t*>(smem + L::ZT);
    const int t = lane;
    const bool rho = BWD ? false : rho_B<12>(t);
    int col[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) col[c] = G::idxA(t, c * 8);
    const uint32_t nomask[4] = {0u, 0u, 0u, 0u};
    constexpr bool SPLIT = !BWD && WIDE;
    constexpr int JOBS = SPLIT ? 2 * TT : TT;
    for (int jb = wave; jb < JOBS; jb += qw::FWAVES) {
      const int k = SPLIT ? jb >> 1 : jb, half = SPLIT ? jb & 1 : 0;
      const int64_t tok = tok0 + min(k, ntok - 1);  // tail tokens recompute the last one
      const uint16_t* xr = x + tok * ldx;
      float v[64];
      u16x2 am{0, 0};  // split: the largest |x_i| of the token, from the bf16 bits
      if constexpr (BWD) {
        // lane t holds columns 64 t .. 64 t + 63 (layout B); columns past
        // in_cols are zero (16-byte loads where a chunk lies inside and the
        // rows are 16-byte aligned, `vec`; else element loads)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int c0 = 64 * t + 8 * q;
          if (vec && c0 + 8 <= in_cols) {
            const u32x4 w = ldg<u32x4>(xr + c0);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              v[8 * q + 2 * p] = bf16lo(w[p]);
              v[8 * q + 2 * p + 1] = bf16hi(w[p]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[8 * q + e] = c0 + e < in_cols ? as_f((uint32_t)xr[c0 + e] << 16) : 0.f;
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if constexpr (SPLIT) {
            // half h: x_lo + x_hi or x_lo - x_hi (the top-bit butterfly first)
            Raw8 rl, rh;
            fetch8<DT_BF16>(xr, col[c], rl);
            fetch8<DT_BF16>(xr, col[c] + 4096, rh);
            am = absmax16(absmax16(absmax16(absmax16(am, rl.a.x), rl.a.y), rl.a.z), rl.a.w);
            am = absmax16(absmax16(absmax16(absmax16(am, rh.a.x), rh.a.y), rh.a.z), rh.a.w);
            float vl[8], vh[8];
            widen8<DT_BF16, false>(rl, vl, nomask, 0u);
            widen8<DT_BF16, false>(rh, vh, nomask, 0u);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[8 * c + e] = half ? vl[e] - vh[e] : vl[e] + vh[e];
          } else {
            // d_in < 4096: the row is zero-extended to 4096
            Raw8 raw{};
            if (col[c] < in_cols) fetch8<DT_BF16>(xr, col[c], raw);
            widen8<DT_BF16, false>(raw, v + 8 * c, nomask, 0u);
          }
        }
        stages_A<12, false>(v, t);
        transpose_AB<12, 64>(scratch, v, t);
        stages_B<12, 2>(v, t);
      }
      int e = 0;
      if constexpr (SPLIT) {
        // every raw sum |(H_4096 (x_lo +- x_hi))_k| <= 8192 max |x_i| <
        // 2^(em+13) with max |x_i| < 2^em (the maximum is exact: no sum of
        // squares that could overflow or underflow fp32); e = em + 12 keeps
        // the staged values (times 2^(14-e)) below 2^15, inside fp16.  Both
        // halves compute the same e.
        const uint32_t mb = wave_max_u32(absmax16(am));
        if (mb) e = bf16_mag_exp(mb) + 12;
      } else {
        // exact power-of-two scale putting max |z| in [2^13, 2^14)
        float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 64; r += 2) a4[(r >> 1) & 3] = max3abs(a4[(r >> 1) & 3], v[r], v[r + 1]);
        float a = fmaxf(fmaxf(a4[0], a4[1]), fmaxf(a4[2], a4[3]));
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) a = fmaxf(a, __shfl_xor(a, s));
        if (a > 0.f) (void)frexpf(a, &e);       // a = m 2^e, m in [0.5, 1)
      }
      // e >= -100 keeps 2^(14-e) and the output factor 2^(e-20) normal fp32
      // numbers (tokens below about 2^-113 are staged with a smaller scale)
      e = e > -100 ? e : -100;
      const float mult = ldexpf(rho ? -1.0f : 1.0f, 14 - e);
      if (lane == 0 && half == 0) texp[k] = e;
      uint16_t* zrow = zt + k * Q::ZW + half * 4096 + t * 64;
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
    const uint16_t* zt = reinterpret_cast<const uint16_t*>(smem + L::ZT);
    for (int kk = tid; kk < Q::ZW; kk += qw::THREADS) {
      uint32_t h[TT];
#pragma unroll
      for (int k = 0; k < TT; ++k) h[k] = zt[k * Q::ZW + kk];
      if constexpr (TT == 8)
        reinterpret_cast<u32x4*>(smem + L::Z)[kk] =
            u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      else
        reinterpret_cast<u32x2*>(smem + L::Z)[kk] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    }
  }
  __syncthreads();  // the staging area becomes the row list / output buffer
  if constexpr (BWD) {
    // rows of F^T (columns of dx) past d_out are never gathered: zero them
    // (d_out here is the number of F^T rows, the adapter's d_in)
    for (int i = tid; i < TT * (Q::NT - d_out); i += qw::THREADS)
      obuf[(i / (Q::NT - d_out)) * L::OSTRIDE + d_out + i % (Q::NT - d_out)] = 0;
  }

  constexpr int TPS = TT / 4;  // tokens per lane of a row's quad
  const int slot = lane & 3;   // lane within the row's quad
  // its tokens slot TPS + i: undo the staging scale 2^(14-e), normalise (wscale
  // times 2^-6 = 1/sqrt(4096))
  float osc[TPS];
#pragma unroll
  for (int i = 0; i < TPS; ++i) osc[i] = ldexpf(wscale, texp[slot * TPS + i] - 20);

  for (int base = 0; base < d_out; base += qw::CHUNK) {
    const int cn = min(qw::CHUNK, d_out - base);
    if (base > 0) {
      for (int i = tid; i < qw::NBKT; i += qw::THREADS) bkt[i] = 0;
      __syncthreads();
      histogram(base, cn);
    }
    __syncthreads();
    // ---- 3. bucket offsets (one wave), then scatter the chunk's rows
    if (wave == 0) {
      uint32_t run = 0;
      for (int b0 = 0; b0 < qw::NBKT; b0 += 64) {
        const uint32_t c = bkt[b0 + lane];
        uint32_t incl = c;
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) {
          const uint32_t o = __shfl_up(incl, s);
          if (lane >= s) incl += o;
        }
        bkt[b0 + lane] = run + incl - c;
        run += __shfl(incl, 63);
      }
    }
    __syncthreads();
    for (int r = tid; r < cn; r += qw::THREADS) {
      const int beg = row_ptr[base + r], end = row_ptr[base + r + 1];
      const uint32_t pos = atomicAdd(&bkt[qw::NBKT - 1 - min(qw_steps(beg, end), qw::NBKT - 1)], 1u);
      rid[pos] = (uint16_t)r;
      rbeg[pos] = beg;
      rend[pos] = end;
    }
    __syncthreads();

    // ---- 4. gather SpMM: group g = 16 sorted rows, one quad of lanes per
    // row; a wave takes groups rr NW + (wave, or NW - 1 - wave on odd rr):
    // snake order, so that long and short groups mix.  The index / value
    // loads run one step ahead, across group boundaries.
    const int ng = nnz > 0 ? (cn + 15) >> 4 : 0;
    if (nnz == 0)  // F = 0: every output is zero
      for (int i = tid; i < TT * cn; i += qw::THREADS) obuf[(i / cn) * L::OSTRIDE + (BWD ? base : 0) + i % cn] = 0;
    struct Row {
      int r, beg, end, nst;
    };
    auto row_of = [&](int rr) {
      const int g = rr * qw::NW + ((rr & 1) ? qw::NW - 1 - wave : wave);
      const int p = 16 * g + (lane >> 2);
      Row w{0, 0, 0, 0};
      if (g < ng && p < cn) {
        w.r = rid[p];
        w.beg = rbeg[p];
        w.end = rend[p];
        w.nst = qw_steps(w.beg, w.end);
      }
      return w;
    };
    // index / value loads of one step, kept in two alternating buffers (even
    // steps in A, odd in B) so that a load is never copied while in flight
    struct Buf {
      u32x4 cw;
      typename V::raw vw;
    };
    // this lane's entries of step s of a row: [(beg & ~3) + 16 s + 4 slot, + 4)
    // The whole aligned 16-byte index block (8 or 16 bytes of values) holding
    // entry jj is read even where the arrays end inside it: an aligned block
    // never straddles a page, and entries outside the row are masked below.
    // Every step issues the same two loads (a step with nothing to do reads
    // block 0) so that the outstanding-load count is the same on every path
    // and a use waits only for its own buffer.
    auto load_step = [&](const Row& w, int s, Buf& b) {
      int jj = (w.beg & ~3) + 16 * s + 4 * slot;
      jj = (s < w.nst && jj < w.end) ? jj : 0;
      b.cw = ldg<u32x4>(reinterpret_cast<const uint8_t*>(col_idx) + 4u * (uint32_t)jj);
      b.vw = V::load(vals, jj);
    };
    auto run_step = [&](const Row& w, int s, const Buf& b, float* acc) {
      const int jc = (w.beg & ~3) + 16 * s + 4 * slot;
      if (s >= w.nst || jc >= w.end) return;
      // the four Z columns first, then their 32 FMAs
      u32x4 cw = b.cw;
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = V::get(b.vw, q);
      if (jc < w.beg || jc + 4 > w.end) {  // the row's first or last quad: drop other entries
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = (jc + q >= w.beg && jc + q < w.end) ? v[q] : 0.f;
          cw[q] &= (uint32_t)(Q::ZW - 1);  // past the arrays' end the index is arbitrary
        }
      }
      // (columns copied out as words: subscripting the loaded vectors with the
      // unrolled loop index was miscompiled into a single 4-byte read)
      constexpr int WPC = TT / 2;  // 32-bit words per column
      uint32_t zc[4][WPC];
      if constexpr (TT == 8) {
        u32x4 zv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) zv[q] = *reinterpret_cast<const u32x4*>(smem + L::Z + (cw[q] << Q::CSH));
        __builtin_memcpy(zc, zv, 64);
      } else {
        u32x2 zv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) zv[q] = *reinterpret_cast<const u32x2*>(smem + L::Z + (cw[q] << Q::CSH));
        __builtin_memcpy(zc, zv, 32);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int w2 = 0; w2 < WPC; ++w2) {
          fma_mix_lo(acc[2 * w2], v[q], zc[q][w2]);
          fma_mix_hi(acc[2 * w2 + 1], v[q], zc[q][w2]);
        }
      }
    };
    Buf A{}, B{};
    Row cur = row_of(0);
    load_step(cur, 0, A);
    for (int rr = 0; rr * qw::NW < ng; ++rr) {
      const Row nxt = row_of(rr + 1);
      float acc[TT];
#pragma unroll
      for (int k = 0; k < TT; ++k) acc[k] = 0.f;
      // steps in pairs (an odd count gets an empty last step); the group after
      // this one starts in buffer A again
      for (int s = 0; s < cur.nst || s == 0; s += 2) {
        load_step(cur, s + 1, B);
        run_step(cur, s, A, acc);
        if (s + 2 < cur.nst) load_step(cur, s + 2, A);
        else load_step(nxt, 0, A);
        run_step(cur, s + 1, B, acc);
      }
      // quad all-reduce: every lane of the quad gets the row's 8 sums
#pragma unroll
      for (int k = 0; k < TT; ++k) {
        acc[k] += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(acc[k]), 0xB1, 0xF, 0xF, true));  // ^1
        acc[k] += as_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u(acc[k]), 0x4E, 0xF, 0xF, true));  // ^2
      }
      const int g = rr * qw::NW + ((rr & 1) ? qw::NW - 1 - wave : wave);
      if (g < ng && 16 * g + (lane >> 2) < cn) {  // lane `slot` writes tokens slot TPS .. slot TPS + TPS - 1
        const int oc = (BWD ? base : 0) + cur.r;
#pragma unroll
        for (int i = 0; i < TPS; ++i) {
          float a = acc[i];
#pragma unroll
          for (int k = 1; k < 4; ++k) a = slot == k ? acc[TPS * k + i] : a;
          obuf[(TPS * slot + i) * L::OSTRIDE + oc] = (uint16_t)(pack_bf16(a * osc[i], 0.f) & 0xffffu);
        }
      }
      cur = nxt;
    }
    __syncthreads();

    // ---- 5. the chunk's outputs, row-contiguous (the backward keeps them on chip)
    if constexpr (!BWD) {
      const int cq = (cn + 7) >> 3;
      for (int i = tid; i < ntok * cq; i += qw::THREADS) {
        const int t = i / cq, q = i - t * cq;
        const uint16_t* src = obuf + t * qw::CHUNK + 8 * q;
        uint16_t* dst = y + (tok0 + t) * ldy + base + 8 * q;
        if (vec && 8 * q + 8 <= cn) {
          stg(dst, *reinterpret_cast<const u32x4*>(src));
        } else {
          for (int e = 0; e < 8 && 8 * q + e < cn; ++e) dst[e] = src[e];
        }
      }
    }
    __syncthreads();  // the next chunk reuses the row list and the output buffer
  }

  // ---- 6. backward only: dx_t = Hn (dy_t F).  The buffer holds (dy_t F) / 64
  // in bf16, so the raw transform of each row finishes it (times pscale:
  // 64 / sqrt(d_in) for a zero-extended row, 1 / sqrt(2) for the halves of a
  // wide one); one wave per token row, or per (token, half) when wide, its
  // transpose scratch in the (now unused) Z tile and row lists.
  if constexpr (BWD) {
    constexpr int JOBS = WIDE ? 2 * TT : TT;
    static_assert(JOBS * G::LDS_ROW * 4 <= L::OUT, "transpose scratch below the output buffer");
    if (wave < JOBS) {
      const int k = WIDE ? wave >> 1 : wave, half = WIDE ? wave & 1 : 0, t = lane;
      float* scratch = reinterpret_cast<float*>(smem) + wave * G::LDS_ROW;
      const uint16_t* orow = obuf + k * Q::NT;
      const uint32_t nomask[4] = {0u, 0u, 0u, 0u};
      float v[64];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        Raw8 raw;
        raw.a = *reinterpret_cast<const u32x4*>(orow + G::idxA(t, c * 8));
        widen8<DT_BF16, false>(raw, v + 8 * c, nomask, 0u);
        if constexpr (WIDE) {
          Raw8 rh;
          rh.a = *reinterpret_cast<const u32x4*>(orow + 4096 + G::idxA(t, c * 8));
          float vh[8];
          widen8<DT_BF16, false>(rh, vh, nomask, 0u);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[8 * c + e] = half ? v[8 * c + e] - vh[e] : v[8 * c + e] + vh[e];
        }
      }
      stages_A<12, false>(v, t);
      transpose_AB<12, 64>(scratch, v, t);
      stages_B<12, 2>(v, t);
      const int c0 = half * 4096 + 64 * t;
      if (k < ntok && c0 < out_cols) {
        const float sg = rho_B<12>(t) ? -pscale : pscale;
#pragma unroll
        for (int e = 0; e < 64; ++e) v[e] *= sg;
        uint16_t* dst = y + (tok0 + k) * ldy + c0;
#pragma unroll
        for (int q = 0; q < 8; ++q) store8<DT_BF16>(dst, 8 * q, v + 8 * q);
      }
    }
  }
}

template <int VALDT, bool BWD, bool WIDE>
static void launch_one(const void* x, int64_t tokens, int64_t ldx, int in_cols, const int32_t* row_ptr,
                       const int32_t* col_idx, const void* vals, int rows, int nnz, void* y, int64_t ldy,
                       int vec, int out_cols, float wscale, float pscale, hipStream_t s) {
  using L = QwLds<BWD, WIDE>;
  static const bool attr = hipFuncSetAttribute((const void*)k_qwha<VALDT, BWD, WIDE>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES) == hipSuccess;
  (void)attr;
  constexpr int TT = QwGeo<BWD, WIDE>::TT;
  const unsigned grid = (unsigned)((tokens + TT - 1) / TT);
  hipLaunchKernelGGL((k_qwha<VALDT, BWD, WIDE>), dim3(grid), dim3(qw::THREADS), L::BYTES, s,
                     (const uint16_t*)x, tokens, ldx, in_cols, row_ptr, col_idx, vals, rows, nnz,
                     (uint16_t*)y, ldy, vec, out_cols, wscale, pscale);
}

template <bool BWD>
static void launch_w(bool wide, int val_dt, const void* x, int64_t tokens, int64_t ldx, int in_cols,
                     const int32_t* row_ptr, const int32_t* col_idx, const void* vals, int rows, int nnz, void* y,
                     int64_t ldy, int vec, int out_cols, float wscale, float pscale, hipStream_t s) {
#define QW_L(VD, WD) launch_one<VD, BWD, WD>(x, tokens, ldx, in_cols, row_ptr, col_idx, vals, rows, nnz, y, ldy, \
                                             vec, out_cols, wscale, pscale, s)
  if (val_dt == DT_BF16) {
    if (wide) QW_L(DT_BF16, true);
    else QW_L(DT_BF16, false);
  } else {
    if (wide) QW_L(DT_F32, true);
    else QW_L(DT_F32, false);
  }
#undef QW_L
}

// Width factors: d_in = 8192 splits on the top index bit (1 / sqrt(2) on
// the 4096-point sums); d_in < 4096 is zero-extended (64 / sqrt(d_in)).
static float qw_width_scale(int64_t d_in) {
  return d_in == 8192 ? (float)(1.0 / std::sqrt(2.0)) : (float)(64.0 / std::sqrt((double)d_in));
}

hipError_t launch_qwha_fwd(const void* x, int64_t tokens, int64_t d_in, int64_t ldx, const int32_t* row_ptr,
                           const int32_t* col_idx, const void* vals, int val_dt, int64_t d_out, int64_t nnz, void* y,
                           int64_t ldy, const void* plan, int64_t plan_bytes, hipStream_t s);

// d_in <= 4096 runs the 16-token matrix-core kernel (qwha_fwd.hip); d_in =
// 8192 the split-transform kernel above
hipError_t launch_qwha(const void* x, int64_t tokens, int64_t d_in, int64_t ldx, const int32_t* row_ptr,
                       const int32_t* col_idx, const void* vals, int val_dt, int64_t d_out, int64_t nnz,
                       void* y, int64_t ldy, const void* plan, int64_t plan_bytes, hipStream_t s) {
  if (d_in <= 4096)
    return launch_qwha_fwd(x, tokens, d_in, ldx, row_ptr, col_idx, vals, val_dt, d_out, nnz, y, ldy, plan,
                           plan_bytes, s);
  // 16-byte output stores need a 16-byte aligned base and row stride
  const int vec_out = ((reinterpret_cast<uintptr_t>(y) & 15u) == 0 && (ldy * 2) % 16 == 0) ? 1 : 0;
  launch_w<false>(d_in == 8192, val_dt, x, tokens, ldx, (int)d_in, row_ptr, col_idx, vals, (int)d_out, (int)nnz,
                  y, ldy, vec_out, 0, qw_width_scale(d_in), 1.0f, s);
  return hipGetLastError();
}

// dx = (dy F) Hn from the CSR of F^T (d_in rows whose entries index the d_out
// columns of dy).
hipError_t launch_qwha_bwd_input(const void* dy, int64_t tokens, int64_t lddy, int64_t d_out,
                                 const int32_t* t_row_ptr, const int32_t* t_col_idx, const void* t_vals,
                                 int val_dt, int64_t d_in, int64_t nnz, void* dx, int64_t lddx, hipStream_t s) {
  // 16-byte dy loads need a 16-byte aligned base and row stride
  const int vec_in = ((reinterpret_cast<uintptr_t>(dy) & 15u) == 0 && (lddy * 2) % 16 == 0) ? 1 : 0;
  launch_w<true>(d_in == 8192, val_dt, dy, tokens, lddy, (int)d_out, t_row_ptr, t_col_idx, t_vals, (int)d_in,
                 (int)nnz, dx, lddx, vec_in, (int)d_in, 1.0f, qw_width_scale(d_in), s);
  return hipGetLastError();
}

}  // namespace whtq
