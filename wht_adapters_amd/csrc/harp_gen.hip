// harp_rotate for a general mixed-radix schedule.
//
// HARP explainer, 2.1: a schedule b = (b_0 .. b_{m-1}) with prod b_t = d; stage t
// applies d / b_t independent orthogonal b_t x b_t blocks, each to the
// coordinates that share every digit but digit t (a stride permutation of
// the coordinates, e.g. 8.8.8.5.2 for d = 5120).  Digit t of index i is
// (i / s_t) mod b_t with s_t = b_0 ... b_{t-1}; block c = i with digit t
// removed (remaining digits in increasing significance), i.e. its
// coordinates are base + k s_t, base = (c mod s_t) + (c / s_t) s_t b_t;
// out_sub[k] = sum_j B[k][j] in_sub[j].  With preconditioning (d a power of
// two), the randomized Hadamard transform Hn S runs first: the sign flips as
// the row is loaded and Hn = (x) H_{2^a} / 2^(a/2) over a split of the index
// bits into digits of at most 16 values, each an in-register Hadamard stage.
//
// One block per tile of tt tokens (as many as fit in LDS, at most 16): the
// tile stays in LDS in fp32 across every stage, one stage per barrier.  A
// stage's work items are (block c, row chunk): a lane holds its chunk of
// the block's coefficients in registers (the whole block when b <= 8, a
// quarter when b > 8; the four lanes of one block sit in one wave, so all
// of them read their inputs before any of them writes) and runs every token
// of the tile through it; for small d the items are spread over tokens too.
// fp32 arithmetic throughout (fp16 blocks are widened exactly); the output
// is rounded once to bf16.  VALU-bound by design: b^2 FMAs per coordinate
// per stage (the radix-16 d = 4096 schedule has its own MFMA kernel).
#include "io.hpp"
#include "launch.hpp"

namespace whtq {

namespace hg {
constexpr int THREADS = 1024;
constexpr int MAXST = 20;          // stages, preconditioning factors included
constexpr int MAXTT = 16;
constexpr int LDS_FLOATS = 38912;  // 152 KB of tile
// one float of padding per 32: strided digit accesses spread over the banks
__device__ __forceinline__ int pos(int i) { return i + (i >> 5); }
inline int pos_h(int i) { return i + (i >> 5); }
}  // namespace hg

struct HgSched {
  int n;                       // stages to run
  int b[hg::MAXST];            // radix
  int s[hg::MAXST];            // stride of the digit
  int had[hg::MAXST];          // 1: fixed Hadamard factor H_b / sqrt(b)
  long long off[hg::MAXST];    // element offset of the stage's blocks
};

template <int BDT>
__device__ __forceinline__ float blk_at(const void* blocks, long long i) {
  if constexpr (BDT == DT_F32) return reinterpret_cast<const float*>(blocks)[i];
  else return (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(blocks)[i]);
}

// N consecutive block coefficients from element e0, widened to fp32: 16-byte
// loads where the run is a whole number of aligned 16-byte pieces (blocks of
// radix 2 to 16 in fp32, 4 to 16 in fp16, whose runs start on such
// boundaries), element loads otherwise
template <int BDT, int N>
__device__ __forceinline__ void blk_run(const void* blocks, long long e0, float* co) {
  constexpr int ESZ = BDT == DT_F32 ? 4 : 2;
  const uint8_t* p = reinterpret_cast<const uint8_t*>(blocks) + e0 * ESZ;
  if constexpr ((N * ESZ) % 16 == 0) {
    if ((reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
#pragma unroll
      for (int v = 0; v < N * ESZ / 16; ++v) {
        const u32x4 w = ldg<u32x4>(p + 16 * v);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (ESZ == 4) {
            co[4 * v + q] = as_f(w[q]);
          } else {
            co[8 * v + 2 * q] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[q] & 0xffffu));
            co[8 * v + 2 * q + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[q] >> 16));
          }
        }
      }
      return;
    }
  }
#pragma unroll
  for (int k = 0; k < N; ++k) co[k] = blk_at<BDT>(blocks, e0 + k);
}

// in-register Sylvester FWHT of B values (B a power of two), scaled by 1/sqrt(B)
template <int B>
__device__ __forceinline__ void had_regs(float (&x)[B]) {
#pragma unroll
  for (int m = 1; m < B; m <<= 1)
#pragma unroll
    for (int k = 0; k < B; ++k)
      if (!(k & m)) bfly(x[k], x[k | m]);
  const float sc = B == 2 ? 0.70710678118654752f : B == 4 ? 0.5f : B == 8 ? 0.35355339059327376f : 0.25f;
#pragma unroll
  for (int k = 0; k < B; ++k) x[k] *= sc;
}

template <int B, int BDT>
__device__ __forceinline__ void hg_stage(float* tile, int ldt, int nt, int d, int s, const void* blocks,
                                         long long off) {
  constexpr int LPB = B <= 8 ? 1 : 4;            // lanes per block
  constexpr int RPL = (B + LPB - 1) / LPB;       // rows per lane
  const int items = (d / B) * LPB;
  // token loop inside the item (coefficients loaded once per tile) when the
  // items fill the block; otherwise items and tokens are spread together
  const bool spread = items < hg::THREADS / 2;
  const int total = spread ? items * nt : items;
  for (int f = threadIdx.x; f < total; f += hg::THREADS) {
    const int it = spread ? f % items : f;
    const int j0 = spread ? f / items : 0, j1 = spread ? j0 + 1 : nt;
    const int c = it / LPB, r0 = (it - c * LPB) * RPL;
    const int base = (c % s) + (c / s) * s * B;
    float co[RPL][B];
    const long long bo = off + (long long)c * B * B;
    if constexpr (RPL * LPB == B) {
      // the lane's rows r0 .. r0 + RPL - 1 are one contiguous run of the block
      blk_run<BDT, RPL * B>(blocks, bo + (long long)r0 * B, &co[0][0]);
    } else {
#pragma unroll
      for (int r = 0; r < RPL; ++r)
#pragma unroll
        for (int k = 0; k < B; ++k) co[r][k] = r0 + r < B ? blk_at<BDT>(blocks, bo + (r0 + r) * B + k) : 0.f;
    }
    // the item's LDS addresses, computed once for all its tokens (rows past
    // the block's end, in the last lane of a split block, write nowhere)
    int ia[B], oa[RPL];
#pragma unroll
    for (int k = 0; k < B; ++k) ia[k] = hg::pos(base + k * s);
#pragma unroll
    for (int r = 0; r < RPL; ++r) oa[r] = r0 + r < B ? hg::pos(base + (r0 + r) * s) : -1;
    for (int j = j0; j < j1; ++j) {
      float* row = tile + j * ldt;
      float xv[B];
#pragma unroll
      for (int k = 0; k < B; ++k) xv[k] = row[ia[k]];
      float yv[RPL];
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        float a = 0.f;
#pragma unroll
        for (int k = 0; k < B; ++k) a = fmaf(co[r][k], xv[k], a);
        yv[r] = a;
      }
#pragma unroll
      for (int r = 0; r < RPL; ++r)
        if (RPL * LPB == B || oa[r] >= 0) row[oa[r]] = yv[r];
    }
  }
}

// A fixed Hadamard factor H_B / sqrt(B) along a digit: one lane per group
// and token, the group's B values through in-register butterflies.
template <int B>
__device__ __forceinline__ void hg_had(float* tile, int ldt, int nt, int d, int s) {
  const int groups = d / B;
  for (int f = threadIdx.x; f < groups * nt; f += hg::THREADS) {
    const int j = f / groups, c = f - j * groups;
    const int base = (c % s) + (c / s) * s * B;
    float* row = tile + j * ldt;
    int ia[B];
#pragma unroll
    for (int k = 0; k < B; ++k) ia[k] = hg::pos(base + k * s);
    float xv[B];
#pragma unroll
    for (int k = 0; k < B; ++k) xv[k] = row[ia[k]];
    had_regs<B>(xv);
#pragma unroll
    for (int k = 0; k < B; ++k) row[ia[k]] = xv[k];
  }
}

template <int BDT, int XDT>
__global__ __launch_bounds__(hg::THREADS) void k_harp_gen(const void* __restrict__ xv_, void* __restrict__ yv_,
                                                         int64_t tokens, int64_t ldx, int64_t ldy, int d, int ldt,
                                                         int tt, const uint32_t* __restrict__ sbits,
                                                         const void* __restrict__ blocks, HgSched sc, int vec) {
  extern __shared__ __align__(16) float tile[];
  const int64_t tok0 = (int64_t)blockIdx.x * tt;
  const int nt = (int)min<int64_t>(tt, tokens - tok0);
  const int nch = (d + 7) >> 3;  // 8-value chunks per row

  // ---- load (signs flipped on the way when preconditioning); rows are bf16
  // or fp32 (XDT), the tile fp32 either way.  Every 8-value chunk of the
  // tile goes to one thread; a thread's chunks are all requested before any
  // is written,
  // so the tile costs one memory latency rather than one per chunk (the
  // tile's tt d values fit in LDS_FLOATS, so a thread has at most LDCH chunks).
  constexpr int LDCH = (hg::LDS_FLOATS / 8 + hg::THREADS - 1) / hg::THREADS;
  {
    constexpr int W = XDT == DT_F32 ? 8 : 4;  // 32-bit words per chunk
    uint32_t raw[LDCH][W];
    const int nf = nt * nch;
#pragma unroll
    for (int u = 0; u < LDCH; ++u) {
      const int f = threadIdx.x + u * hg::THREADS;
      if (f < nf) {
        const int j = f / nch, i0 = 8 * (f - j * nch);
        if (vec && i0 + 8 <= d) {
          if constexpr (XDT == DT_F32) {
            const float* xr = reinterpret_cast<const float*>(xv_) + (tok0 + j) * ldx;
            const u32x4 a = ldg<u32x4>(xr + i0), b = ldg<u32x4>(xr + i0 + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              raw[u][q] = a[q];
              raw[u][4 + q] = b[q];
            }
          } else {
            const uint16_t* xr = reinterpret_cast<const uint16_t*>(xv_) + (tok0 + j) * ldx;
            const u32x4 w = ldg<u32x4>(xr + i0);
#pragma unroll
            for (int q = 0; q < 4; ++q) raw[u][q] = w[q];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < LDCH; ++u) {
      const int f = threadIdx.x + u * hg::THREADS;
      if (f < nf) {
        const int j = f / nch, i0 = 8 * (f - j * nch);
        const uint32_t sb = sbits ? (sbits[i0 >> 5] >> (i0 & 31)) & 0xffu : 0u;
        float v[8];
        if (vec && i0 + 8 <= d) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            v[e] = XDT == DT_F32 ? as_f(raw[u][e]) : ((e & 1) ? bf16hi(raw[u][e >> 1]) : bf16lo(raw[u][e >> 1]));
        } else if constexpr (XDT == DT_F32) {
          const float* xr = reinterpret_cast<const float*>(xv_) + (tok0 + j) * ldx;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = i0 + e < d ? xr[i0 + e] : 0.f;
        } else {
          const uint16_t* xr = reinterpret_cast<const uint16_t*>(xv_) + (tok0 + j) * ldx;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = i0 + e < d ? as_f((uint32_t)xr[i0 + e] << 16) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (i0 + e < d) tile[j * ldt + hg::pos(i0 + e)] = as_f(as_u(v[e]) ^ (((sb >> e) & 1u) << 31));
      }
    }
  }
  __syncthreads();

  // ---- stages
  for (int t = 0; t < sc.n; ++t) {
    if (sc.had[t]) {
      switch (sc.b[t]) {
        case 2: hg_had<2>(tile, ldt, nt, d, sc.s[t]); break;
        case 4: hg_had<4>(tile, ldt, nt, d, sc.s[t]); break;
        case 8: hg_had<8>(tile, ldt, nt, d, sc.s[t]); break;
        case 16: hg_had<16>(tile, ldt, nt, d, sc.s[t]); break;
        default: break;
      }
      __syncthreads();
      continue;
    }
    switch (sc.b[t]) {
#define HG_CASE(B) \
  case B: hg_stage<B, BDT>(tile, ldt, nt, d, sc.s[t], blocks, sc.off[t]); break;
      HG_CASE(2) HG_CASE(3) HG_CASE(4) HG_CASE(5) HG_CASE(6) HG_CASE(7) HG_CASE(8) HG_CASE(9)
      HG_CASE(10) HG_CASE(11) HG_CASE(12) HG_CASE(13) HG_CASE(14) HG_CASE(15) HG_CASE(16)
#undef HG_CASE
      default: break;
    }
    __syncthreads();
  }

  // ---- store: fp32 as is, or rounded once to bf16
  for (int f = threadIdx.x; f < nt * nch; f += hg::THREADS) {
    const int j = f / nch, i0 = 8 * (f - j * nch);
    const float* row = tile + j * ldt;
    if constexpr (XDT == DT_F32) {
      float* yr = reinterpret_cast<float*>(yv_) + (tok0 + j) * ldy;
      if (vec && i0 + 8 <= d) {
        stg(yr + i0, f32x4{row[hg::pos(i0)], row[hg::pos(i0 + 1)], row[hg::pos(i0 + 2)], row[hg::pos(i0 + 3)]});
        stg(yr + i0 + 4,
            f32x4{row[hg::pos(i0 + 4)], row[hg::pos(i0 + 5)], row[hg::pos(i0 + 6)], row[hg::pos(i0 + 7)]});
      } else {
        for (int e = 0; e < 8 && i0 + e < d; ++e) yr[i0 + e] = row[hg::pos(i0 + e)];
      }
    } else {
      uint16_t* yr = reinterpret_cast<uint16_t*>(yv_) + (tok0 + j) * ldy;
      if (vec && i0 + 8 <= d) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = pack_bf16(row[hg::pos(i0 + 2 * q)], row[hg::pos(i0 + 2 * q + 1)]);
        stg(yr + i0, w);
      } else {
        for (int e = 0; e < 8 && i0 + e < d; ++e)
          yr[i0 + e] = (uint16_t)(pack_bf16(row[hg::pos(i0 + e)], 0.f) & 0xffffu);
      }
    }
  }
}

// Entry from the C ABI (arguments validated there): radices each in [2, 16],
// product d <= 8192, precondition only for d a power of two.
template <int BDT, int XDT>
static void launch_hg(const void* x, void* y, int64_t tokens, int64_t ldx, int64_t ldy, int d, int ldt, int tt,
                      const uint32_t* sbits, const void* blocks, const HgSched& sc, int vec, unsigned grid,
                      size_t lds, hipStream_t s) {
  static const bool a = hipFuncSetAttribute((const void*)k_harp_gen<BDT, XDT>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, hg::LDS_FLOATS * 4) ==
                        hipSuccess;
  (void)a;
  hipLaunchKernelGGL((k_harp_gen<BDT, XDT>), dim3(grid), dim3(hg::THREADS), lds, s, x, y, tokens, ldx, ldy, d, ldt,
                     tt, sbits, blocks, sc, vec);
}

hipError_t launch_harp_gen(const void* x, void* y, int xdt, int64_t tokens, int d, int64_t ldx, int64_t ldy,
                           const uint32_t* sbits, int precondition, const int32_t* radices, int n_stages,
                           const void* blocks, int bdt, hipStream_t s) {
  HgSched sc{};
  int n = 0;
  if (precondition) {
    int logd = 0;
    while ((1 << logd) < d) ++logd;
    int stride = 1;
    for (int bits = logd; bits > 0;) {  // digits of 16 values, the last one smaller
      const int e = bits >= 4 ? 4 : bits;
      sc.b[n] = 1 << e;
      sc.s[n] = stride;
      sc.had[n] = 1;
      sc.off[n] = 0;
      stride <<= e;
      bits -= e;
      ++n;
    }
  }
  long long off = 0;
  int stride = 1;
  for (int t = 0; t < n_stages; ++t) {
    sc.b[n] = radices[t];
    sc.s[n] = stride;
    sc.had[n] = 0;
    sc.off[n] = off;
    off += (long long)d * radices[t];
    stride *= radices[t];
    ++n;
  }
  sc.n = n;
  const int ldt = (hg::pos_h(d - 1) + 4) & ~3;
  const int tt = std::max(1, std::min(hg::MAXTT, hg::LDS_FLOATS / ldt));
  const size_t lds = (size_t)tt * ldt * sizeof(float);
  // 16-byte row accesses need a 16-byte aligned base and row stride on both sides
  const int esz = xdt == DT_F32 ? 4 : 2;
  const int vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0 &&
                          (ldx * esz) % 16 == 0 && (ldy * esz) % 16 == 0
                      ? 1 : 0;
  const unsigned grid = (unsigned)((tokens + tt - 1) / tt);
  const uint32_t* sb = precondition ? sbits : nullptr;
  if (bdt == DT_F16 && xdt == DT_F32) launch_hg<DT_F16, DT_F32>(x, y, tokens, ldx, ldy, d, ldt, tt, sb, blocks, sc, vec, grid, lds, s);
  else if (bdt == DT_F16) launch_hg<DT_F16, DT_BF16>(x, y, tokens, ldx, ldy, d, ldt, tt, sb, blocks, sc, vec, grid, lds, s);
  else if (xdt == DT_F32) launch_hg<DT_F32, DT_F32>(x, y, tokens, ldx, ldy, d, ldt, tt, sb, blocks, sc, vec, grid, lds, s);
  else launch_hg<DT_F32, DT_BF16>(x, y, tokens, ldx, ldy, d, ldt, tt, sb, blocks, sc, vec, grid, lds, s);
  return hipGetLastError();
}

}  // namespace whtq
