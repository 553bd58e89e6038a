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
// One block per tile of tt tokens (as many as fit in its share of LDS, at
// most 16): 1024 threads and the whole LDS per block, or for d <= 4717 two
// 512-thread blocks per CU with half of it each, so that one block's row
// loads overlap the other's stages.  The tile stays in LDS in fp32 across
// every stage, one stage per barrier.  A
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
// tile floats per block of nt threads: 1024 threads, one block per CU; 512
// threads, two blocks per CU (half the tile each)
__host__ __device__ constexpr int lds_floats(int nt) { return nt == THREADS ? LDS_FLOATS : LDS_FLOATS / 2; }
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

template <int B, int BDT, int NT>
__device__ __forceinline__ void hg_stage(float* tile, int ldt, int nt, int d, int s, const void* blocks,
                                         long long off) {
  constexpr int LPB = B <= 8 ? 1 : 4;            // lanes per block
  constexpr int RPL = (B + LPB - 1) / LPB;       // rows per lane
  const int items = (d / B) * LPB;
  // token loop inside the item (coefficients loaded once per tile) when the
  // items fill the block; otherwise items and tokens are spread together
  const bool spread = items < NT / 2;
  const int total = spread ? items * nt : items;
  for (int f = threadIdx.x; f < total; f += NT) {
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
template <int B, int NT>
__device__ __forceinline__ void hg_had(float* tile, int ldt, int nt, int d, int s) {
  const int groups = d / B;
  for (int f = threadIdx.x; f < groups * nt; f += NT) {
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

template <int BDT, int XDT, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void k_harp_gen(const void* __restrict__ xv_, void* __restrict__ yv_,
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
  // tile's tt d values fit in lds_floats(NT), so a thread has at most LDCH chunks).
  constexpr int LDCH = (hg::lds_floats(NT) / 8 + NT - 1) / NT;
  {
    constexpr int W = XDT == DT_F32 ? 8 : 4;  // 32-bit words per chunk
    uint32_t raw[LDCH][W];
    const int nf = nt * nch;
#pragma unroll
    for (int u = 0; u < LDCH; ++u) {
      const int f = threadIdx.x + u * NT;
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
      const int f = threadIdx.x + u * NT;
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
        case 2: hg_had<2, NT>(tile, ldt, nt, d, sc.s[t]); break;
        case 4: hg_had<4, NT>(tile, ldt, nt, d, sc.s[t]); break;
        case 8: hg_had<8, NT>(tile, ldt, nt, d, sc.s[t]); break;
        case 16: hg_had<16, NT>(tile, ldt, nt, d, sc.s[t]); break;
        default: break;
      }
      __syncthreads();
      continue;
    }
    switch (sc.b[t]) {
#define HG_CASE(B) \
  case B: hg_stage<B, BDT, NT>(tile, ldt, nt, d, sc.s[t], blocks, sc.off[t]); break;
      HG_CASE(2) HG_CASE(3) HG_CASE(4) HG_CASE(5) HG_CASE(6) HG_CASE(7) HG_CASE(8) HG_CASE(9)
      HG_CASE(10) HG_CASE(11) HG_CASE(12) HG_CASE(13) HG_CASE(14) HG_CASE(15) HG_CASE(16)
#undef HG_CASE
      default: break;
    }
    __syncthreads();
  }

  // ---- store: fp32 as is, or rounded once to bf16
  for (int f = threadIdx.x; f < nt * nch; f += NT) {
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

// ------------------------------------------------- bf16 rows on the matrix cores
//
// bf16 rows (output tolerance 2e-2) of small d take fp16 MFMAs with fp32
// accumulation, as the radix-16 kernel's stages do.  The tile holds TT tokens
// token-fastest: element i of all TT tokens is one slot of 2 TT bytes, each
// token scaled by an exact power of two from its largest |x_i|.  A stage of
// radix b packs P = 16 / b blocks block-diagonally into one 16 x 16 operand
// Bp and computes, per MFMA, D^T = X Bp^T for the 16 token lanes:
//   A = X[token][j]: one transposing LDS read per lane.  ds_read_b64_tr_b16
//       gives lane 4p + e of a 16-lane group halfword e of the 8 bytes
//       addressed by lanes p, p + 4, p + 8 and p + 12; those lanes address
//       token quad p of the inputs j = 4g .. 4g + 3, so lane 4p + e receives
//       token 4p + e of all four;
//   B = Bp^T: lane (k, g) holds row k of Bp at columns 4g .. 4g + 3 (zero
//       outside the row's own block);
//   D^T[token][k]: lane (k, g) holds tokens 4g .. 4g + 3 of output k, one
//       8-byte write into the tile (in place: the same elements were read).
// The P blocks of one MFMA are consecutive blocks c0 .. c0 + P - 1 of one
// run of s blocks (s the digit's stride; a run's blocks share the digits
// above) when s >= P, else P' = floor(P / s) s blocks making whole runs:
// either way an element is a wave-uniform base plus a per-lane offset fixed
// for the stage, so addressing costs a few VALU operations per MFMA.  Each
// wave takes a contiguous range of MFMAs; their coefficients are loaded PD
// MFMAs ahead (unconditional loads, combined when used) and the next MFMA's
// inputs are read before the current one runs.  The MFMA count per token
// grows with the number of stages, not with the radices, and the fixed cost
// per MFMA is several times the VALU kernel's per coefficient, so this form
// is used where it measured faster: d <= 3072 (at 4096 and above, with one
// 8-wave block per CU, the VALU kernel was as fast or faster) and a mean
// radix of at least 4 (radix-2 chains stay on the VALU kernel).
namespace hm {
constexpr int THREADS = 512;
constexpr int PD = 8;  // coefficient loads run PD MFMAs ahead (L2 latency)
constexpr int NW = THREADS / 64;
constexpr int MAXR = 12;  // 16-byte chunks a lane loads per tile (16 tokens, d <= 3072)
__host__ __device__ constexpr int slot(int i) { return i; }
template <int TT>
__host__ __device__ constexpr int tile_bytes(int d) { return (slot(d - 1) + 1) * 2 * TT; }
}  // namespace hm

typedef short hm_s16x4 __attribute__((ext_vector_type(4)));
typedef float hm_f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 hm_f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 hm_tr_read(const uint8_t* smem, int off) {
  const hm_s16x4 v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) hm_s16x4*)(smem + off));
  return __builtin_bit_cast(u32x2, v);
}

// coefficient (row r, column col) of block c, rounded to fp16 bits
template <int BDT>
__device__ __forceinline__ uint32_t hm_coef(const void* blocks, long long i) {
  if constexpr (BDT == DT_F32)
    return __builtin_bit_cast(uint16_t, (_Float16)reinterpret_cast<const float*>(blocks)[i]);
  else
    return reinterpret_cast<const uint16_t*>(blocks)[i];
}


// WIDE: the digit's stride s >= P, P consecutive blocks of one run per MFMA;
// HAD: a fixed Hadamard factor (coefficients computed, nothing loaded)
template <int B, int BDT, int TT, bool WIDE, bool HAD>
__device__ __forceinline__ void hm_stage_w(uint8_t* smem, int d, int st, const void* blocks, long long off, int w,
                                           int lane) {
  constexpr int S = 2 * TT;
  constexpr int P = 16 / B;
  constexpr int PD = hm::PD;
  constexpr int ESZ = BDT == DT_F32 ? 4 : 2;
  const int nblk = d / B;
  const int PP = WIDE ? P : (P / st) * st;      // blocks per MFMA
  const int mpr = WIDE ? (st + P - 1) / P : 1;  // MFMAs per run of st blocks
  const int nmf = WIDE ? (nblk / st) * mpr : (nblk + PP - 1) / PP;
  // the wave's MFMAs: a contiguous range [m0, m1)
  const int per = (nmf + hm::NW - 1) / hm::NW;
  const int m0 = min(nmf, w * per), m1 = min(nmf, m0 + per);
  if (m0 >= m1) return;
  const int g = lane >> 4, l16 = lane & 15;
  // this lane as a source of the transposing read: contraction index ja, token quad qa
  const int ja = 4 * g + (l16 >> 2), qa = l16 & 3;
  const int pa = ja / B, ra = ja - pa * B;
  const bool ina = pa < PP;
  const int da = !ina ? 0 : WIDE ? pa + ra * st : (pa % st) + (pa / st) * st * B + ra * st;
  const int qoff = 8 * ((4 * qa < TT) ? qa : 0);  // token quads past TT read quad 0 (outputs unused)
  const int aoff = da * S + qoff;                 // LDS bytes from the MFMA's base element
  const int pa_s = ina ? pa : 1 << 20;            // block of the input slot (never below nv when unused)
  // this lane as output k = l16 (row rk of block pk), tokens 4g .. 4g + 3
  const int pk = l16 / B, rk = l16 - pk * B;
  const bool ink = pk < PP;
  const int dk = !ink ? 0 : WIDE ? pk + rk * st : (pk % st) + (pk / st) * st * B + rk * st;
  const int ooff = dk * S + 8 * g;
  // row k's coefficients at columns 4g + jj: in block pk for column 4g + jj - pk B in [0, B)
  unsigned cm = 0;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int col = 4 * g + jj - pk * B;
    if (ink && col >= 0 && col < B) cm |= 1u << jj;
  }
  // the lane writes output k for tokens 4g .. 4g + 3 when its block is present
  // (as an operand lane it holds columns 4g .. 4g + 3 of row k: a separate role)
  const int pk_s = (ink && 4 * g < TT) ? pk : 1 << 20;
  const int pk_c = cm != 0u ? pk : 1 << 20;
  const int h2 = (cm & 1u) ? 0 : 1;  // radix 2: the row's two columns are the first or second pair
  // byte offset of the lane's first coefficient within its MFMA's block group
  const uint32_t cboff = cm ? (uint32_t)(pk * B * B + rk * B - pk * B + 4 * g + (B == 2 ? 2 * h2 : 0)) * ESZ : 0u;
  uint32_t hw[2] = {0u, 0u};
  if constexpr (HAD) {
    const float hs = B == 2 ? 0.70710678118654752f : B == 4 ? 0.5f : B == 8 ? 0.35355339059327376f : 0.25f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (cm & (1u << jj)) {
        const int col = 4 * g + jj - pk * B;
        const float v = (__builtin_popcount(rk & col) & 1) ? -hs : hs;
        hw[jj >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v) << (16 * (jj & 1));
      }
  }
  // wave-uniform MFMA state: base element e0, valid blocks nv, first block c0
  int run = WIDE ? m0 / mpr : 0;
  int idx = WIDE ? m0 - run * mpr : m0 * PP;
  auto cur = [&](int& pe0, int& pnv, int& pc0) {
    if constexpr (WIDE) {
      pc0 = run * st + idx * P;
      pnv = min(P, st - idx * P);
      pe0 = idx * P + run * st * B;
    } else {
      pc0 = idx;
      pnv = min(PP, nblk - idx);
      pe0 = idx * B;
    }
  };
  auto step = [&]() {
    if constexpr (WIDE) {
      ++idx;
      run += idx == mpr ? 1 : 0;
      idx = idx == mpr ? 0 : idx;
    } else {
      idx += PP;
    }
  };
  const uint8_t* bbase = reinterpret_cast<const uint8_t*>(blocks) + off * ESZ;
  // one MFMA's coefficients as loaded (unconditional loads: rows without
  // coefficients in the MFMA read its first coefficient)
  struct Raw {
    uint32_t v[4];  // fp16 words or halfwords, or fp32 bits
  };
  auto cload = [&](int pnv, int pc0) {
    Raw r{};
    if constexpr (!HAD) {
      const uint8_t* bp = bbase + (size_t)pc0 * (B * B * ESZ) + (pk_c < pnv ? cboff : 0u);
      if constexpr (BDT == DT_F16) {
        if constexpr (B % 4 == 0) {
          const u32x2 v = ldg<u32x2>(bp);
          r.v[0] = v.x;
          r.v[1] = v.y;
        } else if constexpr (B == 2) {
          r.v[0] = ldg<uint32_t>(bp);
        } else {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) r.v[jj] = ldg<uint16_t>(bp + ((cm >> jj) & 1u) * 2 * jj);
        }
      } else {
        if constexpr (B % 4 == 0) {
          const u32x4 v = ldg<u32x4>(bp);
#pragma unroll
          for (int q = 0; q < 4; ++q) r.v[q] = v[q];
        } else if constexpr (B == 2) {
          const u32x2 v = ldg<u32x2>(bp);
          r.v[0] = v.x;
          r.v[1] = v.y;
        } else {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) r.v[jj] = ldg<uint32_t>(bp + ((cm >> jj) & 1u) * 4 * jj);
        }
      }
    }
    return r;
  };
  auto cword = [&](const Raw& r, int pnv) -> u32x2 {
    const bool ok = pk_c < pnv;
    u32x2 c;
    if constexpr (HAD) {
      c = u32x2{hw[0], hw[1]};
    } else if constexpr (BDT == DT_F16) {
      if constexpr (B % 4 == 0) c = u32x2{r.v[0], r.v[1]};
      else if constexpr (B == 2) c = h2 ? u32x2{0u, r.v[0]} : u32x2{r.v[0], 0u};
      else {
        uint32_t hv[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) hv[jj] = (cm & (1u << jj)) ? (r.v[jj] & 0xffffu) : 0u;
        c = u32x2{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16)};
      }
    } else {
      if constexpr (B % 4 == 0) c = u32x2{pack_f16(as_f(r.v[0]), as_f(r.v[1])), pack_f16(as_f(r.v[2]), as_f(r.v[3]))};
      else if constexpr (B == 2) {
        const uint32_t pw = pack_f16(as_f(r.v[0]), as_f(r.v[1]));
        c = h2 ? u32x2{0u, pw} : u32x2{pw, 0u};
      } else {
        float fv[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) fv[jj] = (cm & (1u << jj)) ? as_f(r.v[jj]) : 0.f;
        c = u32x2{pack_f16(fv[0], fv[1]), pack_f16(fv[2], fv[3])};
      }
    }
    return ok ? c : u32x2{0u, 0u};
  };
  // an MFMA's inputs; slots of blocks missing from a partial MFMA (and MFMAs
  // past the range, nv = 0) read its base element, times zero weights
  auto xread = [&](int pe0, int pnv) { return hm_tr_read(smem, pe0 * S + (pa_s < pnv ? aoff : qoff)); };
  int re0[PD], rnv[PD];
  Raw cq[PD];
#pragma unroll
  for (int u = 0; u < PD; ++u) {
    int c0 = 0;
    re0[u] = 0;
    rnv[u] = 0;
    if (m0 + u < m1) {
      cur(re0[u], rnv[u], c0);
      step();
    }
    cq[u] = cload(rnv[u], c0);
  }
  u32x2 xn = xread(re0[0], rnv[0]);
  for (int base = m0; base < m1; base += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      if (base + u < m1) {
        const int e0 = re0[u], nv = rnv[u];
        const u32x2 xa = xn;
        xn = xread(re0[(u + 1) % PD], rnv[(u + 1) % PD]);  // the next MFMA's inputs: other blocks, other elements
        const u32x2 cw = cword(cq[u], nv);
        int c0 = 0;
        re0[u] = 0;
        rnv[u] = 0;
        if (base + u + PD < m1) {
          cur(re0[u], rnv[u], c0);
          step();
        }
        cq[u] = cload(rnv[u], c0);  // the MFMA PD ahead
        const f32x4 dv = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(hm_f16x4, xa),
                                                               __builtin_bit_cast(hm_f16x4, cw),
                                                               f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        if (pk_s < nv)
          *reinterpret_cast<u32x2*>(smem + e0 * S + ooff) = u32x2{pack_f16(dv[0], dv[1]), pack_f16(dv[2], dv[3])};
      }
    }
  }
}

template <int B, int BDT, int TT>
__device__ __forceinline__ void hm_stage(uint8_t* smem, int d, int st, bool had, const void* blocks, long long off,
                                         int w, int lane) {
  constexpr bool H = B == 2 || B == 4 || B == 8 || B == 16;
  // a fresh copy of the lane index per stage: the per-lane constants of every
  // radix would otherwise be hoisted out of the stage loop and stay live
  asm volatile("" : "+v"(lane));
  if (st >= 16 / B) {
    if (H && had) hm_stage_w<B, BDT, TT, true, H>(smem, d, st, blocks, off, w, lane);
    else hm_stage_w<B, BDT, TT, true, false>(smem, d, st, blocks, off, w, lane);
  } else {
    if (H && had) hm_stage_w<B, BDT, TT, false, H>(smem, d, st, blocks, off, w, lane);
    else hm_stage_w<B, BDT, TT, false, false>(smem, d, st, blocks, off, w, lane);
  }
}

template <int BDT, int TT>
__global__ __launch_bounds__(hm::THREADS) void k_harp_mx(const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                        int64_t tokens, int64_t ldx, int64_t ldy, int d, int lgd,
                                                        const uint32_t* __restrict__ sbits,
                                                        const void* __restrict__ blocks, HgSched sc) {
  constexpr int S = 2 * TT;
  constexpr int GPW = 64 / TT;  // token groups of a wave in the row phases
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* tmax = reinterpret_cast<uint32_t*>(smem + ((hm::tile_bytes<TT>(d) + 15) & ~15));
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int64_t tok0 = (int64_t)blockIdx.x * TT;
  if (threadIdx.x < 16) tmax[threadIdx.x] = 0u;
  __syncthreads();

  // ---- load: lane (token jt, group gq) takes 16-byte chunks cc = (u NW + w) GPW + gq
  // of its token's row (signs flipped on the way when preconditioning)
  const int jt = lane % TT, gq = lane / TT;
  const int nch = d >> 3;
  const bool lact = gq < GPW && tok0 + jt < tokens;
  const uint16_t* xr = x + (tok0 + jt) * ldx;
  u32x4 raw[hm::MAXR];
  uint32_t mb = 0u;
#pragma unroll
  for (int u = 0; u < hm::MAXR; ++u) {
    const int cc = (u * hm::NW + w) * GPW + gq;
    raw[u] = u32x4{0u, 0u, 0u, 0u};
    if (lact && cc < nch) {
      u32x4 v = ldg<u32x4>(xr + 8 * cc);
      if (sbits) {
        const int i0 = 8 * cc;
        const uint32_t sb = (sbits[i0 >> 5] >> (i0 & 31)) & 0xffu;
        v ^= u32x4{pair_mask16(sb), pair_mask16(sb >> 2), pair_mask16(sb >> 4), pair_mask16(sb >> 6)};
      }
      raw[u] = v;
    }
  }
  {
    u16x2 am{0, 0};
#pragma unroll
    for (int u = 0; u < hm::MAXR; ++u) {
      const u32x4 v = raw[u];
      am = absmax16(absmax16(absmax16(absmax16(am, v.x), v.y), v.z), v.w);
    }
    mb = absmax16(am);
  }
  if (lact) atomicMax(&tmax[jt], mb);
  __syncthreads();
  // power-of-two scale per token: ||x|| <= sqrt(d) max |x_i| < 2^e with
  // e = exp(max) + ceil(log2 sqrt(d)), so every stage's values (the stages
  // being orthogonal) stay below 2^14 after multiplying by 2^(14 - e);
  // e >= -112 keeps both factors normal fp32 numbers
  auto tok_exp = [&](int j) {
    const uint32_t m = tmax[j];
    const int e = bf16_mag_exp(m) + lgd;
    return m ? (e > -112 ? e : -112) : 0;
  };
  {
    const float scl = ldexpf(1.0f, 14 - tok_exp(jt));
#pragma unroll
    for (int u = 0; u < hm::MAXR; ++u) {
      const int cc = (u * hm::NW + w) * GPW + gq;
      if (gq < GPW && cc < nch) {
        const u32x4 v = raw[u];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = 8 * cc + 2 * q;
          *reinterpret_cast<_Float16*>(smem + hm::slot(i) * S + 2 * jt) = (_Float16)(bf16lo(v[q]) * scl);
          *reinterpret_cast<_Float16*>(smem + hm::slot(i + 1) * S + 2 * jt) = (_Float16)(bf16hi(v[q]) * scl);
        }
      }
    }
  }
  __syncthreads();

  // ---- stages
  for (int t = 0; t < sc.n; ++t) {
    switch (sc.b[t]) {
#define HM_CASE(BB) \
  case BB: hm_stage<BB, BDT, TT>(smem, d, sc.s[t], sc.had[t] != 0, blocks, sc.off[t], w, lane); break;
      HM_CASE(2) HM_CASE(3) HM_CASE(4) HM_CASE(5) HM_CASE(6) HM_CASE(7) HM_CASE(8) HM_CASE(9)
      HM_CASE(10) HM_CASE(11) HM_CASE(12) HM_CASE(13) HM_CASE(14) HM_CASE(15) HM_CASE(16)
#undef HM_CASE
      default: break;
    }
    __syncthreads();
  }

  // ---- store: transposing reads give lane t of group g token t's elements
  // E + 4g .. E + 4g + 3 (source lane s addresses element E + 4g + s / 4,
  // token quad s % 4); unscale, round to bf16
  {
    const int g = lane >> 4, l16 = lane & 15;
    const int qs = l16 & 3;
    const int qoff = 8 * ((4 * qs < TT) ? qs : 0);
    const bool act = l16 < TT && tok0 + l16 < tokens;
    const float us = ldexpf(1.0f, tok_exp(l16 < TT ? l16 : 0) - 14);
    uint16_t* yr = y + (tok0 + l16) * ldy;
    for (int e0 = 16 * w; e0 < d; e0 += 16 * hm::NW) {
      // d is a multiple of 8: a group past the row's end reads element 0 and stores nothing
      const int ei = e0 + 4 * g;
      const bool in = ei < d;
      const u32x2 hv = hm_tr_read(smem, hm::slot(in ? ei + (l16 >> 2) : 0) * S + qoff);
      if (act && in) {
        // (vector elements copied to scalars first: this compiler's bit_cast
        // of an element of a vector value reads element 0)
        const uint32_t w0 = hv.x, w1 = hv.y;
        const f16x2_t a = __builtin_bit_cast(f16x2_t, w0), b = __builtin_bit_cast(f16x2_t, w1);
        stg<u32x2>(yr + ei, u32x2{pack_bf16((float)a.x * us, (float)a.y * us), pack_bf16((float)b.x * us, (float)b.y * us)});
      }
    }
  }
}

// Entry from the C ABI (arguments validated there): radices each in [2, 16],
// product d <= 8192, precondition only for d a power of two.
template <int BDT, int XDT, int NT>
static void launch_hg(const void* x, void* y, int64_t tokens, int64_t ldx, int64_t ldy, int d, int ldt,
                      const uint32_t* sbits, const void* blocks, const HgSched& sc, int vec, hipStream_t s) {
  static const bool a = hipFuncSetAttribute((const void*)k_harp_gen<BDT, XDT, NT>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, hg::lds_floats(NT) * 4) ==
                        hipSuccess;
  (void)a;
  const int tt = std::max(1, std::min(hg::MAXTT, hg::lds_floats(NT) / ldt));
  const size_t lds = (size_t)tt * ldt * sizeof(float);
  const unsigned grid = (unsigned)((tokens + tt - 1) / tt);
  hipLaunchKernelGGL((k_harp_gen<BDT, XDT, NT>), dim3(grid), dim3(NT), lds, s, x, y, tokens, ldx, ldy, d, ldt, tt,
                     sbits, blocks, sc, vec);
}
template <int NT>
static void launch_hg_dt(const void* x, void* y, int xdt, int bdt, int64_t tokens, int64_t ldx, int64_t ldy, int d,
                         int ldt, const uint32_t* sb, const void* blocks, const HgSched& sc, int vec, hipStream_t s) {
  if (bdt == DT_F16 && xdt == DT_F32) launch_hg<DT_F16, DT_F32, NT>(x, y, tokens, ldx, ldy, d, ldt, sb, blocks, sc, vec, s);
  else if (bdt == DT_F16) launch_hg<DT_F16, DT_BF16, NT>(x, y, tokens, ldx, ldy, d, ldt, sb, blocks, sc, vec, s);
  else if (xdt == DT_F32) launch_hg<DT_F32, DT_F32, NT>(x, y, tokens, ldx, ldy, d, ldt, sb, blocks, sc, vec, s);
  else launch_hg<DT_F32, DT_BF16, NT>(x, y, tokens, ldx, ldy, d, ldt, sb, blocks, sc, vec, s);
}

template <int BDT, int TT>
static void launch_hm(const void* x, void* y, int64_t tokens, int64_t ldx, int64_t ldy, int d, int lgd,
                      const uint32_t* sbits, const void* blocks, const HgSched& sc, unsigned grid, size_t lds,
                      hipStream_t s) {
  static const bool a = hipFuncSetAttribute((const void*)k_harp_mx<BDT, TT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                            160 * 1024) == hipSuccess;
  (void)a;
  hipLaunchKernelGGL((k_harp_mx<BDT, TT>), dim3(grid), dim3(hm::THREADS), lds, s, (const uint16_t*)x, (uint16_t*)y,
                     tokens, ldx, ldy, d, lgd, sbits, blocks, sc);
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
  // 16-byte row accesses need a 16-byte aligned base and row stride on both sides
  const int esz = xdt == DT_F32 ? 4 : 2;
  const int vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) == 0 &&
                          (ldx * esz) % 16 == 0 && (ldy * esz) % 16 == 0
                      ? 1 : 0;
  const uint32_t* sb = precondition ? sbits : nullptr;
  // bf16 rows whose length is a multiple of 8 (16-byte chunks), with 16-byte
  // aligned rows and blocks, d <= 3072 and a mean radix of at least 4: the
  // matrix-core form (16-token tiles), where it measured faster
  int rsum = 0;
  for (int t = 0; t < n; ++t) rsum += sc.b[t];
  const bool mx_fits = hm::tile_bytes<16>(d) <= 96 * 1024;  // d <= 3072
  if (xdt == DT_BF16 && vec && d % 8 == 0 && (reinterpret_cast<uintptr_t>(blocks) & 15u) == 0 && mx_fits &&
      rsum >= 4 * n) {
    int lgd = 0;
    while ((1LL << (2 * lgd)) < d) ++lgd;  // sqrt(d) <= 2^lgd
    const int nch = d / 8, per_round = hm::NW * (64 / 16);
    if ((nch + per_round - 1) / per_round <= hm::MAXR) {
      const size_t lds = (size_t)((hm::tile_bytes<16>(d) + 15) & ~15) + 64;
      const unsigned gm = (unsigned)((tokens + 15) / 16);
      if (bdt == DT_F16) launch_hm<DT_F16, 16>(x, y, tokens, ldx, ldy, d, lgd, sb, blocks, sc, gm, lds, s);
      else launch_hm<DT_F32, 16>(x, y, tokens, ldx, ldy, d, lgd, sb, blocks, sc, gm, lds, s);
      return hipGetLastError();
    }
  }
  // two 512-thread blocks per CU where half the tile still holds 4 tokens
  // (d <= 4717): one block's row loads and stage-start coefficient waits
  // overlap the other's stages; else one 1024-thread block with the whole
  // tile (fewer tokens per tile would multiply the coefficient loads)
  if (hg::lds_floats(512) / ldt >= 4) launch_hg_dt<512>(x, y, xdt, bdt, tokens, ldx, ldy, d, ldt, sb, blocks, sc, vec, s);
  else launch_hg_dt<hg::THREADS>(x, y, xdt, bdt, tokens, ldx, ldy, d, ldt, sb, blocks, sc, vec, s);
  return hipGetLastError();
}

}  // namespace whtq
