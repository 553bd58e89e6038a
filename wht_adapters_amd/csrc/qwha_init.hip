// QWHA adapter initialisation on the device: error coefficients, the
// calibration Gram matrix, activation errors, per-channel selection and
// least-squares refinement.
//
// QWHA explainer, 2.2: AdaAlloc gives each output channel a share of the
// parameter budget in proportion to its activation error (with a minimum),
// keeps the channel's largest-magnitude coefficients, and refinement fits the
// kept values by least squares to the layer output error.  With
// Delta W = F Hn, F_dense = (W - Q(W)) Hn and calibration tokens as rows of x,
// put Z = x Hn and G = Z^T Z (n x n, the rotated input Gram matrix).  Then
//   e_o^2 = ||x Delta W[o]^T||^2 = F_dense[o] G F_dense[o]^T,
// and the least-squares values on a support E solve the normal equations
//   G[E][E] c = (F_dense G)[o][E].
// Everything after G is independent of the number of calibration tokens, and
// G accumulates over calibration batches.
//
// Kernels: W - Q(W) (the transforms and Q are the library's FWHT and
// dequantise-inverse kernels), an fp32 GEMM on MFMA 16x16x4 f32 tiles for G
// (symmetric: upper blocks only, mirrored) and for F_dense G, the per-row
// quadratic form, a per-row bitwise top-k search, and a per-row blocked
// Cholesky solve with the factor held in 4 x 4 register blocks.
#include "io.hpp"
#include "launch.hpp"

namespace whtq {

namespace qi {
constexpr int KMAX = 128;     // largest support a row's refinement takes
constexpr int BT = 128;       // GEMM block tile (M and N)
constexpr int KS = 16;        // GEMM k-step staged in LDS
constexpr int LDT = BT + 16;  // LDS row stride of a k-major tile (conflict-free MFMA operand reads)
}  // namespace qi

// one weight element (bf16, fp16 or fp32) as fp32
template <int WDT>
__device__ __forceinline__ float qi_w_at(const void* w, int64_t i) {
  if constexpr (WDT == DT_F32) {
    return reinterpret_cast<const float*>(w)[i];
  } else {
    const uint16_t b = reinterpret_cast<const uint16_t*>(w)[i];
    return WDT == DT_BF16 ? as_f((uint32_t)b << 16) : (float)__builtin_bit_cast(_Float16, b);
  }
}

// F = W - Q(W), in place over Q(W): a block per row (grid-stride over the
// rows), eight consecutive values per thread and step with 16-byte accesses
// (W with element loads where its rows are not 16-byte aligned).
template <int WDT>
__global__ __launch_bounds__(256) void k_qi_sub(const void* __restrict__ w, int64_t ldw, float* __restrict__ f,
                                                int64_t ldf, int64_t rows, int n, int vec) {
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    float* fr = f + r * ldf;
    const int64_t wr = r * ldw;
    for (int c = 8 * (int)threadIdx.x; c < n; c += 8 * 256) {
      if (c + 8 > n) {  // (n below 8)
        for (int e = c; e < n; ++e) fr[e] = qi_w_at<WDT>(w, wr + e) - fr[e];
        continue;
      }
      float wv[8];
      if (vec) {
        if constexpr (WDT == DT_F32) {
          const f32x4 a = ldg<f32x4>(reinterpret_cast<const float*>(w) + wr + c);
          const f32x4 b = ldg<f32x4>(reinterpret_cast<const float*>(w) + wr + c + 4);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            wv[q] = a[q];
            wv[4 + q] = b[q];
          }
        } else {
          const u32x4 v = ldg<u32x4>(reinterpret_cast<const uint16_t*>(w) + wr + c);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if constexpr (WDT == DT_BF16) {
              wv[2 * q] = bf16lo(v[q]);
              wv[2 * q + 1] = bf16hi(v[q]);
            } else {
              wv[2 * q] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[q] & 0xffffu));
              wv[2 * q + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[q] >> 16));
            }
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) wv[e] = qi_w_at<WDT>(w, wr + c + e);
      }
      f32x4 a = *reinterpret_cast<const f32x4*>(fr + c), b = *reinterpret_cast<const f32x4*>(fr + c + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = wv[q] - a[q];
        b[q] = wv[4 + q] - b[q];
      }
      *reinterpret_cast<f32x4*>(fr + c) = a;
      *reinterpret_cast<f32x4*>(fr + c + 4) = b;
    }
  }
}

hipError_t launch_qi_sub(const void* w, int wdt, int64_t ldw, float* f, int64_t ldf, int64_t rows, int64_t n,
                         hipStream_t s) {
  const unsigned grid = persistent_grid(rows, 8);
  const int esz = wdt == DT_F32 ? 4 : 2;
  const int vec = ((reinterpret_cast<uintptr_t>(w) & 15u) == 0 && (ldw * esz) % 16 == 0) ? 1 : 0;
  if (wdt == DT_F32)
    hipLaunchKernelGGL(k_qi_sub<DT_F32>, dim3(grid), dim3(256), 0, s, w, ldw, f, ldf, rows, (int)n, vec);
  else if (wdt == DT_F16)
    hipLaunchKernelGGL(k_qi_sub<DT_F16>, dim3(grid), dim3(256), 0, s, w, ldw, f, ldf, rows, (int)n, vec);
  else
    hipLaunchKernelGGL(k_qi_sub<DT_BF16>, dim3(grid), dim3(256), 0, s, w, ldw, f, ldf, rows, (int)n, vec);
  return hipGetLastError();
}

// C[m][c] = beta C[m][c] + sum_k A(m, k) B(k, c) in fp32.  B is k-major
// (B[k * ldb + c]); A is m-major (A[m * lda + k]) when AM, else k-major
// (A[k * lda + m]).  Requirements (checked by the callers): N % 128 == 0,
// 16-byte aligned bases and strides; AM: K % 16 == 0 (rows past M read as
// zero and are not stored); k-major A: M % 128 == 0 (k past K read as zero).
// SYM (C = A^T A with A == B, M == N): only the tiles that reach the upper
// triangle are computed (those inside a 128 x 128 diagonal block in full),
// and the others also write their mirror.
//
// Block tile BM x 128 (BM 128 or 64), 256 threads = 4 waves in 2 x 2, each
// wave a (BM / 2) x 64 part as (BM / 32) x 4 MFMA 16x16x4 tiles (operand lane
// l: row/col l % 16, k l / 16; result register r of lane l: row 4 (l / 16) + r,
// col l % 16).  The next k-step's global loads are in flight while the
// current one is multiplied.
template <bool AM, bool SYM, int BM>
__global__ __launch_bounds__(256) void k_qi_gemm(const float* __restrict__ A, int64_t lda,
                                                const float* __restrict__ B, int64_t ldb, float* __restrict__ C,
                                                int64_t ldc, int64_t M, int64_t K, float beta) {
  using namespace qi;
  constexpr int MT = BM / 32;          // MFMA row tiles per wave
  constexpr int AL = BM * KS / 4 / 256;  // float4 loads of A per thread and k-step
  constexpr int BL = BT * KS / 4 / 256;  // and of B
  static_assert(KS == 16, "the scheduling groups below count a 16-deep k-step");
  __shared__ __align__(16) float As[KS][BM + 16];
  __shared__ __align__(16) float Bs[KS][LDT];
  const int bn = blockIdx.x, bm = blockIdx.y;
  if (SYM && bm * BM >= (bn + 1) * BT) return;
  const bool mirror = SYM && (bm * BM) / BT != bn;
  const int64_t m0 = (int64_t)bm * BM, n0 = (int64_t)bn * BT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = (w >> 1) * (BM / 2), wn = (w & 1) * 64;
  const int li = lane & 15, lk = lane >> 4;
  f32x4 acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 ga[AL], gb[BL];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int h = 0; h < BL; ++h) {
      const int e = tid + 256 * h;
      const int64_t kb = k0 + (e >> 5);
      gb[h] = kb < K ? ldg<f32x4>(B + kb * ldb + n0 + (e & 31) * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int h = 0; h < AL; ++h) {
      const int e = tid + 256 * h;
      if constexpr (AM) {
        const int64_t m = m0 + e / (KS / 4);
        ga[h] = m < M ? ldg<f32x4>(A + m * lda + k0 + (e % (KS / 4)) * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        const int64_t kb = k0 + e / (BM / 4);
        ga[h] = kb < K ? ldg<f32x4>(A + kb * lda + m0 + (e % (BM / 4)) * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int h = 0; h < BL; ++h) {
      const int e = tid + 256 * h;
      *reinterpret_cast<f32x4*>(&Bs[e >> 5][(e & 31) * 4]) = gb[h];
    }
#pragma unroll
    for (int h = 0; h < AL; ++h) {
      const int e = tid + 256 * h;
      if constexpr (AM) {
#pragma unroll
        for (int q = 0; q < 4; ++q) As[(e % (KS / 4)) * 4 + q][e / (KS / 4)] = ga[h][q];
      } else {
        *reinterpret_cast<f32x4*>(&As[e / (BM / 4)][(e % (BM / 4)) * 4]) = ga[h];
      }
    }
  };
  load(0);
  for (int64_t k0 = 0; k0 < K; k0 += KS) {
    stage();
    __syncthreads();
    if (k0 + KS < K) load(k0 + KS);
    // all of the k-step's operands first (one LDS wait), then the MFMAs back to back
    float a[KS / 4][MT], b[KS / 4][4];
#pragma unroll
    for (int kk = 0; kk < KS / 4; ++kk) {
#pragma unroll
      for (int i = 0; i < MT; ++i) a[kk][i] = As[4 * kk + lk][wm + i * 16 + li];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[kk][j] = Bs[4 * kk + lk][wn + j * 16 + li];
    }
#pragma unroll
    for (int kk = 0; kk < KS / 4; ++kk)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[kk][i], b[kk][j], acc[i][j], 0, 0, 0);
    // keep that order: the next k-step's global loads, every LDS read, then the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x020, AL + BL, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * (MT + 4), 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * MT * 4, 0);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm + i * 16 + 4 * lk + r, c = n0 + wn + j * 16 + li;
        if (AM && m >= M) continue;
        float v = acc[i][j][r];
        if (beta != 0.f) v = fmaf(beta, C[m * ldc + c], v);
        C[m * ldc + c] = v;
      }
      if (mirror) {
        // the mirror C[c][m .. m + 3]: a lane's four registers are consecutive m
        const int64_t m = m0 + wm + i * 16 + 4 * lk, c = n0 + wn + j * 16 + li;
        f32x4 u = acc[i][j];
        if (beta != 0.f) {
          const f32x4 o = ldg<f32x4>(C + c * ldc + m);
#pragma unroll
          for (int e = 0; e < 4; ++e) u[e] = fmaf(beta, o[e], u[e]);
        }
        stg<f32x4>(C + c * ldc + m, u);
      }
    }
}

// G = beta G + Z^T Z, Z [T][n] (row stride n), n % 128 == 0.  64-row tiles:
// about twice as many upper-triangle tiles as CUs' worth of 128 x 128 ones,
// which evens out the work per CU.
hipError_t launch_qi_gram(const float* z, int64_t T, int64_t n, float* g, float beta, hipStream_t s) {
  const dim3 grid((unsigned)(n / qi::BT), (unsigned)(n / 64));
  hipLaunchKernelGGL((k_qi_gemm<false, true, 64>), grid, dim3(256), 0, s, z, n, z, n, g, n, n, T, beta);
  return hipGetLastError();
}

// P = F G, F [rows][n] (stride ldf), G [n][n] symmetric, P [rows][n] (stride n)
hipError_t launch_qi_fg(const float* f, int64_t ldf, int64_t rows, int64_t n, const float* g, float* p,
                        hipStream_t s) {
  const dim3 grid((unsigned)(n / qi::BT), (unsigned)((rows + qi::BT - 1) / qi::BT));
  hipLaunchKernelGGL((k_qi_gemm<true, false, 128>), grid, dim3(256), 0, s, f, ldf, g, n, p, n, rows, n, 0.f);
  return hipGetLastError();
}

// err[o] = sqrt(max(0, sum_i p[o][i] f[o][i])), one wave per row, n % 256 == 0
__global__ __launch_bounds__(256) void k_qi_qform(const float* __restrict__ f, int64_t ldf,
                                                 const float* __restrict__ p, int64_t rows, int64_t n,
                                                 float* __restrict__ err) {
  const int64_t o = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (o >= rows) return;
  float a = 0.f;
  for (int64_t i = lane * 4; i < n; i += 256) {
    const f32x4 u = ldg<f32x4>(f + o * ldf + i), v = ldg<f32x4>(p + o * n + i);
    a = fmaf(u[0], v[0], a);
    a = fmaf(u[1], v[1], a);
    a = fmaf(u[2], v[2], a);
    a = fmaf(u[3], v[3], a);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) a += __shfl_xor(a, m);
  if (lane == 0) err[o] = __builtin_sqrtf(fmaxf(a, 0.f));
}

hipError_t launch_qi_qform(const float* f, int64_t ldf, const float* p, int64_t rows, int64_t n, float* err,
                           hipStream_t s) {
  hipLaunchKernelGGL(k_qi_qform, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, f, ldf, p, rows, n, err);
  return hipGetLastError();
}

__device__ __forceinline__ uint32_t qi_wave_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true);   // xor 1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true);   // xor 2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true);  // half-row mirror
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true);  // row mirror
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); // row bcast 15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); // row bcast 31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Per row: the k = row_ptr[r+1] - row_ptr[r] (<= n) indices of largest |f|,
// ties to the lower index, ascending, into col_idx[row_ptr[r] ..).  The keys
// are the bit patterns of |f| (non-negative floats order as their patterns).
// The k-th largest key t is built bit by bit from the top: a bit is kept when
// at least k keys are >= the candidate (31 block-wide counts, one barrier
// each, no atomics).  Keys above t are taken, and of the keys equal to t the
// lowest-index ones.  256 threads; thread tid holds the VPT = n / 256
// contiguous values from tid VPT, so block-wide exclusive prefix sums in
// thread order give each thread its output position.
template <int VPT>
__global__ __launch_bounds__(256) void k_qi_select(const float* __restrict__ f, int64_t ldf, int n,
                                                  const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx) {
  __shared__ uint32_t part[2][4];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int base = row_ptr[r];
  const int k = row_ptr[r + 1] - base;
  if (k <= 0 || k > n) return;
  uint32_t key[VPT];
  const float* fr = f + r * ldf + tid * VPT;
  if constexpr (VPT >= 4) {
#pragma unroll
    for (int q = 0; q < VPT; q += 4) {
      const u32x4 v = ldg<u32x4>(fr + q);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[q + e] = v[e] & 0x7fffffffu;
    }
  } else {
#pragma unroll
    for (int q = 0; q < VPT; ++q) key[q] = __builtin_bit_cast(uint32_t, fr[q]) & 0x7fffffffu;
  }
  // block-wide sum; slots alternate so one barrier per call suffices
  auto bsum = [&](uint32_t v, int slot) -> uint32_t {
    v = qi_wave_sum(v);
    if (lane == 0) part[slot][wv] = v;
    __syncthreads();
    return part[slot][0] + part[slot][1] + part[slot][2] + part[slot][3];
  };
  const bool all = k == n;
  uint32_t t = 0;
  if (!all) {
    for (int b = 30; b >= 0; --b) {
      const uint32_t cand = t | (1u << b);
      uint32_t c = 0;
#pragma unroll
      for (int q = 0; q < VPT; ++q) c += key[q] >= cand ? 1u : 0u;
      if (bsum(c, b & 1) >= (uint32_t)k) t = cand;
    }
  }
  uint32_t nties = 0, nabove = 0;
#pragma unroll
  for (int q = 0; q < VPT; ++q) {
    nabove += (all || key[q] > t) ? 1u : 0u;
    nties += (!all && key[q] == t) ? 1u : 0u;
  }
  // exclusive prefix sums in thread order: wave scans, then the wave totals
  __shared__ uint32_t wtot[2][4];
  auto exscan = [&](uint32_t v, int slot) -> uint32_t {
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t u = (uint32_t)__shfl_up((int)incl, o);
      if (lane >= o) incl += u;
    }
    if (lane == 63) wtot[slot][wv] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int w2 = 0; w2 < wv; ++w2) before += wtot[slot][w2];
    return before + incl - v;
  };
  const uint32_t above_total = all ? (uint32_t)k : bsum(nabove, 1);  // slot 0 was the last search step's
  const uint32_t want = (uint32_t)k - above_total;   // keys equal to t that are taken
  const uint32_t tie0 = exscan(nties, 0);
  const uint32_t left = want > tie0 ? want - tie0 : 0u;
  const uint32_t take = all ? 0u : (left < nties ? left : nties);  // this thread's ties that are taken
  uint32_t pos = exscan(nabove + take, 1), seen = 0;
#pragma unroll
  for (int q = 0; q < VPT; ++q) {
    bool s = all || key[q] > t;
    if (!s && key[q] == t) {
      s = seen < take;
      ++seen;
    }
    if (s) col_idx[base + pos++] = tid * VPT + q;
  }
}

hipError_t launch_qi_select(const float* f, int64_t ldf, int64_t rows, int n, const int32_t* row_ptr,
                            int32_t* col_idx, hipStream_t s) {
  const dim3 g((unsigned)rows), b(256);
  switch (n) {
    case 256: hipLaunchKernelGGL(k_qi_select<1>, g, b, 0, s, f, ldf, n, row_ptr, col_idx); break;
    case 512: hipLaunchKernelGGL(k_qi_select<2>, g, b, 0, s, f, ldf, n, row_ptr, col_idx); break;
    case 1024: hipLaunchKernelGGL(k_qi_select<4>, g, b, 0, s, f, ldf, n, row_ptr, col_idx); break;
    case 2048: hipLaunchKernelGGL(k_qi_select<8>, g, b, 0, s, f, ldf, n, row_ptr, col_idx); break;
    case 4096: hipLaunchKernelGGL(k_qi_select<16>, g, b, 0, s, f, ldf, n, row_ptr, col_idx); break;
    case 8192: hipLaunchKernelGGL(k_qi_select<32>, g, b, 0, s, f, ldf, n, row_ptr, col_idx); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Per row r with support E (k = |E| <= KMAX): the normal equations
// G[E][E] c = P[r][E] (P = F_dense G), solved by Cholesky G[E][E] = L L^T,
// L y = b, L^T c = y; vals[row_ptr[r] + a] = c_a.  Rows with k > KMAX get NaN.
//
// Blocked by 4: G[E][E] is padded to kp = 4 ceil(k / 4) with identity rows and
// cut into 4 x 4 blocks; each thread owns up to MAXP blocks of the lower block
// triangle in registers, and the right-hand side rides along as one more
// block row R (its row 0 holds b), so that the factorisation turns it into y
// (forward substitution for free).  Block step J: the owner of (J, J)
// factorises it in registers and publishes L_JJ and its reciprocal diagonal;
// the owners of (I, J), I > J (R included), form L_IJ = A_IJ L_JJ^-T and
// publish it; every owner of (I, K), K > J, subtracts L_IJ L_KJ^T.  Two
// barriers per block step.  Back substitution then walks J downwards: the
// owner of (J, J) solves L_JJ^T c_J = y_J, and the owners of (J, K), K < J,
// subtract L_JK^T c_J from y_K (one writer per K and step).  L never leaves
// the registers; pivots use the reciprocal square root.
__global__ __launch_bounds__(256) void k_qi_refine(const float* __restrict__ g, int64_t n,
                                                  const float* __restrict__ p, const int32_t* __restrict__ row_ptr,
                                                  const int32_t* __restrict__ col_idx, float* __restrict__ vals) {
  constexpr int KM = qi::KMAX, NBM = KM / 4, MAXP = (NBM * (NBM + 1) / 2 + NBM + 255) / 256;
  __shared__ int sidx[KM];
  __shared__ __align__(16) float panel[KM + 4][4];  // L_IJ rows of the current block column; row KM: R
  __shared__ __align__(16) float ljj[16];           // L_JJ row-major
  __shared__ float invd[KM];                         // 1 / L[i][i]
  __shared__ float yv[KM];                           // y, then c
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int base = row_ptr[r];
  const int k = row_ptr[r + 1] - base;
  if (k <= 0) return;
  if (k > KM) {
    for (int i = tid; i < k; i += 256) vals[base + i] = __builtin_nanf("");
    return;
  }
  for (int i = tid; i < KM; i += 256) sidx[i] = i < k ? col_idx[base + i] : 0;
  __syncthreads();
  const int nb = (k + 3) >> 2, npair = nb * (nb + 1) / 2;
  // slot m: a lower block (bi >= bj), an R block (bi == nb), or empty (-1)
  int pbi[MAXP], pbj[MAXP];
  float acc[MAXP][4][4];
  const float* pr = p + r * n;
#pragma unroll
  for (int m = 0; m < MAXP; ++m) {
    const int q = tid + 256 * m;
    int bi = -1, bj = -1;
    if (q < npair) {
      bi = (int)((__builtin_sqrtf(8.f * (float)q + 1.f) - 1.f) * 0.5f);
      while ((bi + 1) * (bi + 2) / 2 <= q) ++bi;
      while (bi * (bi + 1) / 2 > q) --bi;
      bj = q - bi * (bi + 1) / 2;
    } else if (q < npair + nb) {
      bi = nb;
      bj = q - npair;
    }
    pbi[m] = bi;
    pbj[m] = bj;
    // gathers issued unconditionally (indices clamped into the support), patched below
    const int ib = (bi < 0 || bi == nb) ? 0 : bi, jb0 = bj < 0 ? 0 : bj;
    int64_t rowoff[4];
    int colv[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      rowoff[x] = (int64_t)sidx[min(4 * ib + x, k - 1)] * n;
      colv[x] = sidx[min(4 * jb0 + x, k - 1)];
    }
    if (bi == nb) {
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[m][0][y] = 4 * jb0 + y < k ? pr[colv[y]] : 0.f;
#pragma unroll
      for (int x = 1; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[m][x][y] = 0.f;
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[m][x][y] = g[rowoff[x] + colv[y]];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int i = 4 * ib + x, l = 4 * jb0 + y;
          if (bi < 0 || i >= k || l >= k) acc[m][x][y] = (bi >= 0 && i == l) ? 1.f : 0.f;
        }
    }
  }
  for (int J = 0; J < nb; ++J) {
    // (1) the diagonal block
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
      if (pbi[m] != J || pbj[m] != J) continue;
      float(&a)[4][4] = acc[m];
      const float i0 = __builtin_amdgcn_rsqf(a[0][0]);
      a[0][0] *= i0;
      a[1][0] *= i0;
      a[2][0] *= i0;
      a[3][0] *= i0;
      a[1][1] = fmaf(-a[1][0], a[1][0], a[1][1]);
      const float i1 = __builtin_amdgcn_rsqf(a[1][1]);
      a[1][1] *= i1;
      a[2][1] = fmaf(-a[2][0], a[1][0], a[2][1]) * i1;
      a[3][1] = fmaf(-a[3][0], a[1][0], a[3][1]) * i1;
      a[2][2] = fmaf(-a[2][1], a[2][1], fmaf(-a[2][0], a[2][0], a[2][2]));
      const float i2 = __builtin_amdgcn_rsqf(a[2][2]);
      a[2][2] *= i2;
      a[3][2] = fmaf(-a[3][1], a[2][1], fmaf(-a[3][0], a[2][0], a[3][2])) * i2;
      a[3][3] = fmaf(-a[3][2], a[3][2], fmaf(-a[3][1], a[3][1], fmaf(-a[3][0], a[3][0], a[3][3])));
      const float i3 = __builtin_amdgcn_rsqf(a[3][3]);
      a[3][3] *= i3;
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) ljj[4 * x + y] = y <= x ? a[x][y] : 0.f;
      invd[4 * J + 0] = i0;
      invd[4 * J + 1] = i1;
      invd[4 * J + 2] = i2;
      invd[4 * J + 3] = i3;
    }
    __syncthreads();
    // (2) the panel below it: L_IJ = A_IJ L_JJ^-T, row by row
    {
      float L[4][4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&ljj[4 * x]);
        L[x][0] = v[0];
        L[x][1] = v[1];
        L[x][2] = v[2];
        L[x][3] = v[3];
      }
      const float d0 = invd[4 * J], d1 = invd[4 * J + 1], d2 = invd[4 * J + 2], d3 = invd[4 * J + 3];
#pragma unroll
      for (int m = 0; m < MAXP; ++m) {
        if (pbj[m] != J || pbi[m] <= J) continue;
        float(&a)[4][4] = acc[m];
        const int prow = pbi[m] == nb ? KM : 4 * pbi[m];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float l0 = a[x][0] * d0;
          const float l1 = fmaf(-l0, L[1][0], a[x][1]) * d1;
          const float l2 = fmaf(-l1, L[2][1], fmaf(-l0, L[2][0], a[x][2])) * d2;
          const float l3 = fmaf(-l2, L[3][2], fmaf(-l1, L[3][1], fmaf(-l0, L[3][0], a[x][3]))) * d3;
          a[x][0] = l0;
          a[x][1] = l1;
          a[x][2] = l2;
          a[x][3] = l3;
          *reinterpret_cast<f32x4*>(&panel[prow + x][0]) = f32x4{l0, l1, l2, l3};
        }
      }
    }
    __syncthreads();
    // (3) trailing update A_IK -= L_IJ L_KJ^T for the blocks right of column J
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
      if (pbj[m] <= J) continue;  // also skips empty slots (-1)
      const int prow = pbi[m] == nb ? KM : 4 * pbi[m], krow = 4 * pbj[m];
      f32x4 li[4], lk[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        li[x] = *reinterpret_cast<const f32x4*>(&panel[prow + x][0]);
        lk[x] = *reinterpret_cast<const f32x4*>(&panel[krow + x][0]);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          float v = acc[m][x][y];
#pragma unroll
          for (int c = 0; c < 4; ++c) v = fmaf(-li[x][c], lk[y][c], v);
          acc[m][x][y] = v;
        }
    }
  }
  // y (row 0 of the R blocks) to LDS
#pragma unroll
  for (int m = 0; m < MAXP; ++m)
    if (pbi[m] == nb) {
#pragma unroll
      for (int y = 0; y < 4; ++y) yv[4 * pbj[m] + y] = acc[m][0][y];
    }
  __syncthreads();
  for (int J = nb - 1; J >= 0; --J) {
    // L_JJ^T c_J = y_J
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
      if (pbi[m] != J || pbj[m] != J) continue;
      const float(&a)[4][4] = acc[m];
      const float c3 = yv[4 * J + 3] * invd[4 * J + 3];
      const float c2 = fmaf(-a[3][2], c3, yv[4 * J + 2]) * invd[4 * J + 2];
      const float c1 = fmaf(-a[3][1], c3, fmaf(-a[2][1], c2, yv[4 * J + 1])) * invd[4 * J + 1];
      const float c0 = fmaf(-a[3][0], c3, fmaf(-a[2][0], c2, fmaf(-a[1][0], c1, yv[4 * J]))) * invd[4 * J];
      yv[4 * J] = c0;
      yv[4 * J + 1] = c1;
      yv[4 * J + 2] = c2;
      yv[4 * J + 3] = c3;
    }
    __syncthreads();
    // y_K -= L_JK^T c_J for K < J
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
      if (pbi[m] != J || pbj[m] >= J || pbj[m] < 0) continue;
      const float(&a)[4][4] = acc[m];
      const int K = pbj[m];
      const float c0 = yv[4 * J], c1 = yv[4 * J + 1], c2 = yv[4 * J + 2], c3 = yv[4 * J + 3];
#pragma unroll
      for (int y = 0; y < 4; ++y)
        yv[4 * K + y] = fmaf(-a[3][y], c3, fmaf(-a[2][y], c2, fmaf(-a[1][y], c1, fmaf(-a[0][y], c0, yv[4 * K + y]))));
    }
    __syncthreads();
  }
  for (int i = tid; i < k; i += 256) vals[base + i] = yv[i];
}

hipError_t launch_qi_refine(const float* g, int64_t n, const float* p, int64_t rows, const int32_t* row_ptr,
                            const int32_t* col_idx, float* vals, hipStream_t s) {
  hipLaunchKernelGGL(k_qi_refine, dim3((unsigned)rows), dim3(256), 0, s, g, n, p, row_ptr, col_idx, vals);
  return hipGetLastError();
}

}  // namespace whtq
