// Gradient of the QWHA adapter with respect to its coefficient values.
//
// QWHA explainer, 2.1: F is built from a value vector c placed at an index
// list E, and the adapter output is y = (x Hn) F^T.  For the entry e at
// (row o_e, column k_e) of F the gradient of a loss with upstream dy is
//   dc[e] = sum_t dy[t][o_e] * Z[t][k_e],     Z = x Hn,
// a dense-dense product sampled on the support of F.
//
// Three launches on the caller's stream:
//   1. Z = x Hn in fp32 (the FWHT engine, bf16 -> f32) into the workspace;
//   2. k_qwha_dc: the entries are cut into slabs of at most 16384 (16 per
//      lane of a 1024-lane block) and the tokens into slabs of whole
//      4-token tiles; block (entry slab, token slab) keeps its entries'
//      (column, row) pairs and fp32 sums in registers and, per tile, stages
//      the tile's Z rows as Z[k][4 tokens] (one 16-byte column) and the dy
//      values of the slab's rows as dy[o][4 tokens] in LDS, then adds four
//      products per entry; the next tile's global loads are in flight while
//      the current tile is summed.  Per-token-slab partial sums go to the
//      workspace (or straight to dc when there is one token slab);
//   3. k_qwha_dc_reduce: dc[e] = sum of the partials in slab order.
// Every sum runs in a fixed order, so the result is deterministic.
//
// Blocks that share a token slab read the same Z rows; they are placed on
// the same XCD (the hardware deals consecutive blocks out to the 8 XCDs in
// turn), so those rows are fetched once into that XCD's L2.
#include "io.hpp"
#include "launch.hpp"

namespace whtq {

hipError_t launch_wht(int logn, int din, int dout, const void* x, void* y, int64_t rows, int64_t ldx,
                      int64_t ldy, const uint32_t* sbits, int sign_mode, float scale, hipStream_t s);

namespace qg {
constexpr int N = 4096;        // d_in
constexpr int THREADS = 1024;
constexpr int EPL = 16;        // entries per lane
constexpr int EPB = THREADS * EPL;
constexpr int TQ = 4;          // tokens per tile (one 16-byte fp32 column)
constexpr int XCDS = 8;
constexpr int LDS_Z = 0;                    // Z[k][4] fp32, 64 KB
constexpr int LDS_D = N * 16;               // dy[o - o_lo][4] fp32, up to 64 KB; row_ptr at set-up
constexpr int LDS_LIM = LDS_D + N * 16;     // first and last row of the slab
constexpr int LDS_BYTES = LDS_LIM + 16;
constexpr int ZPT = N / THREADS;            // Z columns staged per thread (4)
constexpr int DPT = N / THREADS;            // dy rows staged per thread, at most (4)
}  // namespace qg

struct DcGrid {
  int r_slabs, t_slabs, span, quads_per_slab;
};

// The plan depends on the sizes alone (not on the device), so the workspace
// size is a pure function of (tokens, nnz).
static DcGrid dc_grid(int64_t tokens, int64_t nnz) {
  constexpr int cus = 256;  // one block per compute unit of the target
  DcGrid g;
  g.r_slabs = (int)std::max<int64_t>(1, (nnz + qg::EPB - 1) / qg::EPB);
  g.span = (int)((nnz + g.r_slabs - 1) / g.r_slabs);
  const int64_t quads = (tokens + qg::TQ - 1) / qg::TQ;
  // about one block per CU (each holds 128 KB of LDS), a multiple of the XCD count
  int64_t ts = std::max<int64_t>(1, (cus + g.r_slabs - 1) / g.r_slabs);
  ts = std::min<int64_t>(ts, quads);
  g.quads_per_slab = (int)((quads + ts - 1) / ts);
  g.t_slabs = (int)((quads + g.quads_per_slab - 1) / g.quads_per_slab);
  return g;
}

// Block b -> (entry slab r, token slab p) such that b mod 8 (its XCD) is a
// function of p alone: consecutive runs of blocks on one XCD share p.
__device__ __forceinline__ void dc_block(int b, int r_slabs, int t_slabs, int& r, int& p) {
  const int x = b % qg::XCDS, j = b / qg::XCDS;
  // blocks of XCD x, in order: token slabs x, x + 8, x + 16, ... each for every r
  r = j % r_slabs;
  p = x + qg::XCDS * (j / r_slabs);
  (void)t_slabs;
}

__global__ __launch_bounds__(qg::THREADS) void k_qwha_dc(
    const float* __restrict__ z, int64_t tokens, const uint16_t* __restrict__ dy, int64_t lddy,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int d_out, int nnz, int span,
    int r_slabs, int t_slabs, int quads_per_slab, float* __restrict__ out) {
  extern __shared__ __align__(16) uint8_t smem[];
  f32x4* zq = reinterpret_cast<f32x4*>(smem + qg::LDS_Z);
  f32x4* dq = reinterpret_cast<f32x4*>(smem + qg::LDS_D);
  int* rp = reinterpret_cast<int*>(smem + qg::LDS_D);
  int* lim = reinterpret_cast<int*>(smem + qg::LDS_LIM);
  const int tid = threadIdx.x;
  int r, p;
  dc_block(blockIdx.x, r_slabs, t_slabs, r, p);
  if (p >= t_slabs) return;  // grid rounded up to whole XCD rounds (uniform per block)
  const int e0 = r * span, e1 = min(nnz, e0 + span);

  // ---- set-up: row_ptr in LDS, each entry's row by binary search
  for (int i = tid; i <= d_out; i += qg::THREADS) rp[i] = row_ptr[i];
  __syncthreads();
  // largest o in [0, d_out) with rp[o] <= e (the row holding entry e)
  auto row_of = [&](int e) {
    int pos = 0;
    for (int step = 1 << 12; step > 0; step >>= 1) {
      const int c = pos + step;
      if (c < d_out && rp[c] <= e) pos = c;
    }
    return pos;
  };
  if (tid == 0) {
    lim[0] = row_of(e0);
    lim[1] = row_of(e1 - 1);
  }
  __syncthreads();
  const int o_lo = lim[0], nrows = lim[1] - lim[0] + 1;  // nrows <= d_out <= 4096
  uint32_t ent[qg::EPL];  // column | (row - o_lo) << 16
  float acc[qg::EPL];
  {
    int col[qg::EPL];
#pragma unroll
    for (int i = 0; i < qg::EPL; ++i) {
      const int e = e0 + tid + qg::THREADS * i;
      col[i] = e < e1 ? col_idx[e] & (qg::N - 1) : 0;
    }
    int pos[qg::EPL];
#pragma unroll
    for (int i = 0; i < qg::EPL; ++i) pos[i] = 0;
    // the sixteen searches interleaved, one level at a time
    for (int step = 1 << 12; step > 0; step >>= 1) {
#pragma unroll
      for (int i = 0; i < qg::EPL; ++i) {
        const int e = min(e0 + tid + qg::THREADS * i, e1 - 1);
        const int c = pos[i] + step;
        if (c < d_out && rp[c] <= e) pos[i] = c;
      }
    }
#pragma unroll
    for (int i = 0; i < qg::EPL; ++i) {
      const int o = min(max(pos[i] - o_lo, 0), nrows - 1);
      ent[i] = (uint32_t)col[i] | ((uint32_t)o << 16);
      acc[i] = 0.f;
    }
  }

  // ---- tiles of 4 tokens
  const int64_t quads = (tokens + qg::TQ - 1) / qg::TQ;
  const int64_t q_beg = (int64_t)p * quads_per_slab;
  const int64_t q_end = min<int64_t>(quads, q_beg + quads_per_slab);
  // staged values of one tile: Z columns tid + 1024 m, dy rows o_lo + tid + 1024 m
  float zr[qg::TQ][qg::ZPT];
  u16x2 dr[qg::TQ / 2][qg::DPT];  // bf16 pairs of tokens (2 i, 2 i + 1)
  auto fetch = [&](int64_t q) {
#pragma unroll
    for (int j = 0; j < qg::TQ; ++j) {
      const int64_t t = min<int64_t>(q * qg::TQ + j, tokens - 1);  // past the end: re-read the last token
      const float* zrow = z + t * qg::N;
      const uint16_t* drow = dy + t * lddy + o_lo;
#pragma unroll
      for (int m = 0; m < qg::ZPT; ++m) zr[j][m] = zrow[tid + qg::THREADS * m];
#pragma unroll
      for (int m = 0; m < qg::DPT; ++m) {
        const int o = tid + qg::THREADS * m;
        const uint16_t d = o < nrows ? drow[o] : (uint16_t)0;
        if (j & 1) dr[j >> 1][m].y = d;
        else dr[j >> 1][m].x = d;
      }
    }
  };
  auto stage = [&](int64_t q) {
#pragma unroll
    for (int m = 0; m < qg::ZPT; ++m)
      zq[tid + qg::THREADS * m] = f32x4{zr[0][m], zr[1][m], zr[2][m], zr[3][m]};
    // tokens past the end contribute nothing: their dy is zero
    const int64_t t0 = q * qg::TQ;
#pragma unroll
    for (int m = 0; m < qg::DPT; ++m) {
      const int o = tid + qg::THREADS * m;
      if (o < nrows) {
        f32x4 d;
#pragma unroll
        for (int j = 0; j < qg::TQ; ++j)
          d[j] = t0 + j < tokens ? as_f((uint32_t)((j & 1) ? dr[j >> 1][m].y : dr[j >> 1][m].x) << 16) : 0.f;
        dq[o] = d;
      }
    }
  };
  __syncthreads();  // row_ptr copy no longer needed: its space becomes the dy tile
  if (q_beg < q_end) fetch(q_beg);
  for (int64_t q = q_beg; q < q_end; ++q) {
    stage(q);
    __syncthreads();
    if (q + 1 < q_end) fetch(q + 1);  // in flight while this tile is summed
#pragma unroll
    for (int i = 0; i < qg::EPL; ++i) {
      const f32x4 zc = zq[ent[i] & 0xffffu];
      const f32x4 dc = dq[ent[i] >> 16];
      float a = acc[i];
      a = fmaf(dc[0], zc[0], a);
      a = fmaf(dc[1], zc[1], a);
      a = fmaf(dc[2], zc[2], a);
      a = fmaf(dc[3], zc[3], a);
      acc[i] = a;
    }
    __syncthreads();
  }
  float* dst = out + (int64_t)p * nnz;
#pragma unroll
  for (int i = 0; i < qg::EPL; ++i) {
    const int e = e0 + tid + qg::THREADS * i;
    if (e < e1) dst[e] = acc[i];
  }
}

// dc[e] = sum over token slabs of the partial sums, in slab order.
__global__ __launch_bounds__(256) void k_qwha_dc_reduce(const float* __restrict__ part, int t_slabs, int nnz,
                                                        float* __restrict__ dc) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= nnz) return;
  float s = part[e];
  for (int p = 1; p < t_slabs; ++p) s += part[(int64_t)p * nnz + e];
  dc[e] = s;
}

// t_vals[j] = vals[perm[j]] (the values of F in the entry order of F^T).
template <typename T>
__global__ __launch_bounds__(256) void k_permute(const T* __restrict__ vals, const int32_t* __restrict__ perm,
                                                 int64_t nnz, T* __restrict__ out) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < nnz) out[j] = vals[perm[j]];
}

int64_t qwha_dc_workspace_bytes(int64_t tokens, int64_t nnz) {
  const DcGrid g = dc_grid(tokens, nnz);
  const int64_t zb = tokens * qg::N * 4;
  const int64_t pb = g.t_slabs > 1 ? (int64_t)g.t_slabs * nnz * 4 : 0;
  return ((zb + 255) & ~int64_t(255)) + pb;
}

hipError_t launch_qwha_dc(const void* x, int64_t ldx, const void* dy, int64_t lddy, int64_t tokens,
                          int64_t d_out, const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                          float* dc, void* workspace, hipStream_t s) {
  const DcGrid g = dc_grid(tokens, nnz);
  float* z = reinterpret_cast<float*>(workspace);
  const int64_t zb = ((tokens * qg::N * 4 + 255) & ~int64_t(255));
  float* part = g.t_slabs > 1 ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + zb) : dc;
  hipError_t e = launch_wht(12, DT_BF16, DT_F32, x, z, tokens, ldx, qg::N, nullptr, 0, 1.0f / 64.0f, s);
  if (e != hipSuccess) return e;
  static const bool attr = hipFuncSetAttribute((const void*)k_qwha_dc, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               qg::LDS_BYTES) == hipSuccess;
  (void)attr;
  // whole rounds of 8 token slabs per XCD lane: blocks with p >= t_slabs exit at once
  const int64_t p_rounds = (g.t_slabs + qg::XCDS - 1) / qg::XCDS;
  const unsigned grid = (unsigned)(p_rounds * qg::XCDS * g.r_slabs);
  hipLaunchKernelGGL(k_qwha_dc, dim3(grid), dim3(qg::THREADS), qg::LDS_BYTES, s, z, tokens,
                     (const uint16_t*)dy, lddy, row_ptr, col_idx, (int)d_out, (int)nnz, g.span, g.r_slabs,
                     g.t_slabs, g.quads_per_slab, part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (g.t_slabs > 1) {
    hipLaunchKernelGGL(k_qwha_dc_reduce, dim3((unsigned)((nnz + 255) / 256)), dim3(256), 0, s, part, g.t_slabs,
                       (int)nnz, dc);
    e = hipGetLastError();
  }
  return e;
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_permute(const void* vals, int val_dt, const int32_t* perm, int64_t nnz, void* out,
                          hipStream_t s) {
  const unsigned grid = (unsigned)((nnz + 255) / 256);
  if (val_dt == DT_F32)
    hipLaunchKernelGGL(k_permute<float>, dim3(grid), dim3(256), 0, s, (const float*)vals, perm, nnz, (float*)out);
  else
    hipLaunchKernelGGL(k_permute<uint16_t>, dim3(grid), dim3(256), 0, s, (const uint16_t*)vals, perm, nnz,
                       (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace whtq
