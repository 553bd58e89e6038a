// Gradient of the QWHA adapter with respect to its coefficient values.
//
// QWHA explainer, 2.1: F is built from a value vector c placed at an index
// list E, and the adapter output is y = (x Hn) F^T.  For the entry e at
// (row o_e, column k_e) of F the gradient of a loss with upstream dy is
//   dc[e] = sum_t dy[t][o_e] * Z[t][k_e],     Z = x Hn,
// a dense-dense product sampled on the support of F.
//
// Three launches on the caller's stream:
//   1. k_qwha_z: Z = x Hn in fp32 (the FWHT engine) into the workspace,
//      tile-interleaved (four tokens per 16-byte column); d_in < 4096 is
//      zero-extended, d_in = 8192 transformed as two halves;
//   2. k_qwha_dc: the entries are cut into slabs of at most 16384 (16 per
//      lane of a 1024-lane block, placed so that LDS reads rarely collide,
//      see the slot set-up) and the tokens into slabs of whole 4-token
//      tiles; block (entry slab, token slab) keeps its entries'
//      (column, row) pairs and fp32 sums in registers and, per tile, stages
//      the tile's Z rows as Z[k][4 tokens] (one 16-byte column) and the dy
//      values of the slab's rows as dy[o][4 tokens] (bf16) in LDS, then adds
//      four products per entry; the global loads of the next two tiles are in
//      flight while the current tile is summed.  Per-token-slab partial sums go to the
//      workspace (or straight to dc when there is one token slab);
//   3. k_qwha_dc_reduce: dc[e] = sum of the partials in slab order.
// Every sum runs in a fixed order, so the result is deterministic.
//
// Blocks that share a token slab read the same Z rows; they are placed on
// the same XCD (the hardware deals consecutive blocks out to the 8 XCDs in
// turn), so those rows are fetched once into that XCD's L2.
#include <cmath>

#include "io.hpp"
#include "launch.hpp"

namespace whtq {

namespace qg {
constexpr int N = 4096;        // d_in
constexpr int THREADS = 1024;
constexpr int EPL = 16;        // entries per lane
constexpr int EPB = THREADS * EPL;
constexpr int TQ = 4;          // tokens per tile (one 16-byte fp32 column)
constexpr int XCDS = 8;
constexpr int GROUPS = THREADS / 16;       // 16-lane groups, 16 * EPL entries each
constexpr int GE = 16 * EPL;                // entries per group
constexpr int NRES = 17;                    // column residues mod 16, plus "past the slab"
constexpr int LDS_Z = 0;                    // Z[k][4] fp32, 64 KB; set-up counters before the tiles
constexpr int LDS_D = N * 16;               // dy[o - o_lo][4] bf16, up to 32 KB; set-up tables before
constexpr int LDS_T = LDS_D + N * 16;       // slot table: entry offsets within the slab (u16)
constexpr int LDS_BYTES = LDS_T + EPB * 2;  // 160 KB
// set-up only, in the Z region: residue counters and bases [GROUPS][NRES]
// u32, the slab limits, each entry's column (u16); in the dy region after
// the row_ptr copy: each entry's row (u16)
constexpr int LDS_CNT = 0;
constexpr int LDS_BASE = LDS_CNT + GROUPS * NRES * 4;
constexpr int LDS_LIM = LDS_BASE + GROUPS * NRES * 4;
constexpr int LDS_COL = 16384;
constexpr int LDS_ROW = LDS_D + 16400;
static_assert(LDS_LIM + 8 <= LDS_COL && LDS_COL + 2 * EPB <= LDS_D, "set-up tables in the Z region");
static_assert(LDS_ROW + 2 * EPB <= LDS_T && LDS_D + 4 * (N + 1) <= LDS_ROW, "row table after row_ptr");
constexpr int ZPT = N / THREADS;            // Z columns staged per thread (4)
}  // namespace qg

// Z = x Hn in fp32, four tokens per block, written tile-interleaved:
// zi[quad][k] = (Z[4 quad][k], .., Z[4 quad + 3][k]) as one 16-byte column,
// zeros past the last token, so that a tile of k_qwha_dc is 64 KB of
// contiguous columns that go to LDS as they are loaded.  Each wave
// transforms one token row with the FWHT engine; the rows meet in LDS
// (padded by 4 floats per 64: conflict-free both ways) and leave as columns.
namespace qz {
constexpr int ROW = 4096 + 256;  // padded row, floats
constexpr int LDS_BYTES = 4 * ROW * 4;
}  // namespace qz

// d_in < 4096 is zero-extended (the first d_in outputs of H_4096 [x; 0] are
// H_d x, scale 1 / sqrt(d_in)); d_in = 8192 (WIDE) writes the two halves
// H_4096 (x_lo + x_hi) and H_4096 (x_lo - x_hi) of H_8192 x in turn, the
// quad's columns [h 4096, h 4096 + 4096).
template <bool WIDE>
__global__ __launch_bounds__(256) void k_qwha_z(const uint16_t* __restrict__ x, int64_t tokens, int64_t ldx,
                                                int in_cols, float scale, float* __restrict__ zi) {
  using G = Geo<12>;
  static_assert(4 * G::LDS_ROW <= 4 * qz::ROW, "transpose scratch fits in the row buffer");
  constexpr int ZS = WIDE ? 8192 : 4096;  // columns per quad
  extern __shared__ __align__(16) uint8_t smem[];
  float* lds = reinterpret_cast<float*>(smem);
  const int tid = threadIdx.x, w = tid >> 6, t = tid & 63;
  const int64_t quad = blockIdx.x, tok = quad * 4 + w;
  const uint32_t nomask[4] = {0u, 0u, 0u, 0u};
  const uint16_t* xr = x + (tok < tokens ? tok : tokens - 1) * ldx;
#pragma unroll 1
  for (int h = 0; h < (WIDE ? 2 : 1); ++h) {
    float v[64];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int col = G::idxA(t, c * 8);
      if constexpr (WIDE) {
        Raw8 rl, rh;
        fetch8<DT_BF16>(xr, col, rl);
        fetch8<DT_BF16>(xr, col + 4096, rh);
        float vh[8];
        widen8<DT_BF16, false>(rl, v + 8 * c, nomask, 0u);
        widen8<DT_BF16, false>(rh, vh, nomask, 0u);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * c + e] = h ? v[8 * c + e] - vh[e] : v[8 * c + e] + vh[e];
      } else {
        Raw8 raw{};
        if (col < in_cols) fetch8<DT_BF16>(xr, col, raw);
        widen8<DT_BF16, false>(raw, v + 8 * c, nomask, 0u);
      }
    }
    if (h) __syncthreads();  // the previous half's columns have left the row buffer
    stages_A<12, false>(v, t);
    transpose_AB<12, 64>(lds + w * G::LDS_ROW, v, t);
    stages_B<12, 2>(v, t);
    const float cs = tok < tokens ? (rho_B<12>(t) ? -scale : scale) : 0.0f;
    __syncthreads();  // every wave's transpose scratch is free
    float* row = lds + w * qz::ROW + t * 68;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      *reinterpret_cast<f32x4*>(row + 4 * q) =
          f32x4{v[4 * q] * cs, v[4 * q + 1] * cs, v[4 * q + 2] * cs, v[4 * q + 3] * cs};
    __syncthreads();
    f32x4* dst = reinterpret_cast<f32x4*>(zi) + quad * ZS + h * 4096;
#pragma unroll 4
    for (int m = 0; m < 16; ++m) {
      const int k = tid + 256 * m, ph = k + ((k >> 6) << 2);
      dst[k] = f32x4{lds[ph], lds[qz::ROW + ph], lds[2 * qz::ROW + ph], lds[3 * qz::ROW + ph]};
    }
  }
}

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
  g.quads_per_slab += g.quads_per_slab & 1;  // the kernel runs tiles in pairs
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
    int r_slabs, int t_slabs, int quads_per_slab, int zstride, int kbase, float* __restrict__ out) {
  extern __shared__ __align__(16) uint8_t smem[];
  f32x4* zq = reinterpret_cast<f32x4*>(smem + qg::LDS_Z);
  u32x2* dq = reinterpret_cast<u32x2*>(smem + qg::LDS_D);
  int* rp = reinterpret_cast<int*>(smem + qg::LDS_D);
  uint16_t* slot = reinterpret_cast<uint16_t*>(smem + qg::LDS_T);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(smem + qg::LDS_CNT);
  uint32_t* bas = reinterpret_cast<uint32_t*>(smem + qg::LDS_BASE);
  int* lim = reinterpret_cast<int*>(smem + qg::LDS_LIM);
  uint16_t* coltab = reinterpret_cast<uint16_t*>(smem + qg::LDS_COL);
  uint16_t* rowtab = reinterpret_cast<uint16_t*>(smem + qg::LDS_ROW);
  const int tid = threadIdx.x, grp = tid >> 4, gl = tid & 15;
  int r, p;
  dc_block(blockIdx.x, r_slabs, t_slabs, r, p);
  if (p >= t_slabs) return;  // grid rounded up to whole XCD rounds (uniform per block)
  const int e0 = r * span, e1 = min(nnz, e0 + span);

  // ---- set-up: row_ptr in LDS; each entry's row and column; slot assignment
  for (int i = tid; i <= d_out; i += qg::THREADS) rp[i] = row_ptr[i];
  for (int i = tid; i < qg::GROUPS * qg::NRES; i += qg::THREADS) cnt[i] = 0;
  __syncthreads();
  // largest o in [lo, d_out) with rp[o] <= e, for rp[lo] <= e (the row holding entry e)
  auto row_from = [&](int lo, int e) {
    int pos = lo;
    for (int step = 1 << 12; step > 0; step >>= 1) {
      const int c = pos + step;
      if (c < d_out && rp[c] <= e) pos = c;
    }
    return pos;
  };
  if (tid == 0) {
    lim[0] = row_from(0, e0);
    lim[1] = row_from(0, e1 - 1);
  }
  // Slots.  16-lane group g owns the slab's entries [256 g, 256 g + 256); lane
  // l sums, in its i-th slot, the entry at position 16 l + i of those entries
  // ordered by column mod 16.  With about 16 entries per residue the 16 lanes
  // of one slot then read Z columns in distinct 16-byte LDS bank slots
  // (16-byte reads are served 16 lanes at a time over 64 banks), instead of
  // colliding about 3x as random columns do; the entries of a slot stay
  // within 256 consecutive entries, i.e. a few consecutive rows, so their dy
  // reads are broadcasts or distinct banks too.  Which lane sums an entry
  // does not change its value (the sum runs over tokens in order), so the
  // ranks within a residue may come in any order.
  //
  // Lane l first takes the 16 consecutive entries 256 g + 16 l + j: one
  // binary search finds the row of the first, the rest follow it forward (a
  // new search only where an entry lies past the next row's start), and the
  // rows and columns go to LDS tables indexed by the entry's offset.
  {
    uint32_t res[qg::EPL], rank[qg::EPL];
    const int eb = e0 + qg::GE * grp + qg::EPL * gl;  // this lane's first entry
    int o = row_from(0, min(eb, e1 - 1));
#pragma unroll
    for (int j = 0; j < qg::EPL; ++j) {
      const int e = eb + j;
      const bool ok = e < e1;
      const int cf = ok ? col_idx[e] : 0;
      const int c = cf & (qg::N - 1);
      // this launch covers the columns [kbase, kbase + 4096) of Z; an entry
      // outside them is summed against the window's column c (harmless) and
      // not written (the other window's launch writes it)
      const bool out_win = ok && (cf & ~(qg::N - 1)) != kbase;
      if (ok && o + 1 < d_out && rp[o + 1] <= e) o = row_from(o + 1, e);
      res[j] = ok ? (uint32_t)c & 15u : 16u;
      coltab[qg::GE * grp + qg::EPL * gl + j] = (uint16_t)(c | (out_win ? 0x8000 : 0));
      rowtab[qg::GE * grp + qg::EPL * gl + j] = (uint16_t)o;
    }
#pragma unroll
    for (int j = 0; j < qg::EPL; ++j) rank[j] = atomicAdd(&cnt[grp * qg::NRES + res[j]], 1u);
    __syncthreads();
    if (gl == 0) {
      uint32_t run = 0;
      for (int b = 0; b < qg::NRES; ++b) {
        bas[grp * qg::NRES + b] = run;
        run += cnt[grp * qg::NRES + b];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < qg::EPL; ++j)
      slot[qg::GE * grp + bas[grp * qg::NRES + res[j]] + rank[j]] = (uint16_t)(qg::GE * grp + qg::EPL * gl + j);
  }
  __syncthreads();
  const int o_lo = lim[0], nrows = lim[1] - lim[0] + 1;  // nrows <= d_out <= 4096
  uint32_t ent[qg::EPL];  // column | (row - o_lo) << 16
  uint32_t skip = 0u;     // bit i: entry i lies outside this launch's column window
  float acc[qg::EPL];
#pragma unroll
  for (int i = 0; i < qg::EPL; ++i) {
    const int off = slot[qg::GE * grp + qg::EPL * gl + i];
    const int o = min(max((int)rowtab[off] - o_lo, 0), nrows - 1);
    ent[i] = ((uint32_t)coltab[off] & (qg::N - 1)) | ((uint32_t)o << 16);
    skip |= (uint32_t)(coltab[off] >> 15) << i;
    acc[i] = 0.f;
  }

  // ---- tiles of 4 tokens
  const int q_beg = p * quads_per_slab;  // quads_per_slab is even
  const int q_end = q_beg + quads_per_slab;
  const int last_tok = (int)tokens - 1;
  // Staged values of a tile, fetched two tiles ahead into one of two register
  // sets: Z columns tid + 1024 m and dy row o_lo + min(tid, nrows - 1), each
  // kept as loaded (a 32-bit register per value, every load unconditional) so
  // that nothing waits for them before they are staged.  Rows o_lo + tid +
  // 1024 m, m >= 1 (only slabs of very short rows have them) are read when
  // the tile is staged.
  struct Pre {
    f32x4 z[qg::ZPT];
    uint32_t d[qg::TQ];
  };
  const int last_quad = (last_tok) / qg::TQ;
  // (lane offsets are unsigned 32-bit and row bases block-uniform, so each
  // load is an SGPR base plus one shared VGPR offset)
  const uint32_t drow = (uint32_t)(o_lo + min(tid, nrows - 1));
  auto fetch = [&](int q, Pre& b) {
    // past the end: re-read the last tile (its dy is zeroed when staged)
    const f32x4* zt = reinterpret_cast<const f32x4*>(z) + (int64_t)min(q, last_quad) * zstride + kbase;
#pragma unroll
    for (int m = 0; m < qg::ZPT; ++m) b.z[m] = zt[(uint32_t)(tid + qg::THREADS * m)];
#pragma unroll
    for (int j = 0; j < qg::TQ; ++j) {
      const int t = min(q * qg::TQ + j, last_tok);
      b.d[j] = dy[(int64_t)t * lddy + drow];
    }
  };
  auto stage = [&](int q, const Pre& b) {
#pragma unroll
    for (int m = 0; m < qg::ZPT; ++m) zq[tid + qg::THREADS * m] = b.z[m];
    // tokens past the end contribute nothing: their dy is zero
    const int t0 = q * qg::TQ;
    // dy stays bf16 in LDS (8 bytes per row and tile, widened at the sum):
    // the sums are bound by LDS-to-register bytes, and this cuts them by a
    // quarter
    if (tid < nrows) {
      uint32_t h[qg::TQ];
#pragma unroll
      for (int j = 0; j < qg::TQ; ++j) h[j] = t0 + j <= last_tok ? b.d[j] : 0u;
      dq[tid] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    }
    for (int o = tid + qg::THREADS; o < nrows; o += qg::THREADS) {
      uint32_t h[qg::TQ];
#pragma unroll
      for (int j = 0; j < qg::TQ; ++j) h[j] = t0 + j <= last_tok ? (uint32_t)dy[(int64_t)(t0 + j) * lddy + o_lo + o] : 0u;
      dq[o] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    }
  };
  // the sums, four entries (eight 16-byte LDS reads in flight) at a time
  auto sum_tile = [&]() {
#pragma unroll
    for (int i0 = 0; i0 < qg::EPL; i0 += 4) {
      f32x4 zc[4];
      u32x2 dh[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        zc[u] = zq[ent[i0 + u] & 0xffffu];
        dh[u] = dq[ent[i0 + u] >> 16];
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the 8 LDS reads first
      __builtin_amdgcn_sched_group_barrier(0x002, 32, 0); // then widening and FMAs
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float a = acc[i0 + u];
        a = fmaf(bf16lo(dh[u].x), zc[u][0], a);
        a = fmaf(bf16hi(dh[u].x), zc[u][1], a);
        a = fmaf(bf16lo(dh[u].y), zc[u][2], a);
        a = fmaf(bf16hi(dh[u].y), zc[u][3], a);
        acc[i0 + u] = a;
      }
    }
  };
  __syncthreads();  // row_ptr copy no longer needed: its space becomes the dy tile
  // Every block runs the same even number of tiles and every fetch is
  // unconditional (tiles past the last token have zero dy and re-read valid
  // rows), so the compiler's load counters stay exact: staging a tile waits
  // only for its own loads, not for the set fetched after it.
  Pre A;
  fetch(q_beg, A);
  for (int q = q_beg; q < q_end; ++q) {
    stage(q, A);
    __syncthreads();
    fetch(q + 1, A);  // in flight while this tile is summed
    // keep the loads ahead of the sums (the scheduler would otherwise sink
    // them into the sum and wait for them before the next barrier)
    __builtin_amdgcn_sched_barrier(0);
    sum_tile();
    __syncthreads();
  }
  float* dst = out + (int64_t)p * nnz;
#pragma unroll
  for (int i = 0; i < qg::EPL; ++i) {
    const int e = e0 + slot[qg::GE * grp + qg::EPL * gl + i];
    if (e < e1 && !((skip >> i) & 1u)) dst[e] = acc[i];
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

// Z columns per 4-token quad in the workspace: d_in = 8192 keeps both halves
static int64_t dc_zstride(int64_t d_in) { return d_in == 8192 ? 8192 : qg::N; }

int64_t qwha_dc_workspace_bytes(int64_t tokens, int64_t d_in, int64_t nnz) {
  const DcGrid g = dc_grid(tokens, nnz);
  const int64_t zb = (tokens + 3) / 4 * dc_zstride(d_in) * 16;  // tile-interleaved Z
  const int64_t pb = g.t_slabs > 1 ? (int64_t)g.t_slabs * nnz * 4 : 0;
  return ((zb + 255) & ~int64_t(255)) + pb;
}

template <bool WIDE>
static void launch_z(const void* x, int64_t tokens, int64_t ldx, int in_cols, float scale, float* z, hipStream_t s) {
  static const bool zattr = hipFuncSetAttribute((const void*)k_qwha_z<WIDE>,
                                                hipFuncAttributeMaxDynamicSharedMemorySize, qz::LDS_BYTES) == hipSuccess;
  (void)zattr;
  hipLaunchKernelGGL(k_qwha_z<WIDE>, dim3((unsigned)((tokens + 3) / 4)), dim3(256), qz::LDS_BYTES, s,
                     (const uint16_t*)x, tokens, ldx, in_cols, scale, z);
}

hipError_t launch_qwha_dc(const void* x, int64_t ldx, const void* dy, int64_t lddy, int64_t tokens, int64_t d_in,
                          int64_t d_out, const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                          float* dc, void* workspace, hipStream_t s) {
  const DcGrid g = dc_grid(tokens, nnz);
  const bool wide = d_in == 8192;
  const int64_t zs = dc_zstride(d_in);
  float* z = reinterpret_cast<float*>(workspace);
  const int64_t zb = ((tokens + 3) / 4 * zs * 16 + 255) & ~int64_t(255);
  float* part = g.t_slabs > 1 ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + zb) : dc;
  const float scale = (float)(1.0 / std::sqrt((double)d_in));
  if (wide) launch_z<true>(x, tokens, ldx, (int)d_in, scale, z, s);
  else launch_z<false>(x, tokens, ldx, (int)d_in, scale, z, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static const bool attr = hipFuncSetAttribute((const void*)k_qwha_dc, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               qg::LDS_BYTES) == hipSuccess;
  (void)attr;
  // whole rounds of 8 token slabs per XCD lane: blocks with p >= t_slabs exit at once
  const int64_t p_rounds = (g.t_slabs + qg::XCDS - 1) / qg::XCDS;
  const unsigned grid = (unsigned)(p_rounds * qg::XCDS * g.r_slabs);
  // one launch per 4096-column window of Z (two at d_in = 8192); each entry
  // is written by the launch whose window holds its column
  for (int kb = 0; kb < (wide ? 8192 : qg::N); kb += qg::N) {
    hipLaunchKernelGGL(k_qwha_dc, dim3(grid), dim3(qg::THREADS), qg::LDS_BYTES, s, z, tokens,
                       (const uint16_t*)dy, lddy, row_ptr, col_idx, (int)d_out, (int)nnz, g.span, g.r_slabs,
                       g.t_slabs, g.quads_per_slab, (int)zs, kb, part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
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
