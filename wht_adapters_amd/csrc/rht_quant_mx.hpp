// rht_quantize_rtn for 16-bit rows of n = 4096 or 8192: the first seven
// butterfly stages on the matrix cores.
//
// The forward transform is y = Hn(S w) (HARP explainer, technical summary
// section 1: fixed random signs, then the Sylvester Hadamard transform).
// Sylvester's matrix factors over any split of the index bits
// (H_2^a (x) H_2^b = H_2^(a+b)), so the transform along seven chosen index
// bits is one dense product with H_128, whose +-1 entries are exact in bf16
// and fp16: the raw 16-bit inputs go straight into
// v_mfma_f32_16x16x32_{bf16,f16} (exact products, fp32 accumulation), and
// only the remaining 5 (n = 4096) or 6 (n = 8192) stages run on the VALU:
// one or two in-register stages and four DPP stages.  The quantiser
// epilogue (group absmax -> fp16 scale -> RTN -> packing) is the one of
// rht_quant.hpp.
//
// One wave per row, 64 lanes x R = n/64 values.  Rows stream through LDS:
// while a wave transforms row r, the next row it owns is already being copied
// into its LDS buffer (global_load_lds, one coalesced 1 KB block of the row
// per instruction, non-temporal), so HBM latency hides behind the arithmetic.
//
// Index bits (p0 = least significant):
//   load:  lane l reads NC = R/8 16-byte chunks c (8 consecutive values,
//          p0..p2 = e) from the LDS copy.  Chunk bits c0, c1 -> p4, p5
//          (c3 -> p6 at n = 8192), lane bit 5 -> p3, lane bits 0..3 -> the
//          four bits above the lane's block (twisted, below), chunk bit c2
//          and lane bit 4 -> the two top bits.  In LDS each 1 KB block of the
//          row is stored with its 64 chunks permuted (sig) so that these
//          reads are free of bank conflicts.
//   MFMA:  the B operand of lane l holds B[k][col] with col = lane bits 0..3
//          and k = 8 (l/16) + j, j = 0..7: the eight chunks c2 c1 c0 after an
//          in-register transpose (v_perm), so k = (c0, c1, c2, l4, l5); the
//          four tiles (e0, e1) of one chunk element pair supply k5, k6.  The
//          outputs D[m][col], m = 4 (l/16) + j' plus 16 x out-block, carry
//          the same seven position bits in Sylvester order: c0, c1 in the
//          register slot j', c2 and l4 now on lane bits 4 and 5, l5, e0, e1
//          in the out-block.  Every lane then holds R consecutive positions.
//   DPP:   lane bits 0, 1 (quad_perm), 2 (row_half_mirror, which pairs
//          lanes l and l ^ 7) and 3 (row_ror:8, l ^ 8).  So that l ^ 7 is a
//          butterfly partner, lanes with bit 2 set hold the positions of
//          bits 0 and 1 flipped (the twist).
#pragma once

#include "rht_quant.hpp"

namespace whtq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Streaming (non-temporal) global accesses: every byte is touched once, and
// on MI355X the non-temporal hint lifts a plain read + write stream from about
// 64 % to about 80 % of peak HBM bandwidth.
template <typename V>
__device__ __forceinline__ void stg_stream(void* p, V v) {
  __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
}

template <int LOGN>
struct MxGeo {
  static_assert(LOGN == 12 || LOGN == 13, "matrix-core quantiser: n = 4096 or 8192");
  static constexpr int N = 1 << LOGN;
  static constexpr int R = N / 64;      // values per lane
  static constexpr int LOW = LOGN - 6;  // in-lane position bits
  static constexpr int NC = R / 8;      // 16-byte chunks per lane
  static constexpr int NG = R / 32;     // groups of four tiles (one H128 product each)
  static constexpr int WPB = LOGN == 12 ? 4 : 8;  // waves per block
  static constexpr int THREADS = 64 * WPB;

  // the four position bits above a lane's block, from lane bits 0..3
  __device__ static __forceinline__ int twist(int l) {
    return ((l & 3) ^ ((l & 4) ? 3 : 0)) | (l & 12);
  }
  // first position of the R consecutive outputs lane l holds after the MFMA
  __device__ static __forceinline__ int out_block(int l) { return twist(l) | (l & 48); }
  // position of element 0 of chunk c in lane l (load side)
  __device__ static __forceinline__ int chunk_pos(int l, int c) {
    return (((l >> 5) & 1) << 3) | ((c & 1) << 4) | (((c >> 1) & 1) << 5) | (((c >> 3) & 1) << 6) |
           (twist(l) << LOW) | (((c >> 2) & 1) << (LOW + 4)) | (((l >> 4) & 1) << (LOW + 5));
  }
  static constexpr int chunk_off(int c) {
    return ((c & 1) << 4) | (((c >> 1) & 1) << 5) | (((c >> 3) & 1) << 6) | (((c >> 2) & 1) << (LOW + 4));
  }
  // Coalesced staging (one 1 KB block of the row per copy instruction): lane
  // i of the copy of block b fetches the block's 16-byte chunk sinv(b, i) and
  // it lands in LDS slot i; chunk x of block b sits in slot sig(b, x).  The
  // slots are chosen so that the 16 lanes of a quarter-wave reading one
  // chunk each (they differ in lane bits 0..3) hit 16 distinct 16-byte bank
  // slots.
  static constexpr int sig(int b, int x) {
    return LOGN == 12 ? (((x >> 3) | ((x & 7) << 3)) ^ ((b & 1) << 3))
                      : (((x >> 4) | ((x & 15) << 2)) ^ ((b & 3) << 2));
  }
  __device__ static __forceinline__ int sinv(int b, int i) {
    if constexpr (LOGN == 12) {
      const int y = i ^ ((b & 1) << 3);
      return ((y & 7) << 3) | (y >> 3);
    } else {
      const int y = i ^ ((b & 3) << 2);
      return ((y & 3) << 4) | (y >> 2);
    }
  }
  // n = 4096: slot of chunk c minus slot of chunk 0, the same for every lane
  // (chunk bits c0, c1 land on slot bits 4, 5 and c2 on bit 7)
  static constexpr int slot_step(int c) { return ((c & 1) << 4) | (((c >> 1) & 1) << 5) | (((c >> 2) & 1) << 7); }
  // in-lane position of output register j' of out-block ob of tile group g
  static constexpr int out_off(int g, int ob, int jp) {
    return ((ob >> 1) & 1) | (((ob >> 2) & 1) << 1) | ((g & 1) << 2) | ((ob & 1) << 3) | (jp << 4) |
           ((g >> 1) << 6);
  }
};

template <bool BF16> struct MxOp;
template <> struct MxOp<true> {
  typedef bf16x8_t vec;
  static constexpr uint16_t ONE = 0x3f80, NEG = 0xbf80;
  __device__ static __forceinline__ f32x4 mma(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(vec, a), __builtin_bit_cast(vec, b), c,
                                                   0, 0, 0);
  }
};
template <> struct MxOp<false> {
  typedef f16x8_t vec;
  static constexpr uint16_t ONE = 0x3c00, NEG = 0xbc00;
  __device__ static __forceinline__ f32x4 mma(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(vec, a), __builtin_bit_cast(vec, b), c,
                                                  0, 0, 0);
  }
};

// DPP butterflies over 8 values: x += c * x[partner], partner by CTRL.
#define WHTQ_DPP_HM "row_half_mirror row_mask:0xf bank_mask:0xf"
#define WHTQ_DPP_R8 "row_ror:8 row_mask:0xf bank_mask:0xf"

template <int LANEBIT>
__device__ __forceinline__ void dpp_bfly8_mx(float* v, float k) {
  if constexpr (LANEBIT == 0) WHTQ_DPP8(WHTQ_DPP_Q0);
  else if constexpr (LANEBIT == 1) WHTQ_DPP8(WHTQ_DPP_Q1);
  else if constexpr (LANEBIT == 2) WHTQ_DPP8(WHTQ_DPP_HM);
  else WHTQ_DPP8(WHTQ_DPP_R8);
}

template <int LOGN, int DIN, int BITS, int LOGG>
__global__ __launch_bounds__(MxGeo<LOGN>::THREADS) void k_rht_quant_mx(
    const uint8_t* __restrict__ w, int64_t rows, int64_t ldw_b, const uint32_t* __restrict__ sbits,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales, float inv_sqrt_n) {
  using G = MxGeo<LOGN>;
  using OP = MxOp<DIN == DT_BF16>;
  using QP = QPack<BITS>;
  constexpr int R = G::R, NC = G::NC;
  constexpr int GS = 1 << LOGG;
  constexpr int GL = GS <= R ? GS : R;           // group length inside one lane
  constexpr int NGL = R / GL;                    // groups per lane
  constexpr int SPAN = GS <= R ? 1 : GS / R;     // lanes per group (1, 2 or 4)
  constexpr int ROW_CODE_B = (G::N * BITS) / 8;
  constexpr int LANE_CODE_B = (R * BITS) / 8;
  constexpr int NSC = G::N / GS;
  constexpr float QM = (float)QP::QMAX;
  static_assert(SPAN <= 4, "a group spans at most one quad of lanes");

  const int l = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // sign masks (bit 15 / 31 of each input word), shared by the block's waves:
  // [chunk][lane] x 16 bytes
  __shared__ u32x4 smask[NC * 64];
  // each wave's next row, fetched straight into LDS while the current row is
  // transformed: [chunk][lane] x 16 bytes, the image of the register layout
  __shared__ u32x4 rowbuf[G::WPB][NC * 64];
  const int64_t wave0 = (int64_t)blockIdx.x * G::WPB + wv;
  const int64_t wstride = (int64_t)gridDim.x * G::WPB;
  u32x4* buf = rowbuf[wv];
  // coalesced copies: block b = 64 consecutive chunks; the lane's source
  // chunk within the block depends on b only through b & 1 (n = 4096) or
  // b & 3 (n = 8192)
  constexpr int NV = LOGN == 12 ? 2 : 4;
  int src_off[NV];
#pragma unroll
  for (int q = 0; q < NV; ++q) src_off[q] = G::sinv(q, l) * 16;
  auto fetch_row = [&](int64_t row) {
    const uint8_t* wr = w + row * ldw_b;
#pragma unroll
    for (int b = 0; b < NC; ++b)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(wr + b * 1024 + src_off[b % NV]),
          (__attribute__((address_space(3))) void*)(buf + b * 64), 16, 0, 2 /* nt */);
  };
  // LDS slot of chunk c of lane l; at n = 4096 the chunk bits enter the slot
  // additively (a lane base plus a per-chunk constant), so the reads share
  // one address register
  auto slot_of = [&](int c) {
    if constexpr (LOGN == 12) {
      const int m0 = G::chunk_pos(l, 0) >> 3;
      return (m0 >> 6) * 64 + G::sig(m0 >> 6, m0 & 63) + G::slot_step(c);
    } else {
      const int m = G::chunk_pos(l, c) >> 3;
      return (m >> 6) * 64 + G::sig(m >> 6, m & 63);
    }
  };
  // n = 4096 (a row or two per wave, latency-bound): the first row's copy is
  // in flight while the block builds its sign masks.  n = 8192 (fourteen rows
  // per wave at the benchmark size) measured about 1 % slower that way and
  // copies after the set-up.
  if constexpr (LOGN == 12)
    if (wave0 < rows) fetch_row(wave0);
  {
    // every sign word is requested before any is used, so the block waits
    // for one round trip (overlapping the row copy's), not one per pass
    constexpr int NIT = NC * 64 / G::THREADS;
    static_assert(NIT * G::THREADS == NC * 64, "sign-mask setup: whole passes");
    const uint32_t* sp = sbits != nullptr ? sbits : kNoSigns;
    uint32_t wd[NIT];
    int pos[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int i = threadIdx.x + it * G::THREADS;
      pos[it] = G::chunk_pos(i % 64, i / 64);
      wd[it] = sp[pos[it] >> 5];
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const uint32_t sbyte = (wd[it] >> (pos[it] & 31)) & 0xffu;
      smask[threadIdx.x + it * G::THREADS] = u32x4{pair_mask16(sbyte), pair_mask16(sbyte >> 2),
                                                   pair_mask16(sbyte >> 4), pair_mask16(sbyte >> 6)};
    }
  }
  // a barrier on the LDS writes only (an n = 4096 row copy stays in flight)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if constexpr (LOGN == 13)
    if (wave0 < rows) fetch_row(wave0);

  // the four distinct 16x32 slices of H_128 (A operands): lane l holds
  // row i = l % 16, columns k = 8 (l / 16) + j; T[o0][s] has entries
  // (-1)^(s + popcount(i & k & 15) + o0 * (k >> 4)).  With q = l / 16 and
  // j = 2d + h that exponent is s + o0 q1 + i3 q0 + i1 d0 + i2 d1 + i0 h
  // (bits of q, d, i), so each word is a lane constant with both halves'
  // sign bits (M) flipped by the terms in o0, s and d.
  u32x4 T[2][2];
  {
    constexpr uint32_t M = 0x80008000u;
    const int i = l & 15, q = l >> 4;
    const uint32_t w0 = (uint32_t)OP::ONE * 0x10001u ^ ((i & 1) ? 0x80000000u : 0u);
    const uint32_t e1 = ((i >> 1) & 1) ? M : 0u, e2 = ((i >> 2) & 1) ? M : 0u;
    const uint32_t ed[4] = {0u, e1, e2, e1 ^ e2};
#pragma unroll
    for (int o0 = 0; o0 < 2; ++o0) {
      const uint32_t x = w0 ^ ((((o0 & (q >> 1)) ^ ((i >> 3) & q)) & 1) ? M : 0u);
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int d = 0; d < 4; ++d) T[o0][s][d] = x ^ ed[d] ^ (s ? M : 0u);
    }
  }

  // DPP coefficients and the accumulated sign rho of the lane
  const int tw = G::twist(l);
  float cf[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) cf[b] = ((tw >> b) & 1) ? -1.0f : 1.0f;
  const bool rho = __builtin_popcount(tw) & 1;
  const int ob_lane = G::out_block(l);

  for (int64_t row = wave0; row < rows; row += wstride) {
    u32x4 raw[NC];
    // The copies must have landed before any read of buf.  The compiler sees
    // each global_load_lds as a 16-byte write at its LDS pointer (not the
    // wave's 1 KB), so it may place its own wait after reads it believes do
    // not overlap: wait explicitly.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int c = 0; c < NC; ++c) raw[c] = buf[slot_of(c)];
    // the reads must have returned before the next row's copies overwrite buf
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (row + wstride < rows) fetch_row(row + wstride);
#pragma unroll
    for (int c = 0; c < NC; ++c) raw[c] ^= smask[c * 64 + l];

    // transpose: tile (e, c3) dword d = (chunk 2d, element e | chunk 2d+1, element e)
    u32x4 tile[NC];
#pragma unroll
    for (int c3 = 0; c3 < NC / 8; ++c3)
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          tile[e + 8 * c3][d] = __builtin_amdgcn_perm(raw[8 * c3 + 2 * d + 1][e >> 1], raw[8 * c3 + 2 * d][e >> 1],
                                                      (e & 1) ? 0x07060302u : 0x05040100u);

    // H_128 along (c0, c1, c2, l4, l5, e0, e1) for each tile group g = (e2, c3)
    float v[R];
#pragma unroll
    for (int g = 0; g < G::NG; ++g) {
      f32x4 acc[8];
#pragma unroll
      for (int ob = 0; ob < 8; ++ob) acc[ob] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 b = tile[kb + 4 * (g & 1) + 8 * (g >> 1)];
#pragma unroll
        for (int ob = 0; ob < 8; ++ob)
          acc[ob] = OP::mma(T[ob & 1][__builtin_popcount((ob >> 1) & kb) & 1], b, acc[ob]);
      }
#pragma unroll
      for (int ob = 0; ob < 8; ++ob)
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) v[G::out_off(g, ob, jp)] = acc[ob][jp];
    }
    // in-register stages: p2 (and p6 at n = 8192)
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (!(r & 4)) bfly(v[r], v[r | 4]);
    if constexpr (R == 128) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (!(r & 64)) bfly(v[r], v[r | 64]);
    }
    // DPP stages over lane bits 0..3
#pragma unroll
    for (int r = 0; r < R; r += 8) dpp_bfly8_mx<0>(v + r, cf[0]);
#pragma unroll
    for (int r = 0; r < R; r += 8) dpp_bfly8_mx<1>(v + r, cf[1]);
#pragma unroll
    for (int r = 0; r < R; r += 8) dpp_bfly8_mx<2>(v + r, cf[2]);
#pragma unroll
    for (int r = 0; r < R; r += 8) dpp_bfly8_mx<3>(v + r, cf[3]);

    // ---- epilogue: group absmax -> fp16 scale -> codes
    float mult[NGL];
    uint16_t s16b[NGL];
    bool ovf = false;
#pragma unroll
    for (int k = 0; k < NGL; ++k) {
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e + 1 < GL; e += 2) a4[(e >> 1) & 3] = max3abs(a4[(e >> 1) & 3], v[k * GL + e], v[k * GL + e + 1]);
      float a = __builtin_fmaxf(__builtin_fmaxf(a4[0], a4[1]), __builtin_fmaxf(a4[2], a4[3]));
      a = quad_max(a, SPAN);
      const float s_pre = (a * inv_sqrt_n) / QM;
      const _Float16 h = (_Float16)s_pre;
      const float sf = (float)h;
      const float dv = inv_sqrt_n / __builtin_fmaxf(sf, 1.17549435e-38f);
      const float mm = sf > 0.f ? dv : 0.f;
      mult[k] = rho ? -mm : mm;
      s16b[k] = __builtin_bit_cast(uint16_t, h);
      ovf |= a * mm > QM + 0.25f;
    }
    uint32_t cw[LANE_CODE_B / 4];
    auto codes_of = [&](auto clip) {
      auto q_of = [&](int r) {
        float f = __builtin_fmaf(v[r], mult[r / GL], QP::MAGIC);
        if constexpr (decltype(clip)::value) f = __builtin_amdgcn_fmed3f(f, QP::MAGIC - QM, QP::MAGIC + QM);
        return as_u(f);
      };
      if constexpr (BITS == 3) {
#pragma unroll
        for (int j = 0; j < LANE_CODE_B / 4; ++j) cw[j] = 0u;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t c = q_of(r) & 7u;
          const int bit = 3 * r, wi = bit >> 5, off = bit & 31;
          cw[wi] |= c << off;
          if (off > 29) cw[wi + 1] |= c >> (32 - off);
        }
      } else {
#pragma unroll
        for (int j = 0; j < LANE_CODE_B / 4; ++j) {
          uint32_t acc = 0;
#pragma unroll
          for (int k = 0; k < QP::PER_WORD; ++k) acc = __builtin_amdgcn_alignbit(q_of(j * QP::PER_WORD + k), acc, BITS);
          cw[j] = acc;
        }
      }
    };
    if (__builtin_amdgcn_ballot_w64(ovf)) codes_of(std::true_type{});
    else codes_of(std::false_type{});
    uint8_t* cr = codes + row * (int64_t)ROW_CODE_B + ob_lane * LANE_CODE_B;
    if constexpr (BITS == 3) {  // 24 or 48 bytes a lane: 8-byte aligned
#pragma unroll
      for (int j = 0; j < LANE_CODE_B / 4; j += 2) stg_stream<u32x2>(cr + 4 * j, u32x2{cw[j], cw[j + 1]});
    } else {
#pragma unroll
      for (int j = 0; j < LANE_CODE_B / 4; j += 4)
        stg_stream<u32x4>(cr + 4 * j, u32x4{cw[j], cw[j + 1], cw[j + 2], cw[j + 3]});
    }
    uint16_t* sr = scales + row * (int64_t)NSC;
    if constexpr (SPAN == 1) {
#pragma unroll
      for (int k = 0; k < NGL; ++k) stg_stream<uint16_t>(sr + ob_lane * NGL + k, s16b[k]);
    } else {
      stg_stream<uint16_t>(sr + ob_lane / SPAN, s16b[0]);
    }
  }
}

template <int LOGN, int DIN, int BITS, int LOGG>
static hipError_t run_q_mx(const void* w, int64_t rows, int64_t ldw, const uint32_t* sb, uint8_t* codes,
                           uint16_t* scales, hipStream_t s) {
  using G = MxGeo<LOGN>;
  auto k = k_rht_quant_mx<LOGN, DIN, BITS, LOGG>;
  static const int nb = blocks_per_cu(k, G::THREADS, 0);
  const unsigned grid = persistent_grid((rows + G::WPB - 1) / G::WPB, nb);
  hipLaunchKernelGGL(k, dim3(grid), dim3(G::THREADS), 0, s, (const uint8_t*)w, rows, ldw * 2, sb, codes, scales,
                     (float)(1.0 / __builtin_sqrt((double)(1 << LOGN))));
  return hipGetLastError();
}

}  // namespace whtq
