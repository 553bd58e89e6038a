// harp_build_blocks: the HARP blocks B_{t,c} = Q_{t,c}(theta) G_{b_t} from
// their parameters.
//
// HARP explainer, 2.2: Q is a Givens rotation when b_t = 2 and a Cayley map
// when b_t > 2, G a fixed base mixer (the normalised Sylvester Hadamard for a
// power-of-two radix, else a fixed orthogonal substitute); theta = 0 gives
// B = G.  2.4: the parameters may be stored as int8.  This library's
// readings: Givens Q = [[cos t, -sin t], [sin t, cos t]]; Cayley
// Q = (I - A)(I + A)^-1 = (I + A)^-1 (I - A) (the two factors commute) with
// the skew-symmetric A's strict upper triangle taken row by row from the
// parameters; int8 parameters are s_t * q with one fp32 scale per stage.
//
// One wave per block: lane i holds row i of [I + A | I - A]; Gauss-Jordan
// elimination with the pivot row broadcast by lane shuffles turns it into
// [I | Q] (I + A has the identity as symmetric part, so every pivot is
// nonzero and no row exchange is needed); then row i of Q G is formed from
// the mixer and written.  fp32 throughout.
#include "io.hpp"
#include "launch.hpp"

namespace whtq {

namespace hb {
constexpr int MAXST = 16;
}  // namespace hb

struct HbSched {
  int n;
  int b[hb::MAXST];
  long long poff[hb::MAXST];   // first parameter of the stage
  long long boff[hb::MAXST];   // first block element of the stage
  long long moff[hb::MAXST];   // first mixer element of the stage
  int first[hb::MAXST + 1];    // first block index of the stage (global numbering)
};

enum ParamDt : int { PD_F32 = 0, PD_I8 = 3 };

template <int PDT, int BDT>
__global__ __launch_bounds__(64) void k_harp_build(const void* __restrict__ params, const float* __restrict__ scales,
                                                  const float* __restrict__ mixers, void* __restrict__ blocks,
                                                  HbSched sc) {
  const int g = blockIdx.x, lane = threadIdx.x;
  int t = 0;
  while (t + 1 < sc.n && g >= sc.first[t + 1]) ++t;
  const int b = sc.b[t], c = g - sc.first[t];
  const int np = b == 2 ? 1 : b * (b - 1) / 2;
  const long long p0 = sc.poff[t] + (long long)c * np;
  auto par = [&](int k) -> float {
    if constexpr (PDT == PD_I8) return scales[t] * (float)reinterpret_cast<const int8_t*>(params)[p0 + k];
    else return reinterpret_cast<const float*>(params)[p0 + k];
  };
  // A[i][j] for the row i = lane: parameter i b - i (i + 1) / 2 + (j - i - 1) when i < j
  auto a_at = [&](int i, int j) -> float {
    if (i == j) return 0.f;
    const int lo = i < j ? i : j, hi = i < j ? j : i;
    const float v = par(lo * b - lo * (lo + 1) / 2 + (hi - lo - 1));
    return i < j ? v : -v;
  };

  float q[16];
  if (b == 2) {
    const float th = par(0);
    float sn, cs;
    sincosf(th, &sn, &cs);
    q[0] = lane == 0 ? cs : sn;
    q[1] = lane == 0 ? -sn : cs;
#pragma unroll
    for (int j = 2; j < 16; ++j) q[j] = 0.f;
  } else {
    float m[16], r[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float a = (lane < b && j < b) ? a_at(lane, j) : 0.f;
      const float e = lane == j ? 1.f : 0.f;
      m[j] = e + a;
      r[j] = e - a;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < b) {  // uniform
        float pm[16], pr[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          pm[j] = __shfl(m[j], k);
          pr[j] = __shfl(r[j], k);
        }
        const float inv = 1.0f / pm[k];
        const float f = lane == k ? 0.f : m[k] * inv;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float nm = lane == k ? m[j] * inv : fmaf(-f, pm[j], m[j]);
          const float nr = lane == k ? r[j] * inv : fmaf(-f, pr[j], r[j]);
          m[j] = nm;
          r[j] = nr;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) q[j] = r[j];
  }

  // row `lane` of Q G
  if (lane < b) {
    const float rs = 1.0f / __builtin_sqrtf((float)b);
    const long long o = sc.boff[t] + ((long long)c * b + lane) * b;
    for (int j = 0; j < b; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k < b) {
          const float gk = mixers ? mixers[sc.moff[t] + (long long)k * b + j]
                                  : ((__builtin_popcount((unsigned)(k & j)) & 1) ? -rs : rs);
          acc = fmaf(q[k], gk, acc);
        }
      }
      if constexpr (BDT == DT_F32) reinterpret_cast<float*>(blocks)[o + j] = acc;
      else reinterpret_cast<uint16_t*>(blocks)[o + j] = __builtin_bit_cast(uint16_t, (_Float16)acc);
    }
  }
}

// Entry from the C ABI (validated there): radices in [2, 16], at most 16
// stages, product d; mixers NULL only for power-of-two radices.
hipError_t launch_harp_build(const void* params, int pdt, const float* scales, int64_t d, const int32_t* radices,
                             int n_stages, const float* mixers, void* blocks, int bdt, hipStream_t s) {
  HbSched sc{};
  sc.n = n_stages;
  long long po = 0, bo = 0, mo = 0;
  int first = 0;
  for (int t = 0; t < n_stages; ++t) {
    const int b = radices[t];
    sc.b[t] = b;
    sc.poff[t] = po;
    sc.boff[t] = bo;
    sc.moff[t] = mo;
    sc.first[t] = first;
    po += (d / b) * (long long)(b == 2 ? 1 : b * (b - 1) / 2);
    bo += d * (long long)b;
    mo += (long long)b * b;
    first += (int)(d / b);
  }
  sc.first[n_stages] = first;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)first), dim3(64), 0, s, params, scales, mixers, blocks, sc);
  };
  if (pdt == PD_I8) {
    if (bdt == DT_F16) go(k_harp_build<PD_I8, DT_F16>);
    else go(k_harp_build<PD_I8, DT_F32>);
  } else {
    if (bdt == DT_F16) go(k_harp_build<PD_F32, DT_F16>);
    else go(k_harp_build<PD_F32, DT_F32>);
  }
  return hipGetLastError();
}

}  // namespace whtq
