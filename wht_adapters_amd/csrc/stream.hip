// whtq_stream_probe: a plain 16-byte streaming kernel that reads in_bytes and
// writes out_bytes of device memory, the bandwidth reference a transform
// kernel moving the same bytes is compared against ("% achievable").
// Blocks are split between the two streams in proportion to their bytes, so
// reads and writes proceed together, as in a copy; every access is 16 bytes,
// coalesced and non-temporal (the fastest plain form measured on MI355X).  The reads are XOR-folded
// into a value that is stored only if it equals an improbable constant, which
// keeps every load without writing anything extra.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "launch.hpp"

namespace whtq {

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_stream(const u32x4s* __restrict__ src, int64_t in_units,
                                                u32x4s* __restrict__ dst, int64_t out_units, int read_blocks) {
  const bool reader = (int)blockIdx.x < read_blocks;
  const int64_t nb = reader ? read_blocks : (int64_t)gridDim.x - read_blocks;
  const int64_t b = reader ? blockIdx.x : blockIdx.x - read_blocks;
  const int64_t T = nb * blockDim.x, t0 = b * blockDim.x + threadIdx.x;
  if (reader) {
    u32x4s acc = {0u, 0u, 0u, 0u};
    int64_t i = t0;
    for (; i + 7 * T < in_units; i += 8 * T) {
      u32x4s v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * T);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= v[u];
    }
    for (; i < in_units; i += T) acc ^= __builtin_nontemporal_load(src + i);
    if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0xf39cc060u && acc.w == 0x5ced4b1du &&
        out_units > 0)
      dst[0] = acc;
  } else {
    for (int64_t i = t0; i < out_units; i += T) __builtin_nontemporal_store(u32x4s{(uint32_t)i, 0u, 0u, 0u}, dst + i);
  }
}

hipError_t launch_stream_probe(const void* src, int64_t in_bytes, void* dst, int64_t out_bytes, hipStream_t s) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  const int64_t blocks = (int64_t)device_cu_count(dev) * 16;
  const double frac = (double)in_bytes / (double)(in_bytes + out_bytes);
  int rb = (int)std::llround(frac * (double)blocks);
  if (in_bytes > 0) rb = std::max(rb, 1);
  if (out_bytes > 0) rb = std::min<int>(rb, (int)blocks - 1);
  if (in_bytes == 0) rb = 0;
  const int grid = (out_bytes > 0 || in_bytes > 0) ? (int)blocks : 0;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_stream, dim3(grid), dim3(256), 0, s, (const u32x4s*)src, in_bytes / 16, (u32x4s*)dst,
                     out_bytes / 16, rb);
  return hipGetLastError();
}

}  // namespace whtq
