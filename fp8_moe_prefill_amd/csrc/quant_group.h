// The group-mode activation quantiser as a device function over one (virtual) 256-thread
// block, shared by the quantiser's own kernel and the launch that runs it beside the
// top-k routing (quant_route_kernel): the chunks a thread handles, and so every output,
// depend only on the block index, the block count and the thread index passed in.
#pragma once

#include "common.h"

namespace fp8moe {
namespace qg {

struct F8 {
  float v[8];
};

__device__ __forceinline__ F8 unpack8(uint4 u) {
  F8 f;
  f.v[0] = bf16_lo(u.x); f.v[1] = bf16_hi(u.x);
  f.v[2] = bf16_lo(u.y); f.v[3] = bf16_hi(u.y);
  f.v[4] = bf16_lo(u.z); f.v[5] = bf16_hi(u.z);
  f.v[6] = bf16_lo(u.w); f.v[7] = bf16_hi(u.w);
  return f;
}

__device__ __forceinline__ float amax8(const F8& f) {
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f.v[j]));  // fmaxf skips NaN
  return m;
}

__device__ __forceinline__ uint2 encode8(const F8& f, float inv) {
  uint2 r;
  r.x = e4m3x4(f.v[0] * inv, f.v[1] * inv, f.v[2] * inv, f.v[3] * inv);
  r.y = e4m3x4(f.v[4] * inv, f.v[5] * inv, f.v[6] * inv, f.v[7] * inv);
  return r;
}

// Chunks of 8 consecutive elements per thread: kChunks of them, a whole grid apart, all
// loaded before any is processed (more loads in flight per thread hide the HBM latency);
// the 16 consecutive lanes of a quarter wave hold one 128-group.
constexpr int kChunks = 2;

// Block `block` of `nblocks` 256-thread blocks, thread `tid` (its lane = tid % 64), CH
// chunks per thread: the blocks cover 256 * CH * nblocks >= nchunks chunks.
template <int CH = kChunks>
__device__ __forceinline__ void group_block(const uint4* __restrict__ x, int64_t nchunks,
                                            uint2* __restrict__ q, float* __restrict__ scales,
                                            float* __restrict__ sums, int64_t block,
                                            int64_t nblocks, int tid) {
  const int64_t stride = nblocks * 256;
  const int64_t i0 = block * 256 + tid;
  uint4 u[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int64_t i = i0 + j * stride;
    // nchunks and stride are multiples of 16: groups are all-or-nothing
    u[j] = i < nchunks ? x[i] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int64_t i = i0 + j * stride;
    const F8 f = unpack8(u[j]);
    const float m = max16(amax8(f));
    float s, inv;
    scale_pair(m, s, inv);
    const uint2 c = encode8(f, inv);
    // optional: the sum of the group's code values (the grouped GEMM's offset seed)
    const float gs = sums ? sum16(e4m3_sum8(c.x, c.y)) : 0.f;
    if (i < nchunks) {
      q[i] = c;
      if ((tid & 15) == 0) {
        scales[i >> 4] = s;
        if (sums) sums[i >> 4] = gs;
      }
    }
  }
}

}  // namespace qg
}  // namespace fp8moe
