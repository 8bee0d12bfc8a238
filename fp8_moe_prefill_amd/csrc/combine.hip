// Weighted combine of each token's k expert rows back into token order
// (moe_unpermute_combine):  out[t, :] = sum_{j=0..k-1} w[t, j] * y[pos[t*k + j], :].
//
// "FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant", section 1: the grouped
// GEMM replaces per-token dispatch, so its rows come back in grouped order and must be
// returned to their tokens with the router weights.
//
// HBM-bound gather: one thread per 8 consecutive columns (16-byte bf16 / 32-byte fp32
// loads), up to eight of a token's rows loaded together, the k rows summed in fp32 in
// increasing j -- a fixed order, so the result is deterministic (no atomics).
#include "common.h"
#include "launch.h"

namespace fp8moe {
namespace {

__device__ __forceinline__ void load8(const uint16_t* p, float* f) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}
__device__ __forceinline__ void load8(const float* p, float* f) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void store8(uint16_t* p, const float* f) {
  uint4 u;
  u.x = f32_to_bf16(f[0]) | (f32_to_bf16(f[1]) << 16);
  u.y = f32_to_bf16(f[2]) | (f32_to_bf16(f[3]) << 16);
  u.z = f32_to_bf16(f[4]) | (f32_to_bf16(f[5]) << 16);
  u.w = f32_to_bf16(f[6]) | (f32_to_bf16(f[7]) << 16);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

template <typename YT, typename OT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ w, int64_t T,
                                                      int k, int64_t H, int HB,
                                                      OT* __restrict__ out) {
  const int64_t t = blockIdx.x / HB;
  const int64_t h0 = ((int64_t)(blockIdx.x % HB) * 256 + threadIdx.x) * 8;
  if (h0 >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int j = 0;
  // eight rows at a time: their positions and weights, then all eight row loads in flight
  // together, then the sums in increasing j (the same order as one row at a time)
  for (; j + 8 <= k; j += 8) {
    int64_t row[8];
    float wj[8], f[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      row[u] = pos[t * k + j + u];
      wj[u] = w[t * k + j + u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) load8(y + row[u] * H + h0, f[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj[u], f[u][i], acc[i]);
  }
  for (; j < k; ++j) {
    const int64_t row = pos[t * k + j];
    const float wj = w[t * k + j];
    float f[8];
    load8(y + row * H + h0, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, f[i], acc[i]);
  }
  store8(out + t * H + h0, acc);
}

template <typename YT, typename OT>
hipError_t run(const void* y, const int32_t* pos, const float* w, int64_t T, int k, int64_t H,
               void* out, hipStream_t st) {
  const int HB = (int)((H / 8 + 255) / 256);
  combine_kernel<YT, OT><<<dim3((uint32_t)(T * HB)), 256, 0, st>>>(
      static_cast<const YT*>(y), pos, w, T, k, H, HB, static_cast<OT*>(out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* y, int32_t y_dtype, const int32_t* pos, const float* w,
                          int64_t T, int32_t k, int64_t H, int32_t out_dtype, void* out,
                          hipStream_t st) {
  if (y_dtype == FP8MOE_DTYPE_BF16) {
    if (out_dtype == FP8MOE_DTYPE_BF16) return run<uint16_t, uint16_t>(y, pos, w, T, k, H, out, st);
    return run<uint16_t, float>(y, pos, w, T, k, H, out, st);
  }
  if (out_dtype == FP8MOE_DTYPE_BF16) return run<float, uint16_t>(y, pos, w, T, k, H, out, st);
  return run<float, float>(y, pos, w, T, k, H, out, st);
}

}  // namespace fp8moe
