// Residual add + RMSNorm of the depth stack (fp8moe_rmsnorm).
//
// The FP8 grouped-expert prefill note ("FP8 grouped-expert prefill with on-chip int4-to-e4m3
// dequant", sections 1 and 3) runs its projections and experts inside a stack of
// transformer layers that use RMSNorm; the note prints no formula, so the plain one is
// taken: y = x / sqrt(mean(x^2) + eps), unit gain, with the residual stream and the
// normalised activations stored in bf16.
//
// One wave per row. The sum of squares of the bf16 values (each square exact in fp64) is
// accumulated in fp64, x / sqrt(mean + eps) is formed in fp64 (as x times the row's fp64
// reciprocal) and rounded once to bf16: the correctly rounded bf16 of the exact value
// except when that value lies within a few fp64 ulps of a bf16 rounding midpoint. The
// residual add x + delta of two bf16 values is exact in fp64 and is rounded once to bf16
// the same way. Memory-bound: 2 bytes read per element (4 with the residual), 2 written
// (4 with the residual).
#include "common.h"
#include "launch.h"

namespace fp8moe {
namespace {

// fp64 -> bf16 bits, round to nearest even, in one rounding. The fp32 conversion rounds
// first; that can only go wrong when it lands exactly on a bf16 midpoint (low 16 bits
// 0x8000) from a value that was not one, and then one fp32 ulp back toward the exact value
// restores the side of the midpoint the exact value is on.
__device__ __forceinline__ uint32_t f64_to_bf16(double v) {
  if (v != v) return 0x7FC0u;
  const float f = (float)v;
  uint32_t b = __float_as_uint(f);
  if ((b & 0xFFFFu) == 0x8000u && (double)f != v) {
    const bool up = v > (double)f;
    b = (up == (f > 0.f)) ? b + 1u : b - 1u;
  }
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// 8 bf16 (one uint4) -> 8 doubles
__device__ __forceinline__ void unpack8(const uint4 w, double* d) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d[2 * i] = (double)bf16_lo(u[i]);
    d[2 * i + 1] = (double)bf16_hi(u[i]);
  }
}

__device__ __forceinline__ uint4 pack8(const double* d) {
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = f64_to_bf16(d[2 * i]) | (f64_to_bf16(d[2 * i + 1]) << 16);
  return make_uint4(u[0], u[1], u[2], u[3]);
}

// x_out may alias x (in-place residual update); y aliases neither.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* x, const uint16_t* delta,
                                                      uint16_t* x_out, uint16_t* __restrict__ y,
                                                      int T, int H, double eps) {
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wv;
  if (row >= T) return;
  const int64_t base = (int64_t)row * H;
  const uint4* xr = reinterpret_cast<const uint4*>(x + base);
  const uint4* dr = reinterpret_cast<const uint4*>(delta + base);
  uint4* xo = reinterpret_cast<uint4*>(x_out + base);
  uint4* yr = reinterpret_cast<uint4*>(y + base);
  const int nch = H / 8;
  double ss = 0.0;
  for (int c = lane; c < nch; c += 64) {
    uint4 w = xr[c];
    double v[8];
    unpack8(w, v);
    if (delta) {
      double d[8];
      unpack8(dr[c], d);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += d[i];
      w = pack8(v);
      xo[c] = w;
      unpack8(w, v);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
  }
  ss = wave_sum_f64(ss);
  const double inv = 1.0 / sqrt(ss / (double)H + eps);
  for (int c = lane; c < nch; c += 64) {
    // the same lane wrote this chunk of x_out above, so it reads its own store
    const uint4 w = delta ? xo[c] : xr[c];
    double v[8];
    unpack8(w, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = v[i] * inv;
    yr[c] = pack8(v);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* delta, int64_t T, int64_t H,
                          double eps, uint16_t* x_out, uint16_t* y, hipStream_t st) {
  rmsnorm_kernel<<<dim3((uint32_t)((T + 3) / 4)), 256, 0, st>>>(x, delta, x_out, y, (int)T,
                                                                 (int)H, eps);
  return hipGetLastError();
}

}  // namespace fp8moe
