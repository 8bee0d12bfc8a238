// Residual add + RMSNorm of the depth stack (fp8moe_rmsnorm).
//
// The FP8 grouped-expert prefill note ("FP8 grouped-expert prefill with on-chip int4-to-e4m3
// dequant", sections 1 and 3) runs its projections and experts inside a stack of
// transformer layers that use RMSNorm; the note prints no formula, so the plain one is
// taken: y = x / sqrt(mean(x^2) + eps), unit gain, with the residual stream and the
// normalised activations stored in bf16.
//
// One wave per row. The sum of squares of the bf16 values (each square exact in fp64) is
// accumulated in fp64 and the row's reciprocal 1 / sqrt(mean + eps) is formed in fp64.
// Both outputs are single roundings to bf16 (round to nearest even) of the exact value,
// formed in fp32 where that is provably the same rounding:
// * x + delta: two bf16 values whose exponents differ by at most 15 add exactly in fp32;
//   otherwise the smaller is below 2^-15 of the larger, a bf16 value, so the exact sum and
//   its fp32 rounding lie strictly between the same two bf16 rounding midpoints.
// * x * inv: the fp32 product of x and the fp32-rounded reciprocal is within two fp32 ulps
//   of the exact product, so its bf16 rounding is that of the exact value unless its low
//   16 bits lie within 3 of the midpoint 0x8000 (or it is subnormal, huge or not finite);
//   those elements (about one in 10^4) take the fp64 product and a single fp64 -> bf16
//   rounding instead, as does a whole row whose reciprocal is outside [2^-100, 2^100].
// The result is the correctly rounded bf16 of the exact value except when that value lies
// within a few fp64 ulps of a bf16 midpoint. Memory-bound: 2 bytes read per element (4 with
// the residual), 2 written (4 with the residual); for H <= 4096 a row stays in registers
// between the two passes.
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

// bf16(x + d) of 8 pairs (one uint4 each), a single rounding of the exact sum (above).
__device__ __forceinline__ uint4 add8(const uint4 x, const uint4 d) {
  const uint32_t a[4] = {x.x, x.y, x.z, x.w}, b[4] = {d.x, d.y, d.z, d.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = f32_to_bf16(bf16_lo(a[i]) + bf16_lo(b[i])) |
           (f32_to_bf16(bf16_hi(a[i]) + bf16_hi(b[i])) << 16);
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// ss += v^2 for the 8 bf16 values of w, in element order (each square exact in fp64)
__device__ __forceinline__ void sumsq8(const uint4 w, double& ss) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double lo = (double)bf16_lo(u[i]), hi = (double)bf16_hi(u[i]);
    ss = fma(lo, lo, ss);
    ss = fma(hi, hi, ss);
  }
}

// An fp32 product whose bf16 rounding may differ from that of the exact product: low 16
// bits within 3 of the midpoint, or exponent field 0, 1, 254 or 255.
__device__ __forceinline__ bool near_midpoint(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t e = (b >> 23) & 0xFFu;
  return ((b & 0xFFFFu) - 0x7FFDu) <= 6u || e - 2u >= 252u;
}

// bf16(x * inv) of 8 values: the fp32 product where it rounds the same, else fp64.
__device__ __forceinline__ uint4 scale8(const uint4 w, float inv32, double inv) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf16_lo(u[i]), hi = bf16_hi(u[i]);
    const float plo = lo * inv32, phi = hi * inv32;
    r[i] = bf16x2(plo, phi);
    if (near_midpoint(plo) || near_midpoint(phi))
      r[i] = f64_to_bf16((double)lo * inv) | (f64_to_bf16((double)hi * inv) << 16);
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// bf16(x * inv) of 8 values in fp64 (rows whose reciprocal is outside the fp32 margin)
__device__ __forceinline__ uint4 scale8_f64(const uint4 w, double inv) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = f64_to_bf16((double)bf16_lo(u[i]) * inv) |
           (f64_to_bf16((double)bf16_hi(u[i]) * inv) << 16);
  return make_uint4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ double row_inverse(double ss, int H, double eps) {
  return 1.0 / sqrt(ss / (double)H + eps);
}
__device__ __forceinline__ bool f32_reciprocal_ok(double inv) {
  return inv >= 0x1p-100 && inv <= 0x1p100;
}

// Rows of up to 512 * CPL elements: lane l holds chunks l, l + 64, ... (8 bf16 each) in
// registers, all loads issued at once. x_out may alias x (every load precedes the row's
// stores); y aliases neither.
template <int CPL>
__global__ __launch_bounds__(256) void rmsnorm_reg_kernel(const uint16_t* x, const uint16_t* delta,
                                                          uint16_t* x_out,
                                                          uint16_t* __restrict__ y, int T, int H,
                                                          double eps) {
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wv;
  if (row >= T) return;
  const int64_t base = (int64_t)row * H;
  const int nch = H / 8;
  const uint4* xr = reinterpret_cast<const uint4*>(x + base);
  uint4 v[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    v[j] = c < nch ? xr[c] : make_uint4(0u, 0u, 0u, 0u);
  }
  if (delta) {
    const uint4* dr = reinterpret_cast<const uint4*>(delta + base);
    uint4 d[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      d[j] = c < nch ? dr[c] : make_uint4(0u, 0u, 0u, 0u);
    }
    uint4* xo = reinterpret_cast<uint4*>(x_out + base);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c < nch) {
        v[j] = add8(v[j], d[j]);
        xo[c] = v[j];
      }
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < CPL; ++j)
    if (lane + 64 * j < nch) sumsq8(v[j], ss);
  ss = wave_sum_f64(ss);
  const double inv = row_inverse(ss, H, eps);
  uint4* yr = reinterpret_cast<uint4*>(y + base);
  if (f32_reciprocal_ok(inv)) {  // wave-uniform
    const float inv32 = (float)inv;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c < nch) yr[c] = scale8(v[j], inv32, inv);
    }
  } else {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c < nch) yr[c] = scale8_f64(v[j], inv);
    }
  }
}

// Longer rows: the same arithmetic in two passes over the row; the second pass reads the
// row again (its own stores of x_out with the residual). x_out may alias x; y aliases
// neither.
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
    if (delta) {
      w = add8(w, dr[c]);
      xo[c] = w;
    }
    sumsq8(w, ss);
  }
  ss = wave_sum_f64(ss);
  const double inv = row_inverse(ss, H, eps);
  const bool f32ok = f32_reciprocal_ok(inv);
  const float inv32 = (float)inv;
  for (int c = lane; c < nch; c += 64) {
    // the same lane wrote this chunk of x_out above, so it reads its own store
    const uint4 w = delta ? xo[c] : xr[c];
    yr[c] = f32ok ? scale8(w, inv32, inv) : scale8_f64(w, inv);
  }
}

template <int CPL>
hipError_t launch_reg(const uint16_t* x, const uint16_t* delta, int64_t T, int64_t H, double eps,
                      uint16_t* x_out, uint16_t* y, hipStream_t st) {
  rmsnorm_reg_kernel<CPL><<<dim3((uint32_t)((T + 3) / 4)), 256, 0, st>>>(x, delta, x_out, y,
                                                                           (int)T, (int)H, eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* delta, int64_t T, int64_t H,
                          double eps, uint16_t* x_out, uint16_t* y, hipStream_t st) {
  const int64_t nch = H / 8;
  if (nch <= 64) return launch_reg<1>(x, delta, T, H, eps, x_out, y, st);
  if (nch <= 128) return launch_reg<2>(x, delta, T, H, eps, x_out, y, st);
  if (nch <= 256) return launch_reg<4>(x, delta, T, H, eps, x_out, y, st);
  if (nch <= 512) return launch_reg<8>(x, delta, T, H, eps, x_out, y, st);
  rmsnorm_kernel<<<dim3((uint32_t)((T + 3) / 4)), 256, 0, st>>>(x, delta, x_out, y, (int)T,
                                                                 (int)H, eps);
  return hipGetLastError();
}

}  // namespace fp8moe
