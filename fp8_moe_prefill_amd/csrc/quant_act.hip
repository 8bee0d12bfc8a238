// Dynamic activation quantisation bf16 -> e4m3 (fp8_quant_act).
//
// Group mode: one scale per (row, 128 columns) -- the per-(token, group) activation scale
// of "FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant", section 1.
// Per-tensor mode: one scale for the whole tensor -- FreeToken PR #389, "What this adds"
// (an amax pass, then the cast; one fused launch for small tensors, a reduction plus a
// cast launch above 64k elements, chosen by shape only).
// Row mode: one scale per row (token) -- FreeToken PR #389, "Limits" (row-wise activation
// scales, measured there against the per-tensor route).
// MXFP4 (mxfp4_quant_act): E2M1 codes with one E8M0 scale per 32 consecutive elements --
// the FP4 activations of DeepGEMM issue 338, in the OCP MX v1.0 MXFP4 format.
// Block-128 weights (fp8_quant_weight_block128): one scale per 128 x 128 block of an
// [N, K] weight -- the block-128 e4m3 class of the memra-engine fp8_ffi docs, made at load
// time.
// Scale rule amax/448: memra-engine fp8_ffi module docs.
//
// Both modes are HBM-bound streaming kernels: each thread reads 16-byte chunks (8 bf16),
// two of them in flight at once, and writes 8 bytes per chunk; a 128-group is the 16
// consecutive lanes of a quarter wave, so its amax is a 4-step cross-lane reduction with
// no LDS and no host synchronisation.
#include "common.h"
#include "launch.h"
#include "quant_group.h"

namespace fp8moe {
namespace {

using qg::F8;
using qg::amax8;
using qg::encode8;
using qg::kChunks;
using qg::unpack8;

__global__ __launch_bounds__(256) void quant_group_kernel(const uint4* __restrict__ x,
                                                          int64_t nchunks,
                                                          uint2* __restrict__ q,
                                                          float* __restrict__ scales,
                                                          float* __restrict__ sums) {
  qg::group_block(x, nchunks, q, scales, sums, blockIdx.x, gridDim.x, threadIdx.x);
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int j = 0; j < nw; ++j) r = fmaxf(r, red[j]);
  __syncthreads();
  return r;
}

// Small tensors: one workgroup does the amax pass and the cast.
__global__ __launch_bounds__(1024) void quant_tensor_fused_kernel(const uint4* __restrict__ x,
                                                                 int64_t nchunks,
                                                                 uint2* __restrict__ q,
                                                                 float* __restrict__ block) {
  __shared__ float red[16];
  float m = 0.f;
  for (int64_t i = threadIdx.x; i < nchunks; i += blockDim.x) m = fmaxf(m, amax8(unpack8(x[i])));
  float amax = block_max(m, red);
  float s, inv;
  scale_pair(amax, s, inv);
  if (threadIdx.x == 0) {
    block[0] = amax; block[1] = inv; block[2] = s; block[3] = 0.f;
  }
  for (int64_t i = threadIdx.x; i < nchunks; i += blockDim.x) q[i] = encode8(unpack8(x[i]), inv);
}

// Large tensors, pass 1: per-workgroup partial amax (no atomics: the result does not
// depend on scheduling order).
__global__ __launch_bounds__(256) void quant_tensor_amax_kernel(const uint4* __restrict__ x,
                                                               int64_t nchunks,
                                                               float* __restrict__ partials) {
  __shared__ float red[4];
  float m = 0.f;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nchunks; i += kChunks * stride) {
    uint4 u[kChunks];
#pragma unroll
    for (int j = 0; j < kChunks; ++j)
      u[j] = i + j * stride < nchunks ? x[i + j * stride] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < kChunks; ++j) m = fmaxf(m, amax8(unpack8(u[j])));
  }
  float r = block_max(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = r;
}

// Large tensors, pass 2: every workgroup reduces the partials, then casts its share.
__global__ __launch_bounds__(256) void quant_tensor_cast_kernel(const uint4* __restrict__ x,
                                                               int64_t nchunks,
                                                               const float* __restrict__ partials,
                                                               int npart, uint2* __restrict__ q,
                                                               float* __restrict__ block) {
  __shared__ float red[4];
  float m = 0.f;
  for (int j = threadIdx.x; j < npart; j += 256) m = fmaxf(m, partials[j]);
  float amax = block_max(m, red);
  float s, inv;
  scale_pair(amax, s, inv);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    block[0] = amax; block[1] = inv; block[2] = s; block[3] = 0.f;
  }
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nchunks; i += kChunks * stride) {
    uint4 u[kChunks];
#pragma unroll
    for (int j = 0; j < kChunks; ++j)
      u[j] = i + j * stride < nchunks ? x[i + j * stride] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < kChunks; ++j)
      if (i + j * stride < nchunks) q[i + j * stride] = encode8(unpack8(u[j]), inv);
  }
}

// Row mode: one workgroup per row. The row's amax is a block reduction; the cast pass
// reads the row again (a few KB, still in the caches), so HBM sees it once.
__global__ __launch_bounds__(256) void quant_row_kernel(const uint4* __restrict__ x,
                                                       int64_t nch, uint2* __restrict__ q,
                                                       float* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint4* xr = x + row * nch;
  uint2* qr = q + row * nch;
  float m = 0.f;
  for (int64_t c = threadIdx.x; c < nch; c += 256) m = fmaxf(m, amax8(unpack8(xr[c])));
  const float amax = block_max(m, red);
  float s, inv;
  scale_pair(amax, s, inv);
  if (threadIdx.x == 0) scales[row] = s;
  for (int64_t c = threadIdx.x; c < nch; c += 256) qr[c] = encode8(unpack8(xr[c]), inv);
}

// Block-128 weights: one workgroup per 128 x 128 block. Its 2048 chunks of 8 bf16 (128
// rows x 16 chunks) are held in registers, 8 per thread, across the block's amax
// reduction and the cast; rows past N (the last row block of a ragged N) are skipped.
__global__ __launch_bounds__(256) void quant_block128_kernel(const uint4* __restrict__ w,
                                                            int N, int K,
                                                            uint2* __restrict__ q,
                                                            float* __restrict__ scales) {
  __shared__ float red[4];
  const int nb = blockIdx.y, g = blockIdx.x, G = K / 128;
  const int64_t rs = K / 8;  // chunks per row
  uint4 u[8];
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = threadIdx.x + 256 * j, row = nb * 128 + (c >> 4);
    u[j] = row < N ? w[(int64_t)row * rs + g * 16 + (c & 15)] : make_uint4(0, 0, 0, 0);
    m = fmaxf(m, amax8(unpack8(u[j])));
  }
  const float amax = block_max(m, red);
  float s, inv;
  scale_pair(amax, s, inv);
  if (threadIdx.x == 0) scales[nb * G + g] = s;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = threadIdx.x + 256 * j, row = nb * 128 + (c >> 4);
    if (row < N) q[(int64_t)row * rs + g * 16 + (c & 15)] = encode8(unpack8(u[j]), inv);
  }
}

// MXFP4: one thread per 8 elements, four consecutive lanes per 32-element block. The
// shared exponent is floor(log2(amax)) - 2 clamped to [-127, 127], read straight from
// amax's exponent field (E8M0 byte = field - 2, clamped to [0, 254]; zero and subnormal
// maxima give 0); v / 2^e is an exact multiply, and the E2M1 code of its magnitude is the
// count of the rounding thresholds it passes (a midpoint counts toward the even code).
__device__ __forceinline__ uint32_t e2m1_code(float v, float inv) {
  const float a = fabsf(v * inv);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  const bool neg = (__float_as_uint(v) >> 31) && !(v != v);  // NaN encodes to +0
  return m | (neg ? 8u : 0u);
}

__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint4* __restrict__ x,
                                                         int64_t nchunks,
                                                         uint32_t* __restrict__ q,
                                                         uint8_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  // nchunks is a multiple of 4 and so is every block's first chunk: a quad of lanes is
  // either wholly in range or wholly out
  const uint4 u = i < nchunks ? x[i] : make_uint4(0, 0, 0, 0);
  const F8 f = unpack8(u);
  float m = amax8(f);
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
  const int field = (int)((__float_as_uint(m) >> 23) & 0xFF);
  const uint32_t b = (uint32_t)min(max(field - 2, 0), 254);
  const float inv = __uint_as_float((254u - b) << 23);  // 2^-(b - 127), b <= 252 here
  if (i < nchunks) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= e2m1_code(f.v[j], inv) << (4 * j);
    q[i] = w;
    if ((threadIdx.x & 3) == 0) scales[i >> 2] = (uint8_t)b;
  }
}

}  // namespace

hipError_t launch_quant_mxfp4(const uint16_t* x, int64_t M, int64_t K, uint8_t* q,
                              uint8_t* scales, hipStream_t st) {
  const int64_t nchunks = M * K / 8;
  quant_mxfp4_kernel<<<dim3((uint32_t)((nchunks + 255) / 256)), dim3(256), 0, st>>>(
      reinterpret_cast<const uint4*>(x), nchunks, reinterpret_cast<uint32_t*>(q), scales);
  return hipGetLastError();
}

hipError_t launch_quant_block128(const uint16_t* w, int64_t N, int64_t K, uint8_t* q,
                                 float* scales, hipStream_t st) {
  const dim3 grid((uint32_t)(K / 128), (uint32_t)((N + 127) / 128));
  quant_block128_kernel<<<grid, dim3(256), 0, st>>>(reinterpret_cast<const uint4*>(w), (int)N,
                                                   (int)K, reinterpret_cast<uint2*>(q), scales);
  return hipGetLastError();
}

hipError_t launch_quant_row(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* scales,
                            hipStream_t st) {
  quant_row_kernel<<<dim3((uint32_t)M), dim3(256), 0, st>>>(
      reinterpret_cast<const uint4*>(x), K / 8, reinterpret_cast<uint2*>(q), scales);
  return hipGetLastError();
}

hipError_t launch_quant_group(const uint16_t* x, int64_t M, int64_t K, uint8_t* q,
                              float* scales, float* sums, hipStream_t st) {
  const int64_t nchunks = M * K / 8;
  const int64_t blocks = (nchunks + 256 * kChunks - 1) / (256 * kChunks);
  quant_group_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, st>>>(
      reinterpret_cast<const uint4*>(x), nchunks, reinterpret_cast<uint2*>(q), scales, sums);
  return hipGetLastError();
}

hipError_t launch_quant_tensor(const uint16_t* x, int64_t n, uint8_t* q, float* block,
                               float* partials, hipStream_t st) {
  int64_t nchunks = n / 8;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint2* qv = reinterpret_cast<uint2*>(q);
  if (n <= kQuantFusedMax) {
    quant_tensor_fused_kernel<<<1, 1024, 0, st>>>(xv, nchunks, qv, block);
    return hipGetLastError();
  }
  int64_t want = (nchunks + 256 * 8 - 1) / (256 * 8);  // ~8 chunks per thread
  int npart = (int)(want < kQuantPartials ? want : kQuantPartials);
  quant_tensor_amax_kernel<<<npart, 256, 0, st>>>(xv, nchunks, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t cast_blocks = (nchunks + 256 * kChunks - 1) / (256 * kChunks);
  if (cast_blocks > 8192) cast_blocks = 8192;
  quant_tensor_cast_kernel<<<(uint32_t)cast_blocks, 256, 0, st>>>(xv, nchunks, partials, npart,
                                                                  qv, block);
  return hipGetLastError();
}

}  // namespace fp8moe
