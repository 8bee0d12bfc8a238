// Dense W8A8 projection y = (s_a * s_w) * (qa . qw^T) (fp8_dense_gemm).
//
// FreeToken PR #389, "What this adds": projection weights quantised at load time to e4m3
// with one fp32 scale per tensor, a dynamic per-tensor activation scale, an FP8 x FP8 GEMM.
// memra-engine fp8_ffi module docs: both scales folded into one device scalar, no host sync.
//
// gfx950 design: with per-tensor scales the fp32 accumulator chains through the whole K
// loop inside the MFMA (no per-group fold), and the scalar s_a * s_w is applied once in
// the epilogue from device memory. Workgroup tile 128 x 128, 4 waves in a 2 x 2 grid of
// 64 x 64 (4 x 4 tiles of v_mfma_f32_16x16x128_f8f6f4); both operands are K-contiguous
// and staged through XOR-swizzled LDS, double-buffered with one barrier per 128-wide
// K step.
#include "common.h"
#include "launch.h"

namespace fp8moe {
namespace {

constexpr int TM = 128, TN = 128;

// chunk c of row r at position c ^ (r & 7) ^ ((r >> 3) & 1): conflict-free ds_read_b128 of
// one chunk across 16 consecutive rows
__device__ __forceinline__ int t_off(int r, int c) {
  return r * 128 + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void dense_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ a_blk,
    const uint8_t* __restrict__ W, const float* __restrict__ w_scale, int M, int N, int K,
    int NTN, void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][TM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][TN * 128];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t L = xcd_contiguous(blockIdx.x, gridDim.x);
  const int tm = (int)(L / (uint32_t)NTN), tn = (int)(L % (uint32_t)NTN);
  const int m0 = tm * TM, n0 = tn * TN;
  const int wm = wv >> 1, wn = wv & 1;
  const int q = lane >> 4, c16 = lane & 15;

  // staging: thread -> (row, half of the 128-byte K slice) for A and for W
  const int sr = tid >> 1, sh = tid & 1;
  const uint8_t* a_src = A + (int64_t)min(m0 + sr, M - 1) * K + sh * 64;
  const uint8_t* b_src = W + (int64_t)min(n0 + sr, N - 1) * K + sh * 64;

  v4f acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[t][s] = (v4f){0.f, 0.f, 0.f, 0.f};

  uint4 ra[4], rb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = *reinterpret_cast<const uint4*>(a_src + i * 16);
    rb[i] = *reinterpret_cast<const uint4*>(b_src + i * 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<uint4*>(&sA[0][t_off(sr, sh * 4 + i)]) = ra[i];
    *reinterpret_cast<uint4*>(&sB[0][t_off(sr, sh * 4 + i)]) = rb[i];
  }
  __syncthreads();

  const int KS = K / 128;
  for (int ks = 0; ks < KS; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < KS;
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const uint4*>(a_src + (ks + 1) * 128 + i * 16);
        rb[i] = *reinterpret_cast<const uint4*>(b_src + (ks + 1) * 128 + i * 16);
      }
    }
    v8i bop[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = wn * 64 + s * 16 + c16;
      uint4 lo = *reinterpret_cast<const uint4*>(&sB[cur][t_off(r, 2 * q)]);
      uint4 hi = *reinterpret_cast<const uint4*>(&sB[cur][t_off(r, 2 * q + 1)]);
      bop[s] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = wm * 64 + t * 16 + c16;
      uint4 lo = *reinterpret_cast<const uint4*>(&sA[cur][t_off(r, 2 * q)]);
      uint4 hi = *reinterpret_cast<const uint4*>(&sA[cur][t_off(r, 2 * q + 1)]);
      v8i aop = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc[t][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[s], acc[t][s], 0,
                                                                     0, 0, 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4*>(&sA[cur ^ 1][t_off(sr, sh * 4 + i)]) = ra[i];
        *reinterpret_cast<uint4*>(&sB[cur ^ 1][t_off(sr, sh * 4 + i)]) = rb[i];
      }
    }
    __syncthreads();
  }

  const float scale = a_blk[2] * w_scale[0];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm * 64 + t * 16 + 4 * q + r;
      if (row < M) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int cc = n0 + wn * 64 + s * 16 + c16;
          if (cc < N) {
            const float v = acc[t][s][r] * scale;
            if (OUT_BF16)
              reinterpret_cast<uint16_t*>(out)[(int64_t)row * N + cc] = (uint16_t)f32_to_bf16(v);
            else
              reinterpret_cast<float*>(out)[(int64_t)row * N + cc] = v;
          }
        }
      }
    }
}

}  // namespace

hipError_t launch_dense_gemm(const uint8_t* a, const float* a_blk, const uint8_t* w,
                             const float* w_scale, int64_t M, int64_t N, int64_t K,
                             int32_t out_dtype, void* out, hipStream_t st) {
  const int NTM = (int)((M + TM - 1) / TM), NTN = (int)((N + TN - 1) / TN);
  dim3 grid((uint32_t)(NTM * NTN)), block(256);
  if (out_dtype == FP8MOE_DTYPE_BF16)
    dense_gemm_kernel<true><<<grid, block, 0, st>>>(a, a_blk, w, w_scale, (int)M, (int)N, (int)K,
                                                    NTN, out);
  else
    dense_gemm_kernel<false><<<grid, block, 0, st>>>(a, a_blk, w, w_scale, (int)M, (int)N,
                                                     (int)K, NTN, out);
  return hipGetLastError();
}

}  // namespace fp8moe
