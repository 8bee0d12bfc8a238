// bf16 x bf16 -> fp32 GEMM out = a . w^T (fp8moe_bf16_gemm): the depth stack's router and
// LM head.
//
// The FP8 grouped-expert prefill note ("FP8 grouped-expert prefill with on-chip int4-to-e4m3
// dequant", section 1) gates on the cosine of the final logits; FreeToken PR #389 ("Limits")
// keeps the LM head in bf16. The router that feeds the top-k selection and the LM head are
// therefore plain bf16 GEMMs with fp32 accumulation and fp32 output.
//
// gfx950 design: both operands K-contiguous ("TN"). For N > 128: workgroup tile 128 x 128,
// 4 waves in a 2 x 2 grid of 64 x 64, each 4 x 4 tiles of v_mfma_f32_16x16x32_bf16. One K step is 64
// elements (128 bytes per row), staged through XOR-swizzled LDS, double-buffered with one
// barrier per step; the next step's global loads are in flight during the MFMAs.
#include "common.h"
#include "launch.h"

namespace fp8moe {
namespace {

constexpr int TM = 128, TN = 128;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// 16-byte chunk c of row r at position c ^ (r & 7) ^ ((r >> 3) & 1): conflict-free
// ds_read_b128 of one chunk across 16 consecutive rows
__device__ __forceinline__ int t_off(int r, int c) {
  return r * 128 + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__global__ __launch_bounds__(256, 2) void bf16_gemm_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ W,
                                                           int M, int N, int K, int NTN,
                                                           float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][TM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][TN * 128];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t L = xcd_contiguous(blockIdx.x, gridDim.x);
  const int tm = (int)(L / (uint32_t)NTN), tn = (int)(L % (uint32_t)NTN);
  const int m0 = tm * TM, n0 = tn * TN;
  const int wm = wv >> 1, wn = wv & 1;
  const int q = lane >> 4, c16 = lane & 15;

  // staging: thread -> (row, half of the 128-byte K slice) for A and for W; rows past the
  // end read the last row (their results are never stored)
  const int sr = tid >> 1, sh = tid & 1;
  const uint8_t* a_src =
      reinterpret_cast<const uint8_t*>(A + (int64_t)min(m0 + sr, M - 1) * K) + sh * 64;
  const uint8_t* b_src =
      reinterpret_cast<const uint8_t*>(W + (int64_t)min(n0 + sr, N - 1) * K) + sh * 64;

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

  const int KS = K / 64;
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
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // lane (q, c16) supplies row c16, elements 8q .. 8q+7 of the 32-wide K slice kk
      bf16x8_t bop[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        bop[s] = as_bf16x8(
            *reinterpret_cast<const uint4*>(&sB[cur][t_off(wn * 64 + s * 16 + c16, 4 * kk + q)]));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8_t aop = as_bf16x8(
            *reinterpret_cast<const uint4*>(&sA[cur][t_off(wm * 64 + t * 16 + c16, 4 * kk + q)]));
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[s], acc[t][s], 0, 0, 0);
      }
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

#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm * 64 + t * 16 + 4 * q + r;
      if (row < M) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int cc = n0 + wn * 64 + s * 16 + c16;
          if (cc < N) out[(int64_t)row * N + cc] = acc[t][s][r];
        }
      }
    }
}

// Narrow outputs (N <= 128, the router): a workgroup owns 16 rows and all N columns, its
// four waves split K (interleaved 32-wide steps) and add their partial tiles in a fixed
// order through LDS. Operands come straight from global memory (the N x K weight stays in
// L2); the 128 x 128 tiling above would leave most of the chip idle for such shapes.
template <int NT>
__global__ __launch_bounds__(256) void bf16_gemm_narrow_kernel(const uint16_t* __restrict__ A,
                                                               const uint16_t* __restrict__ W,
                                                               int M, int N, int K,
                                                               float* __restrict__ out) {
  __shared__ v4f part[4][NT][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int m0 = blockIdx.x * 16;
  const uint16_t* a = A + (int64_t)min(m0 + c16, M - 1) * K + 8 * g;
  const uint16_t* w[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) w[t] = W + (int64_t)min(16 * t + c16, N - 1) * K + 8 * g;
  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = 32 * wv; k < K; k += 128) {
    const bf16x8_t av = as_bf16x8(*reinterpret_cast<const uint4*>(a + k));
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          av, as_bf16x8(*reinterpret_cast<const uint4*>(w[t] + k)), acc[t], 0, 0, 0);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) part[wv][t][lane] = acc[t];
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    v4f sum = part[0][t][lane];
#pragma unroll
    for (int q = 1; q < 4; ++q) sum += part[q][t][lane];
    const int col = 16 * t + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + 4 * g + r;
      if (row < M && col < N) out[(int64_t)row * N + col] = sum[r];
    }
  }
}

template <int NT>
hipError_t launch_narrow(const uint16_t* a, const uint16_t* w, int64_t M, int64_t N, int64_t K,
                         float* out, hipStream_t st) {
  bf16_gemm_narrow_kernel<NT><<<dim3((uint32_t)((M + 15) / 16)), 256, 0, st>>>(
      a, w, (int)M, (int)N, (int)K, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16_gemm(const uint16_t* a, const uint16_t* w, int64_t M, int64_t N,
                            int64_t K, float* out, hipStream_t st) {
  switch ((N + 15) / 16) {
    case 1: return launch_narrow<1>(a, w, M, N, K, out, st);
    case 2: return launch_narrow<2>(a, w, M, N, K, out, st);
    case 3: return launch_narrow<3>(a, w, M, N, K, out, st);
    case 4: return launch_narrow<4>(a, w, M, N, K, out, st);
    case 5: return launch_narrow<5>(a, w, M, N, K, out, st);
    case 6: return launch_narrow<6>(a, w, M, N, K, out, st);
    case 7: return launch_narrow<7>(a, w, M, N, K, out, st);
    case 8: return launch_narrow<8>(a, w, M, N, K, out, st);
    default: break;
  }
  const int NTM = (int)((M + TM - 1) / TM), NTN = (int)((N + TN - 1) / TN);
  bf16_gemm_kernel<<<dim3((uint32_t)(NTM * NTN)), 256, 0, st>>>(a, w, (int)M, (int)N, (int)K,
                                                                NTN, out);
  return hipGetLastError();
}

}  // namespace fp8moe
