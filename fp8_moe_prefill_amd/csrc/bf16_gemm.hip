// bf16 x bf16 -> fp32 GEMM out = a . w^T (fp8moe_bf16_gemm): the depth stack's router and
// LM head.
//
// The FP8 grouped-expert prefill note ("FP8 grouped-expert prefill with on-chip int4-to-e4m3
// dequant", section 1) gates on the cosine of the final logits; FreeToken PR #389 ("Limits")
// keeps the LM head in bf16. The router that feeds the top-k selection and the LM head are
// therefore plain bf16 GEMMs with fp32 accumulation and fp32 output.
//
// gfx950 design: both operands K-contiguous ("TN"). For N > 128 the shared TN kernel
// (tn_gemm.h: 128 x 128 tiles, operands DMA'd into LDS in MFMA-native blocks, two
// v_mfma_f32_16x16x32_bf16 per 16 x 16 tile and 64-element K step); narrow outputs take
// the path below.
#include "common.h"
#include "launch.h"
#include "tn_gemm.h"

namespace fp8moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Narrow outputs (N <= 128, the router): a workgroup owns 16 rows and NT (one or two)
// 16-column tiles, its NWN waves split K (interleaved 32-wide steps, so each wave has only
// a few loads to wait for) and add their partial tiles in a fixed order through LDS.
// Operands come straight from global memory (the N x K weight stays in L2); 128 x 128
// tiles would leave most of the chip idle for such shapes. Splitting the columns over
// workgroups doubles the CUs in use at the router's 2048 x 2048 x 64 and halves the bytes
// each CU pulls (12.1 -> 9.6 us); the K split, and so every sum, is unchanged.
constexpr int NWN = 16;
template <int NT>
__global__ __launch_bounds__(NWN * 64) void bf16_gemm_narrow_kernel(const uint16_t* __restrict__ A,
                                                               const uint16_t* __restrict__ W,
                                                               int M, int N, int K,
                                                               float* __restrict__ out) {
  __shared__ v4f part[NWN][NT][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int m0 = blockIdx.x * 16, n0 = blockIdx.y * 16 * NT;
  const uint16_t* a = A + (int64_t)min(m0 + c16, M - 1) * K + 8 * g;
  const uint16_t* w[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) w[t] = W + (int64_t)min(n0 + 16 * t + c16, N - 1) * K + 8 * g;
  v4f acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k = 32 * wv; k < K; k += 32 * NWN) {
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
    for (int q = 1; q < NWN; ++q) sum += part[q][t][lane];
    const int col = n0 + 16 * t + c16;
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
  const uint32_t ny = (uint32_t)((N + 16 * NT - 1) / (16 * NT));
  bf16_gemm_narrow_kernel<NT><<<dim3((uint32_t)((M + 15) / 16), ny), NWN * 64, 0, st>>>(
      a, w, (int)M, (int)N, (int)K, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16_gemm(const uint16_t* a, const uint16_t* w, int64_t M, int64_t N,
                            int64_t K, float* out, hipStream_t st) {
  switch ((N + 15) / 16) {
    case 1: return launch_narrow<1>(a, w, M, N, K, out, st);
    case 2: return launch_narrow<2>(a, w, M, N, K, out, st);
    case 3: return launch_narrow<1>(a, w, M, N, K, out, st);
    case 4: return launch_narrow<2>(a, w, M, N, K, out, st);
    case 5: return launch_narrow<1>(a, w, M, N, K, out, st);
    case 6: return launch_narrow<2>(a, w, M, N, K, out, st);
    case 7: return launch_narrow<1>(a, w, M, N, K, out, st);
    case 8: return launch_narrow<2>(a, w, M, N, K, out, st);
    default: break;
  }
  if (tn::use_big_tiles(M, N))
    return tn::launch<true, false, 2, false, false, true>(reinterpret_cast<const uint8_t*>(a),
                                                          reinterpret_cast<const uint8_t*>(w), M,
                                                          N, 2 * K, nullptr, nullptr, out, st);
  return tn::launch<true, false, 2>(reinterpret_cast<const uint8_t*>(a),
                                    reinterpret_cast<const uint8_t*>(w), M, N, 2 * K, nullptr,
                                    nullptr, out, st);
}

}  // namespace fp8moe
