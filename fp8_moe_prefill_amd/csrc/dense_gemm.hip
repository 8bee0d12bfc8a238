// Dense W8A8 projection y = (s_a * s_w) * (qa . qw^T) (fp8_dense_gemm).
//
// FreeToken PR #389, "What this adds": projection weights quantised at load time to e4m3
// with one fp32 scale per tensor, a dynamic per-tensor activation scale, an FP8 x FP8 GEMM.
// memra-engine fp8_ffi module docs: both scales folded into one device scalar, no host sync.
//
// gfx950 design: with per-tensor scales the fp32 accumulator chains through the whole K
// loop inside the MFMA (no per-group fold), and the scalar s_a * s_w is read from device
// memory and applied once in the epilogue. For M > 16 the GEMM is the shared TN kernel
// (tn_gemm.h: 128 x 128 tiles, or 128 x 192 / 256 x 256 where the shape fills the CUs with
// them; operands DMA'd into LDS); decode shapes (M <= 16) take the
// weight-streaming kernel below (memra-engine fp8_ffi module text draws the same line
// between prefill, m >= 16, and decode).
//
// Row-wise variant (fp8_dense_gemm_rowwise): FreeToken PR #389, "Limits" -- one activation
// scale per row, y = (s_a[m] * s_w) * (qa . qw^T); the same kernels with the scale product
// formed per output row in the epilogue.
//
// Block-128 variant (fp8_block_gemm): memra-engine fp8_ffi docs, the block-128 e4m3 weight
// class read in place -- one weight scale per 128 x 128 block, activations scaled per
// (row, 128-wide K group). Every K step is one scale group: its MFMA starts from zero and
// is folded into the accumulator with (row scale x block scale).
#include "common.h"
#include "launch.h"
#include "tn_gemm.h"

namespace fp8moe {
namespace {

constexpr int kDenseStages = 2;

// Small M (decode: M <= 16). The projection is then a pass over the weight matrix, bound
// by HBM, and 128 x 128 tiles would leave most of the chip idle (N/128 workgroups). A
// workgroup owns 16 weight rows (output columns) and all M <= 16 activation rows; its
// kGemvWaves waves split K in interleaved 128-byte steps, each with all its loads issued
// before its MFMAs, and the partial 16 x 16 tiles are added in a fixed order through LDS.
// One v_mfma_f32_16x16x128_f8f6f4 per step: A = the activation rows (rows >= M read as
// zero), B = 16 weight rows.
constexpr int kGemvWaves = 8;
constexpr int kGemvUnroll = 4;

// a_blk: the per-tensor scale block (s_a = a_blk[2]), or with ROW_SCALE the per-row scales;
// with BLOCK, a_blk is fp32 [M, K/128] and w_scale fp32 [ceil(N/128), K/128]
template <bool OUT_BF16, bool ROW_SCALE, bool BLOCK = false>
__global__ __launch_bounds__(kGemvWaves * 64) void dense_gemv_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ a_blk,
    const uint8_t* __restrict__ W, const float* __restrict__ w_scale, int M, int N, int K,
    void* __restrict__ out) {
  __shared__ v4f part[kGemvWaves][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int n0 = blockIdx.x * 16;
  const bool arow = c16 < M;
  const uint8_t* a = A + (int64_t)(arow ? c16 : 0) * K + 32 * g;
  const uint8_t* w = W + (int64_t)min(n0 + c16, N - 1) * K + 32 * g;
  const int KS = K / 128;
  const int mrow = min(4 * g, M - 1);  // BLOCK: scale rows of this lane (clamped; A is 0 there)
  const float* sa_rows = a_blk + (int64_t)mrow * KS;
  const float* swb_row = w_scale + (int64_t)(n0 / 128) * KS;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  for (int ks0 = wv; ks0 < KS; ks0 += kGemvWaves * kGemvUnroll) {
    uint4 al[kGemvUnroll], ah[kGemvUnroll], bl[kGemvUnroll], bh[kGemvUnroll];
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
      const int ks = ks0 + u * kGemvWaves;
      const bool ok = ks < KS;
      const int64_t o = (int64_t)(ok ? ks : 0) * 128;
      bl[u] = *reinterpret_cast<const uint4*>(w + o);
      bh[u] = *reinterpret_cast<const uint4*>(w + o + 16);
      al[u] = *reinterpret_cast<const uint4*>(a + o);
      ah[u] = *reinterpret_cast<const uint4*>(a + o + 16);
      if (!ok || !arow) al[u] = ah[u] = make_uint4(0, 0, 0, 0);  // adds nothing
    }
    float sc[kGemvUnroll][4];
    if (BLOCK) {
#pragma unroll
      for (int u = 0; u < kGemvUnroll; ++u) {
        const int ks = min(ks0 + u * kGemvWaves, KS - 1);
        const float swb = swb_row[ks];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sc[u][r] = sa_rows[(int64_t)min(r, M - 1 - mrow) * KS + ks] * swb;
      }
    }
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
      const v8i aop = {(int)al[u].x, (int)al[u].y, (int)al[u].z, (int)al[u].w,
                       (int)ah[u].x, (int)ah[u].y, (int)ah[u].z, (int)ah[u].w};
      const v8i bop = {(int)bl[u].x, (int)bl[u].y, (int)bl[u].z, (int)bl[u].w,
                       (int)bh[u].x, (int)bh[u].y, (int)bh[u].z, (int)bh[u].w};
      if (BLOCK) {
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, zero, 0, 0, 0, 0,
                                                                       0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf(p[r], sc[u][r], acc[r]);
      } else {
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, acc, 0, 0, 0, 0, 0, 0);
      }
    }
  }
  part[wv][lane] = acc;
  __syncthreads();
  if (wv != 0) return;
  v4f sum = part[0][lane];
#pragma unroll
  for (int j = 1; j < kGemvWaves; ++j) sum += part[j][lane];
  const float sw0 = BLOCK ? 1.f : w_scale[0];
  const int n = n0 + c16;
  // lane (g, c16) holds out[m = 4g + r][n0 + c16]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * g + r;
    if (m < M && n < N) {
      const float v = BLOCK ? sum[r] : sum[r] * ((ROW_SCALE ? a_blk[m] : a_blk[2]) * sw0);
      if (OUT_BF16)
        reinterpret_cast<uint16_t*>(out)[(int64_t)m * N + n] = (uint16_t)f32_to_bf16(v);
      else
        reinterpret_cast<float*>(out)[(int64_t)m * N + n] = v;
    }
  }
}

template <bool ROW_SCALE, bool BLOCK = false>
hipError_t launch_dense(const uint8_t* a, const float* a_s, const uint8_t* w,
                        const float* w_scale, int64_t M, int64_t N, int64_t K,
                        int32_t out_dtype, void* out, hipStream_t st) {
  if (M <= 16) {  // by shape only, never by values
    const dim3 grid((uint32_t)((N + 15) / 16)), block(kGemvWaves * 64);
    if (out_dtype == FP8MOE_DTYPE_BF16)
      dense_gemv_kernel<true, ROW_SCALE, BLOCK><<<grid, block, 0, st>>>(a, a_s, w, w_scale,
                                                                        (int)M, (int)N, (int)K,
                                                                        out);
    else
      dense_gemv_kernel<false, ROW_SCALE, BLOCK><<<grid, block, 0, st>>>(a, a_s, w, w_scale,
                                                                         (int)M, (int)N, (int)K,
                                                                         out);
    return hipGetLastError();
  }
  if constexpr (!ROW_SCALE && !BLOCK) {
    if (tn::use_big_tiles(M, N)) {
      if (out_dtype == FP8MOE_DTYPE_BF16)
        return tn::launch<false, true, 2, false, false, true>(a, w, M, N, K, a_s, w_scale, out,
                                                              st);
      return tn::launch<false, false, 2, false, false, true>(a, w, M, N, K, a_s, w_scale, out,
                                                             st);
    }
  }
  if constexpr (!BLOCK) {
    if (tn::use_wide_tiles(M, N)) {
      if (out_dtype == FP8MOE_DTYPE_BF16)
        return tn::launch_wide<true, ROW_SCALE>(a, w, M, N, K, a_s, w_scale, out, st);
      return tn::launch_wide<false, ROW_SCALE>(a, w, M, N, K, a_s, w_scale, out, st);
    }
  }
  if (out_dtype == FP8MOE_DTYPE_BF16)
    return tn::launch<false, true, kDenseStages, ROW_SCALE, BLOCK>(a, w, M, N, K, a_s, w_scale,
                                                                   out, st);
  return tn::launch<false, false, kDenseStages, ROW_SCALE, BLOCK>(a, w, M, N, K, a_s, w_scale,
                                                                  out, st);
}

}  // namespace

hipError_t launch_dense_gemm(const uint8_t* a, const float* a_blk, const uint8_t* w,
                             const float* w_scale, int64_t M, int64_t N, int64_t K,
                             int32_t out_dtype, void* out, hipStream_t st) {
  return launch_dense<false>(a, a_blk, w, w_scale, M, N, K, out_dtype, out, st);
}

hipError_t launch_dense_gemm_rowwise(const uint8_t* a, const float* a_scales, const uint8_t* w,
                                     const float* w_scale, int64_t M, int64_t N, int64_t K,
                                     int32_t out_dtype, void* out, hipStream_t st) {
  return launch_dense<true>(a, a_scales, w, w_scale, M, N, K, out_dtype, out, st);
}

hipError_t launch_block_gemm(const uint8_t* a, const float* a_scales, const uint8_t* w,
                             const float* w_scales, int64_t M, int64_t N, int64_t K,
                             int32_t out_dtype, void* out, hipStream_t st) {
  return launch_dense<false, true>(a, a_scales, w, w_scales, M, N, K, out_dtype, out, st);
}

}  // namespace fp8moe
