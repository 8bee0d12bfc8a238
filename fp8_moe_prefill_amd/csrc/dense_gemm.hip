// Dense W8A8 projection y = (s_a * s_w) * (qa . qw^T) (fp8_dense_gemm).
//
// FreeToken PR #389, "What this adds": projection weights quantised at load time to e4m3
// with one fp32 scale per tensor, a dynamic per-tensor activation scale, an FP8 x FP8 GEMM.
// memra-engine fp8_ffi module docs: both scales folded into one device scalar, no host sync.
//
// gfx950 design: with per-tensor scales the fp32 accumulator chains through the whole K
// loop inside the MFMA (no per-group fold), and the scalar s_a * s_w is read from device
// memory and applied once in the epilogue. The GEMM itself is the shared TN kernel
// (tn_gemm.h): 128 x 128 tiles, operands DMA'd into LDS in MFMA-native blocks.
#include "common.h"
#include "launch.h"
#include "tn_gemm.h"

namespace fp8moe {

constexpr int kDenseStages = 2;

hipError_t launch_dense_gemm(const uint8_t* a, const float* a_blk, const uint8_t* w,
                             const float* w_scale, int64_t M, int64_t N, int64_t K,
                             int32_t out_dtype, void* out, hipStream_t st) {
  if (out_dtype == FP8MOE_DTYPE_BF16)
    return tn::launch<false, true, kDenseStages>(a, w, M, N, K, a_blk, w_scale, out, st);
  return tn::launch<false, false, kDenseStages>(a, w, M, N, K, a_blk, w_scale, out, st);
}

}  // namespace fp8moe
