// Internal launchers: one per kernel family. Arguments are already validated by the C ABI
// layer (capi.cpp); each launcher only enqueues work and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fp8moe.h"

namespace fp8moe {

// Elements below which the per-tensor quantiser runs as one fused single-workgroup launch
// (amax pass, then the cast) instead of a grid amax pass followed by a grid cast pass.
constexpr int64_t kQuantFusedMax = 65536;
constexpr int kQuantPartials = 1024;  // max workgroups of the per-tensor amax pass

hipError_t launch_quant_mxfp4(const uint16_t* x, int64_t M, int64_t K, uint8_t* q,
                              uint8_t* scales, hipStream_t st);
hipError_t launch_quant_row(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* scales,
                            hipStream_t st);
hipError_t launch_quant_group(const uint16_t* x, int64_t M, int64_t K, uint8_t* q,
                              float* scales, float* sums, hipStream_t st);
hipError_t launch_quant_tensor(const uint16_t* x, int64_t n, uint8_t* q, float* block,
                               float* partials, hipStream_t st);

// Route/permute: tokens per chunk of the stable counting sort.
constexpr int kRouteChunk = 16;
size_t route_workspace_bytes(int64_t T, int32_t E);
hipError_t launch_route_permute(const float* logits, int64_t T, int32_t E, int32_t k,
                                int32_t* ids, float* w, int32_t* offsets, int32_t* sorted,
                                int32_t* pos, const uint8_t* xq, const float* xs, int64_t H,
                                uint8_t* xq_perm, float* xs_perm, const float* xsum,
                                float* xsum_perm, void* ws, hipStream_t st);
// The routing workspace of the allocation-free call lives in a static device array of
// kRouteScratchBytes per GPU. route_scratch() returns its device address on the current
// device (resolved once per device, then cached); it never allocates.
constexpr size_t kRouteScratchBytes = FP8MOE_ROUTE_SCRATCH_BYTES;
hipError_t route_scratch(void** ptr);
// Group quantisation (with optional code sums) of x [T, H] and routing without gathers,
// the quantiser and the top-k in one launch.
hipError_t launch_quant_route(const uint16_t* x, int64_t H, uint8_t* q, float* scales,
                              float* sums, const float* logits, int64_t T, int32_t E,
                              int32_t k, int32_t* ids, float* w, int32_t* offsets,
                              int32_t* sorted, int32_t* pos, void* ws, hipStream_t st);

hipError_t launch_pack_bank(const uint8_t* w, const float* w_scales, int64_t E, int64_t N,
                            int64_t K, uint8_t* w_packed, float* ws_packed, hipStream_t st, bool fp4_layout = false);

hipError_t launch_grouped_gemm(const uint8_t* a, const float* a_scales, const float* a_sums,
                               const int32_t* sorted, int32_t k_route, const uint8_t* w,
                               const float* w_scales, const int32_t* offsets, int64_t R,
                               int32_t E, int64_t N, int64_t K, int32_t epilogue,
                               int32_t out_dtype, void* out, float* out_scales,
                               float* out_sums, hipStream_t st, bool a_fp4 = false);

hipError_t launch_dense_gemm_rowwise(const uint8_t* a, const float* a_scales, const uint8_t* w,
                                     const float* w_scale, int64_t M, int64_t N, int64_t K,
                                     int32_t out_dtype, void* out, hipStream_t st);
hipError_t launch_block_gemm(const uint8_t* a, const float* a_scales, const uint8_t* w,
                             const float* w_scales, int64_t M, int64_t N, int64_t K,
                             int32_t out_dtype, void* out, hipStream_t st);
hipError_t launch_quant_block128(const uint16_t* w, int64_t N, int64_t K, uint8_t* q,
                                 float* scales, hipStream_t st);
hipError_t launch_dense_gemm(const uint8_t* a, const float* a_blk, const uint8_t* w,
                             const float* w_scale, int64_t M, int64_t N, int64_t K,
                             int32_t out_dtype, void* out, hipStream_t st);

hipError_t launch_combine(const void* y, int32_t y_dtype, const int32_t* pos, const float* w,
                          int64_t T, int32_t k, int64_t H, int32_t out_dtype, void* out,
                          hipStream_t st);

// Depth-stack support kernels.
hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* delta, int64_t T, int64_t H,
                          double eps, uint16_t* x_out, uint16_t* y, hipStream_t st);
hipError_t launch_bf16_gemm(const uint16_t* a, const uint16_t* w, int64_t M, int64_t N,
                            int64_t K, float* out, hipStream_t st);
size_t attention_workspace_bytes(int64_t T, int32_t n_kv);
hipError_t launch_attention(const uint16_t* qkv, int64_t T, int32_t n_q, int32_t n_kv,
                            uint16_t* out, uint16_t* vt, hipStream_t st);

}  // namespace fp8moe
