// C ABI of the FP8 MoE prefill library: host-side argument validation, then the launch.
//
// Every check runs before anything is enqueued, so a failing call has no side effects and
// its status is known synchronously; none of them reads device memory (no host sync).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "fp8moe.h"
#include "launch.h"

namespace {

constexpr int32_t kAbiVersion = 9;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int64_t kMaxGroupedK = 16384;
constexpr int32_t kHeadDim = 128;
constexpr int32_t kMaxHeads = 4096;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t launch_status(hipError_t e) { return e == hipSuccess ? FP8MOE_OK : FP8MOE_ERR_LAUNCH; }

size_t quant_ws(int64_t M, int64_t K, int32_t group) {
  if (group == 0 && M * K > fp8moe::kQuantFusedMax)
    return (size_t)fp8moe::kQuantPartials * sizeof(float);
  return 0;
}

// Argument checks shared by both routing entry points (everything but the workspace).
int32_t check_route(const float* logits, int64_t T, int32_t E, int32_t k, const int32_t* ids,
                    const float* weights, const int32_t* offsets, const int32_t* sorted,
                    const int32_t* pos, const uint8_t* xq, const float* xs, int64_t H,
                    const uint8_t* xq_perm, const float* xs_perm, const float* xsum,
                    const float* xsum_perm) {
  if (!logits || !ids || !weights || !offsets || !sorted || !pos) return FP8MOE_ERR_NULL;
  // the row gather (xq -> xq_perm) and the scale gather (xs -> xs_perm) are independent
  // options, each all-or-nothing; the code-sum gather (xsum -> xsum_perm) rides the scale
  // gather
  if ((xq != nullptr) != (xq_perm != nullptr)) return FP8MOE_ERR_NULL;
  if ((xs != nullptr) != (xs_perm != nullptr)) return FP8MOE_ERR_NULL;
  if ((xsum != nullptr) != (xsum_perm != nullptr)) return FP8MOE_ERR_NULL;
  if (xsum && !xs) return FP8MOE_ERR_NULL;
  if (xsum && (!aligned16(xsum) || !aligned16(xsum_perm))) return FP8MOE_ERR_ALIGN;
  const bool rows = xq != nullptr, scales = xs != nullptr;
  if (T < 1 || E < 1 || E > kMaxE || k < 1 || k > E || k > kMaxK) return FP8MOE_ERR_SHAPE;
  if (T * (int64_t)k >= (int64_t(1) << 31)) return FP8MOE_ERR_SHAPE;
  if ((rows || scales) && (H < FP8MOE_GROUP || H % FP8MOE_GROUP != 0)) return FP8MOE_ERR_SHAPE;
  const void* ptrs[] = {logits, ids, weights, offsets, sorted, pos};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FP8MOE_ERR_ALIGN;
  if (rows && (!aligned16(xq) || !aligned16(xq_perm))) return FP8MOE_ERR_ALIGN;
  if (scales && (!aligned16(xs) || !aligned16(xs_perm))) return FP8MOE_ERR_ALIGN;
  return FP8MOE_OK;
}

}  // namespace

extern "C" {

int32_t fp8moe_abi_version(void) { return kAbiVersion; }

const char* fp8moe_status_str(int32_t status) {
  switch (status) {
    case FP8MOE_OK: return "ok";
    case FP8MOE_ERR_NULL: return "a required pointer is NULL";
    case FP8MOE_ERR_SHAPE: return "a size is out of range or not a required multiple";
    case FP8MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FP8MOE_ERR_WORKSPACE: return "workspace is smaller than fp8moe_workspace_bytes()";
    case FP8MOE_ERR_UNSUPPORTED: return "an enum argument has an unknown value";
    case FP8MOE_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    default: return "unknown status";
  }
}

size_t fp8moe_workspace_bytes(int32_t op, int64_t a, int64_t b, int64_t c) {
  if (op == FP8MOE_OP_QUANT_ACT) {
    if (a < 1 || b < 1 || (c != 0 && c != FP8MOE_GROUP && c != FP8MOE_QUANT_ROW))
      return (size_t)-1;
    return quant_ws(a, b, (int32_t)c);
  }
  if (op == FP8MOE_OP_ROUTE_PERMUTE) {
    if (a < 1 || b < 1 || b > kMaxE || c < 1 || c > b || c > kMaxK) return (size_t)-1;
    return fp8moe::route_workspace_bytes(a, (int32_t)b);
  }
  if (op == FP8MOE_OP_ATTENTION) {
    if (a < 1 || a >= (int64_t(1) << 31) || b < 1 || b > kMaxHeads || c != kHeadDim)
      return (size_t)-1;
    return fp8moe::attention_workspace_bytes(a, (int32_t)b);
  }
  return (size_t)-1;
}

int32_t fp8_quant_act(const void* x, int64_t M, int64_t K, int32_t group, uint8_t* q,
                      float* scales, float* sums, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !q || !scales) return FP8MOE_ERR_NULL;
  if (group != 0 && group != FP8MOE_GROUP && group != FP8MOE_QUANT_ROW)
    return FP8MOE_ERR_UNSUPPORTED;
  if (sums && group != FP8MOE_GROUP) return FP8MOE_ERR_UNSUPPORTED;  // group sums only
  if (sums && !aligned16(sums)) return FP8MOE_ERR_ALIGN;
  if (M < 1 || K < 1 || M > (int64_t(1) << 40) / K) return FP8MOE_ERR_SHAPE;
  if (group == FP8MOE_GROUP && K % FP8MOE_GROUP != 0) return FP8MOE_ERR_SHAPE;
  if (group == FP8MOE_QUANT_ROW && (K % 8 != 0 || M >= (int64_t(1) << 31)))
    return FP8MOE_ERR_SHAPE;
  if (group == 0 && (M * K) % 8 != 0) return FP8MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scales)) return FP8MOE_ERR_ALIGN;
  size_t need = quant_ws(M, K, group);
  if (need > 0 && (!ws || ws_bytes < need)) return FP8MOE_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return FP8MOE_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (group == FP8MOE_GROUP)
    return launch_status(fp8moe::launch_quant_group(xb, M, K, q, scales, sums, st));
  if (group == FP8MOE_QUANT_ROW)
    return launch_status(fp8moe::launch_quant_row(xb, M, K, q, scales, st));
  return launch_status(
      fp8moe::launch_quant_tensor(xb, M * K, q, scales, static_cast<float*>(ws), st));
}

int32_t moe_route_permute(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids,
                          float* weights, int32_t* offsets, int32_t* sorted, int32_t* pos,
                          const uint8_t* xq, const float* xs, int64_t H, uint8_t* xq_perm,
                          float* xs_perm, const float* xsum, float* xsum_perm, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!ws) return FP8MOE_ERR_NULL;
  const int32_t st = check_route(logits, T, E, k, ids, weights, offsets, sorted, pos, xq, xs,
                                 H, xq_perm, xs_perm, xsum, xsum_perm);
  if (st != FP8MOE_OK) return st;
  if (!aligned16(ws)) return FP8MOE_ERR_ALIGN;
  if (ws_bytes < fp8moe::route_workspace_bytes(T, E)) return FP8MOE_ERR_WORKSPACE;
  return launch_status(fp8moe::launch_route_permute(
      logits, T, E, k, ids, weights, offsets, sorted, pos, xq, xs, H, xq_perm, xs_perm, xsum,
      xsum_perm, ws, static_cast<hipStream_t>(stream)));
}

int32_t fp8moe_quant_route(const void* x, int64_t T, int64_t H, uint8_t* q, float* scales,
                           float* sums, const float* logits, int32_t E, int32_t k,
                           int32_t* ids, float* weights, int32_t* offsets, int32_t* sorted,
                           int32_t* pos, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !q || !scales || !ws) return FP8MOE_ERR_NULL;
  if (T < 1 || H < FP8MOE_GROUP || H % FP8MOE_GROUP != 0 || T > (int64_t(1) << 40) / H)
    return FP8MOE_ERR_SHAPE;
  const int32_t st = check_route(logits, T, E, k, ids, weights, offsets, sorted, pos, nullptr,
                                 nullptr, H, nullptr, nullptr, nullptr, nullptr);
  if (st != FP8MOE_OK) return st;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scales) || !aligned16(ws) ||
      (sums && !aligned16(sums)))
    return FP8MOE_ERR_ALIGN;
  if (ws_bytes < fp8moe::route_workspace_bytes(T, E)) return FP8MOE_ERR_WORKSPACE;
  return launch_status(fp8moe::launch_quant_route(
      static_cast<const uint16_t*>(x), H, q, scales, sums, logits, T, E, k, ids, weights,
      offsets, sorted, pos, ws, static_cast<hipStream_t>(stream)));
}

int32_t moe_route_permute_noalloc(const float* logits, int64_t T, int32_t E, int32_t k,
                                  int32_t* ids, float* weights, int32_t* offsets,
                                  int32_t* sorted, int32_t* pos, const uint8_t* xq,
                                  const float* xs, int64_t H, uint8_t* xq_perm, float* xs_perm,
                                  const float* xsum, float* xsum_perm, void* stream) {
  const int32_t st = check_route(logits, T, E, k, ids, weights, offsets, sorted, pos, xq, xs,
                                 H, xq_perm, xs_perm, xsum, xsum_perm);
  if (st != FP8MOE_OK) return st;
  if (fp8moe::route_workspace_bytes(T, E) > fp8moe::kRouteScratchBytes)
    return FP8MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (fp8moe::route_scratch(&ws) != hipSuccess) return FP8MOE_ERR_LAUNCH;
  return launch_status(fp8moe::launch_route_permute(
      logits, T, E, k, ids, weights, offsets, sorted, pos, xq, xs, H, xq_perm, xs_perm, xsum,
      xsum_perm, ws, static_cast<hipStream_t>(stream)));
}

namespace {
int32_t pack_bank(const uint8_t* w, const float* w_scales, int64_t E, int64_t N, int64_t K,
                  uint8_t* w_packed, float* w_scales_packed, void* stream, bool fp4_layout) {
  if (!w || !w_scales || !w_packed || !w_scales_packed) return FP8MOE_ERR_NULL;
  if (E < 1 || E > kMaxE) return FP8MOE_ERR_SHAPE;
  if (N < 64 || N % 64 != 0 || N >= (int64_t(1) << 24)) return FP8MOE_ERR_SHAPE;
  if (K < FP8MOE_GROUP || K % FP8MOE_GROUP != 0 || K > kMaxGroupedK) return FP8MOE_ERR_SHAPE;
  if (N * (K / 2) >= (int64_t(1) << 32)) return FP8MOE_ERR_SHAPE;
  const void* ptrs[] = {w, w_scales, w_packed, w_scales_packed};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FP8MOE_ERR_ALIGN;
  return launch_status(fp8moe::launch_pack_bank(w, w_scales, E, N, K, w_packed, w_scales_packed,
                                                static_cast<hipStream_t>(stream), fp4_layout));
}
}  // namespace

int32_t fp8moe_pack_expert_bank(const uint8_t* w, const float* w_scales, int64_t E, int64_t N,
                                int64_t K, uint8_t* w_packed, float* w_scales_packed,
                                void* stream) {
  return pack_bank(w, w_scales, E, N, K, w_packed, w_scales_packed, stream, false);
}

int32_t fp8moe_pack_expert_bank_mxfp4(const uint8_t* w, const float* w_scales, int64_t E,
                                      int64_t N, int64_t K, uint8_t* w_packed,
                                      float* w_scales_packed, void* stream) {
  return pack_bank(w, w_scales, E, N, K, w_packed, w_scales_packed, stream, true);
}

namespace {
int32_t grouped_gemm(const uint8_t* a, const float* a_scales, const float* a_sums,
                     const int32_t* sorted, int32_t k_route, const uint8_t* w,
                     const float* w_scales, const int32_t* offsets, int64_t R, int32_t E,
                     int64_t N, int64_t K, int32_t epilogue, int32_t out_dtype, void* out,
                     float* out_scales, float* out_sums, void* stream, bool a_fp4) {
  if (epilogue != FP8MOE_EPI_STORE && epilogue != FP8MOE_EPI_SWIGLU_QUANT)
    return FP8MOE_ERR_UNSUPPORTED;
  if (epilogue == FP8MOE_EPI_STORE && out_dtype != FP8MOE_DTYPE_F32 &&
      out_dtype != FP8MOE_DTYPE_BF16)
    return FP8MOE_ERR_UNSUPPORTED;
  if (!w || !w_scales || !offsets) return FP8MOE_ERR_NULL;
  // the row-sized buffers may be NULL when there are no rows (empty arrays)
  if (R != 0 && (!a || !a_scales || !out)) return FP8MOE_ERR_NULL;
  if (R != 0 && epilogue == FP8MOE_EPI_SWIGLU_QUANT && !out_scales) return FP8MOE_ERR_NULL;
  if (R < 0 || R >= (int64_t(1) << 31) || E < 1 || E > kMaxE) return FP8MOE_ERR_SHAPE;
  if (K < FP8MOE_GROUP || K % FP8MOE_GROUP != 0 || K > kMaxGroupedK) return FP8MOE_ERR_SHAPE;
  if (N < 16 || N >= (int64_t(1) << 24)) return FP8MOE_ERR_SHAPE;
  if (epilogue == FP8MOE_EPI_STORE && N % 64 != 0) return FP8MOE_ERR_SHAPE;
  if (epilogue == FP8MOE_EPI_SWIGLU_QUANT && N % 256 != 0) return FP8MOE_ERR_SHAPE;
  if (sorted && (k_route < 1 || R % k_route != 0)) return FP8MOE_ERR_SHAPE;  // R = T * k
  if (R * K >= (int64_t(1) << 32)) return FP8MOE_ERR_SHAPE;  // 32-bit A row offsets
  if (N * (K / 2) >= (int64_t(1) << 32)) return FP8MOE_ERR_SHAPE;  // 32-bit offsets in one expert
  // 32-bit tile indexing: (128-row tiles, one more per expert) x (256-column tiles)
  if (((R + 127) / 128 + E) * ((N + 255) / 256) >= (int64_t(1) << 28)) return FP8MOE_ERR_SHAPE;
  const void* ptrs[] = {a, a_scales, w, w_scales, offsets, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FP8MOE_ERR_ALIGN;
  if ((sorted && !aligned16(sorted)) || (out_scales && !aligned16(out_scales)))
    return FP8MOE_ERR_ALIGN;
  if ((a_sums && !aligned16(a_sums)) || (out_sums && !aligned16(out_sums)))
    return FP8MOE_ERR_ALIGN;
  if (out_sums && epilogue != FP8MOE_EPI_SWIGLU_QUANT) return FP8MOE_ERR_UNSUPPORTED;
  if (R == 0) return FP8MOE_OK;
  return launch_status(fp8moe::launch_grouped_gemm(a, a_scales, a_sums, sorted, k_route, w,
                                                   w_scales, offsets, R, E, N, K, epilogue,
                                                   out_dtype, out, out_scales, out_sums,
                                                   static_cast<hipStream_t>(stream), a_fp4));
}
}  // namespace

int32_t fp8_grouped_expert_gemm(const uint8_t* a, const float* a_scales, const float* a_sums,
                                const int32_t* sorted, int32_t k_route, const uint8_t* w,
                                const float* w_scales, const int32_t* offsets, int64_t R,
                                int32_t E, int64_t N, int64_t K, int32_t epilogue,
                                int32_t out_dtype, void* out, float* out_scales,
                                float* out_sums, void* stream) {
  return grouped_gemm(a, a_scales, a_sums, sorted, k_route, w, w_scales, offsets, R, E, N, K,
                      epilogue, out_dtype, out, out_scales, out_sums, stream, false);
}

int32_t mxfp4_grouped_expert_gemm(const uint8_t* a, const uint32_t* a_scales,
                                  const int32_t* sorted, int32_t k_route, const uint8_t* w,
                                  const float* w_scales, const int32_t* offsets, int64_t R,
                                  int32_t E, int64_t N, int64_t K, int32_t epilogue,
                                  int32_t out_dtype, void* out, float* out_scales,
                                  float* out_sums, void* stream) {
  return grouped_gemm(a, reinterpret_cast<const float*>(a_scales), nullptr, sorted, k_route, w,
                      w_scales, offsets, R, E, N, K, epilogue, out_dtype, out, out_scales,
                      out_sums, stream, true);
}

int32_t mxfp4_quant_act(const void* x, int64_t M, int64_t K, uint8_t* q, uint8_t* scales,
                        void* stream) {
  if (!x || !q || !scales) return FP8MOE_ERR_NULL;
  if (M < 1 || K < 32 || K % 32 != 0 || M > (int64_t(1) << 40) / K) return FP8MOE_ERR_SHAPE;
  if (M * K / 8 >= (int64_t(1) << 31) * 256) return FP8MOE_ERR_SHAPE;  // grid size
  if (!aligned16(x) || !aligned16(q) || !aligned16(scales)) return FP8MOE_ERR_ALIGN;
  return launch_status(fp8moe::launch_quant_mxfp4(static_cast<const uint16_t*>(x), M, K, q,
                                                  scales, static_cast<hipStream_t>(stream)));
}

int32_t fp8_dense_gemm(const uint8_t* a, const float* a_scale_blk, const uint8_t* w,
                       const float* w_scale, int64_t M, int64_t N, int64_t K, int32_t out_dtype,
                       void* out, void* stream) {
  if (out_dtype != FP8MOE_DTYPE_F32 && out_dtype != FP8MOE_DTYPE_BF16)
    return FP8MOE_ERR_UNSUPPORTED;
  if (!a || !a_scale_blk || !w || !w_scale || !out) return FP8MOE_ERR_NULL;
  if (M < 1 || M >= (int64_t(1) << 31) || N < 16 || N % 16 != 0 || N >= (int64_t(1) << 31))
    return FP8MOE_ERR_SHAPE;
  if (K < 128 || K % 128 != 0 || K >= (int64_t(1) << 31)) return FP8MOE_ERR_SHAPE;
  // per-lane 32-bit byte offsets into A and W
  if (M * K >= (int64_t(1) << 32) || N * K >= (int64_t(1) << 32)) return FP8MOE_ERR_SHAPE;
  const void* ptrs[] = {a, a_scale_blk, w, w_scale, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FP8MOE_ERR_ALIGN;
  return launch_status(fp8moe::launch_dense_gemm(a, a_scale_blk, w, w_scale, M, N, K, out_dtype,
                                                 out, static_cast<hipStream_t>(stream)));
}

int32_t fp8_dense_gemm_rowwise(const uint8_t* a, const float* a_scales, const uint8_t* w,
                               const float* w_scale, int64_t M, int64_t N, int64_t K,
                               int32_t out_dtype, void* out, void* stream) {
  if (out_dtype != FP8MOE_DTYPE_F32 && out_dtype != FP8MOE_DTYPE_BF16)
    return FP8MOE_ERR_UNSUPPORTED;
  if (!a || !a_scales || !w || !w_scale || !out) return FP8MOE_ERR_NULL;
  if (M < 1 || M >= (int64_t(1) << 31) || N < 16 || N % 16 != 0 || N >= (int64_t(1) << 31))
    return FP8MOE_ERR_SHAPE;
  if (K < 128 || K % 128 != 0 || K >= (int64_t(1) << 31)) return FP8MOE_ERR_SHAPE;
  if (M * K >= (int64_t(1) << 32) || N * K >= (int64_t(1) << 32)) return FP8MOE_ERR_SHAPE;
  const void* ptrs[] = {a, a_scales, w, w_scale, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FP8MOE_ERR_ALIGN;
  return launch_status(fp8moe::launch_dense_gemm_rowwise(a, a_scales, w, w_scale, M, N, K,
                                                         out_dtype, out,
                                                         static_cast<hipStream_t>(stream)));
}

int32_t fp8_block_gemm(const uint8_t* a, const float* a_scales, const uint8_t* w,
                       const float* w_scales, int64_t M, int64_t N, int64_t K, int32_t out_dtype,
                       void* out, void* stream) {
  if (out_dtype != FP8MOE_DTYPE_F32 && out_dtype != FP8MOE_DTYPE_BF16)
    return FP8MOE_ERR_UNSUPPORTED;
  if (!a || !a_scales || !w || !w_scales || !out) return FP8MOE_ERR_NULL;
  if (M < 1 || M >= (int64_t(1) << 31) || N < 16 || N % 16 != 0 || N >= (int64_t(1) << 31))
    return FP8MOE_ERR_SHAPE;
  if (K < 128 || K % 128 != 0 || K >= (int64_t(1) << 31)) return FP8MOE_ERR_SHAPE;
  if (M * K >= (int64_t(1) << 32) || N * K >= (int64_t(1) << 32)) return FP8MOE_ERR_SHAPE;
  if (K > 16384) return FP8MOE_ERR_SHAPE;  // a tile stages its block scales of all K steps
  const void* ptrs[] = {a, a_scales, w, w_scales, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FP8MOE_ERR_ALIGN;
  return launch_status(fp8moe::launch_block_gemm(a, a_scales, w, w_scales, M, N, K, out_dtype,
                                                 out, static_cast<hipStream_t>(stream)));
}

int32_t fp8_quant_weight_block128(const void* w, int64_t N, int64_t K, uint8_t* q,
                                  float* scales, void* stream) {
  if (!w || !q || !scales) return FP8MOE_ERR_NULL;
  if (N < 1 || N >= (int64_t(1) << 31) || K < 128 || K % 128 != 0 || K >= (int64_t(1) << 31))
    return FP8MOE_ERR_SHAPE;
  if ((N + 127) / 128 >= 65536 || K / 128 >= (int64_t(1) << 31)) return FP8MOE_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(q) || !aligned16(scales)) return FP8MOE_ERR_ALIGN;
  return launch_status(fp8moe::launch_quant_block128(static_cast<const uint16_t*>(w), N, K, q,
                                                     scales, static_cast<hipStream_t>(stream)));
}

int32_t moe_unpermute_combine(const void* y, int32_t y_dtype, const int32_t* pos,
                              const float* weights, int64_t T, int32_t k, int64_t H,
                              int32_t out_dtype, void* out, void* stream) {
  if ((y_dtype != FP8MOE_DTYPE_F32 && y_dtype != FP8MOE_DTYPE_BF16) ||
      (out_dtype != FP8MOE_DTYPE_F32 && out_dtype != FP8MOE_DTYPE_BF16))
    return FP8MOE_ERR_UNSUPPORTED;
  if (!y || !pos || !weights || !out) return FP8MOE_ERR_NULL;
  if (T < 1 || k < 1 || k > kMaxK || H < 8 || H % 8 != 0) return FP8MOE_ERR_SHAPE;
  if (T * (int64_t)k >= (int64_t(1) << 31)) return FP8MOE_ERR_SHAPE;
  const void* ptrs[] = {y, pos, weights, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FP8MOE_ERR_ALIGN;
  return launch_status(fp8moe::launch_combine(y, y_dtype, pos, weights, T, k, H, out_dtype, out,
                                              static_cast<hipStream_t>(stream)));
}

int32_t fp8moe_rmsnorm(const void* x, const void* delta, int64_t T, int64_t H, double eps,
                       void* x_out, void* y, void* stream) {
  if (!x || !y || (delta && !x_out)) return FP8MOE_ERR_NULL;
  if (T < 1 || H < 8 || H % 8 != 0 || T >= (int64_t(1) << 31) || H >= (int64_t(1) << 31) ||
      T > (int64_t(1) << 40) / H)
    return FP8MOE_ERR_SHAPE;
  if (!(eps >= 0.0)) return FP8MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(y) || (delta && (!aligned16(delta) || !aligned16(x_out))))
    return FP8MOE_ERR_ALIGN;
  return launch_status(fp8moe::launch_rmsnorm(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(delta), T, H, eps,
      static_cast<uint16_t*>(delta ? x_out : nullptr), static_cast<uint16_t*>(y),
      static_cast<hipStream_t>(stream)));
}

int32_t fp8moe_bf16_gemm(const void* a, const void* w, int64_t M, int64_t N, int64_t K,
                         float* out, void* stream) {
  if (!a || !w || !out) return FP8MOE_ERR_NULL;
  if (M < 1 || N < 1 || K < 64 || K % 64 != 0) return FP8MOE_ERR_SHAPE;
  if (M >= (int64_t(1) << 31) || N >= (int64_t(1) << 31) || K >= (int64_t(1) << 31))
    return FP8MOE_ERR_SHAPE;
  if (((M + 127) / 128) * ((N + 127) / 128) >= (int64_t(1) << 31)) return FP8MOE_ERR_SHAPE;
  // per-lane 32-bit byte offsets into a and w
  if (2 * M * K >= (int64_t(1) << 32) || 2 * N * K >= (int64_t(1) << 32)) return FP8MOE_ERR_SHAPE;
  if (!aligned16(a) || !aligned16(w) || !aligned16(out)) return FP8MOE_ERR_ALIGN;
  return launch_status(fp8moe::launch_bf16_gemm(static_cast<const uint16_t*>(a),
                                                 static_cast<const uint16_t*>(w), M, N, K, out,
                                                 static_cast<hipStream_t>(stream)));
}

int32_t fp8moe_causal_attention(const void* qkv, int64_t T, int32_t n_q, int32_t n_kv,
                                int32_t head_dim, void* out, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!qkv || !out || !ws) return FP8MOE_ERR_NULL;
  if (head_dim != kHeadDim) return FP8MOE_ERR_SHAPE;
  if (T < 1 || n_kv < 1 || n_q < 1 || n_q > kMaxHeads || n_q % n_kv != 0)
    return FP8MOE_ERR_SHAPE;
  if ((int64_t)(n_q + 2 * n_kv) * head_dim * T >= (int64_t(1) << 31)) return FP8MOE_ERR_SHAPE;
  if (!aligned16(qkv) || !aligned16(out) || !aligned16(ws)) return FP8MOE_ERR_ALIGN;
  if (ws_bytes < fp8moe::attention_workspace_bytes(T, n_kv)) return FP8MOE_ERR_WORKSPACE;
  return launch_status(fp8moe::launch_attention(static_cast<const uint16_t*>(qkv), T, n_q, n_kv,
                                                static_cast<uint16_t*>(out),
                                                static_cast<uint16_t*>(ws),
                                                static_cast<hipStream_t>(stream)));
}

}  // extern "C"
