// Device helpers shared by the HIP kernels of the FP8 MoE prefill library (gfx950).
//
// e4m3 here is OCP e4m3fn: the format the activation scale amax/448 implies (memra-engine
// fp8_ffi module docs, module text: one dynamic scale per tensor, computed as amax/448).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8moe {

constexpr int kGroup = 128;       // K-group of every group-wise scale
constexpr float kE4m3Max = 448.f;
constexpr float kAmaxFloor = 1e-12f;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

// Scale pair of one quantisation group from its amax: s = a/448 and inv = 448/a with
// a = max(amax, 1e-12). Both are IEEE divisions (the library is built without fast-math,
// so '/' is correctly rounded).
__device__ __forceinline__ void scale_pair(float amax, float& s, float& inv) {
  float a = fmaxf(amax, kAmaxFloor);
  s = a / kE4m3Max;
  inv = kE4m3Max / a;
}

// Four fp32 values -> four e4m3 bytes (byte i = value i), round to nearest even,
// saturating to +-448, sign of zero kept, NaN -> 0x7F. The hardware conversion rounds to
// nearest even but does not saturate, so values are clamped first.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  float ca = __builtin_amdgcn_fmed3f(a, -kE4m3Max, kE4m3Max);
  float cb = __builtin_amdgcn_fmed3f(b, -kE4m3Max, kE4m3Max);
  float cc = __builtin_amdgcn_fmed3f(c, -kE4m3Max, kE4m3Max);
  float cd = __builtin_amdgcn_fmed3f(d, -kE4m3Max, kE4m3Max);
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
  r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cc, cd, (int)r, true);
  // NaN policy: 0x7F. (med3 of a NaN input is not guaranteed to stay NaN.)
  if (a != a) r = (r & 0xFFFFFF00u) | 0x7Fu;
  if (b != b) r = (r & 0xFFFF00FFu) | 0x7F00u;
  if (c != c) r = (r & 0xFF00FFFFu) | 0x7F0000u;
  if (d != d) r = (r & 0x00FFFFFFu) | 0x7F000000u;
  return r;
}

// Two finite fp32 values -> two e4m3 bytes (low half of the result), round to nearest even,
// saturating. For values that are finite by construction (no NaN handling).
__device__ __forceinline__ uint32_t e4m3x2_finite(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, -kE4m3Max, kE4m3Max),
                                                    __builtin_amdgcn_fmed3f(b, -kE4m3Max, kE4m3Max),
                                                    0, false) & 0xFFFFu;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> two bf16 (round to nearest even) packed low|high, one instruction.
__device__ __forceinline__ uint32_t bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Max over the 16 lanes that share (lane / 16), in every one of them: four DPP row
// rotations (by 1, 2, 4, 8 lanes within the 16-lane row), VALU only.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                    0xF, 0xF, false));
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_row<0x121>(v));  // row_ror:1
  v = fmaxf(v, dpp_row<0x122>(v));  // row_ror:2
  v = fmaxf(v, dpp_row<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_row<0x128>(v));  // row_ror:8
  return v;
}

// sum over the 16 lanes of a row, every lane ends with the sum (a fixed association order
// for each lane, so the value a given lane holds is deterministic)
__device__ __forceinline__ float sum16(float v) {
  v += dpp_row<0x121>(v);  // row_ror:1
  v += dpp_row<0x122>(v);  // row_ror:2
  v += dpp_row<0x124>(v);  // row_ror:4
  v += dpp_row<0x128>(v);  // row_ror:8
  return v;
}

// sum over each aligned group of 8 lanes, every lane of the group ends with the sum (all
// lanes of the row must be active)
__device__ __forceinline__ float sum8(float v) {
  v += dpp_row<0xB1>(v);   // quad_perm [1,0,3,2]: the lane beside
  v += dpp_row<0x4E>(v);   // quad_perm [2,3,0,1]: the other pair of the quad
  v += dpp_row<0x141>(v);  // row_half_mirror: the other quad of the 8
  return v;
}

// sum of the values of 8 e4m3 codes (two words), in a fixed order
__device__ __forceinline__ float e4m3_sum8(uint32_t lo, uint32_t hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const f2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  const f2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  return ((a.x + a.y) + (b.x + b.y)) + ((c.x + c.y) + (d.x + d.y));
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Workgroup ids are dealt round-robin to the 8 XCDs (each with its own L2). Renumber
// them so that each XCD works through one contiguous range of logical tiles: tiles that
// share operands then run on the same L2.
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t bid, uint32_t nblocks) {
  constexpr uint32_t kXcd = 8;
  uint32_t per = nblocks / kXcd, rem = nblocks % kXcd;
  uint32_t x = bid % kXcd, i = bid / kXcd;
  return x * per + (x < rem ? x : rem) + i;
}

// Logical tile L of an NTM x NTN tile grid, in groups of up to 8 tile rows swept
// column-block by column-block: consecutive L (which run side by side on one XCD, see
// xcd_contiguous) then cover a compact block of 8 x 8 tiles whose A rows and W columns
// stay in that XCD's L2, instead of one tile row against 64 different weight blocks.
__device__ __forceinline__ void grouped_tile(uint32_t L, int NTM, int NTN, int& tm, int& tn) {
  constexpr int GM = 8;
  const uint32_t per_group = (uint32_t)(GM * NTN);
  const int first = (int)(L / per_group) * GM;
  const int gm = min(NTM - first, GM);
  const int r = (int)(L % per_group);
  tm = first + r % gm;
  tn = r / gm;
}

}  // namespace fp8moe
