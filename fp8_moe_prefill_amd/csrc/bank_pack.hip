// One-time repacking of a canonical packed-int4 expert bank into the layout the grouped
// GEMM streams (fp8moe_pack_expert_bank).
//
// Method ("FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant", section 1): the
// int4 bank stays packed and resident; this call only reorders its bytes (and transposes
// its scales) once, when the weights are loaded, so that every K group of every 16 columns
// is one contiguous 1 KB block that one wave-wide load brings in, and the scales of one K
// group are contiguous across columns. Nothing is dequantised or widened. The columns of a
// 64-column group are interleaved over its four blocks so that the GEMM's MFMA lanes end
// up with four consecutive output columns each.
//
// Canonical input: w [E][N][K/2], byte i of row (e, n) holds k = 2i (low nibble) and 2i+1
// (high nibble); w_scales [E][N][K/128].
// Output: block (e, c, g) of 1024 bytes at ((e * N/16 + c) * K/128 + g) * 1024 holds the
// 16 columns n(c, i) = 64 * (c / 4) + 4 * i + c % 4 (i = 0..15: every 4th column of a
// 64-column group, so the four blocks of a group interleave) and k in [128g, 128g + 128).
// Its 16 bytes at 16 * (16h + i) hold column n(c, i), k = 128g + 32h + 0..31, as four
// little-endian words; byte b of word j holds k0 + b in the low nibble and k0 + 4 + b in
// the high nibble (k0 = 128g + 32h + 8j). Scales: [E][K/128][N].
//
// FP4-activation layout (the bank for MXFP4 activations): an FP4 operand lane of the
// gfx950 MFMA holds its 32 values at K positions {b .. b + 15} and {b + 32 .. b + 47} of
// the 128 (b = 64 (q % 2) + 16 (q / 2) for lane block q), and its E8M0 scale covers just
// those. With each lane holding one MX block (32 consecutive K) of the activations, the
// weights must present logical K chunk (16 values) pi(c) = c / 2 + 4 (c % 2) at the
// MFMA's K chunk c: so lane block h holds logical k = 128g + 16h + 0..15 and then
// 128g + 64 + 16h + 0..15 (k0 = 128g + 16h + 64 (j / 2) + 8 (j % 2)).
#include "common.h"
#include "launch.h"

namespace fp8moe {
namespace {

// one thread per output 32-bit word
template <bool FP4_LAYOUT>
__global__ __launch_bounds__(256) void pack_bank_kernel(const uint32_t* __restrict__ w,
                                                        uint32_t* __restrict__ out,
                                                        int64_t words, int N, int K) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= words) return;
  const int G = K / kGroup, NB = N / 16;
  const int j = (int)(o & 3), lane = (int)((o >> 2) & 63);
  const int64_t blk = o >> 8;
  const int g = (int)(blk % G);
  const int64_t ecb = blk / G;
  const int cb = (int)(ecb % NB);
  const int64_t e = ecb / NB;
  const int n = 64 * (cb >> 2) + 4 * (lane & 15) + (cb & 3);
  const int h = lane >> 4;
  const int k0 = g * kGroup + (FP4_LAYOUT ? 16 * h + 64 * (j >> 1) + 8 * (j & 1) : 32 * h + 8 * j);
  // canonical k0 .. k0+7 are the 4 bytes at k0/2: k0 + m sits at bits 4m of this word
  const uint32_t c = w[((e * N + n) * (int64_t)(K / 2) + k0 / 2) >> 2];
  uint32_t r = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t lo = (c >> (4 * b)) & 0xFu, hi = (c >> (16 + 4 * b)) & 0xFu;
    r |= (lo | (hi << 4)) << (8 * b);
  }
  out[o] = r;
}

// [E][N][G] -> [E][G][N], one thread per output element
__global__ __launch_bounds__(256) void pack_scales_kernel(const float* __restrict__ s,
                                                          float* __restrict__ out, int64_t n_out,
                                                          int N, int G) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= n_out) return;
  const int n = (int)(o % N);
  const int64_t eg = o / N;
  const int g = (int)(eg % G);
  const int64_t e = eg / G;
  out[o] = s[(e * N + n) * G + g];
}

}  // namespace

hipError_t launch_pack_bank(const uint8_t* w, const float* w_scales, int64_t E, int64_t N,
                            int64_t K, uint8_t* w_packed, float* ws_packed, hipStream_t st,
                            bool fp4_layout) {
  const int64_t words = E * N * (K / 8);
  const dim3 grid((uint32_t)((words + 255) / 256));
  if (fp4_layout)
    pack_bank_kernel<true><<<grid, 256, 0, st>>>(reinterpret_cast<const uint32_t*>(w),
                                                 reinterpret_cast<uint32_t*>(w_packed), words,
                                                 (int)N, (int)K);
  else
    pack_bank_kernel<false><<<grid, 256, 0, st>>>(reinterpret_cast<const uint32_t*>(w),
                                                  reinterpret_cast<uint32_t*>(w_packed), words,
                                                  (int)N, (int)K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ns = E * N * (K / kGroup);
  pack_scales_kernel<<<dim3((uint32_t)((ns + 255) / 256)), 256, 0, st>>>(
      w_scales, ws_packed, ns, (int)N, (int)(K / kGroup));
  return hipGetLastError();
}

}  // namespace fp8moe
