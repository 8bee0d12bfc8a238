// Grouped FP8 expert GEMM over a resident packed-int4 bank (fp8_grouped_expert_gemm).
//
// Method ("FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant", section 1):
// one GEMM launch covers every expert of the layer; the int4 weights stay packed in
// memory and are turned into e4m3 on-chip; the per-(token, group) activation scale and the
// per-group weight scale are folded into the fp32 accumulator:
//
//   y[i, n] = sum_g  s_a[i, g] * s_w[e, n, g] * sum_{k in g} e4m3(a[i, k]) * q[e, n, k]
//
// gfx950 design:
// * The MFMA is v_mfma_f32_16x16x128_f8f6f4: its K of 128 is exactly one scale group, so
//   each group is one MFMA per 16x16 output tile, followed by the fold
//   acc += P * (s_a * s_w) (two VALU ops per output per group).
// * Workgroup tile 128 rows x 256 accumulator columns, 4 waves side by side along N
//   (each wave: all 128 rows x 64 columns = 8 x 4 MFMA tiles, 128 fp32 accumulators per
//   lane). A (e4m3 rows) is shared by the 4 waves through LDS, double-buffered with one
//   barrier per group; the rows are gathered from token order on the fly when `sorted` is
//   given, so no permuted copy of the activations is ever written.
// * B never touches LDS: each wave reads only its own 64 columns, 16 bytes of packed
//   nibbles per lane per tile per group (coalesced along K), prefetched one group ahead,
//   and converts them in registers.
// * Nibble -> e4m3: e4m3 codes 0x00..0x0F are exactly n * 2^-9 (the subnormals and the
//   first normal binade share the spacing 2^-9), so the int4 value v = -8..7 is encoded
//   exactly as the sign-magnitude code of v * 2^-9: byte = v >= 0 ? v : 0x80 | -v. From
//   a two's-complement nibble n that is n for n < 8 and 0x90 - n for n >= 8: four bytes
//   at a time with one subtract, one select-mask and one v_perm byte select. The 2^9 is
//   folded into the weight scale (exact).
// * The nibble split puts even K in one dword and odd K in the next; the A rows are
//   byte-permuted the same way when staged into LDS, so both MFMA operands agree.
// * One launch covers all experts: the grid is the host-known bound ceil(R/128) + E
//   m-tiles times the n-tiles; each workgroup finds its (expert, m-tile) from the device
//   offsets (a workgroup-wide scan over E) and exits if surplus.
// * Epilogues: STORE writes fp32 or bf16; SWIGLU_QUANT pairs gate columns n and up
//   columns I+n in the same wave, forms h = silu(gate) * up in fp32, takes the per-row
//   amax over the workgroup's 128 h columns (= one 128-group of the down GEMM's K) and
//   writes e4m3 codes plus fp32 scales, so h never goes to HBM in fp32 or bf16.
#include "common.h"
#include "launch.h"

namespace fp8moe {
namespace {

constexpr int BM = 128;      // rows per workgroup tile
constexpr int WCOLS = 64;    // accumulator columns per wave
constexpr int kMaxG = 64;    // K <= 8192
constexpr uint32_t kWeightScaleMul = 512;  // 2^9, see the nibble encoding above

__device__ __forceinline__ int block_inclusive_scan256(int v, int* tmp) {
  int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) tmp[w] = v;
  __syncthreads();
  int add = 0;
  for (int j = 0; j < w; ++j) add += tmp[j];
  __syncthreads();
  return v + add;
}

// Four two's-complement nibbles, one per byte (0..15) -> four e4m3 codes of v * 2^-9.
__device__ __forceinline__ uint32_t nib4_to_e4m3(uint32_t x) {
  uint32_t neg = 0x90909090u - x;                          // 0x80 | (16 - n), no borrows
  uint32_t sel = ((x >> 1) & 0x04040404u) | 0x03020100u;   // byte i <- x.i or neg.i
  return __builtin_amdgcn_perm(neg, x, sel);
}

// 16 packed bytes (32 nibbles, K order) -> MFMA B operand (even K of each 8 first).
__device__ __forceinline__ v8i convert_b(uint4 p) {
  v8i b;
  uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    b[2 * j] = (int)nib4_to_e4m3(w[j] & 0x0F0F0F0Fu);
    b[2 * j + 1] = (int)nib4_to_e4m3((w[j] >> 4) & 0x0F0F0F0Fu);
  }
  return b;
}

// Byte permutation of 8 A bytes [a0..a7] -> [a0 a2 a4 a6 a1 a3 a5 a7], matching the
// even/odd split of the B operand.
__device__ __forceinline__ uint4 permute_a(uint4 v) {
  uint4 r;
  r.x = __builtin_amdgcn_perm(v.y, v.x, 0x06040200u);
  r.y = __builtin_amdgcn_perm(v.y, v.x, 0x07050301u);
  r.z = __builtin_amdgcn_perm(v.w, v.z, 0x06040200u);
  r.w = __builtin_amdgcn_perm(v.w, v.z, 0x07050301u);
  return r;
}

// LDS A tile: [BM rows][8 chunks of 16 B], chunk c of row r stored at c ^ (r & 7) so the
// 8 lanes of each ds_read_b128 phase hit distinct banks.
__device__ __forceinline__ int a_off(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

struct Tile {
  int e, row_begin, rows;
};

template <int EPI, bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As,
    const int32_t* __restrict__ sorted, int k_route, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, const int32_t* __restrict__ offsets, int E, int N, int K,
    int NT, void* __restrict__ out, float* __restrict__ out_scales) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * 128];
  __shared__ __attribute__((aligned(16))) float sAs[kMaxG * BM];
  __shared__ int s_tmp[4];
  __shared__ int s_tile[3];
  __shared__ int s_total;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = K / kGroup;
  const uint32_t L = xcd_contiguous(blockIdx.x, gridDim.x);
  const int mt = (int)(L / (uint32_t)NT), nt = (int)(L % (uint32_t)NT);

  // ---- which expert and which 128-row slice of it this workgroup owns
  {
    int loc[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = tid * 4 + j;
      int c = e < E ? offsets[e + 1] - offsets[e] : 0;
      loc[j] = (c + BM - 1) / BM;
      sum += loc[j];
    }
    int inc = block_inclusive_scan256(sum, s_tmp);
    int run = inc - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (mt >= run && mt < run + loc[j]) {
        int e = tid * 4 + j;
        int rb = offsets[e] + (mt - run) * BM;
        s_tile[0] = e;
        s_tile[1] = rb;
        s_tile[2] = min(BM, offsets[e + 1] - rb);
      }
      run += loc[j];
    }
    if (tid == 255) s_total = inc;
    __syncthreads();
  }
  if (mt >= s_total) return;  // surplus workgroup (uniform)
  const Tile tl = {s_tile[0], s_tile[1], s_tile[2]};

  // ---- A staging: thread -> (row, half row of the 128-byte group slice)
  const int ar = tid >> 1, ahalf = tid & 1;
  const uint8_t* a_row;
  {
    int grow = tl.row_begin + min(ar, tl.rows - 1);
    int64_t src = sorted ? (int64_t)(sorted[grow] / k_route) : (int64_t)grow;
    a_row = A + src * (int64_t)K + ahalf * 64;
  }
  // A scales for every group, transposed to [g][row] in LDS
  for (int i = tid; i < BM * G; i += 256) {
    int r = i / G, g = i - r * G;
    int grow = tl.row_begin + min(r, tl.rows - 1);
    int64_t src = sorted ? (int64_t)(sorted[grow] / k_route) : (int64_t)grow;
    sAs[g * BM + r] = r < tl.rows ? As[src * G + g] : 0.f;
  }

  // ---- B: this wave's 4 column tiles
  const int q = lane >> 4, c16 = lane & 15;
  const uint8_t* b_ptr[4];
  const float* bs_ptr[4];
  int col[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    int cc;
    if (EPI == FP8MOE_EPI_SWIGLU_QUANT) {
      const int I = N / 2;
      cc = (s < 2 ? 0 : I) + nt * 128 + wv * 32 + (s & 1) * 16 + c16;
    } else {
      cc = nt * 256 + wv * WCOLS + s * 16 + c16;
      cc = min(cc, N - 1);
    }
    col[s] = cc;
    int64_t wrow = (int64_t)tl.e * N + cc;
    b_ptr[s] = W + wrow * (K / 2) + q * 16;
    bs_ptr[s] = Ws + wrow * G;
  }

  float acc[8][4][4];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][s][r] = 0.f;

  uint4 areg[4];
  uint4 bp[4];
  float bsc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) areg[i] = *reinterpret_cast<const uint4*>(a_row + i * 16);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bp[s] = *reinterpret_cast<const uint4*>(b_ptr[s]);
    bsc[s] = bs_ptr[s][0];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4*>(&sA[0][a_off(ar, ahalf * 4 + i)]) = permute_a(areg[i]);
  __syncthreads();

  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < G; ++g) {
    const int cur = g & 1;
    const bool more = g + 1 < G;
    uint4 bpn[4];
    float bscn[4];
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        areg[i] = *reinterpret_cast<const uint4*>(a_row + (g + 1) * kGroup + i * 16);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bpn[s] = *reinterpret_cast<const uint4*>(b_ptr[s] + (g + 1) * 64);
        bscn[s] = bs_ptr[s][g + 1];
      }
    }
    v8i bop[4];
    float sw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bop[s] = convert_b(bp[s]);
      sw[s] = bsc[s] * (float)kWeightScaleMul;
    }
    const uint8_t* sa_tile = sA[cur];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int r = t * 16 + c16;
      uint4 lo = *reinterpret_cast<const uint4*>(&sa_tile[a_off(r, 2 * q)]);
      uint4 hi = *reinterpret_cast<const uint4*>(&sa_tile[a_off(r, 2 * q + 1)]);
      v8i aop = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const float4 sa = *reinterpret_cast<const float4*>(&sAs[g * BM + t * 16 + 4 * q]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[s], zero, 0, 0, 0,
                                                                 0, 0, 0);
        acc[t][s][0] = fmaf(p[0], sa.x * sw[s], acc[t][s][0]);
        acc[t][s][1] = fmaf(p[1], sa.y * sw[s], acc[t][s][1]);
        acc[t][s][2] = fmaf(p[2], sa.z * sw[s], acc[t][s][2]);
        acc[t][s][3] = fmaf(p[3], sa.w * sw[s], acc[t][s][3]);
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(&sA[cur ^ 1][a_off(ar, ahalf * 4 + i)]) = permute_a(areg[i]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bp[s] = bpn[s];
        bsc[s] = bscn[s];
      }
    }
    __syncthreads();
  }

  // ---- epilogues. Output element (t, s, r) of this lane: row t*16 + 4q + r, column col[s].
  if (EPI == FP8MOE_EPI_STORE) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = t * 16 + 4 * q + r;
        if (row < tl.rows) {
          const int64_t orow = (int64_t)(tl.row_begin + row) * N;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int cc = nt * 256 + wv * WCOLS + s * 16 + c16;
            if (cc < N) {
              if (OUT_BF16)
                reinterpret_cast<uint16_t*>(out)[orow + cc] = (uint16_t)f32_to_bf16(acc[t][s][r]);
              else
                reinterpret_cast<float*>(out)[orow + cc] = acc[t][s][r];
            }
          }
        }
      }
  } else {
    // SwiGLU + e4m3 per (row, 128 h columns). h column of (t, s', r) is wv*32 + s'*16 + c16.
    float* s_amax = reinterpret_cast<float*>(&sA[0][0]);  // [4 waves][BM]
    float* s_inv = s_amax + 4 * BM;                        // [BM]
    uint8_t* s_codes = &sA[1][0];                          // [BM][128]
    float h[8][2][4];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = 0.f;
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          float gt = acc[t][sp][r], up = acc[t][sp + 2][r];
          float hv = gt / (1.f + __expf(-gt)) * up;
          h[t][sp][r] = hv;
          m = fmaxf(m, fabsf(hv));
        }
        m = max16(m);
        if (c16 == 0) s_amax[wv * BM + t * 16 + 4 * q + r] = m;
      }
    __syncthreads();
    if (tid < BM) {
      float m = fmaxf(fmaxf(s_amax[tid], s_amax[BM + tid]),
                      fmaxf(s_amax[2 * BM + tid], s_amax[3 * BM + tid]));
      float sc, inv;
      scale_pair(m, sc, inv);
      s_inv[tid] = inv;
      if (tid < tl.rows)
        out_scales[(int64_t)(tl.row_begin + tid) * (N / 2 / kGroup) + nt] = sc;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = t * 16 + 4 * q + r;
        const float inv = s_inv[row];
        uint32_t c2 = e4m3x4(h[t][0][r] * inv, h[t][1][r] * inv, 0.f, 0.f);
        s_codes[row * 128 + wv * 32 + c16] = (uint8_t)(c2 & 0xFF);
        s_codes[row * 128 + wv * 32 + 16 + c16] = (uint8_t)((c2 >> 8) & 0xFF);
      }
    __syncthreads();
    const int I = N / 2;
    uint8_t* o8 = reinterpret_cast<uint8_t*>(out);
    for (int i = tid; i < BM * 8; i += 256) {
      const int row = i >> 3, ch = i & 7;
      if (row < tl.rows)
        *reinterpret_cast<uint4*>(&o8[(int64_t)(tl.row_begin + row) * I + nt * 128 + ch * 16]) =
            *reinterpret_cast<const uint4*>(&s_codes[row * 128 + ch * 16]);
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm(const uint8_t* a, const float* a_scales, const int32_t* sorted,
                               int32_t k_route, const uint8_t* w, const float* w_scales,
                               const int32_t* offsets, int64_t R, int32_t E, int64_t N,
                               int64_t K, int32_t epilogue, int32_t out_dtype, void* out,
                               float* out_scales, hipStream_t st) {
  if (R == 0) return hipSuccess;
  const int64_t mtiles = (R + BM - 1) / BM + E;
  const int NT = epilogue == FP8MOE_EPI_SWIGLU_QUANT ? (int)(N / 256) : (int)((N + 255) / 256);
  const int64_t blocks = mtiles * NT;
  dim3 grid((uint32_t)blocks), block(256);
  if (epilogue == FP8MOE_EPI_SWIGLU_QUANT)
    grouped_gemm_kernel<FP8MOE_EPI_SWIGLU_QUANT, false><<<grid, block, 0, st>>>(
        a, a_scales, sorted, k_route, w, w_scales, offsets, E, (int)N, (int)K, NT, out,
        out_scales);
  else if (out_dtype == FP8MOE_DTYPE_BF16)
    grouped_gemm_kernel<FP8MOE_EPI_STORE, true><<<grid, block, 0, st>>>(
        a, a_scales, sorted, k_route, w, w_scales, offsets, E, (int)N, (int)K, NT, out,
        nullptr);
  else
    grouped_gemm_kernel<FP8MOE_EPI_STORE, false><<<grid, block, 0, st>>>(
        a, a_scales, sorted, k_route, w, w_scales, offsets, E, (int)N, (int)K, NT, out,
        nullptr);
  return hipGetLastError();
}

}  // namespace fp8moe
