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
//   acc += P * (s_a * s_w) (two VALU ops per output per group). VALU, not the matrix
//   core, is the scarce unit: at full MFMA rate the fold alone fills the VALU, so every
//   other VALU op in the loop is kept to a minimum.
// * Nibble -> e4m3 in two ops per four weights: e4m3 codes 0x00..0x0F are exactly
//   u * 2^-9 (the subnormals and the first normal binade share the spacing 2^-9), so the
//   offset nibble u = n ^ 8 = q + 8 (q the int4 value) IS the e4m3 code of (q + 8) * 2^-9.
//   The +8 is removed inside the MFMA: its accumulator input is seeded with
//   -8 * 2^-9 * sum_k a_k for that row and group, and that row sum is itself one MFMA of
//   the A tile against a constant all-ones operand (one extra MFMA per 16 rows per group,
//   +6%). The 2^9 is folded into the weight scale (exact). The bank's K-interleaved
//   nibble order makes the low nibbles of a 32-bit word four consecutive k, so a byte
//   split (and, shift+and) gives K-ordered e4m3 bytes with no permutes.
// * Workgroup tile 128 rows x 256 accumulator columns, 4 waves side by side along N
//   (each wave: all 128 rows x 64 columns = 8 x 4 MFMA tiles, 128 fp32 accumulators per
//   lane). A (e4m3 rows, gathered from token order through `sorted` when given), each
//   wave's packed B slice and both scale vectors go straight from global memory into LDS
//   (global_load_lds, no VGPR staging) in two stages, one barrier per group; the stage
//   size keeps LDS under 80 KB so two workgroups share a CU and cover each other's
//   memory waits. Each wave stages exactly the 32 A rows whose sums it computes, so the
//   seeds of group g+1 are formed right after the wave's own loads land, before the
//   group's single barrier.
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

constexpr int BM = 128;        // rows per workgroup tile
constexpr int NW = 4;          // waves per workgroup
constexpr int WCOLS = 64;      // accumulator columns per wave
constexpr int WCOLS_WG = NW * WCOLS;           // 256 accumulator columns per workgroup
constexpr int A_BYTES = BM * kGroup;           // e4m3 A tile of one group
constexpr int BW_BYTES = WCOLS * kGroup / 2;   // packed B slice of one wave, one group
constexpr int B_BYTES = NW * BW_BYTES;
// one pipeline stage: A tile, B slices, A scales (128 rows), weight scales (256 columns)
constexpr int STAGE_BYTES = A_BYTES + B_BYTES + BM * 4 + WCOLS_WG * 4;
constexpr int SMEM_BYTES = 2 * STAGE_BYTES + 2 * BM * 4;  // + row-sum seeds, 2 groups
constexpr float kWeightScaleMul = 512.f;       // 2^9: B codes are (q + 8) * 2^-9
constexpr uint32_t kOnes = 0x38383838u;        // four e4m3 1.0

typedef __attribute__((address_space(3))) void lds_void;

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

// global -> LDS without VGPR staging; lane i of the wave writes lds_block + size * i
// (lds_block is wave-uniform).
__device__ __forceinline__ void g2lds16(const void* g, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_block, 16, 0, 0);
}
__device__ __forceinline__ void g2lds4(const void* g, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_block, 4, 0, 0);
}

// 16 packed bytes (32 int4, K-interleaved words) -> MFMA B operand of (q + 8) * 2^-9.
__device__ __forceinline__ v8i convert_b(uint4 p) {
  v8i b;
  uint32_t w[4] = {p.x ^ 0x88888888u, p.y ^ 0x88888888u, p.z ^ 0x88888888u, p.w ^ 0x88888888u};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    b[2 * j] = (int)(w[j] & 0x0F0F0F0Fu);
    b[2 * j + 1] = (int)((w[j] >> 4) & 0x0F0F0F0Fu);
  }
  return b;
}

// LDS A tile: [BM rows][8 chunks of 16 B], chunk c of row r stored at c ^ (r & 7) so the
// 8 lanes of each ds_read_b128 phase hit distinct banks.
__device__ __forceinline__ int a_off(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

__device__ __forceinline__ v8i lds_a_operand(const uint8_t* tile, int r, int q) {
  uint4 lo = *reinterpret_cast<const uint4*>(&tile[a_off(r, 2 * q)]);
  uint4 hi = *reinterpret_cast<const uint4*>(&tile[a_off(r, 2 * q + 1)]);
  return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
               (int)hi.w};
}

// max over each row of 16 lanes, on the DPP path (no LDS traffic)
__device__ __forceinline__ float max16_dpp(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
  return v;
}

template <int EPI, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As,
    const int32_t* __restrict__ sorted, int k_route, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, const int32_t* __restrict__ offsets, int E, int N, int K,
    int NT, void* __restrict__ out, float* __restrict__ out_scales) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM_BYTES];
  __shared__ int s_tmp[4];
  __shared__ int s_tile[3];
  __shared__ int s_total;
  auto stage_a = [&](int b) { return smem + b * STAGE_BYTES; };
  auto stage_b = [&](int b) { return smem + b * STAGE_BYTES + A_BYTES; };
  auto stage_as = [&](int b) { return reinterpret_cast<float*>(smem + b * STAGE_BYTES + A_BYTES + B_BYTES); };
  auto stage_ws = [&](int b) { return reinterpret_cast<float*>(smem + b * STAGE_BYTES + A_BYTES + B_BYTES + BM * 4); };
  float* const sRA = reinterpret_cast<float*>(smem + 2 * STAGE_BYTES);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int q = lane >> 4, c16 = lane & 15;
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
  const int e = s_tile[0], row_begin = s_tile[1], rows = s_tile[2];

  // ---- sources. Wave wv stages rows 32wv .. 32wv+31 of every A tile (the rows whose
  // sums it also computes, so it needs nobody else's loads for that), chunk p = (4wv+j)*64
  // + lane of the swizzled tile for j = 0..3.
  auto src_row = [&](int r) {
    const int grow = row_begin + min(r, rows - 1);
    return sorted ? sorted[grow] / k_route : grow;
  };
  uint32_t a_src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = (wv * 4 + j) * 64 + lane;
    const int r = p >> 3, c = (p & 7) ^ (r & 7);
    a_src[j] = (uint32_t)src_row(r) * (uint32_t)K + (uint32_t)(c * 16);
  }
  // A scale of row 32wv + lane (lanes 0..31); rows past the tile read a valid row and are
  // never stored
  const float* const as_src = As + (int64_t)src_row(wv * 32 + (lane & 31)) * G;
  // accumulator column j (0..255) of the workgroup -> bank column
  auto bank_col = [&](int j) {
    if (EPI == FP8MOE_EPI_SWIGLU_QUANT)  // j = w*64 + s*16 + c: gate for s < 2, up for s >= 2
      return (((j >> 5) & 1) ? N / 2 : 0) + nt * 128 + (j >> 6) * 32 + (j & 31);
    return min(nt * WCOLS_WG + j, N - 1);
  };
  const uint8_t* const Wexp = W + (int64_t)e * N * (K / 2);
  const float* const ws_src = Ws + ((int64_t)e * N + bank_col(wv * WCOLS + lane)) * G;
  const uint8_t* b_src[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    b_src[s] = Wexp + (int64_t)bank_col(wv * WCOLS + 16 * s + c16) * (K / 2) + q * 16;

  auto load_group = [&](int g, int b) {
    uint8_t* sa = stage_a(b);
#pragma unroll
    for (int j = 0; j < 4; ++j) g2lds16(A + a_src[j] + g * kGroup, sa + (wv * 4 + j) * 1024);
    uint8_t* sb = stage_b(b) + wv * BW_BYTES;
#pragma unroll
    for (int s = 0; s < 4; ++s) g2lds16(b_src[s] + g * 64, sb + s * 1024);
    g2lds4(ws_src + g, reinterpret_cast<uint8_t*>(stage_ws(b) + wv * WCOLS));
    if (lane < 32) g2lds4(as_src + g, reinterpret_cast<uint8_t*>(stage_as(b) + wv * 32));
  };

  // sums of this wave's two 16-row tiles of the A tile in stage b -> sRA[rb] as -sum/64,
  // the accumulator seed that removes the +8 offset of the B codes
  const v8i ones = {(int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes,
                    (int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  auto row_sums = [&](int b, int rb) {
    const uint8_t* ta = stage_a(b);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = wv * 2 + u;
      v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lds_a_operand(ta, t * 16 + c16, q),
                                                                ones, zero, 0, 0, 0, 0, 0, 0);
      if (c16 == 0)
        *reinterpret_cast<float4*>(&sRA[rb * BM + t * 16 + 4 * q]) =
            make_float4(pr[0] * -0.015625f, pr[1] * -0.015625f, pr[2] * -0.015625f,
                        pr[3] * -0.015625f);
    }
  };

  float acc[8][4][4];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][s][r] = 0.f;

  // ---- prologue: group 0 staged, its row sums seeded
  load_group(0, 0);
  __builtin_amdgcn_s_waitcnt(0);  // own LDS loads landed (visible to this wave)
  row_sums(0, 0);
  __syncthreads();

  // ---- main loop, two stages: group g+1 streams into LDS while group g is computed.
  // Each group is 32 steps; step i = 4t + s issues the MFMA of tile (t, s) and folds the
  // MFMA of step i-2 (already complete), so the matrix core and the VALU work side by
  // side; a sched_barrier after every step pins that interleaving.
  for (int g = 0; g < G; ++g) {
    const int b = g & 1;
    const bool next = g + 1 < G;
    if (next) load_group(g + 1, b ^ 1);
    const uint8_t* ta = stage_a(b);
    const uint8_t* tb = stage_b(b) + wv * BW_BYTES;
    const float* ra = sRA + b * BM;
    const float* sag = stage_as(b);
    const float* swg = stage_ws(b) + wv * WCOLS;
    v8i bop[4];
    float sw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bop[s] = convert_b(*reinterpret_cast<const uint4*>(&tb[s * 1024 + lane * 16]));
      sw[s] = swg[s * 16 + c16] * kWeightScaleMul;
    }

    v8i aop[2];
    v4f seed[2];
    float4 sa[2];
    aop[0] = lds_a_operand(ta, c16, q);
    {
      const float4 c4 = *reinterpret_cast<const float4*>(&ra[4 * q]);
      seed[0] = (v4f){c4.x, c4.y, c4.z, c4.w};
    }
    sa[0] = *reinterpret_cast<const float4*>(&sag[4 * q]);
    v4f pb[3];

    auto fold = [&](int i) {
      const int t = i >> 2, s = i & 3;
      const float4 a4 = sa[t & 1];
      const v4f p = pb[i % 3];
      acc[t][s][0] = fmaf(p[0], a4.x * sw[s], acc[t][s][0]);
      acc[t][s][1] = fmaf(p[1], a4.y * sw[s], acc[t][s][1]);
      acc[t][s][2] = fmaf(p[2], a4.z * sw[s], acc[t][s][2]);
      acc[t][s][3] = fmaf(p[3], a4.w * sw[s], acc[t][s][3]);
      // keep the fold at this point of the instruction stream (otherwise it is sunk to the
      // end of the group, and the MFMA results pile up in registers)
      asm volatile("" : "+v"(acc[t][s][0]), "+v"(acc[t][s][1]), "+v"(acc[t][s][2]),
                   "+v"(acc[t][s][3]));
    };

#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int t = i >> 2, s = i & 3;
      if (s == 0 && t < 7) {  // A operand and seed of the next row tile
        aop[(t + 1) & 1] = lds_a_operand(ta, (t + 1) * 16 + c16, q);
        const float4 c4 = *reinterpret_cast<const float4*>(&ra[(t + 1) * 16 + 4 * q]);
        seed[(t + 1) & 1] = (v4f){c4.x, c4.y, c4.z, c4.w};
      }
      if (s == 2 && t < 7)  // A scales of the next row tile (tile t-1's folds are done)
        sa[(t + 1) & 1] = *reinterpret_cast<const float4*>(&sag[(t + 1) * 16 + 4 * q]);
      pb[i % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop[t & 1], bop[s],
                                                                   seed[t & 1], 0, 0, 0, 0, 0, 0);
      if (i >= 2) fold(i - 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    fold(30);
    fold(31);
    __builtin_amdgcn_s_waitcnt(0);  // own loads of group g+1 landed
    if (next) row_sums(b ^ 1, b ^ 1);
    __syncthreads();
  }

  // ---- epilogues. Output element (t, s, r) of this lane: row t*16 + 4q + r, workgroup
  // column wv*64 + s*16 + c16.
  if (EPI == FP8MOE_EPI_STORE && OUT_BF16) {
    // stage the 128 x 256 bf16 tile in LDS, then write whole 512-byte row segments
    uint16_t* s_out = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          s_out[(t * 16 + 4 * q + r) * WCOLS_WG + wv * WCOLS + s * 16 + c16] =
              (uint16_t)f32_to_bf16(acc[t][s][r]);
    __syncthreads();
    const int ncols = min(WCOLS_WG, N - nt * WCOLS_WG);  // multiple of 16
    uint16_t* o16 = reinterpret_cast<uint16_t*>(out);
    for (int i = tid; i < BM * (WCOLS_WG / 8); i += 256) {
      const int row = i >> 5, ch = i & 31;
      if (row < rows && ch * 8 < ncols)
        *reinterpret_cast<uint4*>(&o16[(int64_t)(row_begin + row) * N + nt * WCOLS_WG + ch * 8]) =
            *reinterpret_cast<const uint4*>(&s_out[row * WCOLS_WG + ch * 8]);
    }
  } else if (EPI == FP8MOE_EPI_STORE) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = t * 16 + 4 * q + r;
        if (row < rows) {
          const int64_t orow = (int64_t)(row_begin + row) * N;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int cc = nt * WCOLS_WG + wv * WCOLS + s * 16 + c16;
            if (cc < N) reinterpret_cast<float*>(out)[orow + cc] = acc[t][s][r];
          }
        }
      }
  } else {
    // SwiGLU + e4m3 per (row, 128 h columns). h column of (t, s', r) is wv*32 + s'*16 + c16.
    float* s_amax = reinterpret_cast<float*>(smem);        // [4 waves][BM]
    float* s_inv = s_amax + NW * BM;                        // [BM]
    uint8_t* s_codes = smem + A_BYTES;                      // [BM][128]
    float h[8][2][4];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = 0.f;
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          float gt = acc[t][sp][r], up = acc[t][sp + 2][r];
          float hv = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * up;
          h[t][sp][r] = hv;
          m = fmaxf(m, fabsf(hv));
        }
        m = max16_dpp(m);
        if (c16 == 0) s_amax[wv * BM + t * 16 + 4 * q + r] = m;
      }
    __syncthreads();
    if (tid < BM) {
      float m = fmaxf(fmaxf(s_amax[tid], s_amax[BM + tid]),
                      fmaxf(s_amax[2 * BM + tid], s_amax[3 * BM + tid]));
      float sc, inv;
      scale_pair(m, sc, inv);
      s_inv[tid] = inv;
      if (tid < rows) out_scales[(int64_t)(row_begin + tid) * (N / 2 / kGroup) + nt] = sc;
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
      if (row < rows)
        *reinterpret_cast<uint4*>(&o8[(int64_t)(row_begin + row) * I + nt * 128 + ch * 16]) =
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
  const int NT = epilogue == FP8MOE_EPI_SWIGLU_QUANT ? (int)(N / WCOLS_WG)
                                                     : (int)((N + WCOLS_WG - 1) / WCOLS_WG);
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
