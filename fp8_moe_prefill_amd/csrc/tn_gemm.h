// out[M, N] = scale * (A[M, K] . W[N, K]^T) with both operands K-contiguous ("TN"), for
// e4m3 x e4m3 (the W8A8 projections, fp8_dense_gemm) and bf16 x bf16 (the stack's LM head,
// fp8moe_bf16_gemm).
//
// gfx950 design:
// * Workgroup tile 128 x 128, 4 waves in a 2 x 2 grid of 64 x 64 (4 x 4 MFMA tiles each),
//   or (BIG) 256 x 256, 8 waves in a 2 x 4 grid of 128 x 64 (8 x 4 MFMA tiles each, one
//   workgroup per CU). One K step is 128 bytes of each row: one
//   v_mfma_f32_16x16x128_f8f6f4 per 16 x 16 tile for e4m3, two v_mfma_f32_16x16x32_bf16
//   for bf16. The LDS is what bounds the small tile: per MFMA a 64 x 64 wave tile reads
//   1 KB of operands and the workgroup's DMA writes 0.5 KB, as much LDS time as the CU's
//   matrix cores spend; the 128 x 64 wave tile of BIG reads 0.75 KB and its 256 x 256
//   workgroup tile writes 0.25 KB per MFMA. BIG needs many tiles to fill the CUs, so the
//   launch picks it by shape; so it does the 128 x 192 tiling (WIDE, below).
// * Both operands go straight from global memory into LDS (LDS DMA, no VGPR staging, no
//   LDS writes by the waves), each DMA instruction copying 8 whole 128-byte lines (8 rows
//   of one K step) into 1 KB of LDS; the 16-byte chunks of a row are XOR-swizzled so that
//   the MFMA operand reads (row c of a 16-row tile, chunk 2 g + half for lane g * 16 + c)
//   are free of bank conflicts.
// * A ring of STAGES steps in LDS: the loads of step ks + STAGES - 1 are issued right after
//   the barrier that frees their slot and stream in while step ks is computed; each wave
//   waits for its own loads by count, and the barrier publishes them.
// * Tiles are dealt to XCDs in contiguous ranges and walked in 8 x 8 blocks, so the A rows
//   and W columns of the tiles in flight on an XCD stay in its L2.
// * Output columns are interleaved so that each lane holds four consecutive columns of a
//   row: column tile s of a wave covers columns 4 * c + s of its 64, and a lane writes them
//   with one 8-byte (bf16) or 16-byte (fp32) store.
// * BLOCK (block-128 e4m3 weights with one scale per 128 x 128 block, activations with one
//   scale per row and 128-wide K group): a K step is exactly one scale group, so each
//   step's MFMAs start from zero and their results are folded into the fp32 accumulators
//   with the step's scale products (row scale x block scale). The tile's 128 columns are
//   one weight block, so the block scale is a single scalar per step; the 128 row scales of
//   the step ride the same LDS DMA stream as the A tile, and the tile's block scales of all
//   K steps sit in LDS from the start. A step issues its 16 MFMAs, then the 64 folds; the
//   other wave on the SIMD keeps the matrix core busy meanwhile.
#pragma once

#include <type_traits>

#include "common.h"
#include "lds_dma.h"

namespace fp8moe {
namespace tn {

constexpr int TM = 128, TN = 128;  // tile rows and columns (BIG: 256 x 256)
constexpr int KSTEP = 128;         // bytes of K per step
constexpr int BLK = 1024;          // one operand block: 64 lanes x 16 bytes
constexpr int kMaxBlockSteps = 128;  // BLOCK: K <= 16384

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <int STAGES, int ROWS>
struct Smem {
  uint8_t a[STAGES][ROWS / 8 * BLK];  // ROWS / 16 row tiles x 2 halves
  uint8_t b[STAGES][ROWS / 8 * BLK];  // ROWS / 16 column tiles x 2 halves
  float as[STAGES][TM];               // BLOCK: the step's scales of the tile's 128 rows
  float ws[kMaxBlockSteps];           // BLOCK: the tile's weight-block scale of every K step
};
template <int STAGES>
struct SmemBig {
  uint8_t a[STAGES][32 * BLK];
  uint8_t b[STAGES][32 * BLK];
};

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// LDS holds each operand tile as 128 rows of 128 bytes (one K step), the 16-byte chunk c of
// row r at position c ^ sw(r): any 16 consecutive rows then read one chunk each without
// bank conflicts.
__device__ __forceinline__ int sw(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// W's LDS row rho holds global column col_of(rho) of the tile: wave wn's column tile s,
// lane c reads row 64 wn + 16 s + c, which is column 64 wn + 4 c + s, so each lane ends up
// with four consecutive output columns.
__device__ __forceinline__ int col_of(int rho) {
  return 64 * (rho >> 6) + 4 * (rho & 15) + ((rho >> 4) & 3);
}

// IN_BF16: operands are bf16 (K counts elements, 2 bytes each), else e4m3 bytes.
// OUT_BF16: bf16 output (round to nearest even), else fp32.
// scale_a / scale_w: the e4m3 path multiplies by scale_a[2] * scale_w[0] (the activation
// scale block and the weight scale, both on the device), or with ROW_SCALE by
// scale_a[row] * scale_w[0] (one activation scale per row); with BLOCK, scale_a is fp32
// [M, K/128] (per row and K group) and scale_w fp32 [ceil(N/128), K/128] (per weight
// block), folded per K step; the bf16 path takes no scale.
template <bool IN_BF16, bool OUT_BF16, int STAGES, bool ROW_SCALE = false, bool BLOCK = false,
          bool BIG = false>
__global__ __launch_bounds__(BIG ? 512 : 256, BIG ? 1 : 2) void tn_gemm_kernel(const uint8_t* __restrict__ A,
                                                         const uint8_t* __restrict__ W, int M,
                                                         int N, int row_bytes, int NTM,
                                                         int NTN,
                                                         const float* __restrict__ scale_a,
                                                         const float* __restrict__ scale_w,
                                                         void* __restrict__ out) {
  static_assert(!BIG || (!ROW_SCALE && !BLOCK && STAGES == 2), "BIG: per-tensor scales");
  constexpr int NWAVE = BIG ? 8 : 4;
  constexpr int HALF = NWAVE / 2;     // waves that load A (the rest load W)
  constexpr int WNW = BIG ? 4 : 2;    // waves along N
  constexpr int RT = BIG ? 8 : 4;     // 16-row tiles per wave
  constexpr int TMB = 2 * RT * 16, TNB = WNW * 64;  // workgroup tile
  using SmemT = typename std::conditional<BIG, SmemBig<STAGES>, Smem<STAGES, 128>>::type;
  __shared__ __attribute__((aligned(16))) SmemT sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int g = lane >> 4, c16 = lane & 15;
  const int wm = wv / WNW, wn = wv % WNW;
  const uint32_t L = xcd_contiguous(blockIdx.x, gridDim.x);
  int tm, tn;
  grouped_tile(L, NTM, NTN, tm, tn);
  const int m0 = tm * TMB, n0 = tn * TNB;
  const int KS = row_bytes / KSTEP;

  // DMA duty: 8 instructions per wave and step (the 128 or 256 rows of A and of W, 8 rows
  // per instruction); the first half of the waves loads A, the second W. Instruction j of
  // a wave copies rows 8 (8 (wave % HALF) + j) .. + 7 as whole 128-byte lines: lane l
  // takes row 8 (8 (wave % HALF) + j) + l / 8 and writes LDS position l % 8 of it, holding
  // the line's 16-byte chunk (l % 8) ^ sw(row). voff[j] is that byte offset at K step 0.
  const bool loads_a = wv < HALF;
  const uint8_t* src = loads_a ? A : W;
  uint32_t voff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rho = 8 * (8 * (wv % HALF) + j) + (lane >> 3);  // LDS row of this lane
    int row;
    if (loads_a) row = min(m0 + rho, M - 1);
    else row = min(n0 + col_of(rho), N - 1);
    const int chunk = (lane & 7) ^ sw(rho);
    voff[j] = (uint32_t)row * (uint32_t)row_bytes + 16u * (uint32_t)chunk;
  }
  static_assert(!BLOCK || (!IN_BF16 && !ROW_SCALE && STAGES == 2),
                "block scales: e4m3 operands, two stages (the waits count all loads)");
  // BLOCK: waves 0 and 1 also stage the step's scales of rows 64 wv .. 64 wv + 63 (the
  // activation scales are [M, KS], one per row and K step)
  const uint32_t soff = BLOCK && wv < 2
                            ? (uint32_t)min(m0 + 64 * wv + lane, M - 1) * (uint32_t)KS * 4u
                            : 0u;
  // BLOCK: the tile's 128 columns are one weight block; its scales of all K steps go to
  // LDS once (published by the first step's barrier)
  if constexpr (BLOCK)
    for (int k = tid; k < KS; k += 256) sm.ws[k] = scale_w[(n0 / TN) * KS + k];
  auto issue = [&](int ks) {
    const int st = ks % STAGES;
    uint8_t* dst = (loads_a ? sm.a[st] : sm.b[st]) + (wv % HALF) * 8 * BLK;
#pragma unroll
    for (int j = 0; j < 8; ++j) dma16(src, voff[j] + (uint32_t)(ks * KSTEP), dst + j * BLK);
    if constexpr (BLOCK)
      if (wv < 2) dma4(scale_a, soff + 4u * (uint32_t)ks, &sm.as[st][64 * wv]);
  };
  // operand reads: tile T (16 rows), half h: row 16 T + c16, chunk 2 g + h
  const int x = sw(c16);
  const int rd0 = c16 * KSTEP + (((2 * g) ^ x) << 4);
  const int rd1 = c16 * KSTEP + (((2 * g + 1) ^ x) << 4);

  v4f acc[RT][4];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[t][s] = (v4f){0.f, 0.f, 0.f, 0.f};
  // per-row activation scales of this lane's 16 output rows, loaded now so that their
  // latency is hidden behind the main loop
  float row_scale[4][4];
  if (ROW_SCALE) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        row_scale[t][r] = scale_a[min(m0 + 64 * wm + 16 * t + 4 * g + r, M - 1)];
  }

#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < KS) issue(p);

  for (int ks = 0; ks < KS; ++ks) {
    // this step's blocks are in: only the steps issued after it may still be in flight
    if (STAGES == 3 && ks + 1 < KS) wait_loads<8>();
    else wait_loads<0>();
    lds_barrier();  // every wave's loads of step ks landed; slot (ks - 1) % STAGES is free
    if (ks + STAGES - 1 < KS) issue(ks + STAGES - 1);
    const uint8_t* sa = sm.a[ks % STAGES];
    const uint8_t* sb = sm.b[ks % STAGES];
    if constexpr (IN_BF16) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8_t aop[RT], bop[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          bop[s] = __builtin_bit_cast(bf16x8_t, lds16(sb + (4 * wn + s) * 16 * KSTEP + (h ? rd1 : rd0)));
#pragma unroll
        for (int t = 0; t < RT; ++t)
          aop[t] = __builtin_bit_cast(bf16x8_t, lds16(sa + (RT * wm + t) * 16 * KSTEP + (h ? rd1 : rd0)));
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[t], bop[s], acc[t][s], 0, 0, 0);
      }
    } else if constexpr (BLOCK) {
      v8i aop[4], bop[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 lo = lds16(sb + (4 * wn + s) * 16 * KSTEP + rd0);
        const uint4 hi = lds16(sb + (4 * wn + s) * 16 * KSTEP + rd1);
        bop[s] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint4 lo = lds16(sa + (4 * wm + t) * 16 * KSTEP + rd0);
        const uint4 hi = lds16(sa + (4 * wm + t) * 16 * KSTEP + rd1);
        aop[t] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      // scale products of this lane's rows 64 wm + 16 t + 4 g + r for this step
      const float swb = sm.ws[ks];
      float sc[4][4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float4 a4 = *reinterpret_cast<const float4*>(&sm.as[ks % STAGES][64 * wm + 16 * t + 4 * g]);
        sc[t][0] = a4.x * swb; sc[t][1] = a4.y * swb; sc[t][2] = a4.z * swb; sc[t][3] = a4.w * swb;
      }
      const v4f zero = {0.f, 0.f, 0.f, 0.f};
      v4f pb[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pb[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop[i >> 2], bop[i & 3], zero,
                                                                 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[i >> 2][i & 3][r] = fmaf(pb[i][r], sc[i >> 2][r], acc[i >> 2][i & 3][r]);
    } else {
      // all operands of the step first (2 (RT + 4) reads in flight), then the 4 RT MFMAs
      v8i aop[RT], bop[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 lo = lds16(sb + (4 * wn + s) * 16 * KSTEP + rd0);
        const uint4 hi = lds16(sb + (4 * wn + s) * 16 * KSTEP + rd1);
        bop[s] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint4 lo = lds16(sa + (RT * wm + t) * 16 * KSTEP + rd0);
        const uint4 hi = lds16(sa + (RT * wm + t) * 16 * KSTEP + rd1);
        aop[t] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[t][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop[t], bop[s], acc[t][s],
                                                                       0, 0, 0, 0, 0, 0);
    }
  }

  const float sw0 = IN_BF16 || BLOCK ? 1.f : scale_w[0];
  const float tensor_scale = IN_BF16 || ROW_SCALE || BLOCK ? sw0 : scale_a[2] * sw0;
  const int c0 = n0 + 64 * wn + 4 * c16;
  const bool vec = (c0 + 3 < N) && ((N & 3) == 0);
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + 16 * RT * wm + 16 * t + 4 * g + r;
      if (row >= M) continue;
      const float scale = ROW_SCALE ? row_scale[t & 3][r] * sw0 : tensor_scale;
      const float v0 = acc[t][0][r] * scale, v1 = acc[t][1][r] * scale;
      const float v2 = acc[t][2][r] * scale, v3 = acc[t][3][r] * scale;
      const int64_t o = (int64_t)row * N + c0;
      if (OUT_BF16) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(out) + o;
        if (vec) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(bf16x2(v0, v1), bf16x2(v2, v3));
        } else {
          const float v[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int s = 0; s < 4; ++s)
            if (c0 + s < N) dst[s] = (uint16_t)f32_to_bf16(v[s]);
        }
      } else {
        float* dst = reinterpret_cast<float*>(out) + o;
        if (vec) {
          *reinterpret_cast<float4*>(dst) = make_float4(v0, v1, v2, v3);
        } else {
          const float v[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int s = 0; s < 4; ++s)
            if (c0 + s < N) dst[s] = v[s];
        }
      }
    }
}

// WIDE: 128 x 192 workgroup tile for e4m3 operands, 4 waves in a 2 x 2 grid of 64 x 96
// (4 x 6 MFMA tiles each, 96 accumulators per lane), two workgroups per CU (2 x 80 KB of
// LDS). Per MFMA a 64 x 96 wave tile reads 0.83 KB of operands from LDS (1 KB for 64 x 64)
// and the workgroup's DMA writes 0.42 KB (0.5 KB). Used where 128 x 192 tiles fill the
// two workgroup slots of every CU in one round and 128 x 128 tiles would need a second,
// partly empty one (the 2048 x 4096 x 6144 q/k/v projection: 512 against 768 tiles).
// Every output is the same chain of K-step MFMAs as in the 128 x 128 kernel.
// W's LDS row rho holds tile column col_of_wide(rho): wave wn's column tile s, lane c reads
// row 96 wn + 16 s + c, which is column 96 wn + 4 c + s for s < 4 (each lane: four
// consecutive columns) and 96 wn + 64 + 2 c + (s - 4) for s = 4, 5 (two more).
__device__ __forceinline__ int col_of_wide(int rho) {
  const int wn = rho / 96, r = rho - 96 * wn, s = r >> 4, c = r & 15;
  return 96 * wn + (s < 4 ? 4 * c + s : 64 + 2 * c + (s - 4));
}

template <bool OUT_BF16, bool ROW_SCALE>
__global__ __launch_bounds__(256, 2) void tn_gemm_wide_kernel(const uint8_t* __restrict__ A,
                                                              const uint8_t* __restrict__ W,
                                                              int M, int N, int row_bytes,
                                                              int NTM, int NTN,
                                                              const float* __restrict__ scale_a,
                                                              const float* __restrict__ scale_w,
                                                              void* __restrict__ out) {
  constexpr int RT = 4, CT = 6;                  // 16-row and 16-column tiles per wave
  constexpr int TMB = 128, TNB = 192;            // workgroup tile
  constexpr int NA = TMB / 8, NB = TNB / 8;      // DMA blocks of A and of W per step
  constexpr int PER = (NA + NB) / 4;             // DMA instructions per wave and step
  static_assert((NA + NB) % 4 == 0, "DMA blocks split evenly over the 4 waves");
  struct Ring {
    uint8_t a[2][NA * BLK];
    uint8_t b[2][NB * BLK];
  };
  __shared__ __attribute__((aligned(16))) Ring sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int g = lane >> 4, c16 = lane & 15;
  const int wm = wv >> 1, wn = wv & 1;
  const uint32_t L = xcd_contiguous(blockIdx.x, gridDim.x);
  int tm, tn;
  grouped_tile(L, NTM, NTN, tm, tn);
  const int m0 = tm * TMB, n0 = tn * TNB;
  const int KS = row_bytes / KSTEP;

  // DMA duty: the step's NA + NB blocks (8 rows of 128 bytes each) are dealt to the waves
  // in order, PER per wave: block i < NA is A rows 8 i .. 8 i + 7, the others W rows. Lane
  // l takes row 8 i + l / 8 (of its operand) and writes LDS position l % 8 of it, holding
  // the line's 16-byte chunk (l % 8) ^ sw(row). voff[j] is that byte offset at K step 0.
  uint32_t voff[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = PER * wv + j;
    const bool is_a = i < NA;
    const int rho = 8 * (is_a ? i : i - NA) + (lane >> 3);
    const int row = is_a ? min(m0 + rho, M - 1) : min(n0 + col_of_wide(rho), N - 1);
    const int chunk = (lane & 7) ^ sw(rho);
    voff[j] = (uint32_t)row * (uint32_t)row_bytes + 16u * (uint32_t)chunk;
  }
  auto issue = [&](int ks) {
    const int st = ks & 1;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = PER * wv + j;  // wave-uniform
      if (i < NA) dma16(A, voff[j] + (uint32_t)(ks * KSTEP), sm.a[st] + i * BLK);
      else dma16(W, voff[j] + (uint32_t)(ks * KSTEP), sm.b[st] + (i - NA) * BLK);
    }
  };
  const int x = sw(c16);
  const int rd0 = c16 * KSTEP + (((2 * g) ^ x) << 4);
  const int rd1 = c16 * KSTEP + (((2 * g + 1) ^ x) << 4);

  v4f acc[RT][CT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int s = 0; s < CT; ++s) acc[t][s] = (v4f){0.f, 0.f, 0.f, 0.f};
  float row_scale[RT][4];
  if (ROW_SCALE) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        row_scale[t][r] = scale_a[min(m0 + 64 * wm + 16 * t + 4 * g + r, M - 1)];
  }

  if (KS > 0) issue(0);
  for (int ks = 0; ks < KS; ++ks) {
    wait_loads<0>();
    lds_barrier();  // every wave's loads of step ks landed; the other slot is free
    if (ks + 1 < KS) issue(ks + 1);
    const uint8_t* sa = sm.a[ks & 1];
    const uint8_t* sb = sm.b[ks & 1];
    v8i aop[RT], bop[CT];
#pragma unroll
    for (int s = 0; s < CT; ++s) {
      const uint4 lo = lds16(sb + (CT * wn + s) * 16 * KSTEP + rd0);
      const uint4 hi = lds16(sb + (CT * wn + s) * 16 * KSTEP + rd1);
      bop[s] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const uint4 lo = lds16(sa + (RT * wm + t) * 16 * KSTEP + rd0);
      const uint4 hi = lds16(sa + (RT * wm + t) * 16 * KSTEP + rd1);
      aop[t] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int s = 0; s < CT; ++s)
        acc[t][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop[t], bop[s], acc[t][s],
                                                                     0, 0, 0, 0, 0, 0);
  }

  const float sw0 = scale_w[0];
  const float tensor_scale = ROW_SCALE ? sw0 : scale_a[2] * sw0;
  const int c0 = n0 + 96 * wn + 4 * c16;       // tiles 0..3: four consecutive columns
  const int c1 = n0 + 96 * wn + 64 + 2 * c16;  // tiles 4, 5: two consecutive columns
  const bool vec0 = (c0 + 3 < N) && ((N & 3) == 0);
  const bool vec1 = (c1 + 1 < N) && ((N & 1) == 0);
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + 64 * wm + 16 * t + 4 * g + r;
      if (row >= M) continue;
      const float scale = ROW_SCALE ? row_scale[t][r] * sw0 : tensor_scale;
      float v[CT];
#pragma unroll
      for (int s = 0; s < CT; ++s) v[s] = acc[t][s][r] * scale;
      const int64_t o0 = (int64_t)row * N + c0, o1 = (int64_t)row * N + c1;
      if (OUT_BF16) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(out);
        if (vec0) {
          *reinterpret_cast<uint2*>(dst + o0) = make_uint2(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]));
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            if (c0 + s < N) dst[o0 + s] = (uint16_t)f32_to_bf16(v[s]);
        }
        if (vec1) {
          *reinterpret_cast<uint32_t*>(dst + o1) = bf16x2(v[4], v[5]);
        } else {
#pragma unroll
          for (int s = 0; s < 2; ++s)
            if (c1 + s < N) dst[o1 + s] = (uint16_t)f32_to_bf16(v[4 + s]);
        }
      } else {
        float* dst = reinterpret_cast<float*>(out);
        if (vec0) {
          *reinterpret_cast<float4*>(dst + o0) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            if (c0 + s < N) dst[o0 + s] = v[s];
        }
        if (vec1) {
          *reinterpret_cast<float2*>(dst + o1) = make_float2(v[4], v[5]);
        } else {
#pragma unroll
          for (int s = 0; s < 2; ++s)
            if (c1 + s < N) dst[o1 + s] = v[4 + s];
        }
      }
    }
}

// Compute units of the current device (queried once per device).
inline int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// BIG tiles (one workgroup per CU) when they give every CU at least two of them; fewer
// would leave CUs idle for a whole round. By shape only: both tilings accumulate every
// output over the same K steps in the same order, so the choice never changes a result.
inline bool use_big_tiles(int64_t M, int64_t N) {
  return ((M + 255) / 256) * ((N + 255) / 256) >= 2 * (int64_t)device_cus();
}

// WIDE tiles (128 x 192) when they fit the two workgroup slots of every CU in one round
// and 128 x 128 tiles would not. By shape only, like BIG: the results are the same.
inline bool use_wide_tiles(int64_t M, int64_t N) {
  const int64_t slots = 2 * (int64_t)device_cus(), mt = (M + 127) / 128;
  return mt * ((N + 191) / 192) <= slots && mt * ((N + 127) / 128) > slots;
}

template <bool OUT_BF16, bool ROW_SCALE>
hipError_t launch_wide(const uint8_t* a, const uint8_t* w, int64_t M, int64_t N, int64_t row_bytes,
                       const float* scale_a, const float* scale_w, void* out, hipStream_t st) {
  const int NTM = (int)((M + 127) / 128), NTN = (int)((N + 191) / 192);
  tn_gemm_wide_kernel<OUT_BF16, ROW_SCALE><<<dim3((uint32_t)(NTM * NTN)), 256, 0, st>>>(
      a, w, (int)M, (int)N, (int)row_bytes, NTM, NTN, scale_a, scale_w, out);
  return hipGetLastError();
}

// Enqueue the kernel over ceil(M/128) x ceil(N/128) tiles (BIG: 256 x 256); row_bytes =
// bytes per row of K.
template <bool IN_BF16, bool OUT_BF16, int STAGES, bool ROW_SCALE = false, bool BLOCK = false,
          bool BIG = false>
hipError_t launch(const uint8_t* a, const uint8_t* w, int64_t M, int64_t N, int64_t row_bytes,
                  const float* scale_a, const float* scale_w, void* out, hipStream_t st) {
  constexpr int T = BIG ? 256 : 128;
  const int NTM = (int)((M + T - 1) / T), NTN = (int)((N + T - 1) / T);
  tn_gemm_kernel<IN_BF16, OUT_BF16, STAGES, ROW_SCALE, BLOCK, BIG>
      <<<dim3((uint32_t)(NTM * NTN)), BIG ? 512 : 256, 0, st>>>(
      a, w, (int)M, (int)N, (int)row_bytes, NTM, NTN, scale_a, scale_w, out);
  return hipGetLastError();
}

}  // namespace tn
}  // namespace fp8moe
