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
// * Workgroup tile 128 rows x 512 accumulator columns, 8 waves side by side along N
//   (each wave: all 128 rows x 64 columns = 8 x 4 MFMA tiles, 128 fp32 accumulators per
//   lane; two waves per SIMD). Per K group the tile stages 16 KB of A and 32 KB of packed
//   B for 16.8 MFLOP (330 FLOP per staged byte): the L2-to-CU stream, not HBM, is what
//   this kernel has to keep fed. A (e4m3 rows, gathered from token order through
//   `sorted` when given), each wave's packed B slice and both scale vectors go straight
//   from global memory into LDS (global_load_lds, no VGPR staging) in three stages, two
//   groups in flight, one barrier per group. Each wave stages exactly the 16 A rows whose
//   sums it computes, so the seeds of group g+1 are formed as soon as the wave's own loads
//   land, before the group's single barrier.
// * One launch covers all experts: the grid is the host-known bound ceil(R/128) + E
//   m-tiles times the n-tiles; each workgroup finds its (expert, m-tile) from the device
//   offsets (a workgroup-wide scan over E) and exits if surplus.
// * Epilogues: STORE writes fp32 or bf16; SWIGLU_QUANT pairs gate columns n and up
//   columns I+n in the same wave, forms h = silu(gate) * up in fp32, takes the per-row
//   amax over the workgroup's 128 h columns (= one 128-group of the down GEMM's K) and
//   writes e4m3 codes plus fp32 scales, so h never goes to HBM in fp32 or bf16.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace fp8moe {
namespace {

constexpr int BM = 128;        // rows per workgroup tile
constexpr int NW = 8;          // waves per workgroup
constexpr int NT_THREADS = NW * 64;
constexpr int WCOLS = 64;      // accumulator columns per wave
constexpr int WCOLS_WG = NW * WCOLS;           // 512 accumulator columns per workgroup
constexpr int BW_BYTES = WCOLS * kGroup / 2;   // packed B slice of one wave, one group
constexpr float kWeightScaleMul = 512.f;       // 2^9: B codes are (q + 8) * 2^-9
constexpr uint32_t kOnes = 0x38383838u;        // four e4m3 1.0

// One pipeline stage in LDS: the A tile, the waves' packed B slices, the A scales of the
// 128 rows, the weight scales of the 512 columns, and the row-sum seeds of its group.
// The three stages are distinct __shared__ objects and every access names its stage at
// compile time, so the compiler can tell that the direct-to-LDS loads filling one stage
// never alias the reads of another and does not make those reads wait for the loads.
struct __attribute__((aligned(16))) Stage {
  uint8_t a[BM * kGroup];
  uint8_t b[NW * BW_BYTES];
  float as[BM];
  float ws[WCOLS_WG];
  float ra[BM];
};

// Inclusive scan of one int per thread over the workgroup (NT_THREADS threads).
__device__ __forceinline__ int block_inclusive_scan(int v, int* tmp /*[NW]*/) {
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

// global -> LDS without VGPR staging: lane i of the wave copies `size` bytes from
// base + voff (base wave-uniform, voff per lane) to LDS byte address lds + size * i (lds
// wave-uniform, passed in M0). Issued as inline assembly so that the compiler does not
// track these loads: it would otherwise make LDS reads of the stage being computed wait
// for every load in flight (vmcnt(0)), which serialises the pipeline. The kernel waits
// for them itself, by count, and a workgroup barrier then publishes them. The s_nop is
// the wait state the hardware needs between the write of M0 and the LDS DMA.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, const void* lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "{m0}"(lds_addr(lds)) : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, const void* lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(base), "{m0}"(lds_addr(lds)) : "memory");
}

// bitop3 truth table of (a ^ b) & c, with a, b, c in the 0xF0 / 0xCC / 0xAA positions
constexpr int kXorAnd = (0xF0 ^ 0xCC) & 0xAA;

// 16 packed bytes (32 int4, K-interleaved words) -> MFMA B operand of (q + 8) * 2^-9.
__device__ __forceinline__ v8i convert_b(uint4 p) {
  v8i b;
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // low nibbles: (w ^ 0x88888888) & 0x0F0F0F0F; high nibbles: same on w >> 4
    b[2 * j] = (int)__builtin_amdgcn_bitop3_b32(w[j], 0x08080808u, 0x0F0F0F0Fu, kXorAnd);
    b[2 * j + 1] = (int)__builtin_amdgcn_bitop3_b32(w[j] >> 4, 0x08080808u, 0x0F0F0F0Fu, kXorAnd);
  }
  return b;
}

// LDS A tile: [BM rows][8 chunks of 16 B]. Chunk c of row r is stored at position
// c ^ (r & 7) ^ ((r >> 3) & 1): the 16 rows that one ds_read_b128 touches (same c) then land
// on 16 distinct 16-byte bank groups whether the LDS serves 8 or 16 lanes per cycle.
__device__ __forceinline__ int a_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int a_off(int r, int c) { return r * 128 + ((c ^ a_swz(r)) << 4); }

__device__ __forceinline__ v8i lds_a_operand(const uint8_t* tile, int r, int q) {
  uint4 lo = *reinterpret_cast<const uint4*>(&tile[a_off(r, 2 * q)]);
  uint4 hi = *reinterpret_cast<const uint4*>(&tile[a_off(r, 2 * q + 1)]);
  return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
               (int)hi.w};
}

__device__ __forceinline__ float dpp_xor1(float v) {  // value of lane ^ 1 (quad_perm 1,0,3,2)
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {  // value of lane ^ 2 (quad_perm 2,3,0,1)
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_ror4(float v) {  // row_ror:4 within 16 lanes
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_ror8(float v) {  // row_ror:8 within 16 lanes
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

// m[0..3]: this lane's values of rows 0..3. Returns, in lane c of each 16-lane row, the max
// over those 16 lanes of row 2 * (c & 1) + ((c >> 1) & 1). Five DPP steps instead of sixteen.
__device__ __forceinline__ float row4_max16(const float m[4], int c16) {
  // lane bit 0 picks rows {0,1} (even lanes) or {2,3} (odd lanes)
  const bool odd = c16 & 1;
  float keep0 = odd ? m[2] : m[0], keep1 = odd ? m[3] : m[1];
  float give0 = odd ? m[0] : m[2], give1 = odd ? m[1] : m[3];
  keep0 = fmaxf(keep0, dpp_xor1(give0));
  keep1 = fmaxf(keep1, dpp_xor1(give1));
  // lane bit 1 picks one of the two remaining rows
  const bool b1 = c16 & 2;
  float keep = b1 ? keep1 : keep0, give = b1 ? keep0 : keep1;
  keep = fmaxf(keep, dpp_xor2(give));
  // lanes c, c ^ 4, c ^ 8, c ^ 12 now hold the same row: combine them
  keep = fmaxf(keep, dpp_ror4(keep));
  keep = fmaxf(keep, dpp_ror8(keep));
  return keep;
}

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt
// [11:8])
constexpr int kWaitAll = 0;
constexpr int kWaitVm8 = 8 | (7 << 4) | (0xF << 8);      // vmcnt <= 8, nothing else
constexpr int kWaitLgkm0 = 0xF | (7 << 4) | (3 << 14);   // lgkmcnt == 0, nothing else

// Workgroup barrier without the release fence of __syncthreads(): that fence waits for
// every outstanding global load, including the direct-to-LDS loads of the groups still in
// flight. LDS writes of this wave are drained first (they are the only writes other waves
// read after the barrier); the direct-to-LDS loads are waited for explicitly by count.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
}

template <int EPI, bool OUT_BF16>
__global__ __launch_bounds__(NT_THREADS, 1) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As,
    const int32_t* __restrict__ sorted, int k_route, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, const int32_t* __restrict__ offsets, int E, int N, int K,
    int NT, void* __restrict__ out, float* __restrict__ out_scales) {
  __shared__ Stage st0, st1, st2;
  __shared__ int s_tmp[NW];
  __shared__ int s_tile[3];
  __shared__ int s_total;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in an SGPR
  const int q = lane >> 4, c16 = lane & 15;
  const int G = K / kGroup;
  const int kshift = (k_route & (k_route - 1)) == 0 ? __builtin_ctz(k_route) : -1;
  const uint32_t L = xcd_contiguous(blockIdx.x, gridDim.x);
  const int mt = (int)(L / (uint32_t)NT), nt = (int)(L % (uint32_t)NT);

  // ---- which expert and which 128-row slice of it this workgroup owns
  {
    int loc[2], sum = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int e = tid * 2 + j;
      int c = e < E ? offsets[e + 1] - offsets[e] : 0;
      loc[j] = (c + BM - 1) / BM;
      sum += loc[j];
    }
    int inc = block_inclusive_scan(sum, s_tmp);
    int run = inc - sum;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (mt >= run && mt < run + loc[j]) {
        int e = tid * 2 + j;
        int rb = offsets[e] + (mt - run) * BM;
        s_tile[0] = e;
        s_tile[1] = rb;
        s_tile[2] = min(BM, offsets[e + 1] - rb);
      }
      run += loc[j];
    }
    if (tid == NT_THREADS - 1) s_total = inc;
    __syncthreads();
  }
  if (mt >= s_total) return;  // surplus workgroup (uniform)
  const int e = __builtin_amdgcn_readfirstlane(s_tile[0]);
  const int row_begin = __builtin_amdgcn_readfirstlane(s_tile[1]);
  const int rows = __builtin_amdgcn_readfirstlane(s_tile[2]);

  // ---- sources: wave-uniform bases (advanced per group in scalar registers) plus
  // per-lane 32-bit byte offsets. Wave wv stages rows 16wv .. 16wv+15 of every A tile (the
  // rows whose sums it also computes, so it needs nobody else's loads for that): chunk
  // p = (2wv+j)*64 + lane of the swizzled tile for j = 0, 1.
  auto src_row = [&](int r) {
    const int grow = row_begin + min(r, rows - 1);
    if (!sorted) return grow;
    const int p = sorted[grow];
    if (kshift >= 0) return p >> kshift;  // uniform branch: no division for 2^n experts/token
    return p / k_route;
  };
  uint32_t a_off32[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = (wv * 2 + j) * 64 + lane;
    const int r = p >> 3, c = (p & 7) ^ a_swz(r);
    a_off32[j] = (uint32_t)src_row(r) * (uint32_t)K + (uint32_t)(c * 16);
  }
  // A scale of row 16wv + lane (lanes 0..15; rows past the tile read a valid row and are
  // never stored)
  const uint32_t as_off32 = (uint32_t)src_row(wv * 16 + (lane & 15)) * (uint32_t)G * 4u;
  // accumulator column j (0..511) of the workgroup -> bank column. SwiGLU: the workgroup
  // covers two 128-wide h groups (j >> 8); in each, wave (j >> 6) & 3 holds gate columns
  // for (j >> 5) & 1 == 0 and the matching up columns (I + ...) for (j >> 5) & 1 == 1.
  const int I = N / 2;
  auto bank_col = [&](int j) {
    if (EPI == FP8MOE_EPI_SWIGLU_QUANT)
      return min(((j >> 5) & 1 ? I : 0) + nt * 256 + (j >> 8) * 128 + ((j >> 6) & 3) * 32 +
                     (j & 31),
                 N - 1);
    return min(nt * WCOLS_WG + j, N - 1);
  };
  const uint8_t* const Wexp = W + (int64_t)e * N * (K / 2);
  const float* const Wsexp = Ws + (int64_t)e * N * G;
  const uint32_t ws_off32 = (uint32_t)bank_col(wv * WCOLS + lane) * (uint32_t)G * 4u;
  uint32_t b_off32[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    b_off32[s] = (uint32_t)bank_col(wv * WCOLS + 16 * s + c16) * (uint32_t)(K / 2) +
                 (uint32_t)(q * 16);

  // 8 loads per wave per group (the counted waits below rely on that number)
  auto load_group = [&](int g, Stage& st) {
    const uint8_t* ag = A + g * kGroup;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(ag, a_off32[j], st.a + (wv * 2 + j) * 1024);
    const uint8_t* bg = Wexp + g * (kGroup / 2);
    uint8_t* sb = st.b + wv * BW_BYTES;
#pragma unroll
    for (int s = 0; s < 4; ++s) dma16(bg, b_off32[s], sb + s * 1024);
    dma4(Wsexp + g, ws_off32, st.ws + wv * WCOLS);
    if (lane < 16) dma4(As + g, as_off32, st.as + wv * 16);
  };

  // sum of this wave's 16-row tile of the A tile of stage st -> st.ra as -sum/64, the
  // accumulator seed that removes the +8 offset of the B codes
  const v8i ones = {(int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes,
                    (int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  auto row_sums = [&](Stage& st) {
    v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lds_a_operand(st.a, wv * 16 + c16, q),
                                                              ones, zero, 0, 0, 0, 0, 0, 0);
    if (c16 == 0)
      *reinterpret_cast<float4*>(&st.ra[wv * 16 + 4 * q]) =
          make_float4(pr[0] * -0.015625f, pr[1] * -0.015625f, pr[2] * -0.015625f,
                      pr[3] * -0.015625f);
  };

  float acc[8][4][4];

  // ---- prologue: groups 0 and 1 in flight, the seeds of group 0 formed
  load_group(0, st0);
  if (G > 1) load_group(1, st1);
  if (G > 1)  // own group-0 loads landed (group 1's may still be in flight)
    __builtin_amdgcn_s_waitcnt(kWaitVm8);
  else
    __builtin_amdgcn_s_waitcnt(kWaitAll);
  row_sums(st0);
  lds_barrier();

  // ---- one K group. Three stages: group g is computed while g+1 and g+2 stream into LDS.
  // The group is 32 steps; step i = 4t + s issues the MFMA of tile (t, s) and folds the
  // MFMA of step i-2 (already complete), so the matrix core and the VALU work side by
  // side; a sched_barrier after every step pins that interleaving. The first group
  // initialises the accumulators (no separate zeroing).
  auto group = [&](int g, auto first_tag, Stage& cur, Stage& nx1, Stage& nx2) {
    constexpr bool FIRST = decltype(first_tag)::value;
    const bool has2 = g + 2 < G;
    if (has2) load_group(g + 2, nx2);
    const uint8_t* ta = cur.a;
    const uint8_t* tb = cur.b + wv * BW_BYTES;
    const float* ra = cur.ra;
    const float* sag = cur.as;
    const float* swg = cur.ws + wv * WCOLS;
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
      if (FIRST) {
        acc[t][s][0] = p[0] * (a4.x * sw[s]);
        acc[t][s][1] = p[1] * (a4.y * sw[s]);
        acc[t][s][2] = p[2] * (a4.z * sw[s]);
        acc[t][s][3] = p[3] * (a4.w * sw[s]);
      } else {
        acc[t][s][0] = fmaf(p[0], a4.x * sw[s], acc[t][s][0]);
        acc[t][s][1] = fmaf(p[1], a4.y * sw[s], acc[t][s][1]);
        acc[t][s][2] = fmaf(p[2], a4.z * sw[s], acc[t][s][2]);
        acc[t][s][3] = fmaf(p[3], a4.w * sw[s], acc[t][s][3]);
      }
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
    // own loads of group g+1 landed (group g+2's may still be in flight)
    if (has2)
      __builtin_amdgcn_s_waitcnt(kWaitVm8);
    else
      __builtin_amdgcn_s_waitcnt(kWaitAll);
    if (g + 1 < G) row_sums(nx1);
    lds_barrier();
  };

  // group g uses stage g % 3 (named statically, see Stage)
  group(0, std::true_type{}, st0, st1, st2);
  for (int g = 1; g < G; g += 3) {
    group(g, std::false_type{}, st1, st2, st0);
    if (g + 1 < G) group(g + 1, std::false_type{}, st2, st0, st1);
    if (g + 2 < G) group(g + 2, std::false_type{}, st0, st1, st2);
  }

  // ---- epilogues. Output element (t, s, r) of this lane: row t*16 + 4q + r, workgroup
  // column wv*64 + s*16 + c16.
  if (EPI == FP8MOE_EPI_STORE && OUT_BF16) {
    // stage the bf16 tile in LDS 32 rows at a time (32 KB), then write whole 1 KB row
    // segments
    uint16_t* s_out = reinterpret_cast<uint16_t*>(st0.b);
    const int ncols = min(WCOLS_WG, N - nt * WCOLS_WG);  // multiple of 16
    uint16_t* o16 = reinterpret_cast<uint16_t*>(out);
#pragma unroll
    for (int part = 0; part < 4; ++part) {
#pragma unroll
      for (int t = 2 * part; t < 2 * part + 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int s = 0; s < 4; s += 2) {
            const uint32_t pk = bf16x2(acc[t][s][r], acc[t][s + 1][r]);
            uint16_t* o = &s_out[((t - 2 * part) * 16 + 4 * q + r) * WCOLS_WG + wv * WCOLS +
                                 s * 16 + c16];
            o[0] = (uint16_t)(pk & 0xFFFFu);
            o[16] = (uint16_t)(pk >> 16);
          }
      __syncthreads();
      for (int i = tid; i < 32 * (WCOLS_WG / 8); i += NT_THREADS) {
        const int rl = i >> 6, ch = i & 63, row = 32 * part + rl;
        if (row < rows && ch * 8 < ncols)
          *reinterpret_cast<uint4*>(&o16[(int64_t)(row_begin + row) * N + nt * WCOLS_WG + ch * 8]) =
              *reinterpret_cast<const uint4*>(&s_out[rl * WCOLS_WG + ch * 8]);
      }
      __syncthreads();
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
    // SwiGLU + e4m3 per (row, 128 h columns). Wave wv works on h group hg = wv >> 2 of the
    // workgroup; its h column of (t, s', r) is (wv & 3)*32 + s'*16 + c16 within the group.
    const int hg = wv >> 2;
    float* s_amax = reinterpret_cast<float*>(st0.a);       // [8 waves][BM]
    float* s_inv = s_amax + NW * BM;                        // [2 h groups][BM]
    uint8_t* s_codes = st0.b;                               // [2][BM][128]
    float h[8][2][4];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float m[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        m[r] = 0.f;
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          float gt = acc[t][sp][r], up = acc[t][sp + 2][r];
          float hv = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * up;
          h[t][sp][r] = hv;
          m[r] = fmaxf(m[r], fabsf(hv));
        }
      }
      // max of rows r = 0..3 over the 16 lanes of this row group (transposing butterfly)
      const float mr = row4_max16(m, c16);
      if (c16 < 4) s_amax[wv * BM + t * 16 + 4 * q + 2 * (c16 & 1) + ((c16 >> 1) & 1)] = mr;
    }
    __syncthreads();
    if (tid < 2 * BM) {
      const int g2 = tid >> 7, row = tid & (BM - 1);
      const float* am = s_amax + g2 * 4 * BM + row;
      float m = fmaxf(fmaxf(am[0], am[BM]), fmaxf(am[2 * BM], am[3 * BM]));
      float sc, inv;
      scale_pair(m, sc, inv);
      s_inv[tid] = inv;
      const int hcol = nt * 256 + g2 * 128;
      if (row < rows && hcol < I)
        out_scales[(int64_t)(row_begin + row) * (I / kGroup) + hcol / kGroup] = sc;
    }
    __syncthreads();
    const float* inv_g = s_inv + hg * BM;
    uint8_t* codes_g = s_codes + hg * BM * 128;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = t * 16 + 4 * q + r;
        const float inv = inv_g[row];
        uint32_t c2 = e4m3x2_finite(h[t][0][r] * inv, h[t][1][r] * inv);
        codes_g[row * 128 + (wv & 3) * 32 + c16] = (uint8_t)(c2 & 0xFF);
        codes_g[row * 128 + (wv & 3) * 32 + 16 + c16] = (uint8_t)((c2 >> 8) & 0xFF);
      }
    __syncthreads();
    uint8_t* o8 = reinterpret_cast<uint8_t*>(out);
    for (int i = tid; i < 2 * BM * 8; i += NT_THREADS) {
      const int g2 = i >> 10, row = (i >> 3) & (BM - 1), ch = i & 7;
      const int hcol = nt * 256 + g2 * 128;
      if (row < rows && hcol < I)
        *reinterpret_cast<uint4*>(&o8[(int64_t)(row_begin + row) * I + hcol + ch * 16]) =
            *reinterpret_cast<const uint4*>(&s_codes[(g2 * BM + row) * 128 + ch * 16]);
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
  // SwiGLU: a tile covers 256 h columns (gate and up); otherwise 512 output columns
  const int NT = epilogue == FP8MOE_EPI_SWIGLU_QUANT ? (int)((N / 2 + 255) / 256)
                                                     : (int)((N + WCOLS_WG - 1) / WCOLS_WG);
  const int64_t blocks = mtiles * NT;
  dim3 grid((uint32_t)blocks), block(NT_THREADS);
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
