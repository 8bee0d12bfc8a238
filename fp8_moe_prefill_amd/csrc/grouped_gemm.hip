// Grouped FP8 expert GEMM over a resident packed-int4 bank (fp8_grouped_expert_gemm).
//
// Method ("FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant", section 1):
// one GEMM launch covers every expert of the layer; the int4 weights stay packed in
// memory and are turned into e4m3 on-chip; the per-(token, group) activation scale and the
// per-group weight scale are folded into the fp32 accumulator:
//
//   y[i, n] = sum_g  s_a[g, i] * s_w[e, g, n] * sum_{k in g} e4m3(a[i, k]) * q[e, n, k]
//
// gfx950 design:
// * The MFMA is v_mfma_f32_16x16x128_f8f6f4: its K of 128 is exactly one scale group, so
//   each group is one MFMA per 16x16 output tile, followed by the fold
//   acc += P * (s_a * s_w) (two VALU ops per output per group). On gfx950 an FP8 MFMA of
//   this shape occupies most of the VALU issue slots of its own 32 cycles, so VALU, not the
//   matrix core, is the scarce unit: every VALU op in the loop other than the fold is kept
//   to a minimum.
// * Nibble -> e4m3 in two ops per four weights: e4m3 codes 0x00..0x0F are exactly
//   u * 2^-9 (the subnormals and the first normal binade share the spacing 2^-9), so the
//   offset nibble u = n ^ 8 = q + 8 (q the int4 value) IS the e4m3 code of (q + 8) * 2^-9.
//   The +8 is removed inside the MFMA: its accumulator input is seeded with
//   -8 * 2^-9 * sum_k a_k for that row and group. That row sum is given (the quantiser,
//   or a previous SwiGLU epilogue, emits it beside the codes), or else formed here as one
//   MFMA of the A tile against a constant all-ones operand (one extra MFMA per 16 rows per
//   group). The 2^9 is folded into the weight scale (exact). The prepacked bank stores the
//   nibbles of a 32-bit word so that its low nibbles are four consecutive k and its high
//   nibbles the next four: a byte split gives K-ordered e4m3 bytes with no permutes.
// * Tile 128 rows x 256 accumulator columns per workgroup, 4 waves side by side along N
//   (each wave: all 128 rows x 64 columns = 8 x 4 MFMA tiles, 128 fp32 accumulators per
//   lane), two workgroups per CU (two waves per SIMD, one from each). Per K group a tile
//   stages 16 KB of A and 16 KB of packed B for 8.4 MFLOP. A (e4m3 rows, gathered from token order through `sorted` when given),
//   each wave's packed B slice (one contiguous 1 KB block per 16 columns in the prepacked
//   bank) and both scale vectors (the activation scales per row: by token when the rows
//   are gathered, else contiguous per group in the group-major layout) go
//   straight from global memory into LDS (LDS DMA, no VGPR staging) through two stages:
//   the next group streams in while the current one is computed, one barrier per group.
// * Persistent: the grid is two workgroups per CU and each walks its list of
//   (expert, 128-row, 256-column) tiles as one continuous stream of K groups, so the first
//   loads of a tile overlap the previous tile's tail, and no workgroup pays a cold start
//   per tile. The two workgroups of a CU are independent: one's barrier waits, memory
//   waits and epilogue are covered by the other's MFMA work. Tiles are dealt in contiguous ranges per XCD
//   (each XCD has its own L2), so the m-tiles of one expert, which share B, and the
//   n-tiles of one m-tile, which share A, run on the same L2. Row tiles past the end of an
//   expert's last, partial m-tile are skipped.
// * The expert of each tile comes from the device offsets (a workgroup-wide scan of the
//   per-expert m-tile counts, then a binary search), so one launch covers all experts with
//   no host round trip.
// * Epilogues: STORE writes fp32 or bf16; SWIGLU_QUANT pairs gate columns n and up columns
//   I+n in the same wave, forms h = silu(gate) * up in fp32, takes the per-row amax over the
//   tile's 128 h columns (= one 128-group of the down GEMM's K) and writes e4m3 codes plus
//   fp32 scales, so h never goes to HBM in fp32 or bf16.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "lds_dma.h"

namespace fp8moe {
namespace {

constexpr int BM = 128;        // rows per tile
constexpr int NW = 4;          // waves per workgroup (two workgroups per CU)
constexpr int NT_THREADS = NW * 64;
constexpr int RPW = BM / NW;   // A rows each wave stages (and sums)
constexpr int WCOLS = 64;      // accumulator columns per wave
constexpr int WCOLS_WG = NW * WCOLS;           // 256 accumulator columns per workgroup
constexpr int BW_BYTES = WCOLS * kGroup / 2;   // packed B slice of one wave, one group
constexpr int kBlockBytes = 16 * kGroup / 2;   // prepacked bank block: 16 columns, one group
constexpr float kWeightScaleMul = 512.f;       // 2^9: B codes are (q + 8) * 2^-9
constexpr uint32_t kOnes = 0x38383838u;        // four e4m3 1.0
constexpr int kMaxExperts = 1024;
constexpr int kListedUnits = 64;  // tiles per workgroup looked up once, at the start

// One pipeline stage in LDS: the A tile, the waves' packed B slices, the A scales of the
// 128 rows, the weight scales of the 512 columns, and the row-sum seeds of its group.
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

// Read-only data read with a wave-uniform address through the scalar unit (SMEM): the
// value lands in an SGPR and is waited for with lgkmcnt, never with vmcnt, so it does not
// interact with the counted waits of the LDS DMA pipeline.
__device__ __forceinline__ int sload(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// bitop3 truth table of (a ^ b) & c, with a, b, c in the 0xF0 / 0xCC / 0xAA positions
constexpr int kXorAnd = (0xF0 ^ 0xCC) & 0xAA;

// 16 prepacked bytes (32 int4) -> MFMA B operand of (q + 8) * 2^-9.
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

// FP4 (MXFP4) A tile: 64 bytes per row and group, two rows per 128-byte line (line
// L = r / 2 holds chunks c' = 4 (r % 2) + c, c = 0..3 the 16-byte chunks of row r), chunk
// c' of line L at position c' ^ ((L / 2) % 4): the 16 rows one ds_read_b128 touches (same
// c) then sit in 16 distinct 16-byte bank groups. Lane (q, row) of the MFMA reads chunk q
// of its row: the 32 E2M1 values of block q (K = 32 q .. 32 q + 31 of the group).
__device__ __forceinline__ int a4_pos(int L, int cc) { return cc ^ ((L >> 1) & 3); }
__device__ __forceinline__ v8i lds_a4_operand(const uint8_t* tile, int r, int q) {
  const int L = r >> 1;
  const uint4 v = *reinterpret_cast<const uint4*>(&tile[L * 128 + (a4_pos(L, 4 * (r & 1) + q) << 4)]);
  return (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
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

// Tile (expert, first grouped row, valid rows, n-tile) of a logical tile.
struct TileDesc {
  int e, row_begin, rows, nt;
};

// AF4: the activations are MXFP4 (E2M1 codes, two per byte, with one E8M0 scale per 32
// consecutive K, four per row and group as one 32-bit word in As), and the bank is packed
// in the matching K order (pack_bank with the FP4 layout). The MFMA applies the
// activation scales itself, so the fold is one FMA by the weight scale.
//
// As and Asum: per token, row-major [a_rows, G], when the rows are gathered through
// `sorted`; otherwise group-major [G, R] in grouped row order.
// SUMS: the per-(row, K group) sums of the decoded A codes come in Asum (laid out like As)
// and seed the accumulators directly; otherwise the kernel forms them on the matrix core
// from the staged tile.
template <int EPI, bool OUT_BF16, bool AF4, bool SUMS>
__global__ __launch_bounds__(NT_THREADS, 2) void grouped_gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const float* __restrict__ Asum,
    const int32_t* __restrict__ sorted, int k_route, int a_rows, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, const int32_t* __restrict__ offsets, int R, int E, int N,
    int K, int NT, void* __restrict__ out, float* __restrict__ out_scales,
    float* __restrict__ out_sums) {
  __shared__ Stage ring[2];
  __shared__ int s_mstart[kMaxExperts + 1];  // m-tiles before expert e
  __shared__ int s_tmp[NW];
  __shared__ int s_part[kMaxExperts];  // experts with a small (front) or tiny (back) last m-tile
  __shared__ int s_npart;              // tiny count << 11 | small count
  __shared__ int s_src[NW][RPW];  // pair ids of the rows each wave stages for the next tile
  __shared__ int4 s_units[kListedUnits];  // this workgroup's first tiles: (e, row_begin, rows, nt)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in an SGPR
  const int q = lane >> 4, c16 = lane & 15;
  const int G = K / kGroup;
  const int I = N / 2;
  const int NB = N / 16;  // 16-column blocks of the bank
  const int kshift = (k_route & (k_route - 1)) == 0 ? __builtin_ctz(k_route) : -1;

  // ---- m-tiles per expert. An expert's rows split into 128-row m-tiles. Its last m-tile
  // is "small" when it has at most 64 rows (it runs 4 of the 8 row tiles) and "tiny" with
  // at most 16 (1 row tile); the others are "whole". s_mstart[e] = whole m-tiles before
  // expert e; s_part lists the experts with a small last m-tile from the front (entry i =
  // the i-th such expert) and those with a tiny one from the back (entry 1023 - i), at
  // most one per expert, so 1024 entries hold both. 4 experts per thread, E <= 1024.
  {
    constexpr int EPT = kMaxExperts / NT_THREADS;
    int nwh[EPT], cls[EPT], sum_w = 0, sum_p = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid * EPT + j;
      const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
      const int rem = c % BM;
      cls[j] = rem == 0 ? 0 : rem <= 16 ? 2048 : rem <= BM / 2 ? 1 : 0;  // tiny << 11 | small
      nwh[j] = c / BM + (rem > BM / 2 ? 1 : 0);
      sum_w += nwh[j];
      sum_p += cls[j];
    }
    int run_w = block_inclusive_scan(sum_w, s_tmp) - sum_w;
    int run_p = block_inclusive_scan(sum_p, s_tmp) - sum_p;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid * EPT + j;
      if (e < E && cls[j] == 1) s_part[run_p & 2047] = e;
      if (e < E && cls[j] == 2048) s_part[kMaxExperts - 1 - (run_p >> 11)] = e;
      run_w += nwh[j];
      run_p += cls[j];
      if (e < E) s_mstart[e + 1] = run_w;
      if (e == E - 1) s_npart = run_p;
    }
    if (tid == 0) s_mstart[0] = 0;
    __syncthreads();
  }

  // ---- this workgroup's work units. Tiles are (m-tile, n-tile) pairs, n-tile fastest.
  // Whole, small and tiny tiles are dealt separately so that every XCD gets an even share
  // of each: XCD x (workgroups x, x + nx, ...) owns a contiguous range of each class,
  // lists them whole first, then small, then tiny, and its workgroups take every
  // nwg_x-th entry of that list. (The launcher keeps the tile count below 2^28, so 32-bit
  // tile indices do not overflow.)
  const int npart = __builtin_amdgcn_readfirstlane(s_npart);
  const int n_whole = __builtin_amdgcn_readfirstlane(s_mstart[E]) * NT;
  const int n_small = (npart & 2047) * NT, n_tiny = (npart >> 11) * NT;
  const int nx = min(8, (int)gridDim.x);
  const int x = (int)blockIdx.x % nx, u = (int)blockIdx.x / nx;
  const int nwg_x = ((int)gridDim.x - x + nx - 1) / nx;
  const int wb_x = n_whole * x / nx, nw_x = n_whole * (x + 1) / nx - wb_x;
  const int sb_x = n_small * x / nx, ns_x = n_small * (x + 1) / nx - sb_x;
  const int tb_x = n_tiny * x / nx, nt_x = n_tiny * (x + 1) / nx - tb_x;

  // j-th unit of this workgroup: entry u + j * nwg_x. Wave-uniform scalar walk (a binary
  // search over the m-tile starts, scalar loads of the offsets); tile_of below serves the
  // first kListedUnits units from the list formed once at the start.
  auto tile_walk = [&](int j) {
    const int l = u + j * nwg_x;
    TileDesc d;
    if (l < nw_x) {
      const int L = wb_x + l, mt = L / NT;
      d.nt = L - mt * NT;
      int lo = 0, hi = E;  // s_mstart[lo] <= mt < s_mstart[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (__builtin_amdgcn_readfirstlane(s_mstart[mid]) <= mt) lo = mid;
        else hi = mid;
      }
      d.e = lo;
      d.row_begin =
          sload(offsets + lo) + (mt - __builtin_amdgcn_readfirstlane(s_mstart[lo])) * BM;
    } else {
      const bool small = l < nw_x + ns_x;
      const int L = small ? sb_x + (l - nw_x) : tb_x + (l - nw_x - ns_x), i = L / NT;
      d.nt = L - i * NT;
      d.e = __builtin_amdgcn_readfirstlane(s_part[small ? i : kMaxExperts - 1 - i]);
      d.row_begin = sload(offsets + d.e) +
                    (__builtin_amdgcn_readfirstlane(s_mstart[d.e + 1]) -
                     __builtin_amdgcn_readfirstlane(s_mstart[d.e])) * BM;
    }
    d.rows = min(BM, sload(offsets + d.e + 1) - d.row_begin);
    return d;
  };
  // The same lookup for unit j = tid, one per lane, all lanes at once (vector loads), into
  // s_units: the per-tile walk above costs a chain of dependent LDS and scalar-memory
  // round trips at every tile boundary.
  {
    const int j = tid;
    const int l = u + j * nwg_x;
    if (j < kListedUnits && l < nw_x + ns_x + nt_x) {
      int e, row_begin, nt;
      if (l < nw_x) {
        const int L = wb_x + l, mt = L / NT;
        nt = L - mt * NT;
        int lo = 0, hi = E;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_mstart[mid] <= mt) lo = mid;
          else hi = mid;
        }
        e = lo;
        row_begin = offsets[lo] + (mt - s_mstart[lo]) * BM;
      } else {
        const bool small = l < nw_x + ns_x;
        const int L = small ? sb_x + (l - nw_x) : tb_x + (l - nw_x - ns_x), i = L / NT;
        nt = L - i * NT;
        e = s_part[small ? i : kMaxExperts - 1 - i];
        row_begin = offsets[e] + (s_mstart[e + 1] - s_mstart[e]) * BM;
      }
      s_units[j] = make_int4(e, row_begin, min(BM, offsets[e + 1] - row_begin), nt);
    }
    __syncthreads();
  }
  auto tile_of = [&](int j) {
    if (j >= kListedUnits) return tile_walk(j);  // uniform
    const int4 v = s_units[j];
    TileDesc d;
    d.e = __builtin_amdgcn_readfirstlane(v.x);
    d.row_begin = __builtin_amdgcn_readfirstlane(v.y);
    d.rows = __builtin_amdgcn_readfirstlane(v.z);
    d.nt = __builtin_amdgcn_readfirstlane(v.w);
    return d;
  };
  // units [0, j_small) are whole, [j_small, j_tiny) small, [j_tiny, my_tiles) tiny
  auto units_below = [&](int n) { return n > u ? (n - u + nwg_x - 1) / nwg_x : 0; };
  const int j_small = units_below(nw_x), j_tiny = units_below(nw_x + ns_x);
  const int my_tiles = units_below(nw_x + ns_x + nt_x);
  if (my_tiles == 0) return;  // uniform
  const int total_steps = my_tiles * G;

  // Columns. In the prepacked bank, block b of 16 columns holds bank columns
  // 64*(b/4) + 4*i + b%4 (i = 0..15), so MFMA tile s of a wave reading block 4k + s gives
  // lane c16 bank column 64k + 4*c16 + s: each lane ends up with 4 consecutive columns.
  // STORE: wave wv of n-tile nt covers the 64 columns 64k.., k = 4nt + wv.
  // SWIGLU: the tile covers h columns 128nt..128nt+127; wave wv covers the 64-column h
  // group k = 2nt + (wv >> 1), pairs 2*(wv & 1) + {0, 1} of every 4: tiles 0, 1 read gate
  // blocks 4k + 2*(wv & 1) + {0, 1}, tiles 2, 3 the matching up blocks (I/64 groups on),
  // so lane c16 holds gate and up of h columns 64k + 4*c16 + 2*(wv & 1) + {0, 1}.
  const int NG = N / 64;  // 64-column groups of the bank
  auto tile_block = [&](int nt, int s) {  // bank block of MFMA tile s of this wave
    int b;
    if (EPI == FP8MOE_EPI_SWIGLU_QUANT)
      b = 4 * (2 * nt + (wv >> 1) + (s >= 2 ? I / 64 : 0)) + 2 * (wv & 1) + (s & 1);
    else
      b = 4 * (4 * nt + wv) + s;
    return min(b, 4 * NG - 1);
  };
  auto ws_col = [&](int nt, int l) {  // weight-scale column staged by lane l of this wave
    int c;
    if (EPI == FP8MOE_EPI_SWIGLU_QUANT)
      c = (l >= 32 ? I : 0) + 64 * (2 * nt + (wv >> 1)) + 4 * ((l & 31) >> 1) + 2 * (wv & 1) +
          (l & 1);
    else
      c = 64 * (4 * nt + wv) + l;
    return min(c, N - 1);
  };

  // ---- DMA stream state: the tile whose groups are being loaded, and the next one (its
  // descriptor, and the pair ids of its rows brought into LDS by the wave's own loads one
  // group ahead, older than that group's loads, so the group's counted wait covers them)
  TileDesc pend = tile_of(0);
  auto fetch_rows = [&](const TileDesc& d) {
    if (sorted && lane < RPW)
      dma4(sorted, (uint32_t)max(min(d.row_begin + min(wv * RPW + lane, d.rows - 1), R - 1), 0) * 4u,
           &s_src[wv][0]);
  };
  fetch_rows(pend);
  wait_all_loads();

  constexpr int A_DMA = AF4 ? RPW / 16 : RPW / 8;  // A tile DMA instructions per wave
  const int a_row_bytes = AF4 ? K / 2 : K;
  uint32_t a_off32[A_DMA] = {}, as_off32 = 0, ws_off32 = 0;
  uint32_t b_blk[4] = {0, 0, 0, 0};  // byte offset of this wave's 4 column blocks in its expert
  const uint8_t* w_exp = W;
  const float* ws_exp = Ws;
  const uint32_t lane16 = (uint32_t)lane * 16u;

  // The loads of one K group are prepared once per group (dma_prepare: the tile bookkeeping
  // and the group's uniform source bases) and issued one instruction at a time (dma_issue,
  // k = 0..10) between the MFMA steps of the group being computed. Issued together, the 88
  // loads of a CU's eight waves queue in the memory pipeline for about a thousand cycles and
  // stall the waves that issue them; spread out, the queue stays short.
  int lj = 0, lg = -1;  // tile (of this workgroup's list) and K group being loaded
  const uint8_t* ld_a = A;
  const uint8_t* ld_b = W;
  const float* ld_ws = Ws;
  int64_t ld_as = 0;
  auto dma_prepare = [&]() {
    if (++lg == G) {
      lg = 0;
      ++lj;
    }
    const int gd = lg;
    if (gd == 0) {
      // a new tile enters the stream: set up its sources from the prefetched descriptor
      const TileDesc t = pend;
#pragma unroll
      for (int j = 0; j < A_DMA; ++j) {
        // row (of this wave's RPW) and 16-byte chunk staged by this lane
        int rl, c;
        if (AF4) {
          const int L = wv * (RPW / 2) + 8 * j + (lane >> 3);  // LDS line of the tile
          const int cc = a4_pos(L, lane & 7);                   // chunk held at slot lane & 7
          rl = 2 * L + (cc >> 2) - wv * RPW;
          c = cc & 3;
        } else {
          rl = 8 * j + (lane >> 3);
          c = (lane & 7) ^ a_swz(rl);
        }
        int src;
        if (sorted) {
          const int p = s_src[wv][rl];
          src = kshift >= 0 ? (p >> kshift) : (p / k_route);  // uniform branch
        } else {
          src = t.row_begin + min(wv * RPW + rl, t.rows - 1);
        }
        src = max(min(src, a_rows - 1), 0);
        a_off32[j] = (uint32_t)src * (uint32_t)a_row_bytes + (uint32_t)(c * 16);
      }
      if (sorted) {  // per-token scales and sums, row-major [a_rows, G]: the token's row
        const int p = s_src[wv][lane & (RPW - 1)];
        const int tok = max(min(kshift >= 0 ? (p >> kshift) : (p / k_route), a_rows - 1), 0);
        as_off32 = (uint32_t)tok * (uint32_t)G * 4u;
      } else {  // group-major [G, R] in grouped row order
        as_off32 = (uint32_t)max(
            min(t.row_begin + min(wv * RPW + (lane & (RPW - 1)), t.rows - 1), R - 1), 0) * 4u;
      }
      ws_off32 = (uint32_t)ws_col(t.nt, lane) * 4u;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        b_blk[s] = (uint32_t)tile_block(t.nt, s) * (uint32_t)G * kBlockBytes;
      w_exp = W + (int64_t)t.e * NB * G * kBlockBytes;
      ws_exp = Ws + (int64_t)t.e * G * N;
      // the LDS reads of s_src above complete before any later load may refill it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    // the next tile enters the stream at the next group: fetch its descriptor and rows now,
    // before this group's loads
    if (gd == G - 1 && lj + 1 < my_tiles) {
      pend = tile_of(lj + 1);
      fetch_rows(pend);
    }
    ld_a = A + gd * (AF4 ? kGroup / 2 : kGroup);
    ld_b = w_exp + gd * kBlockBytes;
    ld_ws = ws_exp + (int64_t)gd * N;
    // group gd of the rows' scales (and sums): column gd of the per-token arrays, or row gd
    // of the group-major ones
    ld_as = sorted ? (int64_t)gd : (int64_t)gd * R;
  };
  // load k of the prepared group into stage st: the wave's four bank blocks first (they
  // may come from HBM), then its rows of the A tile, the weight scales, and the rows'
  // activation scales and code sums
  auto dma_issue = [&](int k, Stage& st) {
    if (k < 4) {
      dma16(ld_b + b_blk[k], lane16, st.b + wv * BW_BYTES + k * 1024);
    } else if (k < 4 + A_DMA) {
      dma16(ld_a, a_off32[k - 4], st.a + (wv * A_DMA + k - 4) * 1024);
    } else if (k == 4 + A_DMA) {
      dma4(ld_ws, ws_off32, st.ws + wv * WCOLS);
    } else if (k == 5 + A_DMA) {
      if (lane < RPW) dma4(As + ld_as, as_off32, st.as + wv * RPW);
    } else if (k == 6 + A_DMA) {
      // given code sums replace the in-kernel row sums: they land where the seeds go
      if (SUMS && lane < RPW) dma4(Asum + ld_as, as_off32, st.ra + wv * RPW);
    }
  };
  constexpr int N_DMA = 7 + A_DMA;  // loads per wave and K group

  // sum of this wave's 16-row tile of the A tile of stage st -> st.ra as -sum/64, the
  // accumulator seed that removes the +8 offset of the B codes
  const v8i ones = {(int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes,
                    (int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // AF4: this lane's E8M0 scale for A row r (block q) of stage st, in bits 7..0
  auto a4_scale = [&](const Stage& st, int r) {
    return (int)(__float_as_uint(st.as[r]) >> (8 * q));
  };
  auto row_sums = [&](Stage& st) {
    if constexpr (SUMS) {  // this wave's rows' sums arrived with its own loads: sum -> seed
      if (lane < RPW) st.ra[wv * RPW + lane] *= -0.015625f;
      return;
    }
#pragma unroll
    for (int h = 0; h < RPW / 16; ++h) {
      const int r0 = wv * RPW + h * 16;
      v4f pr;
      if (AF4)  // MXFP4 rows, scaled by the MFMA (the ones operand's scale is 2^0)
        pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            lds_a4_operand(st.a, r0 + c16, q), ones, zero, 4, 0, 0, a4_scale(st, r0 + c16), 0,
            127);
      else
        pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lds_a_operand(st.a, r0 + c16, q),
                                                              ones, zero, 0, 0, 0, 0, 0, 0);
      // the MFMA reads every lane's operands (and, scaled, every lane's scale): pin it here,
      // with all lanes active, so that it is not sunk into the one-lane-per-row store below
      asm volatile("" : "+v"(pr));
      if (c16 == 0)
        *reinterpret_cast<float4*>(&st.ra[r0 + 4 * q]) =
            make_float4(pr[0] * -0.015625f, pr[1] * -0.015625f, pr[2] * -0.015625f,
                        pr[3] * -0.015625f);
    }
  };

  float acc[8][4][4];

  // ---- one K group of the current tile from stage `cur`; tmax = row tiles in use.
  // The group is 32 steps; step i = 4t + s issues the MFMA of tile (t, s) and folds the
  // MFMA of step i-2 (already complete), so the matrix core and the VALU work side by
  // side; a sched_barrier after every step pins that interleaving. The first group of a
  // tile initialises the accumulators (no separate zeroing).
  auto group = [&](auto first_tag, auto tmax_tag, const Stage& cur, auto&& issue) {
    constexpr bool FIRST = decltype(first_tag)::value;
    constexpr int tmax = decltype(tmax_tag)::value;
    // MFMA step after which load k of the next group is issued: spread over the first two
    // thirds of the group's steps (all up front when the group is a single row tile)
    constexpr int kIssueStride = tmax == 8 ? 2 : tmax == 4 ? 1 : 0;
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
      // staged scale of this lane's column in tile s (see ws_col)
      const int wi = EPI == FP8MOE_EPI_SWIGLU_QUANT ? (s >= 2 ? 32 : 0) + 2 * c16 + (s & 1)
                                                    : 4 * c16 + s;
      sw[s] = swg[wi] * kWeightScaleMul;
    }

    v8i aop[2];
    v4f seed[2];
    float4 sa[2];
    int sx[2];  // AF4: the E8M0 scale of this lane's A row and block, per row tile
    auto a_op = [&](int r) { return AF4 ? lds_a4_operand(ta, r, q) : lds_a_operand(ta, r, q); };
    aop[0] = a_op(c16);
    {
      const float4 c4 = *reinterpret_cast<const float4*>(&ra[4 * q]);
      seed[0] = (v4f){c4.x, c4.y, c4.z, c4.w};
    }
    if (AF4) sx[0] = a4_scale(cur, c16);
    else sa[0] = *reinterpret_cast<const float4*>(&sag[4 * q]);
    v4f pb[3];

    auto fold = [&](int i) {
      const int t = i >> 2, s = i & 3;
      const v4f p = pb[i % 3];
      if (AF4) {  // the activation scales are already inside P
        if (FIRST) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[t][s][r] = p[r] * sw[s];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[t][s][r] = fmaf(p[r], sw[s], acc[t][s][r]);
        }
        asm volatile("" : "+v"(acc[t][s][0]), "+v"(acc[t][s][1]), "+v"(acc[t][s][2]),
                     "+v"(acc[t][s][3]));
        return;
      }
      const float4 a4 = sa[t & 1];
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
      if (t < tmax) {  // uniform
        if (s == 0 && t + 1 < tmax) {  // A operand and seed of the next row tile
          aop[(t + 1) & 1] = a_op((t + 1) * 16 + c16);
          const float4 c4 = *reinterpret_cast<const float4*>(&ra[(t + 1) * 16 + 4 * q]);
          seed[(t + 1) & 1] = (v4f){c4.x, c4.y, c4.z, c4.w};
          if (AF4) sx[(t + 1) & 1] = a4_scale(cur, (t + 1) * 16 + c16);
        }
        if (!AF4 && s == 2 && t + 1 < tmax)  // A scales of the next row tile (tile t-1's folds are done)
          sa[(t + 1) & 1] = *reinterpret_cast<const float4*>(&sag[(t + 1) * 16 + 4 * q]);
        if (AF4)
          pb[i % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              aop[t & 1], bop[s], seed[t & 1], 4, 0, 0, sx[t & 1], 0, 127);
        else
          pb[i % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              aop[t & 1], bop[s], seed[t & 1], 0, 0, 0, 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < N_DMA; ++k)
        if (k * kIssueStride == i) issue(k);
      if (i >= 2 && ((i - 2) >> 2) < tmax) fold(i - 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (tmax == 8) {
      fold(30);
      fold(31);
    }
  };

  // ---- epilogue of a finished tile. Output element (t, s, r) of this lane: row
  // t*16 + 4q + r, workgroup column wv*64 + s*16 + c16. `scr` is the stage the tile's last
  // group was computed from: free until the loads of a later group are issued into it.
  auto epilogue = [&](const TileDesc& t, Stage& scr) {
    const int rows = t.rows, row_begin = t.row_begin, nt = t.nt;
    const int tmax = (rows + 15) >> 4;
    if (EPI == FP8MOE_EPI_STORE) {
      // each lane holds 4 consecutive output columns (tiles s = 0..3) of rows t*16 + 4q + r:
      // 16 lanes cover 64 consecutive columns of a row, so every store instruction writes
      // whole 128 B (bf16) or 256 B (fp32) row segments, straight from registers
      // (q4 is opaque to the compiler, so the row indices below are formed here and not
      // hoisted out of the tile loops, where they would stay live across the main loop)
      int q4 = 4 * q;
      asm volatile("" : "+v"(q4));
      const int col0 = nt * WCOLS_WG + wv * WCOLS + 4 * c16;
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        if (t8 >= tmax) break;  // uniform
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = t8 * 16 + q4 + r;
          if (row < rows && col0 < N) {
            const int64_t o = (int64_t)(row_begin + row) * N + col0;
            if (OUT_BF16)
              *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + o) =
                  make_uint2(bf16x2(acc[t8][0][r], acc[t8][1][r]),
                             bf16x2(acc[t8][2][r], acc[t8][3][r]));
            else
              *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + o) =
                  make_float4(acc[t8][0][r], acc[t8][1][r], acc[t8][2][r], acc[t8][3][r]);
          }
        }
      }
    } else {
      // SwiGLU + e4m3 per (row, 128 h columns): the tile is one 128-wide h group; lane c16 of
      // wave wv holds h columns 64*(wv >> 1) + 4*c16 + 2*(wv & 1) + s' (s' = 0, 1) of rows
      // t*16 + 4q + r (gate in tile s', up in tile s' + 2). h overwrites the gate
      // accumulators.
      float* s_amax = reinterpret_cast<float*>(scr.a);      // [NW waves][BM]
      float* s_inv = s_amax + NW * BM;                       // [BM]
      uint8_t* s_codes = scr.b;                              // [BM][128]
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        if (t8 >= tmax) break;  // uniform
        float m[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          m[r] = 0.f;
#pragma unroll
          for (int sp = 0; sp < 2; ++sp) {
            const float gt = acc[t8][sp][r], up = acc[t8][sp + 2][r];
            const float hv = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * up;
            acc[t8][sp][r] = hv;
            m[r] = fmaxf(m[r], fabsf(hv));
          }
        }
        // max of rows r = 0..3 over the 16 lanes of this row group (transposing butterfly)
        const float mr = row4_max16(m, c16);
        if (c16 < 4) s_amax[wv * BM + t8 * 16 + 4 * q + 2 * (c16 & 1) + ((c16 >> 1) & 1)] = mr;
      }
      lds_barrier();
      const int hcol = nt * 128;
      if (tid < BM) {
        const int row = tid;
        float m = s_amax[row];
#pragma unroll
        for (int w = 1; w < NW; ++w) m = fmaxf(m, s_amax[w * BM + row]);
        float sc, inv;
        scale_pair(m, sc, inv);
        s_inv[row] = inv;
        if (row < rows && hcol < I) out_scales[(int64_t)(hcol / kGroup) * R + row_begin + row] = sc;
      }
      lds_barrier();
      const int hc = 64 * (wv >> 1) + 4 * c16 + 2 * (wv & 1);  // this lane's h column pair
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        if (t8 >= tmax) break;  // uniform
        const float4 inv4 = *reinterpret_cast<const float4*>(&s_inv[t8 * 16 + 4 * q]);
        const float inv[4] = {inv4.x, inv4.y, inv4.z, inv4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = t8 * 16 + 4 * q + r;
          const uint32_t c2 = e4m3x2_finite(acc[t8][0][r] * inv[r], acc[t8][1][r] * inv[r]);
          *reinterpret_cast<uint16_t*>(&s_codes[row * 128 + hc]) = (uint16_t)c2;
        }
      }
      lds_barrier();
      uint8_t* o8 = reinterpret_cast<uint8_t*>(out);
      static_assert(BM * 8 % NT_THREADS == 0, "every lane takes part in every pass (sum8)");
      for (int i = tid; i < BM * 8; i += NT_THREADS) {  // the 8 lanes i .. i + 7 share a row
        const int row = i >> 3, ch = i & 7;
        const uint4 c = *reinterpret_cast<const uint4*>(&s_codes[row * 128 + ch * 16]);
        if (row < rows && hcol < I)
          *reinterpret_cast<uint4*>(&o8[(int64_t)(row_begin + row) * I + hcol + ch * 16]) = c;
        if (out_sums) {  // the row's 128 code values summed (the down GEMM's offset seed)
          const float v = sum8(e4m3_sum8(c.x, c.y) + e4m3_sum8(c.z, c.w));
          if (ch == 0 && row < rows && hcol < I)
            out_sums[(int64_t)(hcol / kGroup) * R + row_begin + row] = v;
        }
      }
      lds_barrier();
    }
  };

  // ---- prologue: group 0 loaded, its seeds formed
  dma_prepare();
  for (int k = 0; k < N_DMA; ++k) dma_issue(k, ring[0]);
  wait_all_loads();
  row_sums(ring[0]);
  lds_barrier();

  // ---- the stream of K groups: group s is computed from stage s % 2 while group s+1
  // streams into the other stage (issued as soon as the barrier frees it). Two workgroups
  // share each CU, so one workgroup's waits, barriers and epilogue overlap the other's
  // compute. Tiles are consecutive runs of G groups; the first group of a tile initialises
  // the accumulators, the epilogue follows its last group.
  int s = 0;
  auto step = [&](auto first_tag, auto tmax_tag) {
    const int stage = s & 1;
    const bool more = s + 1 < total_steps;
    if (more) dma_prepare();
    group(first_tag, tmax_tag, ring[stage], [&](int k) {
      if (more) dma_issue(k, ring[stage ^ 1]);
    });
    wait_all_loads();  // own loads of group s+1 landed
    if (more) row_sums(ring[stage ^ 1]);
    lds_barrier();
    ++s;
  };
  auto unit = [&](int j, auto tmax_tag) {
    const TileDesc cur = tile_of(j);  // before the accumulators are live
    step(std::true_type{}, tmax_tag);
    for (int g = 1; g < G; ++g) step(std::false_type{}, tmax_tag);
    epilogue(cur, ring[(s + 1) & 1]);
  };
  for (int j = 0; j < j_small; ++j) unit(j, std::integral_constant<int, 8>{});
  for (int j = j_small; j < j_tiny; ++j) unit(j, std::integral_constant<int, 4>{});
  for (int j = j_tiny; j < my_tiles; ++j) unit(j, std::integral_constant<int, 1>{});
}

// ---- Few rows per expert (decode-sized batches) ----
// When the routed rows average only a few per expert, nearly every tile of the kernel above
// is a single 16-row MFMA tile whose K groups are waited for one at a time: the kernel then
// runs at the latency of one group's loads per group, not at HBM speed. This variant cuts
// each expert's rows into units of 16 (one MFMA row tile) x 256 accumulator columns and
// keeps three K groups of a unit in flight through a four-deep ring of compact stages (the
// 16 A rows, the waves' packed B slices, the scales). Every output is formed by the same
// MFMAs, seeds and fold, in the same order, as in the kernel above.
constexpr int R16 = 16;        // rows per unit
constexpr int kRows16PerExpert = 16;  // used when R <= 16 E (measured crossover: 32 E)
constexpr int kRing16 = 4;     // stages in flight
struct __attribute__((aligned(16))) Stage16 {
  uint8_t a[R16 * kGroup];     // 16 rows, chunks swizzled as in the big tile (a_off)
  uint8_t b[NW * BW_BYTES];    // each wave's packed B slice
  float ws[WCOLS_WG];          // weight scales of the 256 columns (as staged by ws_col)
  float as[R16];               // activation scales of the 16 rows
  float ra[R16];               // row-sum seeds (given code sums, scaled in place)
};

template <int EPI, bool OUT_BF16, bool SUMS>
__global__ __launch_bounds__(NT_THREADS, 2) void grouped_rows16_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const float* __restrict__ Asum,
    const int32_t* __restrict__ sorted, int k_route, int a_rows, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, const int32_t* __restrict__ offsets, int R, int E, int N,
    int K, int NT, void* __restrict__ out, float* __restrict__ out_scales,
    float* __restrict__ out_sums) {
  __shared__ Stage16 ring[kRing16];
  __shared__ int s_tmp[NW];
  __shared__ float s_amax[NW * R16];
  __shared__ float s_inv[R16];
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[R16 * 128];
  extern __shared__ int s_ustart[];  // [E + 1]: units of 16 rows before expert e

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, c16 = lane & 15;
  const int G = K / kGroup;
  const int I = N / 2;
  const int NB = N / 16;
  const int NG = N / 64;
  const int kshift = (k_route & (k_route - 1)) == 0 ? __builtin_ctz(k_route) : -1;

  {  // units per expert, ceil(count / 16), and their exclusive scan (4 experts per thread)
    constexpr int EPT = kMaxExperts / NT_THREADS;
    int nu[EPT], sum = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid * EPT + j;
      nu[j] = e < E ? (offsets[e + 1] - offsets[e] + R16 - 1) / R16 : 0;
      sum += nu[j];
    }
    int run = block_inclusive_scan(sum, s_tmp) - sum;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid * EPT + j;
      if (e < E) s_ustart[e] = run;
      run += nu[j];
      if (e == E - 1) s_ustart[E] = run;
    }
    __syncthreads();
  }
  // units (16-row chunk, n-tile), n-tile fastest, dealt to the XCDs in contiguous ranges;
  // the workgroups of XCD x take every nwg_x-th unit of its range
  const int n_units = __builtin_amdgcn_readfirstlane(s_ustart[E]) * NT;
  const int nx = min(8, (int)gridDim.x);
  const int x = (int)blockIdx.x % nx, u = (int)blockIdx.x / nx;
  const int nwg_x = ((int)gridDim.x - x + nx - 1) / nx;
  const int ub_x = n_units * x / nx, nu_x = n_units * (x + 1) / nx - ub_x;

  auto tile_block = [&](int nt, int s) {  // bank block of MFMA tile s of this wave
    int b;
    if (EPI == FP8MOE_EPI_SWIGLU_QUANT)
      b = 4 * (2 * nt + (wv >> 1) + (s >= 2 ? I / 64 : 0)) + 2 * (wv & 1) + (s & 1);
    else
      b = 4 * (4 * nt + wv) + s;
    return min(b, 4 * NG - 1);
  };
  auto ws_col = [&](int nt, int l) {  // weight-scale column staged by lane l of this wave
    int c;
    if (EPI == FP8MOE_EPI_SWIGLU_QUANT)
      c = (l >= 32 ? I : 0) + 64 * (2 * nt + (wv >> 1)) + 4 * ((l & 31) >> 1) + 2 * (wv & 1) +
          (l & 1);
    else
      c = 64 * (4 * nt + wv) + l;
    return min(c, N - 1);
  };
  const v8i ones = {(int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes,
                    (int)kOnes, (int)kOnes, (int)kOnes, (int)kOnes};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const uint32_t lane16 = (uint32_t)lane * 16u;
  constexpr int NPER = SUMS ? 8 : 7;  // loads per wave and K group

  for (int l = u; l < nu_x; l += nwg_x) {
    const int L = ub_x + l, mt = L / NT, nt = L - mt * NT;
    int lo = 0, hi = E;  // s_ustart[lo] <= mt < s_ustart[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(s_ustart[mid]) <= mt) lo = mid;
      else hi = mid;
    }
    const int e = lo;
    const int row_begin =
        sload(offsets + e) + (mt - __builtin_amdgcn_readfirstlane(s_ustart[e])) * R16;
    const int rows = min(R16, sload(offsets + e + 1) - row_begin);

    // this wave's bank blocks and weight-scale columns, and their first groups' loads: they
    // do not depend on the unit's rows, so they go out before the row lookups below
    const uint32_t ws_off32 = (uint32_t)ws_col(nt, lane) * 4u;
    uint32_t b_blk[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) b_blk[s] = (uint32_t)tile_block(nt, s) * (uint32_t)G * kBlockBytes;
    const uint8_t* w_exp = W + (int64_t)e * NB * G * kBlockBytes;
    const float* ws_exp = Ws + (int64_t)e * G * N;
    auto issue_b = [&](int g) {  // 5 loads
      Stage16& st = ring[g % kRing16];
      const uint8_t* bsrc = w_exp + g * kBlockBytes;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        dma16(bsrc + b_blk[s], lane16, st.b + wv * BW_BYTES + s * 1024);
      dma4(ws_exp + (int64_t)g * N, ws_off32, st.ws + wv * WCOLS);
    };
    // every wave is done with the ring (the previous unit's last group) before it refills,
    // and nothing of the previous unit is still counted against this unit's waits
    wait_all_loads();
    lds_barrier();
#pragma unroll
    for (int p = 0; p < kRing16 - 1; ++p)
      if (p < G) issue_b(p);

    // rows 4 wv .. 4 wv + 3 of the unit: A (lanes 0..31, one 16-byte chunk each), the
    // activation scales and code sums (lanes 0..3)
    int tok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int gr = row_begin + min(4 * wv + i, rows - 1);  // grouped row (uniform)
      int t;
      if (sorted) {
        const int p = sload(sorted + gr);
        t = kshift >= 0 ? (p >> kshift) : (p / k_route);
      } else {
        t = gr;
      }
      tok[i] = max(min(t, a_rows - 1), 0);
    }
    auto pick = [&](int i) { return i == 0 ? tok[0] : i == 1 ? tok[1] : i == 2 ? tok[2] : tok[3]; };
    const int ra_i = (lane >> 3) & 3;  // A: lanes 0..31 stage row 4 wv + lane / 8
    const int rl = 4 * wv + ra_i;
    const uint32_t a_off32 =
        (uint32_t)pick(ra_i) * (uint32_t)K + (uint32_t)(((lane & 7) ^ a_swz(rl)) * 16);
    const int rs_i = lane & 3;         // scales and sums: lanes 0..3 stage row 4 wv + lane
    const uint32_t as_off32 =
        sorted ? (uint32_t)pick(rs_i) * (uint32_t)G * 4u
               : (uint32_t)max(min(row_begin + min(4 * wv + rs_i, rows - 1), R - 1), 0) * 4u;
    auto issue_a = [&](int g) {  // 2 loads, 3 with the code sums
      Stage16& st = ring[g % kRing16];
      if (lane < 32) dma16(A + g * kGroup, a_off32, st.a + wv * 4 * kGroup);
      const int64_t sg = sorted ? (int64_t)g : (int64_t)g * R;
      if (lane < 4) dma4(As + sg, as_off32, st.as + 4 * wv);
      if (SUMS && lane < 4) dma4(Asum + sg, as_off32, st.ra + 4 * wv);
    };
#pragma unroll
    for (int p = 0; p < kRing16 - 1; ++p)
      if (p < G) issue_a(p);
    auto issue = [&](int g) {
      issue_b(g);
      issue_a(g);
    };

    float acc[4][4];
    for (int g = 0; g < G; ++g) {
      // this group's loads landed; those of at most two later groups stay in flight (the
      // first group waits for all of the prologue, whose loads went out B first)
      const int later = g == 0 ? 0 : min(kRing16 - 2, G - 1 - g);
      if (later >= 2) wait_loads<2 * NPER>();
      else if (later == 1) wait_loads<NPER>();
      else wait_loads<0>();
      Stage16& cur = ring[g % kRing16];
      if (SUMS && lane < 4) cur.ra[4 * wv + lane] *= -0.015625f;
      lds_barrier();  // the group is in for every wave; stage (g - 1) % 4 is free
      if (g + kRing16 - 1 < G) issue(g + kRing16 - 1);

      const uint8_t* tb = cur.b + wv * BW_BYTES;
      v8i bop[4];
      float sw[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bop[s] = convert_b(*reinterpret_cast<const uint4*>(&tb[s * 1024 + lane * 16]));
        const int wi = EPI == FP8MOE_EPI_SWIGLU_QUANT ? (s >= 2 ? 32 : 0) + 2 * c16 + (s & 1)
                                                      : 4 * c16 + s;
        sw[s] = cur.ws[wv * WCOLS + wi] * kWeightScaleMul;
      }
      const v8i aop = lds_a_operand(cur.a, c16, q);
      v4f seed;
      if constexpr (SUMS) {
        const float4 c4 = *reinterpret_cast<const float4*>(&cur.ra[4 * q]);
        seed = (v4f){c4.x, c4.y, c4.z, c4.w};
      } else {
        const v4f pr =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, ones, zero, 0, 0, 0, 0, 0, 0);
        seed = (v4f){pr[0] * -0.015625f, pr[1] * -0.015625f, pr[2] * -0.015625f,
                     pr[3] * -0.015625f};
      }
      const float4 a4 = *reinterpret_cast<const float4*>(&cur.as[4 * q]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[s], seed, 0, 0,
                                                                       0, 0, 0, 0);
        if (g == 0) {
          acc[s][0] = p[0] * (a4.x * sw[s]);
          acc[s][1] = p[1] * (a4.y * sw[s]);
          acc[s][2] = p[2] * (a4.z * sw[s]);
          acc[s][3] = p[3] * (a4.w * sw[s]);
        } else {
          acc[s][0] = fmaf(p[0], a4.x * sw[s], acc[s][0]);
          acc[s][1] = fmaf(p[1], a4.y * sw[s], acc[s][1]);
          acc[s][2] = fmaf(p[2], a4.z * sw[s], acc[s][2]);
          acc[s][3] = fmaf(p[3], a4.w * sw[s], acc[s][3]);
        }
      }
    }

    // epilogue: output element (s, r) of this lane is row 4 q + r of the unit
    if (EPI == FP8MOE_EPI_STORE) {
      const int col0 = nt * WCOLS_WG + wv * WCOLS + 4 * c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * q + r;
        if (row < rows && col0 < N) {
          const int64_t o = (int64_t)(row_begin + row) * N + col0;
          if (OUT_BF16)
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + o) =
                make_uint2(bf16x2(acc[0][r], acc[1][r]), bf16x2(acc[2][r], acc[3][r]));
          else
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + o) =
                make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
        }
      }
    } else {
      // SwiGLU + e4m3 per (row, the unit's 128 h columns), as in the kernel above
      float m[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        m[r] = 0.f;
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          const float gt = acc[sp][r], up = acc[sp + 2][r];
          const float hv = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * up;
          acc[sp][r] = hv;
          m[r] = fmaxf(m[r], fabsf(hv));
        }
      }
      const float mr = row4_max16(m, c16);
      if (c16 < 4) s_amax[wv * R16 + 4 * q + 2 * (c16 & 1) + ((c16 >> 1) & 1)] = mr;
      lds_barrier();
      const int hcol = nt * 128;
      if (tid < R16) {
        float mx = s_amax[tid];
#pragma unroll
        for (int w = 1; w < NW; ++w) mx = fmaxf(mx, s_amax[w * R16 + tid]);
        float sc, inv;
        scale_pair(mx, sc, inv);
        s_inv[tid] = inv;
        if (tid < rows && hcol < I) out_scales[(int64_t)(hcol / kGroup) * R + row_begin + tid] = sc;
      }
      lds_barrier();
      const int hc = 64 * (wv >> 1) + 4 * c16 + 2 * (wv & 1);  // this lane's h column pair
      const float4 inv4 = *reinterpret_cast<const float4*>(&s_inv[4 * q]);
      const float inv[4] = {inv4.x, inv4.y, inv4.z, inv4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t c2 = e4m3x2_finite(acc[0][r] * inv[r], acc[1][r] * inv[r]);
        *reinterpret_cast<uint16_t*>(&s_codes[(4 * q + r) * 128 + hc]) = (uint16_t)c2;
      }
      lds_barrier();
      if (tid < R16 * 8) {  // waves 0 and 1, all lanes: the 8 lanes tid .. tid + 7 share a row
        const int row = tid >> 3, ch = tid & 7;
        const uint4 c = *reinterpret_cast<const uint4*>(&s_codes[row * 128 + ch * 16]);
        uint8_t* o8 = reinterpret_cast<uint8_t*>(out);
        if (row < rows && hcol < I)
          *reinterpret_cast<uint4*>(&o8[(int64_t)(row_begin + row) * I + hcol + ch * 16]) = c;
        if (out_sums) {
          const float v = sum8(e4m3_sum8(c.x, c.y) + e4m3_sum8(c.z, c.w));
          if (ch == 0 && row < rows && hcol < I)
            out_sums[(int64_t)(hcol / kGroup) * R + row_begin + row] = v;
        }
      }
      // the next unit's first barrier orders these LDS reads before s_amax is rewritten
    }
  }
}

int cu_count() {
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

}  // namespace

namespace {
template <bool AF4, bool SUMS>
hipError_t launch_grouped(const uint8_t* a, const float* a_scales, const float* a_sums,
                          const int32_t* sorted, int32_t k_route, const uint8_t* w,
                          const float* w_scales, const int32_t* offsets, int64_t R, int32_t E,
                          int64_t N, int64_t K, int32_t epilogue, int32_t out_dtype, void* out,
                          float* out_scales, float* out_sums, hipStream_t st) {
  if (R == 0) return hipSuccess;
  const int64_t mtiles = (R + BM - 1) / BM + E;  // bound on the m-tiles over all experts
  // SwiGLU: a tile covers 128 h columns (gate and up); otherwise 256 output columns
  const int NT = epilogue == FP8MOE_EPI_SWIGLU_QUANT ? (int)((N / 2 + 127) / 128)
                                                     : (int)((N + WCOLS_WG - 1) / WCOLS_WG);
  if (mtiles * NT >= (int64_t(1) << 28)) return hipErrorInvalidValue;  // 32-bit tile indexing
  const int a_rows = (int)(sorted ? R / k_route : R);
  dim3 block(NT_THREADS);
  if constexpr (!AF4) {
    // a few rows per expert on average (decode-sized batches): 16-row units, deeper ring
    if (R <= kRows16PerExpert * (int64_t)E) {
      const int64_t units = ((R + R16 - 1) / R16 + E) * NT;  // bound over all experts
      dim3 g((uint32_t)std::min<int64_t>(2 * (int64_t)cu_count(), units));
      const size_t dyn = (size_t)(E + 1) * sizeof(int);
      if (epilogue == FP8MOE_EPI_SWIGLU_QUANT)
        grouped_rows16_kernel<FP8MOE_EPI_SWIGLU_QUANT, false, SUMS><<<g, block, dyn, st>>>(
            a, a_scales, a_sums, sorted, k_route, a_rows, w, w_scales, offsets, (int)R, E,
            (int)N, (int)K, NT, out, out_scales, out_sums);
      else if (out_dtype == FP8MOE_DTYPE_BF16)
        grouped_rows16_kernel<FP8MOE_EPI_STORE, true, SUMS><<<g, block, dyn, st>>>(
            a, a_scales, a_sums, sorted, k_route, a_rows, w, w_scales, offsets, (int)R, E,
            (int)N, (int)K, NT, out, nullptr, nullptr);
      else
        grouped_rows16_kernel<FP8MOE_EPI_STORE, false, SUMS><<<g, block, dyn, st>>>(
            a, a_scales, a_sums, sorted, k_route, a_rows, w, w_scales, offsets, (int)R, E,
            (int)N, (int)K, NT, out, nullptr, nullptr);
      return hipGetLastError();
    }
  }
  const int64_t grid = std::min<int64_t>(2 * (int64_t)cu_count(), mtiles * NT);
  dim3 g((uint32_t)grid);
  if (epilogue == FP8MOE_EPI_SWIGLU_QUANT)
    grouped_gemm_kernel<FP8MOE_EPI_SWIGLU_QUANT, false, AF4, SUMS><<<g, block, 0, st>>>(
        a, a_scales, a_sums, sorted, k_route, a_rows, w, w_scales, offsets, (int)R, E, (int)N,
        (int)K, NT, out, out_scales, out_sums);
  else if (out_dtype == FP8MOE_DTYPE_BF16)
    grouped_gemm_kernel<FP8MOE_EPI_STORE, true, AF4, SUMS><<<g, block, 0, st>>>(
        a, a_scales, a_sums, sorted, k_route, a_rows, w, w_scales, offsets, (int)R, E, (int)N,
        (int)K, NT, out, nullptr, nullptr);
  else
    grouped_gemm_kernel<FP8MOE_EPI_STORE, false, AF4, SUMS><<<g, block, 0, st>>>(
        a, a_scales, a_sums, sorted, k_route, a_rows, w, w_scales, offsets, (int)R, E, (int)N,
        (int)K, NT, out, nullptr, nullptr);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_grouped_gemm(const uint8_t* a, const float* a_scales, const float* a_sums,
                               const int32_t* sorted, int32_t k_route, const uint8_t* w,
                               const float* w_scales, const int32_t* offsets, int64_t R,
                               int32_t E, int64_t N, int64_t K, int32_t epilogue,
                               int32_t out_dtype, void* out, float* out_scales,
                               float* out_sums, hipStream_t st, bool a_fp4) {
  if (a_fp4)
    return launch_grouped<true, false>(a, a_scales, nullptr, sorted, k_route, w, w_scales,
                                       offsets, R, E, N, K, epilogue, out_dtype, out,
                                       out_scales, out_sums, st);
  if (a_sums)
    return launch_grouped<false, true>(a, a_scales, a_sums, sorted, k_route, w, w_scales,
                                       offsets, R, E, N, K, epilogue, out_dtype, out,
                                       out_scales, out_sums, st);
  return launch_grouped<false, false>(a, a_scales, nullptr, sorted, k_route, w, w_scales,
                                      offsets, R, E, N, K, epilogue, out_dtype, out, out_scales,
                                      out_sums, st);
}

}  // namespace fp8moe
