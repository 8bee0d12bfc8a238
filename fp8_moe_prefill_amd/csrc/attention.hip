// Causal grouped-query attention of the depth stack (fp8moe_causal_attention).
//
// The FP8 grouped-expert prefill note ("FP8 grouped-expert prefill with on-chip int4-to-e4m3
// dequant", sections 1 and 3) quantises the q/k/v/o projections around an attention core
// that stays in bf16. Its plain reading: softmax(q k^T / sqrt(d)) v per query head over the
// causal prefix, query head h reading kv head h / (n_q / n_kv), no rotary embedding, bf16
// inputs and output, fp32 softmax and accumulation.
//
// gfx950 design (one pass over the keys with a running max, so the T x T score matrix never
// leaves registers):
// * a workgroup owns one kv head, 16 queries and four query heads of that kv head's group,
//   one per wave (small query blocks: more workgroups in flight for the causal
//   imbalance); the K tile and the transposed V tile of 64 keys are staged once in LDS
//   (K in two stages, V^T in three) and shared by the four waves; a tile's global loads
//   are issued two tiles ahead into one of two register sets (one tile of compute is
//   shorter than the load latency). The loads are buffer loads whose per-lane offsets are
//   fixed for the whole kernel: only the scalar base moves from tile to tile, and keys past
//   T read as zero (the range check of the buffer descriptor), so staging costs no vector
//   ALU work;
// * each wave computes S^T = K Q^T (v_mfma_f32_16x16x32_bf16, keys as rows), so a lane's
//   scores all belong to one query: the running max, the rescale of the output and the
//   row sum need no lane exchange except the 4-lane max per tile; the causal mask only
//   exists in the code of the last (diagonal) tile of a query block;
// * O^T = V^T P^T: P leaves the S^T accumulators as the B operand directly (same lane),
//   split into two bf16 terms hi + lo so that the product keeps the fp32 softmax's
//   accuracy (a single bf16 rounding of the weights would cost 2^-9 relative). The
//   accumulator layout puts keys 4g..4g+3 and 16+4g..16+4g+3 of each 32-key step in lane
//   group g, so the V^T tile is stored in LDS in that key order: one 16-byte read per
//   lane is one A operand;
// * software pipelining inside a wave: iteration kt issues the score MFMAs of tile kt,
//   then the P.V MFMAs of tile kt - 1 while its VALU computes the softmax of tile kt (the
//   two are independent), so the matrix core and the VALU of one wave work side by side.
//   Tile kt - 1's rescale by its running max is applied at the start of iteration kt,
//   before any MFMA, so that the score MFMAs, the softmax and the P.V MFMAs sit in one
//   basic block the compiler can interleave. Per output element the rescales and adds run
//   in the same order as without the pipelining. The third V^T stage lets tile kt + 1 be
//   staged while tile kt - 1's V^T is still being read: one barrier per tile;
// * V is transposed once per layer into a [n_kv][d][T_pad] workspace by a small kernel
//   (zero-filled past T), so V^T tiles load as contiguous rows.
// Workgroups are paired heavy with light (see the rank mapping) against the causal
// imbalance.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace fp8moe {
namespace {

constexpr int D = 128;        // head dim
constexpr int QB = 16;        // queries per workgroup
constexpr int KT = 64;        // keys per tile
constexpr int KS = D * 2;      // K tile row stride in LDS (bytes)
constexpr int VS = KT * 2;     // V^T tile row stride in LDS (bytes): 64 keys
// Dword 3 of a raw buffer descriptor on gfx9 data-parallel parts: 32-bit data format, no
// swizzle, no index stride.
constexpr int kBufferWord3 = 0x00020000;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// LDS layouts. K tile: row `key` (256 B) holds 16 chunks of 16 B, chunk c at position
// c ^ (key % 16). V^T tile: row d (128 B) holds 8 chunks of 16 B; chunk 4c + g holds keys
// 32c + 4g .. +3, then 32c + 16 + 4g .. +3 (the key order of the P operand), at position
// (4c + g) ^ (d % 8). On gfx950 both measured free of bank conflicts for the 16-byte
// operand reads (16 rows x 4 chunks per instruction) and for the staging writes, where
// rows padded by 16 B, or an XOR that also folds in bit 3 of the row, measured 2-way.
__device__ __forceinline__ int v_swz(int d) { return d & 7; }

// max / sum of v over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes that hold the
// same query): two lane-swap instructions of gfx950, no LDS round trip
__device__ __forceinline__ float max4q(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4q(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// [T, ld] column block of V (kv head j, 64 columns) -> vt[j][d][t], zero for t in
// [T, Tp). 16-byte loads of 8 columns, transposed through LDS, 16-byte stores of 8 keys.
__global__ __launch_bounds__(256) void v_transpose_kernel(const uint16_t* __restrict__ qkv,
                                                          int T, int ld, int v_col0, int Tp,
                                                          uint16_t* __restrict__ vt) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][64 + 2];  // [column][key]
  const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 64;  // c: column within the V block
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int r = q >> 3, cc = (q & 7) * 8;  // key r of the tile, columns cc .. cc + 7
    const int t = t0 + r;
    u32x4 v = (u32x4){0u, 0u, 0u, 0u};
    if (t < T) v = *reinterpret_cast<const u32x4*>(qkv + (int64_t)t * ld + v_col0 + c0 + cc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[cc + 2 * e][r] = (uint16_t)(v[e] & 0xFFFFu);
      tile[cc + 2 * e + 1][r] = (uint16_t)(v[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int c = q >> 3, kk = (q & 7) * 8;  // column c, keys kk .. kk + 7
    u32x4 w;  // (132 c + 2 kk + 4 e) bytes: 4-byte aligned pairs of keys
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = *reinterpret_cast<const uint32_t*>(&tile[c][kk + 2 * e]);
    *reinterpret_cast<u32x4*>(vt + (int64_t)(c0 + c) * Tp + t0 + kk) = w;
  }
}

__global__ __launch_bounds__(256, 2) void attention_kernel(const uint16_t* __restrict__ qkv,
                                                           const uint16_t* __restrict__ vt,
                                                           uint16_t* __restrict__ out, int T,
                                                           int ld, int n_q, int n_kv, int Tp,
                                                           int n_hg, float c_log2) {
  __shared__ __attribute__((aligned(16))) uint8_t sK[2][KT * KS];
  __shared__ __attribute__((aligned(16))) uint8_t sV[3][D * VS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int rep = n_q / n_kv;
  const int nqb = (T + QB - 1) / QB;
  const int per_qb = n_kv * n_hg;
  // Work ranks by weight: rank 0 = the latest query block (most keys). The first half of
  // the grid takes ranks 0, 1, ... and the second half the lightest first, so the two
  // workgroups that share a CU (blocks b and b + half are dispatched to the same slot
  // position) carry one heavy and one light block: every CU gets about the same number
  // of key tiles.
  const int nblk = (int)gridDim.x, half = (nblk + 1) / 2;
  const int b = (int)blockIdx.x;
  const int rank = b < half ? b : nblk - 1 - (b - half);
  const int qb = nqb - 1 - rank / per_qb;
  const int rest = rank % per_qb;
  const int j = rest / n_hg, hg = rest % n_hg;
  const int hr = hg * 4 + wv;               // head within the kv group
  const bool live = hr < rep;               // a wave past the group's heads only helps load
  const int h = j * rep + min(hr, rep - 1);
  const int q0 = qb * QB;
  const int nkt = min(q0 + QB - 1, T - 1) / KT + 1;
  const int qi = q0 + c16;  // this lane's query

  // Q fragment: lane (g, c16) holds query q0 + c16, dims 32 kk + 8 g .. +7
  bf16x8_t qf[4];
  {
    const int t = min(qi, T - 1);
    const uint16_t* src = qkv + (int64_t)t * ld + h * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(src + 32 * kk));
  }

  // Staging of one key tile: K rows (64 x 256 B) and V^T rows (128 x 128 B), 4 chunks of
  // 16 B each per thread. Thread chunk c = tid + 256 i: K row c / 16, bytes 16 (c % 16);
  // V^T row d = c / 8, keys 8 (c % 8) .. +7.
  const int64_t k_bytes = (int64_t)T * ld * 2;  // < 2^32 (checked by the caller)
  const char* kbase = reinterpret_cast<const char*>(qkv + (n_q + j) * D);
  const char* vbase = reinterpret_cast<const char*>(vt + (int64_t)j * D * Tp);
  const uint32_t k_voff = (uint32_t)((tid >> 4) * ld * 2 + (tid & 15) * 16);
  const uint32_t k_step = (uint32_t)(16 * ld * 2);  // 16 rows: i -> i + 1
  const uint32_t v_voff = (uint32_t)((tid >> 3) * Tp * 2 + (tid & 7) * 16);
  const uint32_t v_step = (uint32_t)(32 * Tp * 2);  // 32 rows
  const int v_bytes_max = (int)((int64_t)D * Tp * 2);
  // LDS destinations: K chunk c % 16 of row c / 16 (+ 16 rows per i, same position); the
  // two 8-byte halves of a V^T chunk (keys 8m .. 8m+3 and 8m+4 .. 8m+7, m = c % 8) go to
  // chunks 4(m / 4) + 2(m % 2) and that + 1, half (m / 2) % 2 of each (+ 32 rows per i).
  const int k_lds = (tid >> 4) * KS + (((tid & 15) ^ (tid >> 4)) << 4);
  int v_lds0, v_lds1;
  {
    const int d = tid >> 3, m = tid & 7;
    const int ch0 = 4 * (m >> 2) + 2 * (m & 1), hf = ((m >> 1) & 1) * 8;
    v_lds0 = d * VS + ((ch0 ^ v_swz(d)) << 4) + hf;
    v_lds1 = d * VS + (((ch0 + 1) ^ v_swz(d)) << 4) + hf;
  }
  u32x4 rk0[4], rv0[4], rk1[4], rv1[4];
  auto load_tile = [&](auto set_tag, int kt) {
    constexpr int S = decltype(set_tag)::value;
    u32x4* rk = S ? rk1 : rk0;
    u32x4* rv = S ? rv1 : rv0;
    const int64_t k_off = (int64_t)kt * KT * ld * 2;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kbase + k_off), (short)0, (int)(k_bytes - k_off), kBufferWord3);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(vbase + kt * KT * 2), (short)0, v_bytes_max - kt * KT * 2,
        kBufferWord3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rk[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            kr, (int)(k_voff + i * k_step), 0, 0));
      rv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            vr, (int)(v_voff + i * v_step), 0, 0));
    }
  };
  auto store_tile = [&](auto set_tag, int kbuf, int vbuf) {
    constexpr int S = decltype(set_tag)::value;
    const u32x4* rk = S ? rk1 : rk0;
    const u32x4* rv = S ? rv1 : rv0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&sK[kbuf][k_lds + 16 * KS * i]) = rk[i];
      *reinterpret_cast<u32x2*>(&sV[vbuf][v_lds0 + 32 * VS * i]) = rv[i].xy;
      *reinterpret_cast<u32x2*>(&sV[vbuf][v_lds1 + 32 * VS * i]) = rv[i].zw;
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using F = std::false_type;
  using Tr = std::true_type;

  // A-operand offsets: K rows 16 s + c16, chunk 4 kk + g; V^T rows 16 dt + c16, chunk
  // 4c + g
  int k_rd[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) k_rd[kk] = c16 * KS + (((4 * kk + g) ^ c16) << 4);
  const int v_rd0 = c16 * VS + (((0 + g) ^ v_swz(c16)) << 4);
  const int v_rd1 = c16 * VS + (((4 + g) ^ v_swz(c16)) << 4);

  v4f o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  // tile kt: loaded into register set kt % 2 at iteration kt - 2 (the prologue for tiles 0
  // and 1), stored into K stage kt % 2 and V^T stage kt % 3 during iteration kt - 1 (the
  // prologue for tile 0), published by that iteration's barrier; its scores and softmax
  // are computed at iteration kt, its P.V at iteration kt + 1
  load_tile(I0{}, 0);
  store_tile(I0{}, 0, 0);
  if (nkt > 1) load_tile(I1{}, 1);
  __syncthreads();

  // P of the previous tile (register set by tile parity) and its rescale factor: tile kt's
  // P.V runs at iteration kt + 1, beside the softmax of tile kt + 1
  u32x4 pbs0[2], pls0[2], pbs1[2], pls1[2];
  float alpha_prev = 1.f;
  int vs = 0;  // V^T stage of tile kt: kt % 3
  auto rescale = [&](float alpha) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {  // uniform: some query's max moved
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }
  };
  auto pv = [&](auto set_tag, int vbuf) {
    const u32x4* pb = decltype(set_tag)::value ? pbs1 : pbs0;
    const u32x4* pl = decltype(set_tag)::value ? pls1 : pls0;
    // O^T[d 16 dt + 4 g + r][query c16] += V^T P^T over two 32-key steps
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8_t a = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &sV[vbuf][(c ? v_rd1 : v_rd0) + 16 * dt * VS]));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(pb[c]), o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(pl[c]), o[dt], 0, 0, 0);
      }
    }
  };

  auto step = [&](auto par_tag, auto diag_tag, auto first_tag, int kt) {
    constexpr int P = decltype(par_tag)::value;  // kt % 2
    constexpr bool DIAG = decltype(diag_tag)::value;  // the last tile: keys past a query
    constexpr bool FIRST = decltype(first_tag)::value;  // kt == 0: no previous tile
    const int cur = P;
    // the output as of tile kt - 2, rescaled to the running max of tile kt - 1, before
    // tile kt - 1's P.V is added below
    if (!FIRST) rescale(alpha_prev);
    const int vs_prev = vs == 0 ? 2 : vs - 1, vs_next = vs == 2 ? 0 : vs + 1;
    if (!DIAG && kt + 2 < nkt) load_tile(par_tag, kt + 2);  // set P held tile kt
    // tile kt + 1 into the K stage of tile kt - 1 and the V^T stage of tile kt - 2, both
    // read for the last time in iteration kt - 1
    if (!DIAG) store_tile(std::integral_constant<int, P ^ 1>{}, cur ^ 1, vs_next);

    // S^T[key 16 s + 4 g + r][query c16]
    v4f st[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      st[s] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8_t a = as_bf16x8(
            *reinterpret_cast<const u32x4*>(&sK[cur][k_rd[kk] + 16 * s * KS]));
        st[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], st[s], 0, 0, 0);
      }
    }

    // online softmax in the log2 domain (c_log2 > 0, so the max commutes with the scale)
    if (DIAG) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kt * KT + 16 * s + 4 * g + r > qi) st[s][r] = -INFINITY;
    }
    float mx = st[0][0];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[s][r]);
    const float m_new = fmaxf(m_run, max4q(mx) * c_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    // p enters P.V as hi + lo, two bf16 terms (about 16 significant bits): the product
    // keeps fp32-level accuracy on the bf16 matrix cores
    u32x4* pb = P ? pbs1 : pbs0;
    u32x4* pl = P ? pls1 : pls0;
    float ls = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int rp = 0; rp < 2; ++rp) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[s][2 * rp], c_log2, -m_new));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[s][2 * rp + 1], c_log2, -m_new));
        ls += p0 + p1;
        const uint32_t hw = bf16x2(p0, p1);
        pb[s >> 1][2 * (s & 1) + rp] = hw;
        pl[s >> 1][2 * (s & 1) + rp] = bf16x2(p0 - bf16_lo(hw), p1 - bf16_hi(hw));
      }
    l_part = l_part * alpha + ls;
    // the previous tile's P.V (its V^T stage vs_prev), then, at the diagonal tile, this
    // tile's own
    if (!FIRST) pv(std::integral_constant<int, P ^ 1>{}, vs_prev);
    alpha_prev = alpha;
    if (DIAG) {
      rescale(alpha);
      pv(par_tag, vs);
    }
    vs = vs_next;
    if (!DIAG) __syncthreads();
  };
  // tiles 0 .. nkt - 2 are whole (no key past any query of the block), tile nkt - 1 is
  // the diagonal one
  const int nfull = nkt - 1;
  using T0 = std::true_type;
  if (nfull == 0) {
    step(I0{}, Tr{}, T0{}, 0);
  } else {
    step(I0{}, F{}, T0{}, 0);
    int kt = 1;
    for (; kt + 1 < nfull; kt += 2) {
      step(I1{}, F{}, F{}, kt);
      step(I0{}, F{}, F{}, kt + 1);
    }
    if (kt < nfull) {
      step(I1{}, F{}, F{}, kt);
      step(I0{}, Tr{}, F{}, kt + 1);
    } else {
      step(I1{}, Tr{}, F{}, kt);
    }
  }

  if (!live || qi >= T) return;
  const float inv = 1.f / sum4q(l_part);
  uint16_t* dst = out + (int64_t)qi * (n_q * D) + h * D + 4 * g;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const v4f v = o[dt] * inv;
    *reinterpret_cast<uint2*>(dst + 16 * dt) = make_uint2(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]));
  }
}

}  // namespace

size_t attention_workspace_bytes(int64_t T, int32_t n_kv) {
  const int64_t Tp = (T + KT - 1) / KT * KT;
  return (size_t)n_kv * D * Tp * sizeof(uint16_t);
}

hipError_t launch_attention(const uint16_t* qkv, int64_t T, int32_t n_q, int32_t n_kv,
                            uint16_t* out, uint16_t* vt, hipStream_t st) {
  const int ld = (n_q + 2 * n_kv) * D;
  const int Tp = (int)((T + KT - 1) / KT * KT);
  v_transpose_kernel<<<dim3((uint32_t)(Tp / 64), (uint32_t)(n_kv * D / 64)), 256, 0, st>>>(
      qkv, (int)T, ld, (n_q + n_kv) * D, Tp, vt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rep = n_q / n_kv, n_hg = (rep + 3) / 4;
  const int nqb = (int)((T + QB - 1) / QB);
  const float c_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  attention_kernel<<<dim3((uint32_t)(nqb * n_kv * n_hg)), 256, 0, st>>>(
      qkv, vt, out, (int)T, ld, n_q, n_kv, Tp, n_hg, c_log2);
  return hipGetLastError();
}

}  // namespace fp8moe
