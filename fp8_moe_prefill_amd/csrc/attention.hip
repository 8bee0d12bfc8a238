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
//   (double-buffered) and shared by the four waves; a tile's global loads are issued two
//   tiles ahead into one of two register sets (one tile of compute is shorter than the
//   load latency);
// * each wave computes S^T = K Q^T (v_mfma_f32_16x16x32_bf16, keys as rows), so a lane's
//   scores all belong to one query: the running max, the rescale of the output and the
//   row sum need no lane exchange except the 4-lane max per tile;
// * O^T = V^T P^T: P leaves the S^T accumulators as the B operand directly (same lane),
//   split into two bf16 terms hi + lo so that the product keeps the fp32 softmax's
//   accuracy (a single bf16 rounding of the weights would cost 2^-9 relative); V^T comes
//   from LDS; the output accumulators are again per query;
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
constexpr int NQT = 1;        // 16-query MFMA tiles per wave
constexpr int QB = 16 * NQT;  // queries per workgroup
constexpr int KT = 64;        // keys per tile
constexpr int KS = D * 2 + 16;   // K tile row stride in LDS (bytes): 256 + 16 pad
constexpr int VS = KT * 2;       // V^T tile row stride in LDS (bytes): 64 keys, no pad
// V^T tile rows are XOR-swizzled in 8-byte slots (4 keys): slot s of row d sits at
// position s ^ (d % 16), so the 16 rows one operand read touches hit distinct banks.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

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

// [T, ld] column block of V (kv head j) -> vt[j][d][t], zero for t in [T, Tp)
__global__ __launch_bounds__(256) void v_transpose_kernel(const uint16_t* __restrict__ qkv,
                                                          int T, int ld, int v_col0, int Tp,
                                                          uint16_t* __restrict__ vt) {
  __shared__ uint16_t tile[64][65];
  const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 64;  // c: column within the V block
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int t = t0 + r;
    tile[r][tx] = t < T ? qkv[(int64_t)t * ld + v_col0 + c0 + tx] : (uint16_t)0;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) vt[(int64_t)(c0 + r) * Tp + t0 + tx] = tile[tx][r];
}

__global__ __launch_bounds__(256, 2) void attention_kernel(const uint16_t* __restrict__ qkv,
                                                           const uint16_t* __restrict__ vt,
                                                           uint16_t* __restrict__ out, int T,
                                                           int ld, int n_q, int n_kv, int Tp,
                                                           int n_hg, float c_log2) {
  __shared__ __attribute__((aligned(16))) uint8_t sK[2][KT * KS];
  __shared__ __attribute__((aligned(16))) uint8_t sV[2][D * VS];
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

  // Q fragments: lane (g, c16) holds query q0 + 16 qt + c16, dims 32 kk + 8 g .. +7
  bf16x8_t qf[NQT][4];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int t = min(q0 + 16 * qt + c16, T - 1);
    const uint16_t* src = qkv + (int64_t)t * ld + h * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[qt][kk] = as_bf16x8(*reinterpret_cast<const uint4*>(src + 32 * kk));
  }

  // staging of one key tile: K rows (64 x 256 B) and V^T rows (128 x 128 B), 4 chunks of
  // 16 B each per thread
  const uint16_t* kbase = qkv + (n_q + j) * D;
  const uint16_t* vbase = vt + (int64_t)j * D * Tp;
  // two register sets for tiles in flight: the global loads of a tile are issued two
  // iterations before it is used (one iteration of compute does not cover the load
  // latency); set indices are compile-time constants, so they stay in registers
  // (native vector types: arrays of the HIP uint4 struct were kept in scratch memory)
  u32x4 rk0[4], rv0[4], rk1[4], rv1[4];
  auto load_tile = [&](auto set_tag, int kt) {
    constexpr int S = decltype(set_tag)::value;
    u32x4* rk = S ? rk1 : rk0;
    u32x4* rv = S ? rv1 : rv0;
    const int k0 = kt * KT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int key = min(k0 + (c >> 4), T - 1);
      rk[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * ld + (c & 15) * 8);
      rv[i] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)(c >> 3) * Tp + k0 + (c & 7) * 8);
    }
  };
  auto store_tile = [&](auto set_tag, int buf) {
    constexpr int S = decltype(set_tag)::value;
    const u32x4* rk = S ? rk1 : rk0;
    const u32x4* rv = S ? rv1 : rv0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<u32x4*>(&sK[buf][(c >> 4) * KS + (c & 15) * 16]) = rk[i];
      // 16-byte chunk j of row d holds slots 2j, 2j + 1: they land as chunk j ^ (sg / 2),
      // in swapped order when sg is odd
      const int d = c >> 3, sg = d & 15;
      const u32x4 v = (sg & 1) ? rv[i].zwxy : rv[i];
      *reinterpret_cast<u32x4*>(&sV[buf][d * VS + ((c & 7) ^ (sg >> 1)) * 16]) = v;
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  v4f o[NQT][8];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[qt][dt] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run[NQT], l_part[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) m_run[qt] = -INFINITY, l_part[qt] = 0.f;

  // tile kt: loaded into register set kt % 2 at iteration kt - 2 (the prologue for tiles 0
  // and 1), stored into LDS stage kt % 2 at the end of iteration kt - 1, computed at
  // iteration kt
  load_tile(I0{}, 0);
  store_tile(I0{}, 0);
  if (nkt > 1) load_tile(I1{}, 1);
  __syncthreads();

  auto step = [&](auto par_tag, int kt) {
    constexpr int P = decltype(par_tag)::value;  // kt % 2
    const int cur = P;
    if (kt + 2 < nkt) load_tile(par_tag, kt + 2);  // set P held tile kt, already in LDS

    // S^T[key 16 s + 4 g + r][query 16 qt + c16], s = 16-key subtile
    v4f st[NQT][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) st[qt][s] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8_t a = as_bf16x8(
            *reinterpret_cast<const uint4*>(&sK[cur][(16 * s + c16) * KS + kk * 64 + g * 16]));
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
          st[qt][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[qt][kk], st[qt][s], 0, 0, 0);
      }
    }

    // online softmax in the log2 domain; only the last tile can hold keys past a query
    const bool diag = kt == nkt - 1;
    bf16x8_t pb[NQT][2], pl[NQT][2];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int qi = q0 + 16 * qt + c16;
      float mx = -INFINITY;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = st[qt][s][r] * c_log2;
          if (diag && kt * KT + 16 * s + 4 * g + r > qi) v = -INFINITY;
          st[qt][s][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = max4q(mx);
      const float m_new = fmaxf(m_run[qt], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_new);
      m_run[qt] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // p enters P.V as hi + lo, two bf16 terms (about 16 significant bits): the
          // product keeps fp32-level accuracy on the bf16 matrix cores
          const float p = __builtin_amdgcn_exp2f(st[qt][s][r] - m_new);
          const __bf16 hi = (__bf16)p;
          ls += p;
          pb[qt][s >> 1][4 * (s & 1) + r] = hi;
          pl[qt][s >> 1][4 * (s & 1) + r] = (__bf16)(p - (float)hi);
        }
      l_part[qt] = l_part[qt] * alpha + ls;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {  // uniform: some query's max moved
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[qt][dt] *= alpha;
      }
    }

    // O^T[d 16 dt + 4 g + r][query 16 qt + c16] += V^T P^T over two 32-key steps; the key
    // slots of lane group g are 32 c + 4 g + 0..3 and 32 c + 16 + 4 g + 0..3 for both
    // operands
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint8_t* vrow = &sV[cur][(16 * dt + c16) * VS];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + ((8 * c + g) ^ c16) * 8);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + ((8 * c + 4 + g) ^ c16) * 8);
        const bf16x8_t a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
          o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[qt][c], o[qt][dt], 0, 0, 0);
          o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl[qt][c], o[qt][dt], 0, 0, 0);
        }
      }
    }

    if (kt + 1 < nkt) store_tile(std::integral_constant<int, P ^ 1>{}, cur ^ 1);
    __syncthreads();
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    step(I0{}, kt);
    if (kt + 1 < nkt) step(I1{}, kt + 1);
  }

  if (!live) return;
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const float l = sum4q(l_part[qt]);
    const int qi = q0 + 16 * qt + c16;
    if (qi >= T) continue;
    const float inv = 1.f / l;
    uint16_t* dst = out + (int64_t)qi * (n_q * D) + h * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const v4f v = o[qt][dt] * inv;
      *reinterpret_cast<uint2*>(dst + 16 * dt) = make_uint2(bf16x2(v[0], v[1]), bf16x2(v[2], v[3]));
    }
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
