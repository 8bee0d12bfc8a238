// Top-k routing and the grouping of routed (token, expert) pairs by expert
// (moe_route_permute).
//
// "FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant", section 1, replaces one
// dispatch per routed token with one grouped expert GEMM per layer. That GEMM needs the
// routed pairs grouped by expert and each expert's row range, computed on the device so
// the host never waits for the routing.
//
// Design: a stable counting sort with no order-dependent atomics, so every output is a
// pure function of the logits.
//   1. topk_hist:  one wave per token selects the top k by (logit desc, expert asc): each
//                  pick is the wave maximum of the order-preserving logit bits (32-bit, DPP
//                  max steps), then the lowest expert index holding it (a ballot); a
//                  workgroup of 16 waves owns a chunk of 16 tokens and counts its pairs per
//                  expert in LDS (integer adds commute).
//   2. chunk_scan: one workgroup per expert scans that expert's per-chunk counts (for
//                  small count tables the scatter workgroups do this themselves).
//   3. scatter:    one workgroup per chunk recomputes the expert offsets (a scan over E),
//                  ranks each pair among the chunk's earlier pairs of the same expert and
//                  writes sorted[] and pos[].
//   4. gather:     optional copies of the e4m3 rows and (group-major) scales into grouped
//                  order.
// A batch of one chunk (at most 16 tokens, decode sizes) skips steps 2 and 3 as launches:
// its top-k workgroup scans its own histogram and places the pairs itself.
#include <mutex>

#include "common.h"
#include "launch.h"
#include "quant_group.h"

namespace fp8moe {
namespace {

// Workspace of the allocation-free routing call (per-chunk expert counts and the expert
// totals). Every GPU the library runs on holds its own copy until the process ends. In
// host code this name only stands in for the array: the device address comes from
// hipGetSymbolAddress, per device, in route_scratch().
static __device__ __align__(256) uint8_t scratch[kRouteScratchBytes];

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;

// Inclusive scan of one int per thread over a 256-thread workgroup.
__device__ __forceinline__ int block_inclusive_scan256(int v, int* tmp /*[4]*/) {
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

// Orderable bits of a logit: a larger value is a larger unsigned number (negatives flipped,
// -0 taken as +0, since they compare equal); -inf stays above 0, the mark of a taken expert.
__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b << 1) == 0u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_value(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false));
}

// Largest value of the wave, wave-uniform: row_shr steps carry each 16-lane row's maximum
// into its last lane, row_bcast:15 and row_bcast:31 carry them into lane 63; VALU only.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max<0x111>(v);  // row_shr:1
  v = dpp_max<0x112>(v);  // row_shr:2
  v = dpp_max<0x114>(v);  // row_shr:4
  v = dpp_max<0x118>(v);  // row_shr:8
  v = dpp_max<0x142>(v);  // row_bcast:15
  v = dpp_max<0x143>(v);  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// Rank of a routed pair among the earlier pairs of its chunk routed to the same expert, the
// order a stable grouping keeps. A token's k picks are distinct experts, so those earlier
// pairs are one per earlier token of the chunk that picked the expert: with bit t of
// `mask` set when token t of the chunk picked it (set by LDS ORs, which commute), the rank
// is the number of bits below the pair's own token.
__device__ __forceinline__ int chunk_rank(uint32_t mask, int token_in_chunk) {
  static_assert(kRouteChunk <= 32, "one mask bit per token of the chunk");
  return __popc(mask & ((1u << token_in_chunk) - 1u));
}

// Top-k of each token and the per-chunk expert histogram. A workgroup owns a chunk of
// kRouteChunk tokens, one wave per token (the k picks of a token are a dependent chain,
// so the tokens of a chunk run side by side); lane e holds experts e, e+64, ... The wave
// picks the k best one at a time: the wave maximum of the orderable values of the untaken
// experts, then, among the experts holding it, the lowest index (a ballot per lane slot,
// the lowest slot and lane first), whose value is cleared.
//
// One chunk only (T <= kRouteChunk, offsets given): the grouping follows in the same
// workgroup. The exclusive scan of the histogram is the expert offsets, and routed pair i
// (token-major) goes to grouped row offsets[e] + the number of pairs j < i routed to the
// same expert e (chunk_rank): the rows the separate scan and scatter launches give a first
// chunk.
template <int NJ>  // experts per lane: E <= 64 * NJ
__device__ __forceinline__ void topk_hist_block(const float* __restrict__ logits, int64_t T,
                                                int E, int k, int32_t* __restrict__ ids,
                                                float* __restrict__ wts,
                                                int32_t* __restrict__ cnt, int64_t blk,
                                                int* hist /* LDS [kMaxE] */,
                                                int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ sorted,
                                                int32_t* __restrict__ pos) {
  static_assert(kMaxE == kRouteChunk * 64, "one expert per thread in the one-chunk scan");
  __shared__ uint32_t s_mask[kMaxE];  // one chunk: bit t set if token t picked the expert
  __shared__ int s_wtot[kRouteChunk];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += kRouteChunk * 64) {
    hist[e] = 0;
    if (offsets != nullptr) s_mask[e] = 0u;
  }
  int pick = -1;  // this lane's expert, lanes < k of a wave with a token
  __syncthreads();
  const int64_t t = blk * kRouteChunk + wv;
  if (t < T) {  // wave-uniform
    // orderable values of this lane's experts; a taken expert's becomes 0
    uint32_t val[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      float lv = e < E ? logits[t * E + e] : -INFINITY;
      if (lv != lv) lv = -INFINITY;  // NaN ranks as -inf: every pick stays a valid expert
      val[j] = e < E ? order_bits(lv) : 0u;
    }
    float my_v = -INFINITY, top_v = 0.f;
    int my_i = 0;
    for (int s = 0; s < k; ++s) {
      uint32_t best = val[0];
#pragma unroll
      for (int j = 1; j < NJ; ++j) best = max(best, val[j]);
      const uint32_t m = wave_max_u32(best);
      // the lowest expert index holding m: slot j first (experts 64 j + lane), then lane
      int bi = 0;
#pragma unroll
      for (int j = NJ - 1; j >= 0; --j) {
        const uint64_t hit = __ballot(val[j] == m);
        if (hit) bi = 64 * j + (int)__builtin_ctzll(hit);
      }
      bi = __builtin_amdgcn_readfirstlane(bi);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        if (bi == lane + 64 * j) val[j] = 0u;
      const float bv = order_value(m);
      if (lane == s) {
        my_v = bv;
        my_i = bi;
      }
      if (s == 0) top_v = bv;
    }
    // renormalised softmax over the k picks
    const float ex = lane < k ? expf(my_v - top_v) : 0.f;
    float sum = ex;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane < k) {
      ids[t * k + lane] = my_i;
      wts[t * k + lane] = ex / sum;
      atomicAdd(&hist[my_i], 1);
      if (offsets != nullptr) atomicOr(&s_mask[my_i], 1u << wv);  // blk = 0: token wv
      pick = my_i;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteChunk * 64)
    cnt[blk * E + e] = hist[e];
  if (offsets == nullptr) return;  // uniform (a kernel argument)
  // exclusive scan of the histogram, one expert per thread: within each wave, then the
  // totals of the earlier waves
  const int e = threadIdx.x;
  const int v = e < E ? hist[e] : 0;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o);
    if (lane >= o) inc += u;
  }
  if (lane == 63) s_wtot[wv] = inc;
  __syncthreads();
  for (int j = 0; j < wv; ++j) inc += s_wtot[j];
  if (e < E) {
    hist[e] = inc - v;  // thread e alone read hist[e], before the barrier
    offsets[e] = inc - v;
  }
  if (e == E - 1) offsets[E] = inc;  // = T * k
  __syncthreads();
  if (pick >= 0) {  // pair wv * k + lane
    const int row = hist[pick] + chunk_rank(s_mask[pick], wv);
    sorted[row] = wv * k + lane;
    pos[wv * k + lane] = row;
  }
}


template <int NJ>
__global__ __launch_bounds__(kRouteChunk * 64) void topk_hist_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ wts, int32_t* __restrict__ cnt, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
  __shared__ int hist[kMaxE];
  topk_hist_block<NJ>(logits, T, E, k, ids, wts, cnt, blockIdx.x, hist, offsets, sorted, pos);
}

// The group quantiser and the top-k selection in one launch: they are independent (the
// activations and the router logits), the top-k is bound by its dependent pick chains and
// the quantiser by HBM, so the first C workgroups (one chunk of tokens each) pick while
// the rest quantise, each of those acting as four 256-thread quantiser blocks, each
// thread with kQuantRouteChunks chunks in flight (as many as the standalone quantiser's:
// with the 32-bit pick, four or eight measured slower). Every output is the one the two
// separate launches produce.
constexpr int kQuantRouteChunks = 2;
template <int NJ>
__global__ __launch_bounds__(kRouteChunk * 64) void quant_topk_kernel(
    const uint4* __restrict__ x, int64_t nchunks, uint2* __restrict__ q,
    float* __restrict__ scales, float* __restrict__ sums, int64_t nqblocks,
    const float* __restrict__ logits, int64_t T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ wts, int32_t* __restrict__ cnt, int64_t C, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
  static_assert(kRouteChunk * 64 == 4 * 256, "one workgroup = four quantiser blocks");
  __shared__ int hist[kMaxE];
  const int64_t b = blockIdx.x;
  if (b < C) {
    topk_hist_block<NJ>(logits, T, E, k, ids, wts, cnt, b, hist, offsets, sorted, pos);
  } else {
    const int tid = (int)threadIdx.x;
    qg::group_block<kQuantRouteChunks>(x, nchunks, q, scales, sums, (b - C) * 4 + (tid >> 8),
                                       nqblocks, tid & 255);
  }
}

// One workgroup per expert: exclusive scan of its count over the chunks (in place) and
// the expert's total.
__global__ __launch_bounds__(256) void chunk_scan_kernel(int32_t* __restrict__ cnt, int64_t C,
                                                         int E, int32_t* __restrict__ tot) {
  __shared__ int tmp[4];
  __shared__ int tile_sum;
  const int e = blockIdx.x;
  int carry = 0;
  for (int64_t base = 0; base < C; base += 256) {
    int64_t c = base + threadIdx.x;
    int v = c < C ? cnt[c * E + e] : 0;
    int inc = block_inclusive_scan256(v, tmp);
    if (c < C) cnt[c * E + e] = carry + inc - v;
    if (threadIdx.x == 255) tile_sum = inc;
    __syncthreads();
    carry += tile_sum;
    __syncthreads();
  }
  if (threadIdx.x == 0) tot[e] = carry;
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ ids,
                                                      int64_t T, int E, int k,
                                                      const int32_t* __restrict__ cbase,
                                                      const int32_t* __restrict__ tot,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted,
                                                      int32_t* __restrict__ pos) {
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_e[kRouteChunk * kMaxK];
  __shared__ uint32_t s_mask[kMaxE];  // bit t: token t of the chunk picked the expert
  __shared__ int tmp[4];
  for (int e = threadIdx.x; e < E; e += 256) s_mask[e] = 0u;  // ordered by the scan's barriers
  // expert offsets: exclusive scan of the totals, 4 experts per thread
  int loc[4];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int e = threadIdx.x * 4 + j;
    loc[j] = e < E ? tot[e] : 0;
    sum += loc[j];
  }
  int inc = block_inclusive_scan256(sum, tmp);
  int run = inc - sum;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int e = threadIdx.x * 4 + j;
    if (e < E) s_off[e] = run;
    run += loc[j];
  }
  if (threadIdx.x == 255) s_off[E] = inc;  // = T*k
  const int64_t c = blockIdx.x;
  const int64_t p0 = c * kRouteChunk * k;
  int64_t pend = (c + 1) * kRouteChunk;
  if (pend > T) pend = T;
  const int np = (int)(pend * k - p0);
  for (int i = threadIdx.x; i < np; i += 256) {
    const int e = ids[p0 + i];
    s_e[i] = e;
    atomicOr(&s_mask[e], 1u << (i / k));
  }
  __syncthreads();
  if (c == 0)
    for (int e = threadIdx.x; e <= E; e += 256) offsets[e] = s_off[e];
  for (int i = threadIdx.x; i < np; i += 256) {
    const int e = s_e[i];
    const int rank = chunk_rank(s_mask[e], i / k);
    int row = s_off[e] + cbase[c * E + e] + rank;
    sorted[row] = (int32_t)(p0 + i);
    pos[p0 + i] = row;
  }
}

// Small count tables (C * E <= kScanInScatter, E <= 256): the scan is done by the scatter
// workgroups themselves, one launch fewer. Workgroup c sums the raw table: every expert's
// total (for the expert offsets) and its count over the chunks before c (the chunk's base),
// 256 / E threads per expert over interleaved chunks, then adds the slices in a fixed order.
// The rows come out identical to the separate scan and scatter (integer sums).
constexpr int64_t kScanInScatter = 65536;
__global__ __launch_bounds__(256) void scatter_scan_kernel(const int32_t* __restrict__ ids,
                                                           int64_t T, int E, int k,
                                                           const int32_t* __restrict__ cnt,
                                                           int64_t C,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted,
                                                           int32_t* __restrict__ pos) {
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_base[256];
  __shared__ int s_tot[256], s_bef[256];
  __shared__ int s_e[kRouteChunk * kMaxK];
  __shared__ uint32_t s_mask[256];  // bit t: token t of the chunk picked the expert
  __shared__ int tmp[4];
  const int64_t c = blockIdx.x;
  const int t = threadIdx.x;
  const int S = 256 / E;  // threads per expert
  if (t < E) s_mask[t] = 0u;  // ordered by the barriers below
  {
    const int e = t % E, sl = t / E;
    int tot = 0, bef = 0;
    if (sl < S) {
#pragma unroll 8
      for (int64_t cc = sl; cc < C; cc += S) {
        const int v = cnt[cc * E + e];
        tot += v;
        bef += cc < c ? v : 0;
      }
    }
    s_tot[t] = tot;
    s_bef[t] = bef;
  }
  __syncthreads();
  if (t < E) {
    int tot = 0, bef = 0;
    for (int sl = 0; sl < S; ++sl) {
      tot += s_tot[sl * E + t];
      bef += s_bef[sl * E + t];
    }
    s_base[t] = bef;
    s_tot[t] = tot;  // slice 0 of expert t is only read by thread t, above
  }
  __syncthreads();
  // expert offsets: exclusive scan of the totals, one expert per thread
  const int tv = t < E ? s_tot[t] : 0;
  const int inc = block_inclusive_scan256(tv, tmp);
  if (t < E) s_off[t] = inc - tv;
  if (t == 255) s_off[E] = inc;  // = T*k
  const int64_t p0 = c * kRouteChunk * k;
  int64_t pend = (c + 1) * kRouteChunk;
  if (pend > T) pend = T;
  const int np = (int)(pend * k - p0);
  for (int i = t; i < np; i += 256) {
    const int e = ids[p0 + i];
    s_e[i] = e;
    atomicOr(&s_mask[e], 1u << (i / k));
  }
  __syncthreads();
  if (c == 0)
    for (int e = t; e <= E; e += 256) offsets[e] = s_off[e];
  for (int i = t; i < np; i += 256) {
    const int e = s_e[i];
    const int rank = chunk_rank(s_mask[e], i / k);
    const int row = s_off[e] + s_base[e] + rank;
    sorted[row] = (int32_t)(p0 + i);
    pos[p0 + i] = row;
  }
}

// Grouped row i <- token sorted[i] / k: its e4m3 row (H bytes), 16 bytes per thread.
__global__ __launch_bounds__(256) void gather_rows_kernel(const int32_t* __restrict__ sorted,
                                                          int k, int64_t R, int64_t H,
                                                          const uint4* __restrict__ xq,
                                                          uint4* __restrict__ xq_perm) {
  const int64_t per_row = H / 16;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = j / per_row;
  if (row < R) {
    const int64_t tok = sorted[row] / k;
    xq_perm[j] = xq[tok * per_row + (j - row * per_row)];
  }
}

// Scales of grouped row i, group-major: xs_perm[g * R + i] = xs[(sorted[i] / k) * G + g].
// One thread per (g, i), consecutive threads on consecutive grouped rows.
// [T, G] per-token values -> [G, R] group-major in grouped row order, for the scales and,
// when given, the code sums in the same pass
__global__ __launch_bounds__(256) void gather_scales_kernel(const int32_t* __restrict__ sorted,
                                                            int k, int64_t R, int64_t G,
                                                            const float* __restrict__ xs,
                                                            float* __restrict__ xs_perm,
                                                            const float* __restrict__ xsum,
                                                            float* __restrict__ xsum_perm) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < R * G) {
    const int64_t g = j / R, row = j - g * R;
    const int64_t src = (int64_t)(sorted[row] / k) * G + g;
    // copied as 32-bit words: the same gather serves fp32 scales and packed E8M0 bytes
    reinterpret_cast<uint32_t*>(xs_perm)[j] = reinterpret_cast<const uint32_t*>(xs)[src];
    if (xsum) xsum_perm[j] = xsum[src];
  }
}

}  // namespace

hipError_t route_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t route_workspace_bytes(int64_t T, int32_t E) {
  int64_t C = (T + kRouteChunk - 1) / kRouteChunk;
  size_t n = (size_t)(C * E + E) * sizeof(int32_t);
  return (n + 255) & ~(size_t)255;
}

namespace {

// chunk scan, scatter and the optional gathers, after the top-k and histogram launch
hipError_t launch_route_tail(int64_t T, int32_t E, int32_t k, const int32_t* ids,
                             int32_t* offsets, int32_t* sorted, int32_t* pos, const uint8_t* xq,
                             const float* xs, int64_t H, uint8_t* xq_perm, float* xs_perm,
                             const float* xsum, float* xsum_perm, void* ws, hipStream_t st) {
  const int64_t C = (T + kRouteChunk - 1) / kRouteChunk;
  int32_t* cnt = static_cast<int32_t*>(ws);
  int32_t* tot = cnt + C * E;
  hipError_t e = hipSuccess;
  if (C == 1) {
    // one chunk: the top-k workgroup has already written offsets, sorted and pos
  } else if (E <= 256 && C * E <= kScanInScatter) {
    scatter_scan_kernel<<<dim3((uint32_t)C), 256, 0, st>>>(ids, T, E, k, cnt, C, offsets,
                                                           sorted, pos);
  } else {
    chunk_scan_kernel<<<dim3((uint32_t)E), 256, 0, st>>>(cnt, C, E, tot);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    scatter_kernel<<<dim3((uint32_t)C), 256, 0, st>>>(ids, T, E, k, cnt, tot, offsets, sorted,
                                                      pos);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t R = T * k;
  if (xq != nullptr) {
    const int64_t n = R * (H / 16);
    gather_rows_kernel<<<dim3((uint32_t)((n + 255) / 256)), 256, 0, st>>>(
        sorted, k, R, H, reinterpret_cast<const uint4*>(xq), reinterpret_cast<uint4*>(xq_perm));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (xs != nullptr) {
    const int64_t n = R * (H / kGroup);
    gather_scales_kernel<<<dim3((uint32_t)((n + 255) / 256)), 256, 0, st>>>(
        sorted, k, R, H / kGroup, xs, xs_perm, xsum, xsum_perm);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_route_permute(const float* logits, int64_t T, int32_t E, int32_t k,
                                int32_t* ids, float* w, int32_t* offsets, int32_t* sorted,
                                int32_t* pos, const uint8_t* xq, const float* xs, int64_t H,
                                uint8_t* xq_perm, float* xs_perm, const float* xsum,
                                float* xsum_perm, void* ws, hipStream_t st) {
  int64_t C = (T + kRouteChunk - 1) / kRouteChunk;
  int32_t* cnt = static_cast<int32_t*>(ws);
  const dim3 grid((uint32_t)C), block(kRouteChunk * 64);
  // one chunk: the top-k workgroup also writes the grouping
  int32_t* o1 = C == 1 ? offsets : nullptr;
  int32_t* s1 = C == 1 ? sorted : nullptr;
  int32_t* p1 = C == 1 ? pos : nullptr;
  if (E <= 64)
    topk_hist_kernel<1><<<grid, block, 0, st>>>(logits, T, E, k, ids, w, cnt, o1, s1, p1);
  else if (E <= 256)
    topk_hist_kernel<4><<<grid, block, 0, st>>>(logits, T, E, k, ids, w, cnt, o1, s1, p1);
  else
    topk_hist_kernel<16><<<grid, block, 0, st>>>(logits, T, E, k, ids, w, cnt, o1, s1, p1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_route_tail(T, E, k, ids, offsets, sorted, pos, xq, xs, H, xq_perm, xs_perm,
                           xsum, xsum_perm, ws, st);
}

hipError_t launch_quant_route(const uint16_t* x, int64_t H, uint8_t* q, float* scales,
                              float* sums, const float* logits, int64_t T, int32_t E,
                              int32_t k, int32_t* ids, float* w, int32_t* offsets,
                              int32_t* sorted, int32_t* pos, void* ws, hipStream_t st) {
  const int64_t C = (T + kRouteChunk - 1) / kRouteChunk;
  const int64_t nchunks = T * H / 8;
  // quantiser workgroups of four 256-thread blocks, each thread kQuantRouteChunks chunks
  const int64_t nq = (nchunks + 4 * 256 * kQuantRouteChunks - 1) / (4 * 256 * kQuantRouteChunks);
  int32_t* cnt = static_cast<int32_t*>(ws);
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint2* qv = reinterpret_cast<uint2*>(q);
  const dim3 grid((uint32_t)(C + nq)), block(kRouteChunk * 64);
  int32_t* o1 = C == 1 ? offsets : nullptr;  // one chunk: the grouping in the same launch
  int32_t* s1 = C == 1 ? sorted : nullptr;
  int32_t* p1 = C == 1 ? pos : nullptr;
  if (E <= 64)
    quant_topk_kernel<1><<<grid, block, 0, st>>>(xv, nchunks, qv, scales, sums, 4 * nq, logits,
                                                  T, E, k, ids, w, cnt, C, o1, s1, p1);
  else if (E <= 256)
    quant_topk_kernel<4><<<grid, block, 0, st>>>(xv, nchunks, qv, scales, sums, 4 * nq, logits,
                                                  T, E, k, ids, w, cnt, C, o1, s1, p1);
  else
    quant_topk_kernel<16><<<grid, block, 0, st>>>(xv, nchunks, qv, scales, sums, 4 * nq,
                                                   logits, T, E, k, ids, w, cnt, C, o1, s1, p1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_route_tail(T, E, k, ids, offsets, sorted, pos, nullptr, nullptr, H, nullptr,
                           nullptr, nullptr, nullptr, ws, st);
}

}  // namespace fp8moe
