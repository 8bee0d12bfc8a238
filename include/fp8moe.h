/*
 * fp8moe.h -- C ABI of the FP8 (OCP e4m3fn) MoE prefill library for AMD Instinct
 * MI355X (gfx950).
 *
 * The library computes the hot path of an FP8 grouped-expert MoE prefill layer and the
 * W8A8 dense projections next to it:
 *
 *   fp8_quant_act            bf16 activations -> e4m3 codes + fp32 scales
 *   moe_route_permute        router logits -> top-k experts, weights, expert offsets,
 *                            the grouped (permuted) row order
 *   fp8_grouped_expert_gemm  one launch over all experts: e4m3 rows x packed-int4 bank
 *                            (dequantised to e4m3 on-chip), scales folded into the fp32
 *                            accumulator; optional fused SwiGLU + e4m3 requantisation
 *   fp8_dense_gemm           W8A8 GEMM with per-tensor activation and weight scales
 *   moe_unpermute_combine    weighted sum of each token's k expert rows
 *   fp8moe_quant_route       fp8_quant_act (group mode) and moe_route_permute of one
 *                            layer in one call (the quantiser beside the top-k)
 *
 * quantisation variants of those ([P2] "Limits"; [P4] the block-128 e4m3 class):
 *
 *   fp8_dense_gemm_rowwise     W8A8 GEMM with one activation scale per row
 *   fp8_quant_weight_block128  bf16 weight -> e4m3 codes + one fp32 scale per 128 x 128
 *   fp8_block_gemm             e4m3 GEMM on block-128 weights, per-(row, 128) activations
 *   mxfp4_quant_act            bf16 activations -> MXFP4 (E2M1 codes + E8M0 scale per 32)
 *   fp8moe_pack_expert_bank_mxfp4  the expert bank packed for MXFP4 activations
 *   mxfp4_grouped_expert_gemm  the grouped expert GEMM with MXFP4 activations
 *
 * and, for the depth stack those layers sit in ([P1] section 3):
 *
 *   fp8moe_rmsnorm           residual add + RMSNorm, bf16 in and out
 *   fp8moe_bf16_gemm         bf16 x bf16 -> fp32 GEMM (router, LM head)
 *   fp8moe_causal_attention  causal grouped-query attention, bf16 in and out
 *
 * Sources (by page title and section):
 *   [P1] "FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant"
 *        (octopusresearch.org), section 1 Contribution.
 *   [P2] FreeToken PR #389 "load-time per-tensor FP8 dense projections (W8A8 via
 *        _scaled_mm)", sections "What this adds" and "Limits".
 *   [P3] DeepGEMM issue 338 (mirrored as #166), "[RFC] Support FP4 (E2M1) activation
 *        dispatch in MegaMoE", body (E2M1 activations to halve the dispatch buffer and run
 *        an MXF4 main loop).
 *   [P4] memra-engine fp8_ffi module docs (docs.rs), module text and struct Fp8Scratch.
 *   [P1] section 3 also names the depth stacks (L = 8 and 12) the note measures.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major, densely packed, owned by the
 *     caller. The library never allocates, frees or synchronises; scratch memory is a
 *     caller-provided workspace whose size fp8moe_workspace_bytes() reports.
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call only enqueues work
 *     on that stream and returns; there is no device-to-host synchronisation inside any
 *     call ([P2] "No host sync anywhere"; [P4] "no host sync anywhere"), so every call
 *     can be captured into a HIP graph.
 *   - Arguments are validated on the host before anything is enqueued; a non-zero status
 *     means nothing was launched. Value problems (NaN inputs, all-zero groups) are not
 *     errors: they follow the documented numeric policy, since checking them would need
 *     a host sync.
 *   - bf16 tensors are passed as `const void*` holding IEEE bf16 bit patterns.
 *   - e4m3 means OCP e4m3fn bytes: max 448, NaN = 0x7F/0xFF, no infinities.
 *     Quantisation rounds to nearest even, saturates to +-448 and keeps the sign of zero.
 *   - Alignment: every pointer must be 16-byte aligned.
 *   - Calls on different streams touching disjoint memory may run concurrently; the
 *     library keeps no global mutable state, except the device array behind
 *     moe_route_permute_noalloc (the one entry point that takes no workspace).
 */
#ifndef FP8MOE_H
#define FP8MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------------ */
#define FP8MOE_OK 0
#define FP8MOE_ERR_NULL (-1)         /* a required pointer is NULL                   */
#define FP8MOE_ERR_SHAPE (-2)        /* a size is out of range or not a multiple     */
#define FP8MOE_ERR_ALIGN (-3)        /* a pointer is not 16-byte aligned              */
#define FP8MOE_ERR_WORKSPACE (-4)    /* workspace smaller than fp8moe_workspace_bytes */
#define FP8MOE_ERR_UNSUPPORTED (-5)  /* an enum argument has an unknown value         */
#define FP8MOE_ERR_LAUNCH (-6)       /* the HIP runtime rejected a kernel launch      */

/* ---- enums ------------------------------------------------------------------- */
#define FP8MOE_GROUP 128             /* the K-group of every group-wise scale        */
#define FP8MOE_QUANT_ROW (-1)        /* fp8_quant_act group: one scale per row        */

#define FP8MOE_DTYPE_F32 0
#define FP8MOE_DTYPE_BF16 1

#define FP8MOE_EPI_STORE 0           /* write the folded fp32 accumulator            */
#define FP8MOE_EPI_SWIGLU_QUANT 1    /* h = silu(gate) * up, then e4m3 per (row,128)  */

/* ops for fp8moe_workspace_bytes */
#define FP8MOE_OP_QUANT_ACT 0
#define FP8MOE_OP_ROUTE_PERMUTE 1
#define FP8MOE_OP_ATTENTION 2

/* Version of this ABI (bumped on any signature change). */
int32_t fp8moe_abi_version(void);

/* Human-readable text of a status code (static storage, never NULL). */
const char* fp8moe_status_str(int32_t status);

/*
 * fp8moe_workspace_bytes -- device scratch an entry point needs.
 *   op = FP8MOE_OP_QUANT_ACT:      a = M, b = K, c = group (128, 0 or FP8MOE_QUANT_ROW)
 *   op = FP8MOE_OP_ROUTE_PERMUTE:  a = T, b = E, c = k
 *   op = FP8MOE_OP_ATTENTION:      a = T, b = n_kv, c = head_dim (128)
 * Returns 0 for an op that needs none, (size_t)-1 for invalid arguments.
 */
size_t fp8moe_workspace_bytes(int32_t op, int64_t a, int64_t b, int64_t c);

/*
 * fp8_quant_act -- dynamic activation quantisation to e4m3.
 *
 * [P1] section 1: a per-(token, group) activation scale; [P2] "What this adds": a
 * dynamic per-tensor activation scale (an amax pass, then the cast); [P4] module text:
 * the scale is amax/448; struct Fp8Scratch: a 4-float block {amax, quant mul, scale}.
 *
 *   x       bf16 [M, K]
 *   group   FP8MOE_GROUP (128): one scale per (row, 128 consecutive columns);
 *           0: one scale for the whole tensor;
 *           FP8MOE_QUANT_ROW: one scale per row ([P2] "Limits": row-wise scales)
 *   q       out, e4m3 [M, K]
 *   scales  out; group=128: fp32 [M, K/128], scale of (row m, group g) at m*K/128 + g;
 *           group=0: fp32[4] = {amax, 448/a, a/448, 0} with a = max(amax, 1e-12);
 *           FP8MOE_QUANT_ROW: fp32 [M], the scale a/448 of each row
 *   sums    optional out (group=128 only, else NULL): fp32 [M, K/128], the sum of the
 *           e4m3 code values of each (row, group), sum_k e4m3(q[m, k]) unscaled, in a fixed
 *           order in fp32. fp8_grouped_expert_gemm takes them (gathered into grouped order
 *           by moe_route_permute) in place of summing the rows itself.
 *   ws      workspace of fp8moe_workspace_bytes(FP8MOE_OP_QUANT_ACT, M, K, group)
 *           bytes (may be NULL if that is 0)
 * Arithmetic (fp32): a = max(max|x| over the group, 1e-12); s = a/448 and
 * inv = 448/a, both correctly rounded; q = e4m3(x * inv). NaN inputs encode to 0x7F
 * and are skipped by the amax.
 * Constraints: M >= 1, K >= 1; group=128 needs K % 128 == 0; group=0 needs
 * M*K % 8 == 0; FP8MOE_QUANT_ROW needs K % 8 == 0 and M < 2^31.
 */
int32_t fp8_quant_act(const void* x, int64_t M, int64_t K, int32_t group, uint8_t* q,
                      float* scales, float* sums, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_permute -- top-k routing and grouping of the routed (token, expert) pairs.
 *
 * [P1] section 1: per-token expert dispatch is replaced by one grouped GEMM per layer,
 * which needs the routed pairs grouped by expert with per-expert row offsets computed
 * on the device (no host round trip).
 *
 *   logits   fp32 [T, E]
 *   ids      out, int32 [T, k]: experts of token t by descending logit; equal logits
 *            go to the lower expert index first
 *   weights  out, fp32 [T, k]: softmax over the k selected logits (the top-k
 *            renormalised softmax)
 *   offsets  out, int32 [E+1]: expert e owns grouped rows offsets[e] .. offsets[e+1]-1;
 *            offsets[0] = 0, offsets[E] = T*k
 *   sorted   out, int32 [T*k]: grouped row i holds pair p = sorted[i] = t*k + j; within
 *            an expert pairs keep increasing p (a stable order)
 *   pos      out, int32 [T*k]: pos[p] = the grouped row of pair p
 *   xq, xq_perm    optional pair (both NULL or both set): e4m3 rows [T, H] gathered into
 *                  grouped order, xq_perm = e4m3 [T*k, H]
 *   xs, xs_perm    optional pair (both NULL or both set): fp32 scales [T, H/128] gathered
 *                  into grouped order, GROUP-MAJOR: xs_perm[g * T*k + i] is the scale of
 *                  group g of grouped row i (the layout fp8_grouped_expert_gemm reads)
 *   xsum, xsum_perm  optional pair, only with xs: fp32 code sums [T, H/128] (from
 *                  fp8_quant_act) gathered like the scales into [H/128, T*k]
 *   H              row width of xq / xs (needed when either pair is set)
 *   ws       workspace of fp8moe_workspace_bytes(FP8MOE_OP_ROUTE_PERMUTE, T, E, k)
 * Constraints: T >= 1, 1 <= E <= 1024, 1 <= k <= min(E, 32), T*k < 2^31;
 * H % 128 == 0 when gathering. Every output is a pure function of the inputs (no
 * order-dependent atomics), so repeated calls give identical bytes.
 */
int32_t moe_route_permute(const float* logits, int64_t T, int32_t E, int32_t k,
                          int32_t* ids, float* weights, int32_t* offsets, int32_t* sorted,
                          int32_t* pos, const uint8_t* xq, const float* xs, int64_t H,
                          uint8_t* xq_perm, float* xs_perm, const float* xsum,
                          float* xsum_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * fp8moe_quant_route -- fp8_quant_act in group mode (FP8MOE_GROUP, optional code sums)
 * of the layer's activations and moe_route_permute (no gathers) of its router logits in
 * one call.
 *
 * [P1] section 1 runs the activation quantiser and the routing/grouping ahead of the one
 * grouped GEMM per layer. The two read different inputs, so the library runs the
 * quantiser and the top-k selection in one launch (the top-k waits on dependent picks,
 * the quantiser on HBM) and then the rest of the routing (for T <= 16 that launch also
 * groups the pairs, and no other follows).
 *
 *   x, q, scales, sums   as fp8_quant_act with M = T, K = H, group = FP8MOE_GROUP
 *                        (sums may be NULL)
 *   logits .. pos        as moe_route_permute (no gathers: its xq/xs pairs are absent)
 *   ws                   workspace of fp8moe_workspace_bytes(FP8MOE_OP_ROUTE_PERMUTE, T,
 *                        E, k) bytes (the group quantiser needs none)
 * Every output is the one the two separate calls write, byte for byte.
 * Constraints: those of both calls: T >= 1, H >= 128, H % 128 == 0, T*H < 2^40,
 * 1 <= E <= 1024, 1 <= k <= min(E, 32), T*k < 2^31. x, q, scales, sums and ws 16-byte
 * aligned.
 */
int32_t fp8moe_quant_route(const void* x, int64_t T, int64_t H, uint8_t* q, float* scales,
                           float* sums, const float* logits, int32_t E, int32_t k,
                           int32_t* ids, float* weights, int32_t* offsets, int32_t* sorted,
                           int32_t* pos, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_permute_noalloc -- moe_route_permute without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, outputs, constraints and results are those of moe_route_permute, byte for
 * byte (the same kernels run). The workspace is a static device array of
 * FP8MOE_ROUTE_SCRATCH_BYTES that every GPU the library runs on holds from its first use
 * until the process ends; its device address is looked up once per device, on the first
 * call made with that device current. The call allocates and frees nothing.
 *   - Limit: fp8moe_workspace_bytes(FP8MOE_OP_ROUTE_PERMUTE, T, E, k) must not exceed
 *     FP8MOE_ROUTE_SCRATCH_BYTES (4 MiB: e.g. T = 65536 tokens at E = 256); larger calls
 *     return FP8MOE_ERR_WORKSPACE and launch nothing.
 *   - Every call on one GPU shares that GPU's array, and each call overwrites all of the
 *     part it reads before reading it (nothing carries over between calls). Calls that
 *     overlap in time on one GPU (different streams with no ordering between them) race
 *     on the array and give undefined results; order them on one stream, or use
 *     moe_route_permute with a workspace per stream.
 *   - FP8MOE_ERR_LAUNCH also reports a failure to look up the array's address.
 */
#define FP8MOE_ROUTE_SCRATCH_BYTES ((size_t)4 << 20)
int32_t moe_route_permute_noalloc(const float* logits, int64_t T, int32_t E, int32_t k,
                                  int32_t* ids, float* weights, int32_t* offsets,
                                  int32_t* sorted, int32_t* pos, const uint8_t* xq,
                                  const float* xs, int64_t H, uint8_t* xq_perm, float* xs_perm,
                                  const float* xsum, float* xsum_perm, void* stream);

/*
 * fp8moe_pack_expert_bank -- one-time repacking of a packed-int4 expert bank (and its
 * scales) into the layout fp8_grouped_expert_gemm streams. A byte permutation and a
 * transpose: nothing is dequantised or widened, the bank stays at 4 bits per weight.
 *
 * [P1] section 1: the int4 bank stays packed and resident and is converted to e4m3
 * on-chip; its nibble order and block layout are this library's choice (the pages fix
 * neither), made so that one wave-wide load brings one contiguous 1 KB block.
 *
 *   w                canonical bank, packed int4 [E, N, K/2], two's complement -8..7:
 *                    byte i of row (e, n) holds k = 2i in its low nibble and k = 2i+1 in
 *                    its high nibble
 *   w_scales         fp32 [E, N, K/128]
 *   w_packed         out, E*N*K/2 bytes. Block (e, c, g) of 1024 bytes, at byte
 *                    ((e * N/16 + c) * K/128 + g) * 1024, holds the 16 columns
 *                    n(c, i) = 64*(c/4) + 4*i + c%4 (i = 0..15) and k in [128g, 128g+128):
 *                    its 16 bytes at 16 * (16h + i) are column n(c, i),
 *                    k = 128g + 32h + 0..31, as four little-endian 32-bit words; byte b of
 *                    word j holds k0 + b in the low nibble and k0 + 4 + b in the high
 *                    nibble, k0 = 128g + 32h + 8j
 *   w_scales_packed  out, fp32 [E, K/128, N] (the scales of one K group contiguous)
 * The outputs must not overlap the inputs. Constraints: 1 <= E <= 1024, N % 64 == 0,
 * 128 <= K <= 16384, K % 128 == 0, N*K/2 < 2^32.
 */
int32_t fp8moe_pack_expert_bank(const uint8_t* w, const float* w_scales, int64_t E, int64_t N,
                                int64_t K, uint8_t* w_packed, float* w_scales_packed,
                                void* stream);

/*
 * fp8_grouped_expert_gemm -- one launch over every expert.
 *
 * [P1] section 1: a single grouped expert GEMM per layer; int4 weights turned into
 * e4m3 on-chip without unpacking the resident packed-int4 bank; one dynamic activation
 * scale per (token, K group), applied inside the fp32 accumulation.
 *
 * For grouped row i in expert e's range [offsets[e], offsets[e+1]) and column n:
 *   y[i, n] = sum_g s_a(i, g) * w_scales[e, n, g]
 *                   * sum_{k in group g} e4m3(a[r, k]) * int4(w[e, n, k])
 * with r = i, or r = sorted[i] / k_route when `sorted` is given. With `sorted` the A rows
 * are gathered on the fly from token order, and so are their scales and code sums: the
 * quantiser's outputs are read as they are, with no permuted copy of any of them.
 *
 *   a          e4m3 [Ra, K]  (Ra = R without `sorted`, Ra = R / k_route with it)
 *   a_scales   without `sorted`: fp32 [K/128, R], group-major, s_a(i, g) = a_scales[g*R + i];
 *              with it: fp32 [Ra, K/128] per token (fp8_quant_act's scales),
 *              s_a(i, g) = a_scales[r * K/128 + g]
 *   a_sums     NULL, or the sums of the e4m3 code values of each (row, group), laid out as
 *              a_scales (fp8_quant_act's sums with `sorted`, or a previous SWIGLU_QUANT
 *              launch's out_sums without it). The kernel otherwise sums the rows itself
 *              on the matrix core (one extra MFMA per 16 rows and group), a sum that may
 *              drop the lowest bits of tiny codes; both ways stay within the error bound.
 *   sorted     NULL, or int32 [R] pair ids from moe_route_permute
 *   k_route    experts per token (used only with `sorted`; R must then be a multiple of
 *              it, R = T * k_route)
 *   w          the bank as laid out by fp8moe_pack_expert_bank
 *   w_scales   its scales, fp32 [E, K/128, N] (fp8moe_pack_expert_bank's w_scales_packed)
 *   offsets    int32 [E+1] on the device (from moe_route_permute), offsets[E] = R
 *   R          total grouped rows (the host-side bound; not read back from offsets)
 *   epilogue   FP8MOE_EPI_STORE: out is [R, N] in out_dtype (fp32 or bf16, RNE);
 *              FP8MOE_EPI_SWIGLU_QUANT: N = 2I with gate columns 0..I-1 and up columns
 *              I..2I-1; h = silu(gate) * up in fp32 is quantised like fp8_quant_act
 *              (group 128) into out = e4m3 [R, I] and out_scales = fp32 [I/128, R],
 *              group-major like a_scales (ready to be the next GEMM's a_scales), and,
 *              when out_sums is not NULL, the code sums of h into out_sums = fp32
 *              [I/128, R] (ready to be the next GEMM's a_sums); out_sums must be NULL
 *              with STORE
 * Constraints: R >= 0 (R = 0 is a no-op; the row-sized buffers a, a_scales, a_sums, sorted,
 * out, out_scales, out_sums may then be NULL), 1 <= E <= 1024, K % 128 == 0,
 * 128 <= K <= 16384, R*K < 2^32, N*K/2 < 2^32, (ceil(R/128) + E) * ceil(N/256) < 2^28;
 * STORE: N % 64 == 0; SWIGLU_QUANT: N % 256 == 0.
 */
int32_t fp8_grouped_expert_gemm(const uint8_t* a, const float* a_scales,
                                const float* a_sums, const int32_t* sorted, int32_t k_route,
                                const uint8_t* w, const float* w_scales,
                                const int32_t* offsets, int64_t R, int32_t E, int64_t N,
                                int64_t K, int32_t epilogue, int32_t out_dtype, void* out,
                                float* out_scales, float* out_sums, void* stream);

/*
 * fp8_dense_gemm -- W8A8 projection y = (s_a * s_w) * (qa . qw^T).
 *
 * [P2] "What this adds": e4m3 weights with one fp32 scale per tensor, a dynamic
 * per-tensor activation scale, an FP8 x FP8 GEMM; [P4] module text: the two scales are
 * folded into one device scalar, with no host sync.
 *
 *   a            e4m3 [M, K] (from fp8_quant_act with group = 0)
 *   a_scale_blk  fp32[4] scale block from fp8_quant_act; element 2 (s_a) is used
 *   w            e4m3 [N, K]
 *   w_scale      fp32[1] on the device, s_w
 *   out          [M, N] fp32 or bf16 (RNE) per out_dtype
 * Constraints: M >= 1, N % 16 == 0, K % 128 == 0, M*K < 2^32, N*K < 2^32.
 */
int32_t fp8_dense_gemm(const uint8_t* a, const float* a_scale_blk, const uint8_t* w,
                       const float* w_scale, int64_t M, int64_t N, int64_t K,
                       int32_t out_dtype, void* out, void* stream);

/*
 * fp8_dense_gemm_rowwise -- W8A8 projection with one activation scale per row,
 * y[m, n] = (s_a[m] * s_w) * (qa[m] . qw[n]).
 *
 * [P2] "Limits": row-wise activation scales, measured there against the per-tensor route
 * (the same shapes, GEMM only).
 *
 *   a          e4m3 [M, K] (from fp8_quant_act with group = FP8MOE_QUANT_ROW)
 *   a_scales   fp32 [M] on the device, s_a of each row
 *   w, w_scale, out, out_dtype: as fp8_dense_gemm
 * Constraints: as fp8_dense_gemm.
 */
int32_t fp8_dense_gemm_rowwise(const uint8_t* a, const float* a_scales, const uint8_t* w,
                               const float* w_scale, int64_t M, int64_t N, int64_t K,
                               int32_t out_dtype, void* out, void* stream);

/*
 * fp8_quant_weight_block128 -- load-time quantisation of a weight to the block-128 e4m3
 * class: one fp32 scale per 128 x 128 block.
 *
 * [P4] fp8_blk_mmq_native_enabled / st_e4m3_blk_enabled: the block-128 e4m3 weight class
 * ("the Qwen-official FP8 class") with its own grid of block scales, read in place.
 *
 *   w       bf16 [N, K]
 *   q       out, e4m3 [N, K]
 *   scales  out, fp32 [ceil(N/128), K/128]; block (nb, g) covers rows 128 nb .. 128 nb + 127
 *           (fewer in the last row block when N % 128 != 0) and columns 128 g .. 128 g + 127
 * Arithmetic: fp8_quant_act's rule over each block. Constraints: N >= 1, K % 128 == 0,
 * ceil(N/128) < 65536.
 */
int32_t fp8_quant_weight_block128(const void* w, int64_t N, int64_t K, uint8_t* q,
                                  float* scales, void* stream);

/*
 * fp8_block_gemm -- e4m3 GEMM on block-128 weights:
 *   y[m, n] = sum_g s_a[m, g] * s_w[n / 128, g] * (qa[m, 128 g ..] . qw[n, 128 g ..]).
 *
 * [P4]: the block-128 e4m3 weight class read natively by a per-block FP8 tile. The pages do
 * not give the activation scaling of that path; this takes the per-(row, 128-wide K group)
 * scales of fp8_quant_act with group = 128 ([P1] section 1), so both scales are constant
 * inside every 128-wide K group and are folded into the fp32 accumulator group by group.
 *
 *   a          e4m3 [M, K] (fp8_quant_act, group = 128)
 *   a_scales   fp32 [M, K/128] (fp8_quant_act's group-mode layout)
 *   w          e4m3 [N, K], w_scales fp32 [ceil(N/128), K/128] (fp8_quant_weight_block128)
 *   out        [M, N] fp32 or bf16 (RNE) per out_dtype
 * Constraints: as fp8_dense_gemm, and K <= 16384.
 */
int32_t fp8_block_gemm(const uint8_t* a, const float* a_scales, const uint8_t* w,
                       const float* w_scales, int64_t M, int64_t N, int64_t K, int32_t out_dtype,
                       void* out, void* stream);

/*
 * mxfp4_quant_act -- bf16 activations -> MXFP4: E2M1 codes with one E8M0 scale per 32
 * consecutive elements.
 *
 * [P3]: E2M1 activations (packed by a pre-dispatch kernel) for an MXF4 main loop. The
 * pages give no formula; this is the OCP Microscaling (MX) v1.0 MXFP4 definition:
 * e = floor(log2(max |x| over the 32)) - 2 clamped to [-127, 127] (an all-zero block
 * takes -127), scale byte e + 127, code = E2M1(x / 2^e) rounded to nearest with ties to
 * the even code and magnitudes above 6 saturating to 6. The sign of zero is kept; NaN
 * inputs are skipped by the maximum and encode to +0; inputs are otherwise finite.
 *
 *   x       bf16 [M, K]
 *   q       out, [M, K/2] bytes: element 2i in the low nibble of byte i (bit 3 = sign)
 *   scales  out, [M, K/32] E8M0 bytes. With K % 128 == 0 the four bytes of a
 *           (row, 128-column group) form one 32-bit word, so moe_route_permute gathers
 *           them as its fp32 `xs` ([M, K/128] words) into the group-major layout that
 *           mxfp4_grouped_expert_gemm reads.
 * Constraints: M >= 1, K % 32 == 0.
 */
int32_t mxfp4_quant_act(const void* x, int64_t M, int64_t K, uint8_t* q, uint8_t* scales,
                        void* stream);

/*
 * fp8moe_pack_expert_bank_mxfp4 -- fp8moe_pack_expert_bank for the MXFP4-activation GEMM:
 * the same blocks and scales, with the 16-value K chunks of every 128-group in the order
 * the gfx950 MFMA pairs with an FP4 operand (chunk c of the MFMA's K holds logical chunk
 * c / 2 + 4 (c % 2)). Arguments and constraints as fp8moe_pack_expert_bank.
 */
int32_t fp8moe_pack_expert_bank_mxfp4(const uint8_t* w, const float* w_scales, int64_t E,
                                      int64_t N, int64_t K, uint8_t* w_packed,
                                      float* w_scales_packed, void* stream);

/*
 * mxfp4_grouped_expert_gemm -- fp8_grouped_expert_gemm with MXFP4 activations ([P3]: FP4
 * E2M1 activations into the grouped expert GEMM; [P1] section 1 for the rest):
 *   y[i, n] = sum_g s_w[e, g, n] * sum_{k in g} x(a[i, k]) * q[e, n, k],
 * x(a) = E2M1 value * 2^(its block's E8M0 byte - 127). The MFMA applies the activation
 * block scales itself; the weight scale is folded per 128-group as in the e4m3 GEMM.
 *
 *   a          MXFP4 codes [rows, K/2] (mxfp4_quant_act), rows in token order when `sorted`
 *              is given (gathered on the fly), else already grouped
 *   a_scales   uint32 words, the four E8M0 bytes of (row, 128-group) as one word: with
 *              `sorted`, mxfp4_quant_act's scales viewed as [rows, K/128] words; without
 *              it, group-major [K/128, R] in grouped order (e.g. moe_route_permute's xs_perm
 *              of those words)
 *   w, w_scales  from fp8moe_pack_expert_bank_mxfp4
 *   everything else as fp8_grouped_expert_gemm (epilogues, output layouts including
 *   out_sums, constraints); there is no a_sums (the kernel sums the scaled rows itself)
 */
int32_t mxfp4_grouped_expert_gemm(const uint8_t* a, const uint32_t* a_scales,
                                  const int32_t* sorted, int32_t k_route, const uint8_t* w,
                                  const float* w_scales, const int32_t* offsets, int64_t R,
                                  int32_t E, int64_t N, int64_t K, int32_t epilogue,
                                  int32_t out_dtype, void* out, float* out_scales,
                                  float* out_sums, void* stream);

/*
 * moe_unpermute_combine -- out[t, :] = sum_{j=0..k-1} weights[t, j] * y[pos[t*k+j], :]
 *
 * [P1] section 1: the grouped GEMM's rows are returned to token order and weighted by
 * the router. The sum runs in fp32 in increasing j; no atomics, so the result is
 * deterministic.
 *
 *   y        [T*k, H] in y_dtype (fp32 or bf16), grouped order
 *   pos      int32 [T*k] from moe_route_permute
 *   weights  fp32 [T, k]
 *   out      [T, H] in out_dtype (fp32 or bf16, RNE)
 * Constraints: T >= 1, 1 <= k <= 32, H % 8 == 0.
 */
int32_t moe_unpermute_combine(const void* y, int32_t y_dtype, const int32_t* pos,
                              const float* weights, int64_t T, int32_t k, int64_t H,
                              int32_t out_dtype, void* out, void* stream);

/*
 * fp8moe_rmsnorm -- residual add and RMSNorm of one depth-stack block boundary.
 *
 * [P1] sections 1 and 3: the FP8 projections and grouped experts run inside a stack of
 * pre-norm transformer layers with RMSNorm; the pages print no formula, so the plain
 * one is used, with unit gain:
 *   delta == NULL:  y = bf16(x / sqrt(mean(x^2) + eps))
 *   delta != NULL:  x_out = bf16(x + delta), then y = bf16(x_out / sqrt(mean(x_out^2) + eps))
 * Both roundings are single roundings (round to nearest even) of the exact value, up to
 * the fp64 summation order of the mean.
 *
 *   x        bf16 [T, H]
 *   delta    NULL, or bf16 [T, H] added to x
 *   eps      added to the mean square (the stack uses 1e-6)
 *   x_out    out (only with delta), bf16 [T, H]; may be x itself (in-place update)
 *   y        out, bf16 [T, H]; must not overlap x, delta or x_out
 * Constraints: T >= 1, H >= 8, H % 8 == 0, T*H < 2^40, eps >= 0.
 */
int32_t fp8moe_rmsnorm(const void* x, const void* delta, int64_t T, int64_t H, double eps,
                       void* x_out, void* y, void* stream);

/*
 * fp8moe_bf16_gemm -- out = a . w^T in fp32 from bf16 operands (fp32 accumulation).
 *
 * [P1] section 1 gates the stack on its final logits; [P2] "Limits": the LM head stays
 * bf16. Used for the router logits and the LM head.
 *
 *   a    bf16 [M, K]
 *   w    bf16 [N, K]
 *   out  fp32 [M, N]
 * Constraints: M >= 1, N >= 1, K >= 64, K % 64 == 0, M, N, K < 2^31,
 * ceil(M/128) * ceil(N/128) < 2^31, 2*M*K < 2^32, 2*N*K < 2^32.
 */
int32_t fp8moe_bf16_gemm(const void* a, const void* w, int64_t M, int64_t N, int64_t K,
                         float* out, void* stream);

/*
 * fp8moe_causal_attention -- causal grouped-query attention over a fused qkv tensor.
 *
 * [P1] sections 1 and 3: the attention core between the FP8 q/k/v and o projections
 * stays bf16. Reading used: no rotary embedding; query head h reads kv head
 * h / (n_q / n_kv); o[t, h] = sum_{s <= t} softmax_s(q[t, h] . k[s, kv] / sqrt(d)) v[s, kv]
 * with scores, softmax and the sum in fp32. The softmax weights enter the product with v
 * on the bf16 matrix cores as two bf16 terms, hi = bf16(p) and lo = bf16(p - hi) (about
 * 16 significant bits), so that product keeps close to fp32 accuracy; the row sum of the
 * weights is taken in fp32.
 *
 *   qkv   bf16 [T, (n_q + 2 n_kv) * d]: row t = [q heads | k heads | v heads], head-major
 *   out   out, bf16 [T, n_q * d], head-major
 *   ws    workspace of fp8moe_workspace_bytes(FP8MOE_OP_ATTENTION, T, n_kv, d) bytes
 *         (v transposed per kv head)
 * Constraints: T >= 1, d == 128, n_kv >= 1, n_q % n_kv == 0, (n_q + 2 n_kv) * d * T < 2^31.
 */
int32_t fp8moe_causal_attention(const void* qkv, int64_t T, int32_t n_q, int32_t n_kv,
                                int32_t head_dim, void* out, void* ws, size_t ws_bytes,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8MOE_H */
