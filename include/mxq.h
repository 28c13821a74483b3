/*
 * mxq.h -- C ABI of libmxq: float8 quantization kernels for MoE token and expert
 * buffers on AMD Instinct MI355X (gfx950).
 *
 * Sources:
 *   "[mxfp8 MoE training] Support mxfp8 all to all in expert parallel"
 *   (torchtitan PR 1765), Summary: the expert-parallel all-to-all payload is
 *   quantized to mxfp8, the e4m3 data and the e8m0 scales travel in two
 *   all_to_all_single calls, and the receiver decodes them back to the input's
 *   precision.  mxq_quantize_mx / mxq_dequantize_mx are the two ends of that
 *   exchange; the buffers they produce and consume are exactly the ones sent.
 *
 *   "[moe training] fix uncoalesced global accesses in per group rowwise scaling
 *   kernel" (torchao PR 2761), Summary and Performance tables: a per-expert-group
 *   float8 scaling kernel over a (tokens, hidden) bf16 tensor whose fp8 output
 *   feeds the LHS of a scaled grouped GEMM, written either in one layout or in
 *   the transposed one and then transformed.  mxq_group_scale_fp8 is that kernel
 *   with both output layouts; mxq_transpose_u8 is the transform.
 *
 * Formats.  bf16 = bfloat16.  e4m3 = OCP FP8 E4M3 ("fn": bias 7, max 448, no
 * infinity, S.1111.111 = NaN).  e8m0 = OCP E8M0 scale, value 2^(c-127), 0xFF =
 * NaN.  MXFP8 = blocks of 32 consecutive elements along the last dimension
 * sharing one e8m0 scale (OCP Microscaling v1.0).
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers (memory of the current HIP device), except
 *     where a comment says otherwise.  Tensors are dense and row-major with no
 *     padding between rows.  Base pointers must be 16-byte aligned
 *     (MXQ_ERR_ALIGN otherwise); hipMalloc / torch allocations are.
 *   - Ownership: the caller owns every buffer.  The library allocates nothing,
 *     frees nothing, retains no pointer after the call returns and keeps no
 *     state between calls; it is safe to call from several host threads.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns without waiting.
 *   - Argument errors are detected on the host, before anything is enqueued,
 *     and returned as an mxq_status; the output buffers are then untouched.
 *     A failed launch returns MXQ_ERR_HIP (see mxq_last_hip_error).  Faults
 *     inside kernels surface, HIP-style, at the caller's next synchronisation.
 *   - Results are bitwise deterministic: every reduction is a max.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_ABI_VERSION 1

typedef enum mxq_status {
    MXQ_OK = 0,
    MXQ_ERR_NULL = 1,        /* a required pointer is NULL                          */
    MXQ_ERR_SHAPE = 2,       /* a size is negative, too large, or not a multiple    */
    MXQ_ERR_ALIGN = 3,       /* a base pointer is not 16-byte aligned               */
    MXQ_ERR_LAYOUT = 4,      /* unknown mxq_layout value                            */
    MXQ_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required          */
    MXQ_ERR_HIP = 6,         /* a HIP runtime call failed (launch, device query)    */
    MXQ_ERR_NOT_IMPLEMENTED = 7,
    MXQ_ERR_DTYPE = 8,       /* unknown mxq_out_dtype value                         */
    MXQ_ERR_RULE = 9         /* unknown mxq_scale_rule value or group flag          */
} mxq_status;

typedef enum mxq_layout {
    MXQ_LAYOUT_ROW = 0,      /* q[m*K + k]: same layout as X (K-contiguous)          */
    MXQ_LAYOUT_COL = 1       /* q[k*M + m]: transposed (token-contiguous), i.e. the
                                (K, M) row-major operand of a GEMM that contracts
                                over the tokens of each group                        */
} mxq_layout;

typedef enum mxq_scale_rule {
    MXQ_SCALE_FLOOR = 0,     /* OCP MX v1.0: shared exponent floor(log2 amax) - 8;
                                elements above 448 once scaled saturate             */
    MXQ_SCALE_RCEIL = 1      /* round the scale up: the smallest e with
                                amax <= 448 * 2^e, so nothing saturates             */
} mxq_scale_rule;

typedef enum mxq_group_flags {
    MXQ_GROUP_POW2_SCALE = 1,    /* multipliers rounded down to a power of two      */
    MXQ_GROUP_INVERSE_SCALE = 2  /* store 1/s (dequantization factor) instead of s  */
} mxq_group_flags;

typedef enum mxq_out_dtype {
    MXQ_OUT_BF16 = 0,        /* bfloat16, rounded to nearest even from the fp32 sum  */
    MXQ_OUT_F32 = 1          /* the fp32 sum itself                                  */
} mxq_out_dtype;

/* MXQ_ABI_VERSION of the built library. */
int mxq_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* mxq_status_string(int status);

/* hipError_t of the most recent MXQ_ERR_HIP returned on the calling thread
 * (0 if none). */
int mxq_last_hip_error(void);

/*
 * MXFP8 quantization of one all-to-all payload.
 * Source: "[mxfp8 MoE training] Support mxfp8 all to all in expert parallel",
 * Summary (the payload is encoded as MXFP8 before the exchange: an e4m3 buffer
 * and an e8m0 buffer).
 *
 *   x_bf16  (M, K) bf16 input, row-major.
 *   q_e4m3  (M, K) uint8 output: e4m3 codes, row-major (the "e4m3 data" buffer).
 *   s_e8m0  (M, K/32) uint8 output: e8m0 codes, row-major, unswizzled; scale b
 *           of row m covers x[m, 32b .. 32b+31] (the "e8m0 scales" buffer).
 *
 * For each block: amax = max |x|; the scale code is floor(log2(amax)) - 8 + 127,
 * clamped to [0, 254] (amax 0 or subnormal gives 0); each element is divided by
 * the scale (exact) and rounded to the nearest e4m3 value, ties to even,
 * saturating at +-448, sign kept (-0 -> 0x80).  A block containing Inf or NaN
 * gets scale 0xFF and every code 0x7F.
 *
 * Requires K % 32 == 0 (MXQ_ERR_SHAPE), M >= 0, K >= 0, M*K <= 2^40.
 * M == 0 or K == 0 is a no-op that returns MXQ_OK.  A token-row split of Q and S
 * (the all-to-all's input splits) keeps every block whole.
 */
mxq_status mxq_quantize_mx(const void* x_bf16, int64_t M, int64_t K,
                           void* q_e4m3, void* s_e8m0, void* stream);

/*
 * MXFP8 dequantization of one received payload back to bf16.
 * Source: "[mxfp8 MoE training] Support mxfp8 all to all in expert parallel",
 * Summary (after the exchange the receiver decodes both buffers back to bf16).
 *
 *   q_e4m3  (M, K) uint8 e4m3 codes; s_e8m0 (M, K/32) uint8 e8m0 codes, both as
 *           produced by mxq_quantize_mx (or received from a peer).
 *   y_bf16  (M, K) bf16 output, row-major.
 *
 * y = e4m3(q) * 2^(s-127) rounded once to bf16 (nearest, ties to even,
 * subnormals kept, overflow to +-Inf).  For s >= 3 the product is exact.
 * A NaN code (0x7F, 0xFF) or scale 0xFF gives bf16 NaN 0x7FC0.
 * Requires K % 32 == 0; M == 0 or K == 0 is a no-op.
 */
mxq_status mxq_dequantize_mx(const void* q_e4m3, const void* s_e8m0, int64_t M, int64_t K,
                             void* y_bf16, void* stream);

/*
 * MXFP8 variants: the scale rule and the blocking axis.
 * Source: "[mxfp8 MoE training] Support mxfp8 all to all in expert parallel",
 * Summary (the e4m3 + e8m0 encoding of the payload).  The pages name mxfp8
 * only; the two choices below are what the format leaves to its user: how the
 * shared exponent is rounded, and along which dimension 32 elements share it
 * (blocks along the token dimension are what a GEMM contracting over tokens,
 * the weight gradient of a MoE layer, consumes).
 *
 *   axis 1: blocks of 32 consecutive elements of a row; s_e8m0 is (M, K/32)
 *           row-major exactly as for mxq_quantize_mx.  Requires K % 32 == 0.
 *   axis 0: blocks of 32 consecutive rows of one column; s_e8m0 is (M/32, K)
 *           row-major, S[a][k] covering x[32a .. 32a+31][k].  Requires
 *           M % 32 == 0, K % 4 == 0, K <= 2^24 and (M/32)*ceil(K/1024) < 2^31.
 *   Any other axis value: MXQ_ERR_LAYOUT.
 *   q_e4m3 is (M, K) row-major (X's layout) for both axes.
 *   rule: MXQ_SCALE_FLOOR (the rule of mxq_quantize_mx) or MXQ_SCALE_RCEIL
 *         (scale code = E - 8 + (mantissa of amax > 1.75), i.e. the smallest
 *         power-of-two scale with amax / scale <= 448), both clamped to
 *         [0, 254]; anything else: MXQ_ERR_RULE.  Rounding, signs, NaN/Inf
 *         blocks (scale 0xFF, codes 0x7F) as for mxq_quantize_mx.
 * mxq_quantize_mx_ex(x, M, K, 1, MXQ_SCALE_FLOOR, ...) produces the same bytes as
 * mxq_quantize_mx.  mxq_dequantize_mx_ex decodes either axis exactly as
 * mxq_dequantize_mx (the rule does not change decoding).  Shape and size errors
 * as for mxq_quantize_mx; M == 0 or K == 0 is a no-op.
 */
mxq_status mxq_quantize_mx_ex(const void* x_bf16, int64_t M, int64_t K, int axis, int rule,
                              void* q_e4m3, void* s_e8m0, void* stream);
mxq_status mxq_dequantize_mx_ex(const void* q_e4m3, const void* s_e8m0, int64_t M, int64_t K,
                                int axis, void* y_bf16, void* stream);

/*
 * Bytes of device workspace mxq_group_scale_fp8 needs for these sizes (0 for
 * invalid sizes).  The workspace holds the call's chunk table, per-chunk column
 * maxima and arrival counters; its contents need no initialisation, are
 * meaningless after the call, and two calls in flight at once must not share it.
 */
size_t mxq_group_scale_workspace_bytes(int64_t M, int64_t K, int32_t G);

/*
 * Per-expert-group float8 scaling of a token tensor.
 * Source: "[moe training] fix uncoalesced global accesses in per group rowwise
 * scaling kernel", Summary (per-group scaling whose output is the LHS operand of
 * the scaled grouped GEMM; row-major or column-major output).
 *
 *   x_bf16          (M, K) bf16 tokens, row-major; the tokens of group g are the
 *                   rows [end[g-1], end[g]) (end[-1] = 0).
 *   group_end_offs  DEVICE int32[G]: cumulative end offsets, non-decreasing,
 *                   end[G-1] == M by contract.  They are read only on the device
 *                   (no device-to-host copy, no host synchronisation).  Offsets
 *                   outside the contract are clamped, not trapped: end[g] is
 *                   taken as min(M, max(end[0..g], 0)); rows at or past the
 *                   last clamped end belong to no group and get code 0x00.
 *   G               number of groups, >= 1; empty groups are allowed.
 *   out_layout      MXQ_LAYOUT_ROW: q is (M, K); MXQ_LAYOUT_COL: q is (K, M).
 *   q_e4m3          uint8 e4m3 output in out_layout.
 *   scales          DEVICE float[G*K] output, (G, K) row-major: the multiplier s
 *                   applied before the cast (dequantize as e4m3(q) / s).
 *   workspace       DEVICE scratch of at least
 *                   mxq_group_scale_workspace_bytes(M, K, G) bytes, 16-B aligned.
 *
 * For each group g and column k: amax = max |x[r,k]| over the group's rows;
 * s = 448 / max(amax, 1e-12) in binary32 (correctly rounded); q = e4m3 of the
 * binary32 product x*s, nearest, ties to even, saturating at +-448.  An empty
 * group has amax 0.  A column holding Inf or NaN gets s = NaN and q = 0x7F.
 *
 * Requires K % 8 == 0, 0 <= M <= 2^31 - 1024, K <= 2^23, 1 <= G <= 2^20, and
 * the tile count (about (M/128 + G) * K/512) below 2^31 (MXQ_ERR_SHAPE otherwise).
 * K == 0 is a no-op; M == 0 still writes the (G, K) scales.
 *
 * Three methods, all giving the same bytes; the first two are picked on the
 * host from the sizes alone (mxq_set_group_scale_knobs can force any of them):
 *   "hold"    X read once, tiles held on chip until their group's scales are
 *             known: row-major output, and column-major output while the
 *             average group spans at least eight 128-row blocks (four when X
 *             is 512 MB or more);
 *   "two-pass" an amax pass, a finalize pass and a quantize pass, X read
 *             twice: column-major output with more groups (three launches
 *             for G <= 256, a fourth, a plan launch, beyond);
 *   "split"   two streaming launches (column maxima per 128-row block, then
 *             reduce + quantize; needs G <= 256): only when forced, as it was
 *             never measured faster than the other two.
 */
mxq_status mxq_group_scale_fp8(const void* x_bf16, int64_t M, int64_t K,
                               const int32_t* group_end_offs, int32_t G, int out_layout,
                               void* q_e4m3, float* scales,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Group-scaling variants: mxq_group_scale_fp8 with `flags`, a bitwise OR of
 *   MXQ_GROUP_POW2_SCALE     the multiplier is rounded down to a power of two,
 *                            s' = 2^floor(log2 s) (so amax * s' <= 448 still and
 *                            x * s' is exact); the codes use s';
 *   MXQ_GROUP_INVERSE_SCALE  `scales` receives the dequantization factor 1/s
 *                            (one correctly rounded binary32 division; NaN stays
 *                            NaN) instead of the multiplier; the codes do not
 *                            change.
 * flags == 0 is exactly mxq_group_scale_fp8.  Any other bit: MXQ_ERR_RULE.
 * Source: "[moe training] fix uncoalesced global accesses in per group rowwise
 * scaling kernel", Summary (the per-group scaling of the grouped GEMM's
 * operands); the pages fix neither the rounding of the scale nor which of s and
 * 1/s is stored, so both are offered.  Arguments, sizes, errors, workspace
 * (the same mxq_group_scale_workspace_bytes) and clamping as for
 * mxq_group_scale_fp8.
 */
mxq_status mxq_group_scale_fp8_ex(const void* x_bf16, int64_t M, int64_t K,
                                  const int32_t* group_end_offs, int32_t G, int out_layout, int flags,
                                  void* q_e4m3, float* scales,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * mxq_group_scale_fp8_ex without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It allocates nothing and calls no
 * allocating routine: its scratch is a static device array of 16 MiB per GPU
 * that the library holds until the process ends (the address is looked up
 * once per device, on the first call there).
 *   Arguments, results, flags and errors as mxq_group_scale_fp8_ex, plus
 *   MXQ_ERR_WORKSPACE when mxq_group_scale_workspace_bytes(M, K, G) exceeds
 *   16 MiB (checked on the host before anything is enqueued; for example
 *   (16640, 5120) needs at most 5.3 MB at 128 groups).
 * Every call on one GPU uses that GPU's single array: calls that overlap on
 * one GPU (different streams, or several host threads) race and must not be
 * issued; calls in stream order on one stream are fine.
 */
mxq_status mxq_group_scale_fp8_noalloc(const void* x_bf16, int64_t M, int64_t K,
                                       const int32_t* group_end_offs, int32_t G, int out_layout,
                                       int flags, void* q_e4m3, float* scales, void* stream);

/*
 * Test and tuning hook, not for production code: overrides how
 * mxq_group_scale_fp8 / mxq_group_scale_fp8_ex route their work, for every
 * later call in the process (the bytes written never depend on it, only the
 * route and the speed).
 *   method       0 = automatic (the default), 1 = hold, 2 = two-pass, 3 = split
 *                (G <= 256; otherwise the automatic choice).
 *   hold_tiles   the hold method's limit on tiles of one group held on chip at
 *                once (larger groups go through its deferred pass); < 0 = the
 *                device's resident capacity less 16 (the default); 0 defers
 *                every group.
 *   wait_us      bound on each of the hold method's waits, in microseconds;
 *                < 0 = 2000 (the default); 0 makes every waiting tile take its
 *                fallback at once.
 *   strip_block  the hold method's launch order (strips per block of
 *                consecutive workgroups); <= 0 = 1 (the default).
 * MXQ_ERR_RULE for a method outside 0..3.  It is a process-wide setting that
 * concurrent calls read without synchronisation: change it only while no
 * group-scaling call is being issued.
 */
mxq_status mxq_set_group_scale_knobs(int method, int hold_tiles, int64_t wait_us, int strip_block);

/*
 * Test and tuning hook, not for production code: the hold method's route
 * counters from the last mxq_group_scale_fp8 / _ex call that used `workspace`
 * with these sizes and layout, read after synchronising `stream`:
 *   counters[0]  tiles whose wait for their group's scales ran out (they then
 *                went to the deferred pass, or to a strip rescue: the first such
 *                tile of a (group, strip) reads the strip's maxima from X once
 *                and publishes the scales, and the others wait for those);
 *   counters[1]  strips whose maxima were read again from X.
 * Both are 0 when every group's tiles were resident together.  Meaningless
 * after a call that took another method, or with M == 0 or K == 0.  Argument
 * errors as mxq_group_scale_fp8 (MXQ_ERR_NULL for counters == NULL).
 */
mxq_status mxq_group_scale_route_counters(const void* workspace, size_t workspace_bytes, int64_t M, int64_t K,
                                          int32_t G, int out_layout, uint32_t* counters, void* stream);

/*
 * Byte transpose: out (C, R) = in (R, C)^T, both row-major.  The layout
 * transform between the two outputs of mxq_group_scale_fp8.
 * Source: "[moe training] fix uncoalesced global accesses in per group rowwise
 * scaling kernel", Summary (write one layout, then transform to the other).
 * Any R, C >= 0 with R*C <= 2^40; R == 0 or C == 0 is a no-op; in and out must not
 * overlap.
 */
mxq_status mxq_transpose_u8(const void* in, int64_t R, int64_t C, void* out, void* stream);

/*
 * Bytes of device workspace mxq_scaled_grouped_mm needs for these sizes (0 for
 * invalid sizes).  It holds the call's tile list, built on the device from the
 * group offsets; contents need no initialisation, are meaningless after the
 * call, and two calls in flight at once must not share it.
 */
size_t mxq_grouped_mm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t G);

/*
 * Grouped product of MXFP8 operands: Y[m, :] = X[m, :] W_g^T for every token row
 * m of group g.
 * Sources: "[float8] add float8 rowwise MoE prototype" (torchtitan PR 1245),
 * Summary (the routed experts' grouped_mm becomes dynamic quantization plus a
 * scaled grouped GEMM); "[mxfp8 MoE training] Support mxfp8 all to all in expert
 * parallel", Performance table (MXFP8 for the grouped GEMMs); "[moe training]
 * fix uncoalesced global accesses in per group rowwise scaling kernel", Summary
 * (the group-ordered token tensor is the GEMM's left operand).
 *
 *   xq_e4m3 (M, K) uint8   token E4M3 codes, row-major;
 *   xs_e8m0 (M, K/32) uint8 their E8M0 block scales (block b of row m covers
 *           k = 32b .. 32b+31) -- exactly what mxq_quantize_mx writes for X;
 *   wq_e4m3 (G, N, K) uint8 expert weights' E4M3 codes, W_g = wq[g] is (N, K)
 *           row-major (the layout of an nn.Linear weight: K contiguous);
 *   ws_e8m0 (G, N, K/32) uint8 their E8M0 block scales (mxq_quantize_mx of the
 *           (G*N, K) weight);
 *   group_end_offs DEVICE int32[G]: cumulative end offsets of the token groups,
 *           clamped exactly as in mxq_group_scale_fp8 (running maximum, cut to
 *           [0, M]); read on the device only;
 *   out_dtype MXQ_OUT_BF16 or MXQ_OUT_F32;
 *   y       (M, N) output, row-major, bf16 or fp32.  Rows at or past the last
 *           clamped end belong to no group and are written as zeros.
 *   workspace DEVICE scratch of mxq_grouped_mm_workspace_bytes(M, N, K, G) bytes.
 *
 * Arithmetic: each operand value is its E4M3 code times its block's power-of-two
 * scale; the hardware forms the exact products, sums them in fp32 (blocks of 64
 * k at a time) and the result is rounded once to the output type.  Against the
 * exact sum of the same products the fp32 error is a few units in the last place
 * of sum_k |x w|.  Codes 0x7F / 0xFF (E4M3 NaN) and scale 0xFF (E8M0 NaN) are
 * outside the contract: the result of a row/column that meets one is
 * unspecified (mxq_quantize_mx emits them only for blocks holding Inf or NaN).
 *
 * Requires K > 0 and K % 128 == 0, N % 8 == 0, 0 <= M < 2^31, 0 <= N < 2^31,
 * K <= 2^23, 1 <= G <= 4095 (MXQ_ERR_SHAPE otherwise); M == 0 or N == 0 is a
 * no-op.  All buffers 16-byte aligned except group_end_offs (4-byte).
 */
mxq_status mxq_scaled_grouped_mm(const void* xq_e4m3, const void* xs_e8m0, const void* wq_e4m3,
                                 const void* ws_e8m0, const int32_t* group_end_offs, int64_t M,
                                 int64_t N, int64_t K, int32_t G, int out_dtype, void* y,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused dispatch pack: the all-to-all send buffer of an expert-parallel MoE
 * layer, built in one call on the device.
 * Source: "[mxfp8 MoE training] Support mxfp8 all to all in expert parallel",
 * Summary (the routed tokens are quantized to mxfp8 and exchanged as e4m3 data
 * plus e8m0 scales).  Sorting the token-expert pairs by expert and packing each
 * row's two parts together is this library's reading of "quantize straight into
 * the send buffer": rows for expert e (and so for the rank that owns e) are
 * contiguous, and one buffer with one split per destination carries both parts.
 *
 *   x_bf16          (M, K) bf16 tokens, row-major.
 *   expert_ids      DEVICE int32 (M, topk): expert of slot j of token t at
 *                   [t*topk + j].  Ids outside [0, E) drop that pair.
 *   packed          (M*topk, K + K/32) uint8 output rows: row r holds the MX
 *                   encoding (as mxq_quantize_mx) of token src_pair[r] / topk,
 *                   its K e4m3 codes then its K/32 e8m0 scales.
 *   group_end_offs  DEVICE int32[E] output: cumulative end row of each expert
 *                   (the group offsets mxq_scaled_grouped_mm_packed and the group
 *                   scaling take).
 *   src_pair        DEVICE int32[M*topk] output: the pair index t*topk + j of
 *                   each row (for the return trip); -1 for rows at or past
 *                   group_end_offs[E-1].
 *   workspace       DEVICE scratch of mxq_dispatch_pack_workspace_bytes(M, K,
 *                   topk, E) bytes, 16-B aligned, no initialisation needed.
 *
 * Order: by expert, and within an expert by pair index (a stable sort), so the
 * result is deterministic.  Rows at or past the last end are not written.
 * Requires K % 256 == 0 (8-byte aligned rows), 0 < K <= 2^23, 1 <= topk <= 64,
 * 1 <= E <= 1024, M*topk < 2^31 - 256 (MXQ_ERR_SHAPE).  x and packed 16-byte
 * aligned, the int32 arrays 4-byte aligned (MXQ_ERR_ALIGN).  M == 0 writes
 * only group_end_offs (all zero).
 */
size_t mxq_dispatch_pack_workspace_bytes(int64_t M, int64_t K, int32_t topk, int32_t E);
mxq_status mxq_dispatch_pack_mx(const void* x_bf16, int64_t M, int64_t K, const int32_t* expert_ids,
                                int32_t topk, int32_t E, void* packed, int32_t* group_end_offs,
                                int32_t* src_pair, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * mxq_scaled_grouped_mm with the token operand read straight from a packed
 * buffer as mxq_dispatch_pack_mx writes it (rows of K e4m3 codes followed by
 * K/32 e8m0 scales, row stride K + K/32 bytes): the receiver multiplies the
 * payload as received, with no dequantization and no unpacking.
 * Source: "[mxfp8 MoE training] Support mxfp8 all to all in expert parallel",
 * Summary (the receiver of the mxfp8 payload), and the grouped product of
 * mxq_scaled_grouped_mm.
 *
 *   packed  (M, K + K/32) uint8, 16-byte aligned.  Everything else, the result
 *           and every error as for mxq_scaled_grouped_mm (same workspace size),
 *           plus K % 512 == 0 (MXQ_ERR_SHAPE) so that every packed row is
 *           16-byte aligned.  Bit-identical to mxq_scaled_grouped_mm on the
 *           unpacked codes and scales.
 */
mxq_status mxq_scaled_grouped_mm_packed(const void* packed, const void* wq_e4m3, const void* ws_e8m0,
                                        const int32_t* group_end_offs, int64_t M, int64_t N, int64_t K,
                                        int32_t G, int out_dtype, void* y, void* workspace,
                                        size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
