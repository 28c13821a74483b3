// api.hip -- the C ABI of libmxq (declared in include/mxq.h): host-side argument
// validation, then the kernel launches on the caller's stream.  No allocation,
// no synchronisation, no state beyond a thread-local copy of the last HIP error.
#include <hip/hip_runtime.h>

#include "../../include/mxq.h"
#include "internal.hpp"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Largest element count accepted by the flat kernels (keeps every index in range
// of 64-bit arithmetic with a wide margin; 2^40 elements is 2 TB of bf16).
constexpr int64_t kMaxElems = (int64_t)1 << 40;

mxq_status check_2d(int64_t M, int64_t K)
{
    if (M < 0 || K < 0) return MXQ_ERR_SHAPE;
    if (M > 0 && K > kMaxElems / M) return MXQ_ERR_SHAPE;
    return MXQ_OK;
}

mxq_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return MXQ_OK;
    g_last_hip_error = (int)e;
    return MXQ_ERR_HIP;
}

}  // namespace

extern "C" {

int mxq_abi_version(void) { return MXQ_ABI_VERSION; }

const char* mxq_status_string(int status)
{
    switch (status) {
    case MXQ_OK: return "MXQ_OK";
    case MXQ_ERR_NULL: return "MXQ_ERR_NULL: a required pointer is NULL";
    case MXQ_ERR_SHAPE: return "MXQ_ERR_SHAPE: invalid size (negative, too large or not a required multiple)";
    case MXQ_ERR_ALIGN: return "MXQ_ERR_ALIGN: a base pointer is not 16-byte aligned";
    case MXQ_ERR_LAYOUT: return "MXQ_ERR_LAYOUT: unknown output layout";
    case MXQ_ERR_WORKSPACE: return "MXQ_ERR_WORKSPACE: workspace missing or too small";
    case MXQ_ERR_HIP: return "MXQ_ERR_HIP: a HIP runtime call failed";
    case MXQ_ERR_NOT_IMPLEMENTED: return "MXQ_ERR_NOT_IMPLEMENTED";
    case MXQ_ERR_DTYPE: return "MXQ_ERR_DTYPE: unknown output data type";
    case MXQ_ERR_RULE: return "MXQ_ERR_RULE: unknown scale rule or flag";
    default: return "unknown mxq_status";
    }
}

int mxq_last_hip_error(void) { return g_last_hip_error; }

mxq_status mxq_quantize_mx(const void* x_bf16, int64_t M, int64_t K, void* q_e4m3, void* s_e8m0, void* stream)
{
    mxq_status st = check_2d(M, K);
    if (st != MXQ_OK) return st;
    if (K % 32 != 0) return MXQ_ERR_SHAPE;
    if (M == 0 || K == 0) return MXQ_OK;
    if (!x_bf16 || !q_e4m3 || !s_e8m0) return MXQ_ERR_NULL;
    if (!aligned16(x_bf16) || !aligned16(q_e4m3) || !aligned16(s_e8m0)) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_mx_quantize(x_bf16, M, K, q_e4m3, s_e8m0, false, (hipStream_t)stream));
}

// Sizes of the MX variants: axis 1 as the plain codec; axis 0 needs whole 32-row
// blocks, 4-column lanes, and keeps its buffer resources (32 rows) and grid in range.
static mxq_status check_mx_ex(int64_t M, int64_t K, int axis)
{
    mxq_status st = check_2d(M, K);
    if (st != MXQ_OK) return st;
    if (axis != 0 && axis != 1) return MXQ_ERR_LAYOUT;
    if (axis == 1) return K % 32 == 0 ? MXQ_OK : MXQ_ERR_SHAPE;
    if (M % 32 != 0 || K % 4 != 0 || K > ((int64_t)1 << 24)) return MXQ_ERR_SHAPE;
    if ((M / 32) * ((K + 1023) / 1024) >= ((int64_t)1 << 31)) return MXQ_ERR_SHAPE;
    return MXQ_OK;
}

mxq_status mxq_quantize_mx_ex(const void* x_bf16, int64_t M, int64_t K, int axis, int rule, void* q_e4m3,
                              void* s_e8m0, void* stream)
{
    mxq_status st = check_mx_ex(M, K, axis);
    if (st != MXQ_OK) return st;
    if (rule != MXQ_SCALE_FLOOR && rule != MXQ_SCALE_RCEIL) return MXQ_ERR_RULE;
    if (M == 0 || K == 0) return MXQ_OK;
    if (!x_bf16 || !q_e4m3 || !s_e8m0) return MXQ_ERR_NULL;
    if (!aligned16(x_bf16) || !aligned16(q_e4m3) || !aligned16(s_e8m0)) return MXQ_ERR_ALIGN;
    const bool rceil = rule == MXQ_SCALE_RCEIL;
    if (axis == 1)
        return hip_status(mxq::launch_mx_quantize(x_bf16, M, K, q_e4m3, s_e8m0, rceil, (hipStream_t)stream));
    return hip_status(mxq::launch_mx_quantize_dim0(x_bf16, M, K, q_e4m3, s_e8m0, rceil, (hipStream_t)stream));
}

mxq_status mxq_dequantize_mx_ex(const void* q_e4m3, const void* s_e8m0, int64_t M, int64_t K, int axis,
                                void* y_bf16, void* stream)
{
    mxq_status st = check_mx_ex(M, K, axis);
    if (st != MXQ_OK) return st;
    if (M == 0 || K == 0) return MXQ_OK;
    if (!q_e4m3 || !s_e8m0 || !y_bf16) return MXQ_ERR_NULL;
    if (!aligned16(q_e4m3) || !aligned16(s_e8m0) || !aligned16(y_bf16)) return MXQ_ERR_ALIGN;
    if (axis == 1) return hip_status(mxq::launch_mx_dequantize(q_e4m3, s_e8m0, M, K, y_bf16, (hipStream_t)stream));
    return hip_status(mxq::launch_mx_dequantize_dim0(q_e4m3, s_e8m0, M, K, y_bf16, (hipStream_t)stream));
}

mxq_status mxq_dequantize_mx(const void* q_e4m3, const void* s_e8m0, int64_t M, int64_t K, void* y_bf16,
                             void* stream)
{
    mxq_status st = check_2d(M, K);
    if (st != MXQ_OK) return st;
    if (K % 32 != 0) return MXQ_ERR_SHAPE;
    if (M == 0 || K == 0) return MXQ_OK;
    if (!q_e4m3 || !s_e8m0 || !y_bf16) return MXQ_ERR_NULL;
    if (!aligned16(q_e4m3) || !aligned16(s_e8m0) || !aligned16(y_bf16)) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_mx_dequantize(q_e4m3, s_e8m0, M, K, y_bf16, (hipStream_t)stream));
}

// Group scaling limits: rows fit the int32 offsets with room for chunk rounding;
// K keeps every launch dimension in range.
static const int64_t kGroupMaxRows = ((int64_t)1 << 31) - 1024;
static const int64_t kGroupMaxK = (int64_t)1 << 23;
static const int64_t kGroupMaxG = (int64_t)1 << 20;

static mxq_status check_group_sizes(int64_t M, int64_t K, int64_t G)
{
    mxq_status st = check_2d(M, K);
    if (st != MXQ_OK) return st;
    if (M > kGroupMaxRows || K > kGroupMaxK || K % 8 != 0) return MXQ_ERR_SHAPE;
    if (G < 1 || G > kGroupMaxG) return MXQ_ERR_SHAPE;
    if (!mxq::group_scale_sizes_ok(M, K, G)) return MXQ_ERR_SHAPE;
    return MXQ_OK;
}

size_t mxq_group_scale_workspace_bytes(int64_t M, int64_t K, int32_t G)
{
    if (check_group_sizes(M, K, G) != MXQ_OK) return 0;
    return mxq::group_scale_workspace_bytes(M, K, G);
}

mxq_status mxq_group_scale_fp8(const void* x_bf16, int64_t M, int64_t K, const int32_t* group_end_offs, int32_t G,
                               int out_layout, void* q_e4m3, float* scales, void* workspace,
                               size_t workspace_bytes, void* stream)
{
    return mxq_group_scale_fp8_ex(x_bf16, M, K, group_end_offs, G, out_layout, 0, q_e4m3, scales, workspace,
                                  workspace_bytes, stream);
}

mxq_status mxq_group_scale_fp8_ex(const void* x_bf16, int64_t M, int64_t K, const int32_t* group_end_offs,
                                  int32_t G, int out_layout, int flags, void* q_e4m3, float* scales,
                                  void* workspace, size_t workspace_bytes, void* stream)
{
    mxq_status st = check_group_sizes(M, K, G);
    if (st != MXQ_OK) return st;
    if (out_layout != MXQ_LAYOUT_ROW && out_layout != MXQ_LAYOUT_COL) return MXQ_ERR_LAYOUT;
    if ((flags & ~(MXQ_GROUP_POW2_SCALE | MXQ_GROUP_INVERSE_SCALE)) != 0) return MXQ_ERR_RULE;
    if (K == 0) return MXQ_OK;
    if (!group_end_offs || !scales) return MXQ_ERR_NULL;
    if (M > 0 && (!x_bf16 || !q_e4m3)) return MXQ_ERR_NULL;
    if (!aligned16(scales) || (M > 0 && (!aligned16(x_bf16) || !aligned16(q_e4m3)))) return MXQ_ERR_ALIGN;
    if (((uintptr_t)group_end_offs & 3u) != 0) return MXQ_ERR_ALIGN;
    const size_t need = mxq::group_scale_workspace_bytes(M, K, G);
    if (!workspace || workspace_bytes < need) return MXQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_group_scale(x_bf16, (int)M, (int)K, group_end_offs, (int)G, out_layout, flags,
                                              q_e4m3, scales, workspace, (hipStream_t)stream));
}

mxq_status mxq_group_scale_fp8_noalloc(const void* x_bf16, int64_t M, int64_t K, const int32_t* group_end_offs,
                                       int32_t G, int out_layout, int flags, void* q_e4m3, float* scales,
                                       void* stream)
{
    mxq_status st = check_group_sizes(M, K, G);
    if (st != MXQ_OK) return st;
    if (out_layout != MXQ_LAYOUT_ROW && out_layout != MXQ_LAYOUT_COL) return MXQ_ERR_LAYOUT;
    if ((flags & ~(MXQ_GROUP_POW2_SCALE | MXQ_GROUP_INVERSE_SCALE)) != 0) return MXQ_ERR_RULE;
    if (K == 0) return MXQ_OK;
    if (!group_end_offs || !scales) return MXQ_ERR_NULL;
    if (M > 0 && (!x_bf16 || !q_e4m3)) return MXQ_ERR_NULL;
    if (!aligned16(scales) || (M > 0 && (!aligned16(x_bf16) || !aligned16(q_e4m3)))) return MXQ_ERR_ALIGN;
    if (((uintptr_t)group_end_offs & 3u) != 0) return MXQ_ERR_ALIGN;
    if (mxq::group_scale_workspace_bytes(M, K, G) > mxq::kNoAllocScratchBytes) return MXQ_ERR_WORKSPACE;
    void* ws = nullptr;
    const hipError_t e = mxq::group_scale_scratch(&ws);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(mxq::launch_group_scale(x_bf16, (int)M, (int)K, group_end_offs, (int)G, out_layout, flags,
                                              q_e4m3, scales, ws, (hipStream_t)stream));
}

mxq_status mxq_set_group_scale_knobs(int method, int hold_tiles, int64_t wait_us, int strip_block)
{
    if (method < 0 || method > 3) return MXQ_ERR_RULE;
    mxq::set_group_scale_knobs(method, hold_tiles, wait_us < 0 ? -1 : (long)wait_us, strip_block);
    return MXQ_OK;
}

mxq_status mxq_group_scale_route_counters(const void* workspace, size_t workspace_bytes, int64_t M, int64_t K,
                                          int32_t G, int out_layout, uint32_t* counters, void* stream)
{
    mxq_status st = check_group_sizes(M, K, G);
    if (st != MXQ_OK) return st;
    if (out_layout != MXQ_LAYOUT_ROW && out_layout != MXQ_LAYOUT_COL) return MXQ_ERR_LAYOUT;
    if (!counters) return MXQ_ERR_NULL;
    if (!workspace || workspace_bytes < mxq::group_scale_workspace_bytes(M, K, G)) return MXQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MXQ_ERR_ALIGN;
    return hip_status(mxq::group_scale_route_counters(workspace, M, K, G, out_layout, counters, (hipStream_t)stream));
}

mxq_status mxq_transpose_u8(const void* in, int64_t R, int64_t C, void* out, void* stream)
{
    mxq_status st = check_2d(R, C);
    if (st != MXQ_OK) return st;
    if (R == 0 || C == 0) return MXQ_OK;
    if (!in || !out) return MXQ_ERR_NULL;
    if (!aligned16(in) || !aligned16(out)) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_transpose_u8(in, R, C, out, (hipStream_t)stream));
}

static mxq_status check_grouped_mm_sizes(int64_t M, int64_t N, int64_t K, int64_t G)
{
    if (M < 0 || N < 0 || K <= 0) return MXQ_ERR_SHAPE;
    if (!mxq::grouped_mm_sizes_ok(M, N, K, G)) return MXQ_ERR_SHAPE;
    return MXQ_OK;
}

size_t mxq_grouped_mm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t G)
{
    if (check_grouped_mm_sizes(M, N, K, G) != MXQ_OK) return 0;
    return mxq::grouped_mm_workspace_bytes(M, N, G);
}

mxq_status mxq_scaled_grouped_mm(const void* xq_e4m3, const void* xs_e8m0, const void* wq_e4m3,
                                 const void* ws_e8m0, const int32_t* group_end_offs, int64_t M,
                                 int64_t N, int64_t K, int32_t G, int out_dtype, void* y,
                                 void* workspace, size_t workspace_bytes, void* stream)
{
    mxq_status st = check_grouped_mm_sizes(M, N, K, G);
    if (st != MXQ_OK) return st;
    if (out_dtype != MXQ_OUT_BF16 && out_dtype != MXQ_OUT_F32) return MXQ_ERR_DTYPE;
    if (M == 0 || N == 0) return MXQ_OK;
    if (!xq_e4m3 || !xs_e8m0 || !wq_e4m3 || !ws_e8m0 || !group_end_offs || !y) return MXQ_ERR_NULL;
    if (!aligned16(xq_e4m3) || !aligned16(xs_e8m0) || !aligned16(wq_e4m3) || !aligned16(ws_e8m0) ||
        !aligned16(y))
        return MXQ_ERR_ALIGN;
    if (((uintptr_t)group_end_offs & 3u) != 0) return MXQ_ERR_ALIGN;
    const size_t need = mxq::grouped_mm_workspace_bytes(M, N, G);
    if (!workspace || workspace_bytes < need) return MXQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_grouped_mm(xq_e4m3, xs_e8m0, wq_e4m3, ws_e8m0, group_end_offs, (int)M, (int)N,
                                             (int)K, (int)G, y, out_dtype == MXQ_OUT_F32, workspace,
                                             (hipStream_t)stream));
}

// Dispatch pack limits: pairs and their block histograms fit the int32 indices.
static mxq_status check_dispatch_sizes(int64_t M, int64_t K, int64_t topk, int64_t E)
{
    mxq_status st = check_2d(M, K);
    if (st != MXQ_OK) return st;
    if (K <= 0 || K % 256 != 0 || K > ((int64_t)1 << 23)) return MXQ_ERR_SHAPE;
    if (topk < 1 || topk > 64 || E < 1 || E > mxq::dispatch_max_experts()) return MXQ_ERR_SHAPE;
    if (M * topk >= ((int64_t)1 << 31) - 256) return MXQ_ERR_SHAPE;
    if ((M * topk + 255) / 256 * E >= ((int64_t)1 << 31)) return MXQ_ERR_SHAPE;
    return MXQ_OK;
}

size_t mxq_dispatch_pack_workspace_bytes(int64_t M, int64_t K, int32_t topk, int32_t E)
{
    if (check_dispatch_sizes(M, K, topk, E) != MXQ_OK) return 0;
    return mxq::dispatch_workspace_bytes(M * topk, E);
}

mxq_status mxq_dispatch_pack_mx(const void* x_bf16, int64_t M, int64_t K, const int32_t* expert_ids, int32_t topk,
                                int32_t E, void* packed, int32_t* group_end_offs, int32_t* src_pair,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    mxq_status st = check_dispatch_sizes(M, K, topk, E);
    if (st != MXQ_OK) return st;
    if (!group_end_offs || !workspace) return !group_end_offs ? MXQ_ERR_NULL : MXQ_ERR_WORKSPACE;
    if (M > 0 && (!x_bf16 || !expert_ids || !packed || !src_pair)) return MXQ_ERR_NULL;
    if (((uintptr_t)group_end_offs & 3u) != 0 || !aligned16(workspace)) return MXQ_ERR_ALIGN;
    if (M > 0 && (!aligned16(x_bf16) || !aligned16(packed) || ((uintptr_t)expert_ids & 3u) != 0 ||
                  ((uintptr_t)src_pair & 3u) != 0))
        return MXQ_ERR_ALIGN;
    if (workspace_bytes < mxq::dispatch_workspace_bytes(M * topk, E)) return MXQ_ERR_WORKSPACE;
    hipError_t e = mxq::launch_dispatch_order(expert_ids, M * topk, E, src_pair, group_end_offs, workspace,
                                              (hipStream_t)stream);
    if (e == hipSuccess)
        e = mxq::launch_mx_dispatch_pack(x_bf16, K, src_pair, topk, group_end_offs, E, packed, M * topk,
                                         (hipStream_t)stream);
    return hip_status(e);
}

mxq_status mxq_scaled_grouped_mm_packed(const void* packed, const void* wq_e4m3, const void* ws_e8m0,
                                        const int32_t* group_end_offs, int64_t M, int64_t N, int64_t K, int32_t G,
                                        int out_dtype, void* y, void* workspace, size_t workspace_bytes,
                                        void* stream)
{
    mxq_status st = check_grouped_mm_sizes(M, N, K, G);
    if (st != MXQ_OK) return st;
    if (K % 512 != 0) return MXQ_ERR_SHAPE;        // 16-byte aligned packed rows
    if (out_dtype != MXQ_OUT_BF16 && out_dtype != MXQ_OUT_F32) return MXQ_ERR_DTYPE;
    if (M == 0 || N == 0) return MXQ_OK;
    if (!packed || !wq_e4m3 || !ws_e8m0 || !group_end_offs || !y) return MXQ_ERR_NULL;
    if (!aligned16(packed) || !aligned16(wq_e4m3) || !aligned16(ws_e8m0) || !aligned16(y)) return MXQ_ERR_ALIGN;
    if (((uintptr_t)group_end_offs & 3u) != 0) return MXQ_ERR_ALIGN;
    const size_t need = mxq::grouped_mm_workspace_bytes(M, N, G);
    if (!workspace || workspace_bytes < need) return MXQ_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MXQ_ERR_ALIGN;
    const uint32_t ldp = (uint32_t)(K + K / 32);
    const uint8_t* base = static_cast<const uint8_t*>(packed);
    return hip_status(mxq::launch_grouped_mm_strided(base, base + K, ldp, ldp, wq_e4m3, ws_e8m0, group_end_offs,
                                                     (int)M, (int)N, (int)K, (int)G, y, out_dtype == MXQ_OUT_F32,
                                                     workspace, (hipStream_t)stream));
}

}  // extern "C"
