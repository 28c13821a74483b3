// internal.hpp -- launchers shared between the kernel files and the C ABI layer.
// Arguments reaching these functions have already been validated by api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mxq {

hipError_t launch_mx_quantize(const void* x, int64_t M, int64_t K, void* q, void* s, bool rceil, hipStream_t stream);
hipError_t launch_mx_dispatch_pack(const void* x, int64_t K, int32_t* src_pair, int topk, const int32_t* group_end,
                                   int E, void* packed, int64_t nrows, hipStream_t stream);
int dispatch_max_experts();
size_t dispatch_workspace_bytes(int64_t P, int32_t E);
hipError_t launch_dispatch_order(const int32_t* ids, int64_t P, int E, int32_t* src_pair, int32_t* group_end,
                                 void* workspace, hipStream_t stream);
hipError_t launch_mx_quantize_dim0(const void* x, int64_t M, int64_t K, void* q, void* s, bool rceil,
                                   hipStream_t stream);
hipError_t launch_mx_dequantize_dim0(const void* q, const void* s, int64_t M, int64_t K, void* y,
                                     hipStream_t stream);
hipError_t launch_mx_dequantize(const void* q, const void* s, int64_t M, int64_t K, void* y, hipStream_t stream);

bool group_scale_sizes_ok(int64_t M, int64_t K, int64_t G);
size_t group_scale_workspace_bytes(int64_t M, int64_t K, int32_t G);
bool group_split_sizes_ok(int64_t M, int64_t K, int64_t G);
size_t group_split_workspace_bytes(int64_t M, int64_t K, int32_t G);
hipError_t launch_group_split(const void* x, int M, int K, const int32_t* offs, int G, int layout, int flags, void* q,
                              float* scales, void* workspace, hipStream_t stream);
// Route overrides for tests (process-wide): method 0 auto, 1 hold, 2 two-pass, 3 split;
// hold_tiles < 0, wait_us < 0 and strip_block <= 0 select the defaults.
void set_group_scale_knobs(int method, int hold_tiles, long wait_us, int strip_block);
// The allocation-free variant's scratch: a static device array of this many
// bytes per device, its address on the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t group_scale_scratch(void** ptr);
// The hold method's route counters of the last call that used this workspace
// (synchronises the stream).
hipError_t group_scale_route_counters(const void* workspace, int64_t M, int64_t K, int64_t G, int layout,
                                     uint32_t* out, hipStream_t stream);
hipError_t launch_group_scale(const void* x, int M, int K, const int32_t* offs, int G, int layout, int flags,
                              void* q, float* scales, void* workspace, hipStream_t stream);

int grouped_mm_max_groups();
bool grouped_mm_sizes_ok(int64_t M, int64_t N, int64_t K, int64_t G);
size_t grouped_mm_workspace_bytes(int64_t M, int64_t N, int32_t G);
hipError_t launch_grouped_mm(const void* xq, const void* xs, const void* wq, const void* ws,
                             const int32_t* offs, int M, int N, int K, int G, void* y, bool f32_out,
                             void* workspace, hipStream_t stream);
// Token operand with explicit row strides in bytes (codes ldx, scales ldxs; both multiples of 16).
hipError_t launch_grouped_mm_strided(const void* xq, const void* xs, uint32_t ldx, uint32_t ldxs, const void* wq,
                                     const void* ws, const int32_t* offs, int M, int N, int K, int G, void* y,
                                     bool f32_out, void* workspace, hipStream_t stream);

hipError_t launch_transpose_u8(const void* in, int64_t R, int64_t C, void* out, hipStream_t stream);

}  // namespace mxq
