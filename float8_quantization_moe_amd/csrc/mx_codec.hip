// mx_codec.hip -- MXFP8 quantize / dequantize of an expert-parallel all-to-all
// payload on gfx950.
//
// "[mxfp8 MoE training] Support mxfp8 all to all in expert parallel", Summary:
// the payload is quantized to mxfp8 (e4m3 data + e8m0 scales), both buffers are
// exchanged, and the receiver decodes them back into bf16, the input precision.  The
// kernels below produce / consume exactly those two buffers.
//
// Both kernels are flat streaming passes over M*K elements (an HBM-bound byte
// codec, no contraction): the (M, K) row-major tensor is a sequence of 32-element
// blocks, and the e8m0 buffer (M, K/32) is indexed by the same flat block number.
// Each lane owns one 16-byte chunk of bf16 (8 elements) per step, four
// consecutive lanes own one block, so every wave-wide load or store is one
// contiguous run of memory.  The block amax is a packed 16-bit integer max of
// |bits| (positive bf16 order equals integer order; Inf/NaN sort above every
// finite value) finished across the quad with DPP.
#include "device_common.hpp"
#include "internal.hpp"

namespace mxq {

constexpr int kCodecThreads = 256;
constexpr int kCodecUnroll = 4;   // independent 16-byte loads in flight per lane

// One 16-byte chunk (8 bf16) -> 8 E4M3 codes; returns the block's E8M0 code in *scode.
// RCEIL selects the round-up scale rule (see mx_scale_code).
template <bool RCEIL>
__device__ __forceinline__ uint2 quantize_chunk(uint4 v, uint32_t* scode)
{
    const uint32_t m0 = v.x & 0x7FFF7FFFu, m1 = v.y & 0x7FFF7FFFu;
    const uint32_t m2 = v.z & 0x7FFF7FFFu, m3 = v.w & 0x7FFF7FFFu;
    const uint32_t pm = pk_max_u16(pk_max_u16(m0, m1), pk_max_u16(m2, m3));
    uint32_t amax = (pm & 0xFFFFu) > (pm >> 16) ? (pm & 0xFFFFu) : (pm >> 16);
    amax = quad_max_u32(amax);

    const uint32_t code = mx_scale_code<RCEIL>(amax);
    if (amax >= 0x7F80u) {                       // Inf or NaN in the block
        *scode = 0xFFu;
        return make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    }
    *scode = code;
    // Saturation bound 448 * 2^(code-127) as a bf16 magnitude, in both halves.
    const uint32_t L = ((code + 8u) << 7) | 0x60u;
    const uint32_t LL = L | (L << 16);
    const float scale = pow2_from_biased(code);
    const uint32_t t0 = (v.x & 0x80008000u) | pk_min_u16(m0, LL);
    const uint32_t t1 = (v.y & 0x80008000u) | pk_min_u16(m1, LL);
    const uint32_t t2 = (v.z & 0x80008000u) | pk_min_u16(m2, LL);
    const uint32_t t3 = (v.w & 0x80008000u) | pk_min_u16(m3, LL);
    v2i16 lo = {0, 0}, hi = {0, 0};
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(v2bf16, t0), scale, false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(v2bf16, t1), scale, true);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(v2bf16, t2), scale, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(v2bf16, t3), scale, true);
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

template <bool RCEIL>
__global__ __launch_bounds__(kCodecThreads)
void mx_quantize_kernel(const uint4* __restrict__ x, uint2* __restrict__ q, uint8_t* __restrict__ s,
                        int64_t nchunks)
{
    const int64_t per_block = (int64_t)kCodecThreads * kCodecUnroll;
    for (int64_t base = (int64_t)blockIdx.x * per_block + threadIdx.x; base < nchunks;
         base += (int64_t)gridDim.x * per_block) {
        uint4 v[kCodecUnroll];
#pragma unroll
        for (int u = 0; u < kCodecUnroll; ++u) {
            const int64_t c = base + (int64_t)u * kCodecThreads;
            v[u] = c < nchunks ? load_nt(x + c) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kCodecUnroll; ++u) {
            const int64_t c = base + (int64_t)u * kCodecThreads;
            uint32_t code;
            const uint2 out = quantize_chunk<RCEIL>(v[u], &code);   // whole quads are in or out of range
            if (c < nchunks) {
                store_nt(out, q + c);
                if ((threadIdx.x & 3) == 0) s[c >> 2] = (uint8_t)code;
            }
        }
    }
}

// 8 E4M3 codes of one block (scale code sc) -> 8 bf16.
__device__ __forceinline__ uint4 dequantize_chunk(uint2 qv, uint32_t sc)
{
    const float scale = pow2_from_biased(sc);
    const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qv.x, scale, false));
    const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qv.x, scale, true));
    const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qv.y, scale, false));
    const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qv.y, scale, true));
    uint4 r = make_uint4(a, b, c, d);
    if (sc == 0xFFu || (nan_code_bytes(qv.x) | nan_code_bytes(qv.y))) {
        // NaN scale or NaN codes: write the canonical bf16 NaN for those elements.
        uint32_t w[4] = {a, b, c, d};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t code = ((i < 4 ? qv.x : qv.y) >> (8 * (i & 3))) & 0xFFu;
            if (sc == 0xFFu || (code & 0x7Fu) == 0x7Fu) {
                const int sh = 16 * (i & 1);
                w[i >> 1] = (w[i >> 1] & ~(0xFFFFu << sh)) | (0x7FC0u << sh);
            }
        }
        r = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return r;
}

__global__ __launch_bounds__(kCodecThreads)
void mx_dequantize_kernel(const uint2* __restrict__ q, const uint8_t* __restrict__ s, uint4* __restrict__ y,
                          int64_t nchunks)
{
    const int64_t per_block = (int64_t)kCodecThreads * kCodecUnroll;
    for (int64_t base = (int64_t)blockIdx.x * per_block + threadIdx.x; base < nchunks;
         base += (int64_t)gridDim.x * per_block) {
        uint2 qv[kCodecUnroll];
        uint32_t sc[kCodecUnroll];
#pragma unroll
        for (int u = 0; u < kCodecUnroll; ++u) {
            const int64_t c = base + (int64_t)u * kCodecThreads;
            const bool in = c < nchunks;
            qv[u] = in ? load_nt(q + c) : make_uint2(0, 0);
            sc[u] = in ? (uint32_t)s[c >> 2] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kCodecUnroll; ++u) {
            const int64_t c = base + (int64_t)u * kCodecThreads;
            if (c < nchunks) store_nt(dequantize_chunk(qv[u], sc[u]), y + c);
        }
    }
}

// Dispatch pack: row r of the packed buffer (row stride ldp = K + K/32 bytes)
// is the MX encoding of token src_pair[r] / topk, its K codes followed by its
// K/32 scales, exactly the bytes mxq_quantize_mx writes for that token.  Rows
// at or past the last expert's end are not written; their src_pair becomes -1.
// One workgroup per packed row (grid-stride over rows): the source token is one
// uniform load, and the row's K/8 chunks go through the codec's quantizer
// kCodecThreads * kCodecUnroll at a time (a quad of lanes per 32-block).
__global__ __launch_bounds__(kCodecThreads)
void mx_dispatch_pack_kernel(const uint4* __restrict__ x, int K8, int32_t* src_pair, int topk,
                             const int32_t* __restrict__ group_end, int E, uint8_t* __restrict__ packed,
                             int64_t ldp, int64_t nrows)
{
    const int64_t total = group_end[E - 1];
    const int64_t K = (int64_t)K8 * 8;
    for (int64_t r = blockIdx.x; r < nrows; r += gridDim.x) {
        if (r >= total) {                              // uniform
            if (threadIdx.x == 0) src_pair[r] = -1;
            continue;
        }
        const uint4* xr = x + (int64_t)(src_pair[r] / topk) * K8;
        uint8_t* dst = packed + r * ldp;
        for (int c0 = 0; c0 < K8; c0 += kCodecThreads * kCodecUnroll) {
            uint4 v[kCodecUnroll];
#pragma unroll
            for (int u = 0; u < kCodecUnroll; ++u) {
                const int cc = c0 + u * kCodecThreads + (int)threadIdx.x;
                v[u] = cc < K8 ? load_nt(xr + cc) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < kCodecUnroll; ++u) {
                const int cc = c0 + u * kCodecThreads + (int)threadIdx.x;
                uint32_t code;
                const uint2 out = quantize_chunk<false>(v[u], &code);   // whole quads are in or out (K8 % 4 == 0)
                if (cc < K8) {
                    store_nt(out, (uint2*)(dst + (int64_t)cc * 8));
                    if ((threadIdx.x & 3) == 0) dst[K + (cc >> 2)] = (uint8_t)code;
                }
            }
        }
    }
}

hipError_t launch_mx_dispatch_pack(const void* x, int64_t K, int32_t* src_pair, int topk, const int32_t* group_end,
                                   int E, void* packed, int64_t nrows, hipStream_t stream)
{
    if (nrows == 0 || K == 0) return hipSuccess;
    const unsigned grid = (unsigned)(nrows < (1 << 22) ? nrows : (1 << 22));
    hipLaunchKernelGGL(mx_dispatch_pack_kernel, dim3(grid), dim3(kCodecThreads), 0, stream, (const uint4*)x,
                       (int)(K / 8), src_pair, topk, group_end, E, (uint8_t*)packed, K + K / 32, nrows);
    return hipGetLastError();
}

// Grid for a flat pass: one block per kCodecThreads * kCodecUnroll chunks, capped
// (the kernels loop over any remainder).
static unsigned codec_grid(int64_t nchunks)
{
    const int64_t per_block = (int64_t)kCodecThreads * kCodecUnroll;
    int64_t blocks = (nchunks + per_block - 1) / per_block;
    const int64_t cap = 1 << 22;
    return (unsigned)(blocks < cap ? blocks : cap);
}

hipError_t launch_mx_quantize(const void* x, int64_t M, int64_t K, void* q, void* s, bool rceil, hipStream_t stream)
{
    const int64_t nchunks = M * K / 8;
    if (rceil)
        hipLaunchKernelGGL(mx_quantize_kernel<true>, dim3(codec_grid(nchunks)), dim3(kCodecThreads), 0, stream,
                           (const uint4*)x, (uint2*)q, (uint8_t*)s, nchunks);
    else
        hipLaunchKernelGGL(mx_quantize_kernel<false>, dim3(codec_grid(nchunks)), dim3(kCodecThreads), 0, stream,
                           (const uint4*)x, (uint2*)q, (uint8_t*)s, nchunks);
    return hipGetLastError();
}

hipError_t launch_mx_dequantize(const void* q, const void* s, int64_t M, int64_t K, void* y, hipStream_t stream)
{
    const int64_t nchunks = M * K / 8;
    hipLaunchKernelGGL(mx_dequantize_kernel, dim3(codec_grid(nchunks)), dim3(kCodecThreads), 0, stream,
                       (const uint2*)q, (const uint8_t*)s, (uint4*)y, nchunks);
    return hipGetLastError();
}

}  // namespace mxq
