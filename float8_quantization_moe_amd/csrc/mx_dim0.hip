// mx_dim0.hip -- MXFP8 with blocks along dim 0: 32 consecutive rows (tokens) of
// one column share an e8m0 scale, on gfx950.
//
// "[mxfp8 MoE training] Support mxfp8 all to all in expert parallel", Summary:
// the payload is encoded as e4m3 data plus e8m0 scales.  Blocks along the token
// dimension are the layout a GEMM that contracts over tokens consumes (the
// weight-gradient product of a MoE layer's backward), so the same format is
// offered with the other blocking axis.  Q keeps X's row-major layout; the
// scales are (M/32, K) row-major: S[a][k] covers x[32a .. 32a+31][k].
//
// One lane owns 4 columns (8 bytes of bf16) of one 32-row block: 32 loads of 8
// bytes, so a wave reads 512 contiguous bytes of each row.  The column maxima
// are packed 16-bit maxima of |bits|, the scale code comes from mx_scale_code,
// and each element is multiplied by the exact power of two 2^(127 - code) in
// binary32 (the code is at most 247, so the factor is a normal number and the
// product is exact unless it underflows, where the e4m3 result is +-0 anyway),
// clamped to +-448 and converted with nearest-even rounding.  Dequantization
// pairs two rows of one column so that each scaled conversion sees one scale,
// then regroups the bf16 pairs into rows with byte permutes.
#include "device_common.hpp"
#include "internal.hpp"

namespace mxq {

constexpr int kD0Threads = 256;                 // 4 waves, each 256 columns of one block
constexpr int kD0Cols = kD0Threads * 4;         // columns per workgroup

typedef __amdgpu_buffer_rsrc_t D0Rsrc;
constexpr uint32_t kD0OOB = 0xFFFFFFF0u;        // above every resource size here (at most 2^31)
constexpr int kD0NonTemporal = 2;               // cache-policy operand of the buffer builtins: nt

// Raw buffer resource over [base, base + bytes): accesses at an offset at or
// past `bytes` read zero or are dropped.
__device__ __forceinline__ D0Rsrc d0_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint2 d0_load8(D0Rsrc r, uint32_t off)
{
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kD0NonTemporal);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t d0_load4(D0Rsrc r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kD0NonTemporal);
}
__device__ __forceinline__ void d0_store8(uint2 v, D0Rsrc r, uint32_t off)
{
    const u32x2 w = {v.x, v.y};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, kD0NonTemporal);
}
__device__ __forceinline__ void d0_store4(uint32_t v, D0Rsrc r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kD0NonTemporal);
}

// Workgroup b: block a = b / ncb of 32 rows, columns [cb * 1024, cb * 1024 + 1024)
// with cb = b % ncb; lane l of the group owns columns k .. k+3, k = cb*1024 + 4l.
template <bool RCEIL>
__global__ __launch_bounds__(kD0Threads)
void mx_quantize_dim0_kernel(const uint16_t* __restrict__ x, int64_t K, int ncb, uint8_t* __restrict__ q,
                             uint8_t* __restrict__ s)
{
    const int64_t a = (int64_t)blockIdx.x / ncb;
    const int64_t k = (int64_t)(blockIdx.x % ncb) * kD0Cols + (int64_t)threadIdx.x * 4;
    const bool in = k < K;                                   // K % 4 == 0: a lane is all in or all out
    const D0Rsrc rx = d0_rsrc(x + a * 32 * K, (uint32_t)(32 * K * 2));
    const uint32_t base = (uint32_t)k * 2u, step = (uint32_t)K * 2u;
    uint2 v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = d0_load8(rx, in ? base + (uint32_t)i * step : kD0OOB);

    uint32_t m0 = 0, m1 = 0;                                 // |bits| maxima: columns (0,1), (2,3)
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        m0 = pk_max_u16(m0, v[i].x & 0x7FFF7FFFu);
        m1 = pk_max_u16(m1, v[i].y & 0x7FFF7FFFu);
    }
    const uint32_t amax[4] = {m0 & 0xFFFFu, m0 >> 16, m1 & 0xFFFFu, m1 >> 16};
    uint32_t codes = 0, nanmask = 0;
    float f[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bool bad = amax[j] >= 0x7F80u;                 // Inf or NaN in the column's block
        const uint32_t c = bad ? 0xFFu : mx_scale_code<RCEIL>(amax[j]);
        codes |= c << (8 * j);
        nanmask |= bad ? 0xFFu << (8 * j) : 0u;
        f[j] = __uint_as_float((254u - (bad ? 127u : c)) << 23);   // 2^(127 - c), a normal binary32
    }

    const D0Rsrc rq = d0_rsrc(q + a * 32 * K, (uint32_t)(32 * K));
    const uint32_t qbase = (uint32_t)k, qstep = (uint32_t)K;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const float y0 = __builtin_amdgcn_fmed3f(bf16_lo_to_f32(v[i].x) * f[0], -448.0f, 448.0f);
        const float y1 = __builtin_amdgcn_fmed3f(bf16_hi_to_f32(v[i].x) * f[1], -448.0f, 448.0f);
        const float y2 = __builtin_amdgcn_fmed3f(bf16_lo_to_f32(v[i].y) * f[2], -448.0f, 448.0f);
        const float y3 = __builtin_amdgcn_fmed3f(bf16_hi_to_f32(v[i].y) * f[3], -448.0f, 448.0f);
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, pk, true);
        const uint32_t w = ((uint32_t)pk & ~nanmask) | (0x7F7F7F7Fu & nanmask);
        d0_store4(w, rq, in ? qbase + (uint32_t)i * qstep : kD0OOB);
    }
    const D0Rsrc rs = d0_rsrc(s + a * K, (uint32_t)K);
    d0_store4(codes, rs, in ? (uint32_t)k : kD0OOB);
}

__global__ __launch_bounds__(kD0Threads)
void mx_dequantize_dim0_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s, int64_t K, int ncb,
                               uint16_t* __restrict__ y)
{
    const int64_t a = (int64_t)blockIdx.x / ncb;
    const int64_t k = (int64_t)(blockIdx.x % ncb) * kD0Cols + (int64_t)threadIdx.x * 4;
    const bool in = k < K;
    const D0Rsrc rs = d0_rsrc(s + a * K, (uint32_t)K);
    const uint32_t codes = d0_load4(rs, in ? (uint32_t)k : kD0OOB);
    const D0Rsrc rq = d0_rsrc(q + a * 32 * K, (uint32_t)(32 * K));
    uint32_t d[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) d[i] = d0_load4(rq, in ? (uint32_t)k + (uint32_t)i * (uint32_t)K : kD0OOB);

    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = pow2_from_biased((codes >> (8 * j)) & 0xFFu);
    bool scale_nan = false;                                  // a scale code 0xFF (NaN) among the 4 columns
#pragma unroll
    for (int j = 0; j < 4; ++j) scale_nan |= ((codes >> (8 * j)) & 0xFFu) == 0xFFu;
    const D0Rsrc ry = d0_rsrc(y + a * 32 * K, (uint32_t)(32 * K * 2));
    const uint32_t ybase = (uint32_t)k * 2u, ystep = (uint32_t)K * 2u;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
        // bytes: column 0 of rows i, i+1, column 1 of rows i, i+1 (and columns 2, 3)
        const uint32_t p01 = __builtin_amdgcn_perm(d[i + 1], d[i], 0x05010400u);
        const uint32_t p23 = __builtin_amdgcn_perm(d[i + 1], d[i], 0x07030602u);
        uint32_t w[4];
        w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p01, sc[0], false));
        w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p01, sc[1], true));
        w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p23, sc[2], false));
        w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p23, sc[3], true));
        // w[j] = (column j, row i) | (column j, row i+1) << 16
        uint2 r0 = make_uint2(__builtin_amdgcn_perm(w[1], w[0], 0x05040100u), __builtin_amdgcn_perm(w[3], w[2], 0x05040100u));
        uint2 r1 = make_uint2(__builtin_amdgcn_perm(w[1], w[0], 0x07060302u), __builtin_amdgcn_perm(w[3], w[2], 0x07060302u));
        if (scale_nan || (nan_code_bytes(d[i]) | nan_code_bytes(d[i + 1])) != 0u) {
            // NaN code (0x7F, 0xFF) or NaN scale (0xFF): the canonical bf16 NaN
            uint32_t o[4] = {r0.x, r0.y, r1.x, r1.y};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = e & 3, row = e >> 2;
                const uint32_t code = ((row ? d[i + 1] : d[i]) >> (8 * j)) & 0xFFu;
                const uint32_t scode = (codes >> (8 * j)) & 0xFFu;
                if ((code & 0x7Fu) == 0x7Fu || scode == 0xFFu) {
                    const int wi = row * 2 + (j >> 1), sh = 16 * (j & 1);
                    o[wi] = (o[wi] & ~(0xFFFFu << sh)) | (0x7FC0u << sh);
                }
            }
            r0 = make_uint2(o[0], o[1]);
            r1 = make_uint2(o[2], o[3]);
        }
        d0_store8(r0, ry, in ? ybase + (uint32_t)i * ystep : kD0OOB);
        d0_store8(r1, ry, in ? ybase + (uint32_t)(i + 1) * ystep : kD0OOB);
    }
}

hipError_t launch_mx_quantize_dim0(const void* x, int64_t M, int64_t K, void* q, void* s, bool rceil,
                                   hipStream_t stream)
{
    const int ncb = (int)((K + kD0Cols - 1) / kD0Cols);
    const unsigned grid = (unsigned)((M / 32) * ncb);
    if (rceil)
        hipLaunchKernelGGL(mx_quantize_dim0_kernel<true>, dim3(grid), dim3(kD0Threads), 0, stream,
                           (const uint16_t*)x, K, ncb, (uint8_t*)q, (uint8_t*)s);
    else
        hipLaunchKernelGGL(mx_quantize_dim0_kernel<false>, dim3(grid), dim3(kD0Threads), 0, stream,
                           (const uint16_t*)x, K, ncb, (uint8_t*)q, (uint8_t*)s);
    return hipGetLastError();
}

hipError_t launch_mx_dequantize_dim0(const void* q, const void* s, int64_t M, int64_t K, void* y,
                                     hipStream_t stream)
{
    const int ncb = (int)((K + kD0Cols - 1) / kD0Cols);
    const unsigned grid = (unsigned)((M / 32) * ncb);
    hipLaunchKernelGGL(mx_dequantize_dim0_kernel, dim3(grid), dim3(kD0Threads), 0, stream, (const uint8_t*)q,
                       (const uint8_t*)s, K, ncb, (uint16_t*)y);
    return hipGetLastError();
}

}  // namespace mxq
