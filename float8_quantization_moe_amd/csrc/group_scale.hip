// group_scale.hip -- per-expert-group float8 scaling of a (tokens, hidden) bf16
// tensor on gfx950, with row-major or transposed (column-major) output.
//
// "[moe training] fix uncoalesced global accesses in per group rowwise scaling
// kernel", Summary and Performance: per-group scaling whose fp8 output is the LHS
// of the scaled grouped GEMM; storing it in the layout the GEMM wants was the
// bottleneck (uncoalesced writes), and for many groups writing the other layout
// and transforming afterwards was faster.
//
// Definition (per group g, column k): amax = max |x| over the group's rows,
// s = 448 / max(amax, 1e-12) in binary32, q = e4m3(binary32(x * s)) with
// nearest-even rounding saturated at +-448; the stored scale is s.
//
// Three launches, no host synchronisation, offsets read on the device only:
//   A  group_amax_kernel   one workgroup per (row chunk, 512-column strip);
//                          packed 16-bit max of |bf16 bits| -> u16 partial per
//                          (chunk, column) in the workspace.  Chunks never cross a
//                          group boundary and are cut at multiples of 128 rows.
//   F  group_scales_kernel one thread per 8 columns of one group: max over the
//                          group's partials, then the binary32 divide; writes the
//                          (G, K) scales, including those of empty groups.
//   B  group_quant_*       one workgroup per (row chunk, column strip): re-reads
//                          x (the read of A was moments earlier, so it largely
//                          comes back from the last-level cache), multiplies,
//                          clamps, converts, stores.  ROW stores 8 bytes per lane
//                          straight from registers (a wave writes 512 contiguous
//                          bytes of one row); COL transposes 4x8-byte register
//                          blocks, stages a 128x128-byte tile in LDS, and writes
//                          128 contiguous bytes per output row.
#include "device_common.hpp"
#include "internal.hpp"

namespace mxq {

constexpr int kGThreads = 256;
constexpr int kAmaxRows = 128;    // rows per amax chunk
constexpr int kRowStrip = 512;    // columns per workgroup for A and for ROW output (64 lanes x 8)
constexpr int kQuantRows = 128;   // rows per quantize chunk (both layouts)
constexpr int kColStrip = 128;    // columns per workgroup for COL output
constexpr int kScaleCols = kGThreads * 8;
constexpr int kUnrollRows = 8;

static_assert(kQuantRows == 128 && kColStrip == 128, "COL staging assumes a 128 x 128 byte tile");

// ------------------------------------------------------------------- A ----
__global__ __launch_bounds__(kGThreads)
void group_amax_kernel(const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ offs, int G,
                       uint16_t* __restrict__ partial)
{
    const Chunk ch = locate_chunk<kAmaxRows>(offs, G, M, (int)blockIdx.x, false);
    if (ch.g < 0) return;                       // same chunk for every wave: uniform exit
    const int lane = lane_id(), wave = (int)(threadIdx.x >> 6);
    const int k = (int)blockIdx.y * kRowStrip + lane * 8;
    uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
    if (k < K) {
        const uint16_t* xk = x + k;
        for (int r = ch.r0 + wave; r < ch.r1; r += 4 * kUnrollRows) {
            uint4 v[kUnrollRows];
#pragma unroll
            for (int u = 0; u < kUnrollRows; ++u) {
                const int rr = r + 4 * u;
                v[u] = rr < ch.r1 ? *(const uint4*)(xk + (int64_t)rr * K) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < kUnrollRows; ++u) {
                m0 = pk_max_u16(m0, v[u].x & 0x7FFF7FFFu);
                m1 = pk_max_u16(m1, v[u].y & 0x7FFF7FFFu);
                m2 = pk_max_u16(m2, v[u].z & 0x7FFF7FFFu);
                m3 = pk_max_u16(m3, v[u].w & 0x7FFF7FFFu);
            }
        }
    }
    __shared__ uint4 red[kGThreads / kWave][kWave];
    red[wave][lane] = make_uint4(m0, m1, m2, m3);
    __syncthreads();
    if (wave == 0 && k < K) {
        uint4 a = red[0][lane];
#pragma unroll
        for (int w = 1; w < kGThreads / kWave; ++w) {
            const uint4 b = red[w][lane];
            a.x = pk_max_u16(a.x, b.x);
            a.y = pk_max_u16(a.y, b.y);
            a.z = pk_max_u16(a.z, b.z);
            a.w = pk_max_u16(a.w, b.w);
        }
        *(uint4*)(partial + (int64_t)blockIdx.x * K + k) = a;
    }
}

// ------------------------------------------------------------------- F ----
__device__ __forceinline__ float group_scale_of(uint32_t amax_bits)
{
    if (amax_bits >= 0x7F80u) return __uint_as_float(0x7FC00000u);   // Inf/NaN in the column
    const float amax = __uint_as_float(amax_bits << 16);
    return 448.0f / fmaxf(amax, 1e-12f);                            // correctly rounded divide
}

__global__ __launch_bounds__(kGThreads)
void group_scales_kernel(int M, int K, const int32_t* __restrict__ offs, int G,
                         const uint16_t* __restrict__ partial, float* __restrict__ scales)
{
    const int g = (int)blockIdx.x;
    int first, count;
    group_chunk_span<kAmaxRows>(offs, G, M, g, &first, &count);
    const int k = ((int)blockIdx.y * kGThreads + (int)threadIdx.x) * 8;
    if (k >= K) return;
    uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
    const uint16_t* p = partial + (int64_t)first * K + k;
    int i = 0;
    for (; i + 4 <= count; i += 4) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *(const uint4*)(p + (int64_t)(i + u) * K);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            m0 = pk_max_u16(m0, v[u].x);
            m1 = pk_max_u16(m1, v[u].y);
            m2 = pk_max_u16(m2, v[u].z);
            m3 = pk_max_u16(m3, v[u].w);
        }
    }
    for (; i < count; ++i) {
        const uint4 v = *(const uint4*)(p + (int64_t)i * K);
        m0 = pk_max_u16(m0, v.x);
        m1 = pk_max_u16(m1, v.y);
        m2 = pk_max_u16(m2, v.z);
        m3 = pk_max_u16(m3, v.w);
    }
    float4 lo, hi;
    lo.x = group_scale_of(m0 & 0xFFFFu); lo.y = group_scale_of(m0 >> 16);
    lo.z = group_scale_of(m1 & 0xFFFFu); lo.w = group_scale_of(m1 >> 16);
    hi.x = group_scale_of(m2 & 0xFFFFu); hi.y = group_scale_of(m2 >> 16);
    hi.z = group_scale_of(m3 & 0xFFFFu); hi.w = group_scale_of(m3 >> 16);
    float4* dst = (float4*)(scales + (int64_t)g * K + k);
    dst[0] = lo;
    dst[1] = hi;
}

// ------------------------------------------------------------------- B ----
struct ColScales {
    float s[8];
    uint32_t nan_lo, nan_hi;   // 0xFF in each byte whose column has a NaN scale
};

__device__ __forceinline__ ColScales load_col_scales(const float* __restrict__ scales, int g, int K, int k)
{
    ColScales cs;
    const float4 a = *(const float4*)(scales + (int64_t)g * K + k);
    const float4 b = *(const float4*)(scales + (int64_t)g * K + k + 4);
    cs.s[0] = a.x; cs.s[1] = a.y; cs.s[2] = a.z; cs.s[3] = a.w;
    cs.s[4] = b.x; cs.s[5] = b.y; cs.s[6] = b.z; cs.s[7] = b.w;
    cs.nan_lo = 0;
    cs.nan_hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (cs.s[i] != cs.s[i]) cs.nan_lo |= 0xFFu << (8 * i);
        if (cs.s[i + 4] != cs.s[i + 4]) cs.nan_hi |= 0xFFu << (8 * i);
    }
    return cs;
}

// 8 bf16 of one row (8 consecutive columns) -> 8 E4M3 codes.
__device__ __forceinline__ uint2 group_quantize_chunk(uint4 v, const ColScales& cs)
{
    // binary32 product (one rounding), clamp to +-448, then nearest-even E4M3
    const float f0 = __builtin_amdgcn_fmed3f(bf16_lo_to_f32(v.x) * cs.s[0], -448.0f, 448.0f);
    const float f1 = __builtin_amdgcn_fmed3f(bf16_hi_to_f32(v.x) * cs.s[1], -448.0f, 448.0f);
    const float f2 = __builtin_amdgcn_fmed3f(bf16_lo_to_f32(v.y) * cs.s[2], -448.0f, 448.0f);
    const float f3 = __builtin_amdgcn_fmed3f(bf16_hi_to_f32(v.y) * cs.s[3], -448.0f, 448.0f);
    const float f4 = __builtin_amdgcn_fmed3f(bf16_lo_to_f32(v.z) * cs.s[4], -448.0f, 448.0f);
    const float f5 = __builtin_amdgcn_fmed3f(bf16_hi_to_f32(v.z) * cs.s[5], -448.0f, 448.0f);
    const float f6 = __builtin_amdgcn_fmed3f(bf16_lo_to_f32(v.w) * cs.s[6], -448.0f, 448.0f);
    const float f7 = __builtin_amdgcn_fmed3f(bf16_hi_to_f32(v.w) * cs.s[7], -448.0f, 448.0f);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f4, f5, 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(f6, f7, hi, true);
    const uint32_t ulo = ((uint32_t)lo & ~cs.nan_lo) | (0x7F7F7F7Fu & cs.nan_lo);
    const uint32_t uhi = ((uint32_t)hi & ~cs.nan_hi) | (0x7F7F7F7Fu & cs.nan_hi);
    return make_uint2(ulo, uhi);
}

__global__ __launch_bounds__(kGThreads)
void group_quant_row_kernel(const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ offs, int G,
                            const float* __restrict__ scales, uint8_t* __restrict__ q)
{
    const Chunk ch = locate_chunk<kQuantRows>(offs, G, M, (int)blockIdx.x, true);
    if (ch.g < 0) return;
    const int lane = lane_id(), wave = (int)(threadIdx.x >> 6);
    const int k = (int)blockIdx.y * kRowStrip + lane * 8;
    if (k >= K) return;
    uint8_t* qk = q + k;
    if (ch.g == G) {                           // rows that belong to no group
        for (int r = ch.r0 + wave; r < ch.r1; r += 4) *(uint2*)(qk + (int64_t)r * K) = make_uint2(0, 0);
        return;
    }
    const ColScales cs = load_col_scales(scales, ch.g, K, k);
    const uint16_t* xk = x + k;
    for (int r = ch.r0 + wave; r < ch.r1; r += 4 * kUnrollRows) {
        uint4 v[kUnrollRows];
#pragma unroll
        for (int u = 0; u < kUnrollRows; ++u) {
            const int rr = r + 4 * u;
            v[u] = rr < ch.r1 ? *(const uint4*)(xk + (int64_t)rr * K) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kUnrollRows; ++u) {
            const int rr = r + 4 * u;
            if (rr < ch.r1) *(uint2*)(qk + (int64_t)rr * K) = group_quantize_chunk(v[u], cs);
        }
    }
}

// Byte offset of (column c, row r) inside a 128 x 128 staging tile: each column is
// 128 contiguous bytes; its eight 16-byte units are XOR-swizzled by bits of the
// column so that the transposed dword writes spread over the LDS banks.
__device__ __forceinline__ int tile_offset(int c, int r)
{
    return c * 128 + ((((r >> 4) ^ (c >> 3)) & 7) << 4) + (r & 15);
}

// Write the staged tile's columns as output rows: column c of the tile goes to
// out + (col0 + c) * ld + row0 + [lo, hi) for the rows [lo, hi) of the tile that
// are valid.  16-byte stores where a unit is whole and aligned, bytes elsewhere.
__device__ __forceinline__ void store_tile_rows(const uint8_t* tile, uint8_t* __restrict__ out, int64_t ld,
                                                int64_t col0, int64_t ncols, int64_t row0, int lo, int hi,
                                                bool aligned16)
{
    for (int i = 0; i < 4; ++i) {
        const int sid = (int)threadIdx.x + kGThreads * i;
        const int c = sid >> 3, seg = sid & 7;
        if (col0 + c >= ncols) continue;
        const int rb = seg * 16;
        const int a = rb > lo ? rb : lo;
        const int b = rb + 16 < hi ? rb + 16 : hi;
        if (a >= b) continue;
        const uint4 val = *(const uint4*)(tile + tile_offset(c, rb));
        uint8_t* dst = out + (col0 + c) * ld + row0 + rb;
        if (aligned16 && a == rb && b == rb + 16) {
            *(uint4*)dst = val;
        } else {
            const uint32_t w[4] = {val.x, val.y, val.z, val.w};
            for (int j = a - rb; j < b - rb; ++j) dst[j] = (uint8_t)(w[j >> 2] >> (8 * (j & 3)));
        }
    }
}

__global__ __launch_bounds__(kGThreads)
void group_quant_col_kernel(const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ offs, int G,
                            const float* __restrict__ scales, uint8_t* __restrict__ q)
{
    const Chunk ch = locate_chunk<kQuantRows>(offs, G, M, (int)blockIdx.x, true);
    if (ch.g < 0) return;
    __shared__ __align__(16) uint8_t tile[kColStrip * kQuantRows];
    const int t = (int)threadIdx.x;
    const int cg = t & 15;                    // 8-column group of the strip
    const int rs = t >> 4;                    // 4-row slot, 0..15
    const int k = (int)blockIdx.y * kColStrip + cg * 8;
    const int a = (ch.r0 / kQuantRows) * kQuantRows;
    const bool live = k < K && ch.g < G;
    ColScales cs;
    if (live) cs = load_col_scales(scales, ch.g, K, k);
    for (int p = 0; p < 2; ++p) {
        uint4 v[4];
        bool in[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = a + p * 64 + rs * 4 + i;
            in[i] = live && row >= ch.r0 && row < ch.r1;
            v[i] = in[i] ? *(const uint4*)(x + (int64_t)row * K + k) : make_uint4(0, 0, 0, 0);
        }
        uint2 qr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) qr[i] = in[i] ? group_quantize_chunk(v[i], cs) : make_uint2(0, 0);
        // 4 rows x 8 columns of bytes -> one dword (4 consecutive rows) per column
        const int r0 = p * 64 + rs * 4;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int sh = 8 * (c & 3);
            uint32_t d = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = c < 4 ? qr[i].x : qr[i].y;
                d |= ((w >> sh) & 0xFFu) << (8 * i);
            }
            *(uint32_t*)(tile + tile_offset(cg * 8 + c, r0)) = d;
        }
    }
    __syncthreads();
    store_tile_rows(tile, q, M, (int64_t)blockIdx.y * kColStrip, K, a, ch.r0 - a, ch.r1 - a, (M & 15) == 0);
}

// --------------------------------------------------------------- launch ---
static int64_t chunk_slots(int64_t M, int R, int64_t G) { return (M + R - 1) / R + G; }

size_t group_scale_workspace_bytes(int64_t M, int64_t K, int32_t G)
{
    const int64_t bytes = chunk_slots(M, kAmaxRows, G) * K * 2;
    return (size_t)((bytes + 255) / 256 * 256);
}

hipError_t launch_group_scale(const void* x, int M, int K, const int32_t* offs, int G, int layout,
                              void* q, float* scales, void* workspace, hipStream_t stream)
{
    uint16_t* partial = (uint16_t*)workspace;
    if (M > 0) {
        const dim3 grid((unsigned)chunk_slots(M, kAmaxRows, G), (unsigned)((K + kRowStrip - 1) / kRowStrip));
        hipLaunchKernelGGL(group_amax_kernel, grid, dim3(kGThreads), 0, stream,
                           (const uint16_t*)x, M, K, offs, G, partial);
    }
    {
        const dim3 grid((unsigned)G, (unsigned)((K + kScaleCols - 1) / kScaleCols));
        hipLaunchKernelGGL(group_scales_kernel, grid, dim3(kGThreads), 0, stream, M, K, offs, G,
                           (const uint16_t*)partial, scales);
    }
    if (M > 0) {
        if (layout == 0) {
            const dim3 grid((unsigned)chunk_slots(M, kQuantRows, G), (unsigned)((K + kRowStrip - 1) / kRowStrip));
            hipLaunchKernelGGL(group_quant_row_kernel, grid, dim3(kGThreads), 0, stream,
                               (const uint16_t*)x, M, K, offs, G, (const float*)scales, (uint8_t*)q);
        } else {
            const dim3 grid((unsigned)chunk_slots(M, kQuantRows, G), (unsigned)((K + kColStrip - 1) / kColStrip));
            hipLaunchKernelGGL(group_quant_col_kernel, grid, dim3(kGThreads), 0, stream,
                               (const uint16_t*)x, M, K, offs, G, (const float*)scales, (uint8_t*)q);
        }
    }
    return hipGetLastError();
}

}  // namespace mxq
