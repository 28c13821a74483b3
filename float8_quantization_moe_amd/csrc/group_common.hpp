// group_common.hpp -- device helpers of the per-group float8 scaling kernels:
// the scale of a column, the binary32 quantizer, coherent cross-workgroup
// accesses, raw buffer accesses and the byte transposes of the column-major
// output.
//
// "[moe training] fix uncoalesced global accesses in per group rowwise scaling
// kernel", Summary: per-group scaling of the grouped GEMM's left operand.
// Per group g and column k: amax = max |x| over the group's rows,
// s = 448 / max(amax, 1e-12) in binary32, q = e4m3(binary32(x * s)) with
// nearest-even rounding saturated at +-448.
#pragma once

#include "device_common.hpp"

namespace mxq {

// ------------------------------------------------------------- helpers ----
// The multiplier of a column: 448 / max(amax, 1e-12) (correctly rounded divide),
// or that rounded down to a power of two (clearing the significand: the
// quotient is always a positive normal, between 448 / bf16 max and 448 / 1e-12).
__device__ __forceinline__ float group_scale_of(uint32_t amax_bits, int pow2)
{
    if (amax_bits >= 0x7F80u) return __uint_as_float(0x7FC00000u);   // Inf/NaN in the column
    const float amax = __uint_as_float(amax_bits << 16);
    const float s = 448.0f / fmaxf(amax, 1e-12f);
    return pow2 ? __uint_as_float(__float_as_uint(s) & 0xFF800000u) : s;
}

// The stored inverse 1/s of a multiplier (one correctly rounded divide; NaN kept).
__device__ __forceinline__ float4 inverse4(float4 m)
{
    const auto inv = [](float v) { return v != v ? v : 1.0f / v; };
    return make_float4(inv(m.x), inv(m.y), inv(m.z), inv(m.w));
}

struct ColScales {
    float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t nan_lo = 0, nan_hi = 0;   // 0xFF in each byte whose column has a NaN scale
};

__device__ __forceinline__ ColScales make_col_scales(float4 a, float4 b)
{
    ColScales cs;
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

__device__ __forceinline__ void max8(uint4& a, uint4 b)
{
    a.x = pk_max_u16(a.x, b.x);
    a.y = pk_max_u16(a.y, b.y);
    a.z = pk_max_u16(a.z, b.z);
    a.w = pk_max_u16(a.w, b.w);
}

__device__ __forceinline__ uint4 abs8(uint4 v)
{
    return make_uint4(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu, v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu);
}

// a = max(a, red[1..n-1][cg]), two LDS rows per step so that few registers are
// live while a tile is held.
__device__ __forceinline__ void max_rows(uint4& a, const uint4* red, int n, int stride)
{
#pragma unroll 1
    for (int r = 1; r < n; r += 2) {
        const uint4 b0 = red[r * stride];
        const uint4 b1 = r + 1 < n ? red[(r + 1) * stride] : make_uint4(0, 0, 0, 0);
        max8(a, b0);
        max8(a, b1);
    }
}

// ---------------------------------------------------- coherent accesses ---
// Relaxed agent-scope atomics: each access reaches the coherence point shared by
// all XCDs, so a value written by a workgroup on one XCD is eventually seen by
// a workgroup polling it on another.
__device__ __forceinline__ void store_coherent(uint4 v, void* p)
{
    unsigned long long* q = (unsigned long long*)p;
    __hip_atomic_store(q, ((unsigned long long)v.y << 32) | v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, ((unsigned long long)v.w << 32) | v.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint4 load_coherent(const void* p)
{
    const unsigned long long* q = (const unsigned long long*)p;
    const unsigned long long a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
}

// ------------------------------------------------------ buffer accesses ---
// Raw buffer accesses through a (base, size) resource: at an offset at or past
// the size a load reads zero and a store is dropped, without touching memory.
// X is read once and the codes written once, so both use the streaming
// (non-temporal) cache policy, which measured about 10 % faster in the hold
// kernel than the default one.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOOB = 0xFFFFFFF0u;      // above every resource size used here (at most 2^31)
constexpr int kNonTemporal = 2;             // cache-policy operand of the buffer builtins: nt
constexpr int kCached = 0;                  // the default policy (lines kept in the caches)

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// `soff` is a wave-uniform byte offset carried in the instruction's scalar
// offset field (no vector register for it).
template <int POLICY = kNonTemporal>
__device__ __forceinline__ uint4 buf_load16(Rsrc r, uint32_t off, uint32_t soff = 0)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, POLICY);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void buf_store8(uint2 v, Rsrc r, uint32_t off, uint32_t soff = 0)
{
    const u32x2 w = {v.x, v.y};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, soff, kNonTemporal);
}

// Workgroup-wide OR of a predicate; every thread of the workgroup must call it.
// Each wave's ballot goes to its own LDS word, which every lane then reads back
// as a broadcast; the closing barrier keeps the next vote's writes behind these
// reads.  (The built-in __syncthreads_or has every lane OR into one LDS word:
// 64 serialised accesses per wave.)  It is also a full workgroup barrier.
template <int NWAVES>
__device__ __forceinline__ bool block_any(bool p, uint32_t* votes)
{
    const bool wave_any = __ballot(p) != 0ull;
    if ((threadIdx.x & 63) == 0) votes[threadIdx.x >> 6] = wave_any ? 1u : 0u;
    __syncthreads();
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < NWAVES; ++i) r |= votes[i];
    __syncthreads();
    return r != 0u;
}

// Inclusive running maximum over the lanes of a wave (values >= 0): DPP row
// shifts within each 16-lane row, then the row broadcasts.
__device__ __forceinline__ int dpp_scan_max(int v)
{
    const auto mx = [](int a, int b) { return a > b ? a : b; };
    v = mx(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true));    // row_shr:1
    v = mx(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true));    // row_shr:2
    v = mx(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true));    // row_shr:4
    v = mx(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true));    // row_shr:8
    v = mx(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));   // row_bcast:15
    v = mx(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));   // row_bcast:31
    return v;
}
// The previous lane's value (0 in lane 0).
__device__ __forceinline__ int dpp_prev_lane(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, 0x138, 0xF, 0xF, true);         // wave_shr:1
}

// Inclusive sum over the lanes of a wave, with the same DPP row shifts and row
// broadcasts.
__device__ __forceinline__ int dpp_scan_add(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);    // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);    // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);    // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);    // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return v;
}

// An opaque copy: the compiler cannot relate the result to its input, so
// offsets derived from it are recomputed where used instead of being kept in
// registers from an earlier phase.
__device__ __forceinline__ int opaque(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Byte offset of (column c, row r) inside the column-layout staging tile
// (256 columns x 128 rows): each column is 128 contiguous bytes whose 16-byte
// units are XOR-swizzled by bits of the column to spread the LDS banks.
__device__ __forceinline__ int col_tile_offset(int c, int r)
{
    return c * 128 + ((((r >> 4) ^ (c >> 3)) & 7) << 4) + (r & 15);
}

// Store bytes [lo, hi) of a 16-byte unit at dst (dst 16-byte aligned when
// `aligned`): the widest naturally aligned pieces that fit, bytes otherwise.
__device__ __forceinline__ void store_partial16(uint4 val, uint8_t* dst, int lo, int hi, bool aligned)
{
    const unsigned long long w[2] = {((unsigned long long)val.y << 32) | val.x,
                                     ((unsigned long long)val.w << 32) | val.z};
    int b = lo;
    while (b < hi) {
        const unsigned long long word = w[b >> 3] >> (8 * (b & 7));
        if (aligned && (b & 7) == 0 && hi - b >= 8) {
            *(unsigned long long*)(dst + b) = word;
            b += 8;
        } else if (aligned && (b & 3) == 0 && hi - b >= 4) {
            *(uint32_t*)(dst + b) = (uint32_t)word;
            b += 4;
        } else if (aligned && (b & 1) == 0 && hi - b >= 2) {
            *(uint16_t*)(dst + b) = (uint16_t)word;
            b += 2;
        } else {
            dst[b] = (uint8_t)word;
            b += 1;
        }
    }
}

__device__ __forceinline__ float4 scales_lo(uint4 a, int pow2)
{
    return make_float4(group_scale_of(a.x & 0xFFFFu, pow2), group_scale_of(a.x >> 16, pow2),
                       group_scale_of(a.y & 0xFFFFu, pow2), group_scale_of(a.y >> 16, pow2));
}
__device__ __forceinline__ float4 scales_hi(uint4 a, int pow2)
{
    return make_float4(group_scale_of(a.z & 0xFFFFu, pow2), group_scale_of(a.z >> 16, pow2),
                       group_scale_of(a.w & 0xFFFFu, pow2), group_scale_of(a.w >> 16, pow2));
}
__device__ __forceinline__ uint4 f4_bits(float4 f)
{
    return make_uint4(__float_as_uint(f.x), __float_as_uint(f.y), __float_as_uint(f.z), __float_as_uint(f.w));
}
__device__ __forceinline__ float4 bits_f4(uint4 u)
{
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}

__device__ __forceinline__ void transpose4x4_bytes(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, uint32_t out[4])
{
    // w_r holds columns 0..3 of row r; out[c] holds rows 0..3 of column c
    const uint32_t t01_lo = __builtin_amdgcn_perm(w1, w0, 0x05010400u);   // w0.0 w1.0 w0.1 w1.1
    const uint32_t t01_hi = __builtin_amdgcn_perm(w1, w0, 0x07030602u);   // w0.2 w1.2 w0.3 w1.3
    const uint32_t t23_lo = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
    const uint32_t t23_hi = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
    out[0] = __builtin_amdgcn_perm(t23_lo, t01_lo, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(t23_lo, t01_lo, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(t23_hi, t01_hi, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(t23_hi, t01_hi, 0x07060302u);
}

}  // namespace mxq
