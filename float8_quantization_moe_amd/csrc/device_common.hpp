// device_common.hpp -- small device helpers shared by the libmxq kernels (gfx950).
//
// Conversions used by the kernels (their rounding was checked exhaustively
// against the reference encoder: every bf16 pattern x every E8M0 scale code for
// quantization, every E4M3 code x every scale code for dequantization):
//   v_cvt_scalef32_pk_fp8_bf16  bf16 pair / 2^e  -> E4M3 pair, nearest-even, no saturation
//   v_cvt_pk_fp8_f32            fp32 pair        -> E4M3 pair, nearest-even, no saturation
//   v_cvt_scalef32_pk_bf16_fp8  E4M3 pair * 2^e  -> bf16 pair, nearest-even, subnormals kept
// "No saturation" means a magnitude that rounds past 448 becomes NaN, so every
// quantizing path clamps to +-448 (times the block scale) before converting.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) 16- and 8-byte global accesses.
__device__ __forceinline__ uint4 load_nt(const uint4* p)
{
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_nt(const uint2* p)
{
    const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void store_nt(uint4 v, uint4* p)
{
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (u32x4*)p);
}
__device__ __forceinline__ void store_nt(uint2 v, uint2* p)
{
    const u32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, (u32x2*)p);
}

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b)
{
    v2u16 r = __builtin_elementwise_max(__builtin_bit_cast(v2u16, a), __builtin_bit_cast(v2u16, b));
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b)
{
    v2u16 r = __builtin_elementwise_min(__builtin_bit_cast(v2u16, a), __builtin_bit_cast(v2u16, b));
    return __builtin_bit_cast(uint32_t, r);
}

// binary32 with the biased exponent e (1..254) and zero mantissa; e == 0 gives 2^-127.
__device__ __forceinline__ float pow2_from_biased(uint32_t e)
{
    return __uint_as_float(e ? (e << 23) : 0x00400000u);
}

// E8M0 code of a block whose largest |bf16| bit pattern is amax (finite).  E is
// amax's biased exponent, so floor(log2 amax) = E - 127 for normal amax.
//   floor rule (OCP MX v1.0): floor(log2 amax) - 8, i.e. code E - 8.
//   RCEIL: the smallest e with amax <= 448 * 2^e.  448 * 2^(E-127-8) is 1.75 *
//     2^(E-127), so e is E - 135 when amax's significand is at most 1.75
//     (mantissa bits <= 0x60) and one more otherwise: code E - 8 + (m > 0x60).
// Both clamp at code 0 (amax zero, subnormal or below the smallest scale).
template <bool RCEIL>
__device__ __forceinline__ uint32_t mx_scale_code(uint32_t amax)
{
    const uint32_t E = (amax >> 7) + (RCEIL && (amax & 0x7Fu) > 0x60u ? 1u : 0u);
    return E > 8u ? E - 8u : 0u;
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Max over each aligned quad of lanes (DPP quad permutations).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v)
{
    uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);           // [2,3,0,1]
    return v > t ? v : t;
}

// Non-zero in each byte lane of the result whose input byte is 0x7F or 0xFF.
__device__ __forceinline__ uint32_t nan_code_bytes(uint32_t q)
{
    uint32_t t = q & 0x7F7F7F7Fu;
    return (t + 0x01010101u) & 0x80808080u;
}

// ------------------------------------------------------------------ scans --
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ int wave_incl_max(int v)
{
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int t = __shfl_up(v, d, kWave);
        if (lane >= d) v = v > t ? v : t;
    }
    return v;
}

__device__ __forceinline__ int wave_incl_sum(int v)
{
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int t = __shfl_up(v, d, kWave);
        if (lane >= d) v += t;
    }
    return v;
}

__device__ __forceinline__ int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

}  // namespace mxq
