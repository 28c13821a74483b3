// transpose.hip -- byte transpose out (C, R) = in (R, C)^T on gfx950.
//
// "[moe training] fix uncoalesced global accesses in per group rowwise scaling
// kernel", Summary: with many groups the scaled fp8 tensor was written in the
// other layout and transformed afterwards; this is that transform, usable in
// either direction between the two outputs of the group-scaling kernel.
//
// One workgroup per 128 x 128-byte tile.  Each lane loads 16 contiguous bytes of
// 4 consecutive rows (a wave reads 8 rows x 128 bytes), transposes the 4 x 16
// byte block in registers into 16 dwords (4 consecutive output columns each),
// writes them into a swizzled LDS tile, and the workgroup then stores 128
// contiguous bytes per output row.  Edge tiles and widths that are not a multiple
// of 16 fall back to byte accesses for the affected pieces.  The 16-byte loads
// and stores use the streaming (non-temporal) policy: every byte is touched once
// (measured 35.5 -> 33.3 us at 5120 x 16640).  Consecutive workgroups take
// consecutive tiles down a tile column, so the workgroups running at once
// (one per XCD in turn) write adjacent pieces of the same output rows (33.0 ->
// 31.5 us; 128 x 256 tiles, two tiles per workgroup and 2-D super-tile orders
// measured the same or slower).  At that point the reads alone run at 78 % and
// the writes alone at 72 % of the HBM peak: the transpose moves as many bytes
// each way, and the turnaround between the two is what is left.
#include "device_common.hpp"
#include "internal.hpp"

namespace mxq {

constexpr int kTThreads = 256;
constexpr int kTile = 128;

// Tile byte (column c, row r): each column's 128 bytes are 8 16-byte pieces,
// permuted by c >> 4 so that the 8 lanes of a half-wave writing the same row
// offset of 8 columns 16 apart hit 8 different pieces (32 different banks).
__device__ __forceinline__ int ttile_offset(int c, int r)
{
    return c * kTile + ((((r >> 4) ^ (c >> 4)) & 7) << 4) + (r & 15);
}

__global__ __launch_bounds__(kTThreads)
void transpose_u8_kernel(const uint8_t* __restrict__ in, int64_t R, int64_t C, uint8_t* __restrict__ out,
                         int64_t tiles_r)
{
    __shared__ __align__(16) uint8_t tile[kTile * kTile];
    const int64_t ti = (int64_t)blockIdx.x % tiles_r, tj = (int64_t)blockIdx.x / tiles_r;
    const int64_t i0 = ti * kTile, j0 = tj * kTile;
    const int t = (int)threadIdx.x;
    const int cg = t & 7;          // 16-byte column group, 0..7
    const int rs = t >> 3;         // 4-row slot, 0..31
    const int64_t c = j0 + cg * 16;
    const bool fast_in = (C & 15) == 0 && c < C;
    uint4 rows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = i0 + rs * 4 + i;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < R) {
            const uint8_t* src = in + r * C + c;
            if (fast_in) {
                v = load_nt((const uint4*)src);
            } else {
                uint32_t w[4] = {0, 0, 0, 0};
                for (int b = 0; b < 16 && c + b < C; ++b) w[b >> 2] |= (uint32_t)src[b] << (8 * (b & 3));
                v = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        rows[i] = v;
    }
    // 4 rows x 16 bytes -> 16 dwords, dword j = byte j of each of the 4 rows
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int sh = 8 * (j & 3);
        uint32_t d = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = (j < 4) ? rows[i].x : (j < 8) ? rows[i].y : (j < 12) ? rows[i].z : rows[i].w;
            d |= ((w >> sh) & 0xFFu) << (8 * i);
        }
        *(uint32_t*)(tile + ttile_offset(cg * 16 + j, rs * 4)) = d;
    }
    __syncthreads();
    // tile column cc (= input column j0 + cc) becomes output row j0 + cc
    const bool aligned_out = (R & 15) == 0;
    const int valid_rows = (int)((R - i0) < kTile ? (R - i0) : kTile);
    for (int i = 0; i < 4; ++i) {
        const int sid = t + kTThreads * i;
        const int cc = sid >> 3, seg = sid & 7;
        if (j0 + cc >= C) continue;
        const int rb = seg * 16;
        if (rb >= valid_rows) continue;
        const int nb = valid_rows - rb < 16 ? valid_rows - rb : 16;
        const uint4 val = *(const uint4*)(tile + ttile_offset(cc, rb));
        uint8_t* dst = out + (j0 + cc) * R + i0 + rb;
        if (aligned_out && nb == 16) {
            store_nt(val, (uint4*)dst);
        } else {
            const uint32_t w[4] = {val.x, val.y, val.z, val.w};
            for (int b = 0; b < nb; ++b) dst[b] = (uint8_t)(w[b >> 2] >> (8 * (b & 3)));
        }
    }
}

hipError_t launch_transpose_u8(const void* in, int64_t R, int64_t C, void* out, hipStream_t stream)
{
    const int64_t tiles_r = (R + kTile - 1) / kTile, tiles_c = (C + kTile - 1) / kTile;
    hipLaunchKernelGGL(transpose_u8_kernel, dim3((unsigned)(tiles_r * tiles_c)), dim3(kTThreads), 0, stream,
                       (const uint8_t*)in, R, C, (uint8_t*)out, tiles_r);
    return hipGetLastError();
}

}  // namespace mxq
