// group_split.hip -- per-expert-group float8 scaling in two streaming passes
// (the "split" method of mxq_group_scale_fp8) on gfx950.
//
// "[moe training] fix uncoalesced global accesses in per group rowwise scaling
// kernel", Summary and Performance: per-group scaling of a (tokens, hidden)
// tensor whose fp8 output is the LHS of the scaled grouped GEMM, stored
// row-major or column-major (the pages found column-major output plus a
// transform faster for many groups).  Per group g and column k: amax = max |x|
// over the group's rows, s = 448 / max(amax, 1e-12) in binary32,
// q = e4m3(binary32(x * s)) nearest-even, saturated at +-448; s is stored.
//
// Two launches over tiles of 128 rows x 128 columns whose rows are aligned
// blocks that ignore group boundaries:
//   amax      every tile takes the column maxima of each group segment in its
//             block and writes them as the partial row b + g of block b and
//             group g (unique: blocks and groups are both ordered);
//   quantize  every tile reduces the partial rows of its groups (the group's
//             blocks, 1 to 43 rows at 16640 x 5120 -- the whole partial array
//             is 1.5 MB and stays in the caches), divides, quantizes and stores
//             whole 128-byte lines in either layout; the first block of a
//             group also stores the group's scales.
// No workgroup ever waits for another and no table is built in between: each
// tile clamps the group ends itself with a DPP wave scan over at most 256
// offsets, loaded ahead of its tile.  Two launches, against the two-pass
// method's three (four with its plan launch); X is read twice (5 bytes moved
// per element against the method's 3).  Only taken when forced: the two-pass
// method measured faster wherever this one would apply (16 to 128 groups at
// 16640 x 5120, 4 to 32 at 16640 x 8192, 8 to 256 at 65536 x 5120).
//
// The quantizer needs no clamp: with s = 448 / max(amax, 1e-12) every product
// x * s is at most 448 (1 + 2^-24) after binary32 rounding, which the E4M3
// conversion rounds to 448 (NaN only starts past 464); a column holding Inf or
// NaN has the NaN scale and its codes are set to 0x7F.
#include "group_common.hpp"
#include "internal.hpp"

namespace mxq {

namespace {

constexpr int kSR = 128;              // rows per block
constexpr int kST = 256;              // threads per workgroup
constexpr int kSW = 128;              // tile width (columns)
constexpr int kMaxGroups = 256;       // group ends held in registers (4 per lane)
constexpr int CG = kSW / 8;           // lanes per row (8 columns each)
constexpr int NS = kST / CG;          // row slots
constexpr int H = kSR / NS;           // consecutive rows per lane
constexpr int kWaves = kST / 64;
// Amax-pass tile width (columns).  Measured at 16640 x 5120, column-major (amax
// pass alone, kernel trace): 128 / 256 / 512 columns take 30.3 / 29.7 / 30.9 us
// at 16 groups and 35.7 / 36.8 / 39.2 us at 128 groups.
constexpr int kSplitAmaxWidth = 256;
static_assert(H == 8 && CG == 16, "tile shape");

// The clamped group ends, end(g) = min(M, max(0, offs[0..g])), of all G <= 256
// groups, held 4 per lane (group 64 j + l in e[j] of lane l) and read with
// readlane.  start(g) = end(g - 1), start(0) = 0.
struct Groups {
    int e[4];
    int nw;       // windows in use
    __device__ void load(const int32_t* __restrict__ offs, int G)
    {
        const int lane = lane_id();
        nw = (G + kWave - 1) / kWave;
#pragma unroll
        for (int j = 0; j < 4; ++j) e[j] = j < nw && 64 * j + lane < G ? offs[64 * j + lane] : 0;
    }
    __device__ void scan(int M)
    {
        int carry = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j >= nw) break;
            int v = dpp_scan_max(e[j] > 0 ? e[j] : 0);
            v = v > carry ? v : carry;
            e[j] = v < M ? v : M;            // min(M, .) commutes with the running maximum
            carry = readlane(e[j], kWave - 1);
        }
    }
    __device__ int end(int g) const
    {
        const int j = g >> 6, l = g & 63;
        if (j == 0) return readlane(e[0], l);
        if (j == 1) return readlane(e[1], l);
        if (j == 2) return readlane(e[2], l);
        return readlane(e[3], l);
    }
    __device__ int start(int g) const { return g == 0 ? 0 : end(g - 1); }
    // first group whose end lies past row r (G if none)
    __device__ int first_past(int r, int G) const
    {
        const int lane = lane_id();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j >= nw) break;
            const unsigned long long m = __ballot(64 * j + lane < G && e[j] > r);
            if (m) return 64 * j + __builtin_ctzll(m);
        }
        return G;
    }
};

template <int T, int LCG>
struct AmaxShared {
    uint4 red[T / 64][LCG];
};

// The amax pass's tiles: 128 rows x AW columns for AT threads (AW / 8 lanes
// per row); wider tiles read longer runs of each row.
template <int AW>
struct AmaxCfg {
    static constexpr int T = AW >= 512 ? 512 : 256;
    static constexpr int LCG = AW / 8 < 64 ? AW / 8 : 64;
    static constexpr int LNS = T / LCG;
    static constexpr int LH = kSR / LNS;
};

struct SplitShared {
    union {
        __align__(16) uint8_t stage[kSW * kSR];          // column-major staging (quantize pass, at the end)
        uint4 red[kWaves][CG];                           // per-wave column maxima (before that)
    };
    float4 scale_lo[CG], scale_hi[CG];                   // a lane's 8 scales, by column group
    __align__(16) uint32_t vote[kWaves];
};

// Column maxima over the row slots: the 4 row slots of a wave first (lanes 16
// apart hold the same columns), then the waves through LDS.  Every lane gets
// the result; the LDS rows are free again on return.
template <int LCG = CG, class Sh>
__device__ __forceinline__ uint4 reduce_slots(uint4 m, int cg, Sh& sh)
{
#pragma unroll
    for (int d = LCG; d < kWave; d <<= 1) {
        uint4 t;
        t.x = (uint32_t)__shfl_xor((int)m.x, d, kWave);
        t.y = (uint32_t)__shfl_xor((int)m.y, d, kWave);
        t.z = (uint32_t)__shfl_xor((int)m.z, d, kWave);
        t.w = (uint32_t)__shfl_xor((int)m.w, d, kWave);
        max8(m, t);
    }
    constexpr int nw = sizeof(sh.red) / sizeof(sh.red[0]);
    if (lane_id() < LCG) sh.red[threadIdx.x / kWave][cg] = m;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < nw; ++r) max8(m, sh.red[r][cg]);
    __syncthreads();
    return m;
}

// 8 bf16 of one row -> 8 E4M3 codes: binary32 product, nearest-even convert
// (no clamp needed, see above).  FIX replaces the codes of NaN-scale columns
// by 0x7F.  The unpacking shift and mask come in as opaque values so that the
// compiler cannot hoist the unpacked tile (64 registers) out of a loop.
template <bool FIX>
__device__ __forceinline__ uint2 quantize8(uint4 v, const ColScales& cs, uint32_t sh16, uint32_t mhi)
{
    const auto lo = [&](uint32_t w) { return __uint_as_float(w << sh16); };
    const auto hi = [&](uint32_t w) { return __uint_as_float(w & mhi); };
    int l = __builtin_amdgcn_cvt_pk_fp8_f32(lo(v.x) * cs.s[0], hi(v.x) * cs.s[1], 0, false);
    l = __builtin_amdgcn_cvt_pk_fp8_f32(lo(v.y) * cs.s[2], hi(v.y) * cs.s[3], l, true);
    int h = __builtin_amdgcn_cvt_pk_fp8_f32(lo(v.z) * cs.s[4], hi(v.z) * cs.s[5], 0, false);
    h = __builtin_amdgcn_cvt_pk_fp8_f32(lo(v.w) * cs.s[6], hi(v.w) * cs.s[7], h, true);
    if (!FIX) return make_uint2((uint32_t)l, (uint32_t)h);
    const uint32_t ul = ((uint32_t)l & ~cs.nan_lo) | (0x7F7F7F7Fu & cs.nan_lo);
    const uint32_t uh = ((uint32_t)h & ~cs.nan_hi) | (0x7F7F7F7Fu & cs.nan_hi);
    return make_uint2(ul, uh);
}

__device__ __forceinline__ uint32_t opaque_u32(uint32_t v)
{
    asm volatile("" : "+v"(v));
    return v;
}


// ------------------------------------------------------------ amax pass ---
template <int AW>
__global__ __launch_bounds__(AmaxCfg<AW>::T)
void group_split_amax_kernel(const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ offs, int G,
                             int S, uint16_t* __restrict__ partial)
{
    using C = AmaxCfg<AW>;
    __shared__ AmaxShared<C::T, C::LCG> sh;
    const int blk = (int)blockIdx.x / S, s = (int)blockIdx.x % S;
    const int cg = (int)threadIdx.x % C::LCG, rs = (int)threadIdx.x / C::LCG;
    const int k = s * AW + cg * 8;
    const int row0 = blk * kSR;
    const int nrows = M - row0 < kSR ? M - row0 : kSR;
    const int row1 = row0 + nrows;
    const int rbase = rs * C::LH;
    Groups gr;
    gr.load(offs, G);                                     // (ahead of the tile: its wait excludes the tile's)
    // rows past M fall outside the resource, columns past K get an offset
    // outside it; both read zero.  Default cache policy: the quantize pass
    // reads X again.
    const Rsrc rx = make_rsrc(x + (int64_t)row0 * K, (uint32_t)nrows * (uint32_t)K * 2u);
    const uint32_t xoff = k < K ? ((uint32_t)rbase * (uint32_t)K + (uint32_t)k) * 2u : kOOB;
    uint4 v[C::LH];
#pragma unroll
    for (int i = 0; i < C::LH; ++i) v[i] = buf_load16<kCached>(rx, xoff, (uint32_t)i * (uint32_t)K * 2u);
    gr.scan(M);
#pragma unroll
    for (int i = 0; i < C::LH; ++i) v[i] = abs8(v[i]);
    for (int g = gr.first_past(row0, G); g < G; ++g) {
        const int st = gr.start(g), en = gr.end(g);
        if (st >= row1) break;
        if (en <= st) continue;
        uint4 m = make_uint4(0, 0, 0, 0);
        if (st <= row0 && en >= row1) {                   // the whole block (uniform)
#pragma unroll
            for (int i = 0; i < C::LH; ++i) max8(m, v[i]);
        } else {
            const int lo = (st > row0 ? st : row0) - row0, hi = (en < row1 ? en : row1) - row0;
#pragma unroll
            for (int i = 0; i < C::LH; ++i)
                max8(m, rbase + i >= lo && rbase + i < hi ? v[i] : make_uint4(0, 0, 0, 0));
        }
        m = reduce_slots<C::LCG>(m, cg, sh);
        if (rs == 0 && k < K) *(uint4*)(partial + (int64_t)(blk + g) * K + k) = m;
    }
}

// -------------------------------------------------------- quantize pass ---
template <int LAYOUT>
__global__ __launch_bounds__(kST)
void group_split_quant_kernel(const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ offs, int G,
                              int S, const uint16_t* __restrict__ partial, float* __restrict__ scales_out, int flags,
                              uint8_t* __restrict__ q)
{
    __shared__ SplitShared sh;
    const int blk = (int)blockIdx.x / S, s = (int)blockIdx.x % S;
    const int nblk = (M + kSR - 1) / kSR;
    const int cg = (int)threadIdx.x % CG, rs = (int)threadIdx.x / CG;
    const int k = s * kSW + cg * 8;
    const int row0 = blk * kSR;
    const int nrows = M - row0 < kSR ? M - row0 : kSR;
    const int row1 = row0 + nrows;
    const int rbase = rs * H;
    Groups gr;
    gr.load(offs, G);
    const Rsrc rx = make_rsrc(x + (int64_t)row0 * K, (uint32_t)nrows * (uint32_t)K * 2u);
    const uint32_t xoff = k < K ? ((uint32_t)rbase * (uint32_t)K + (uint32_t)k) * 2u : kOOB;
    uint4 v[H];
#pragma unroll
    for (int i = 0; i < H; ++i) v[i] = buf_load16<kNonTemporal>(rx, xoff, (uint32_t)i * (uint32_t)K * 2u);
    gr.scan(M);
    const int pow2 = flags & 1, inverse = (flags & 2) != 0;
    const Rsrc rq = make_rsrc(q + (int64_t)row0 * K, (uint32_t)nrows * (uint32_t)K);
    const uint32_t qoff = k < K ? (uint32_t)rbase * (uint32_t)K + (uint32_t)k : kOOB;
    uint2 out[LAYOUT == 1 ? H : 1];
#pragma unroll
    for (int i = 0; i < (LAYOUT == 1 ? H : 1); ++i) out[i] = make_uint2(0, 0);
    int covered = 0;                                      // rows [0, covered) of the block are in a group
    for (int g = gr.first_past(row0, G); g < G; ++g) {
        const int st = gr.start(g), en = gr.end(g);
        if (st >= row1) break;
        if (en <= st) continue;
        const int lo = (st > row0 ? st : row0) - row0, hi = (en < row1 ? en : row1) - row0;
        const int fb = st / kSR, lb = (en - 1) / kSR;
        // the group's partial rows fb + g .. lb + g (this lane: rows rs, rs + NS, ...)
        uint4 a = make_uint4(0, 0, 0, 0);
        if (k < K) {
            const uint16_t* p = partial + (int64_t)(fb + g) * K + k;
            const int n = lb - fb + 1;
            int r = rs;
            for (; r + NS < n; r += 2 * NS) {
                const uint4 b0 = *(const uint4*)(p + (int64_t)r * K);
                const uint4 b1 = *(const uint4*)(p + (int64_t)(r + NS) * K);
                max8(a, b0);
                max8(a, b1);
            }
            if (r < n) max8(a, *(const uint4*)(p + (int64_t)r * K));
        }
        a = reduce_slots(a, cg, sh);
        if (rs == 0) {
            const float4 lo4 = scales_lo(a, pow2), hi4 = scales_hi(a, pow2);
            sh.scale_lo[cg] = lo4;
            sh.scale_hi[cg] = hi4;
            if (blk == fb && k < K) {                     // the group's first block stores its scales
                float* dst = scales_out + (int64_t)g * K + k;
                *(float4*)dst = inverse ? inverse4(lo4) : lo4;
                *(float4*)(dst + 4) = inverse ? inverse4(hi4) : hi4;
            }
        }
        __syncthreads();
        const ColScales cs = make_col_scales(sh.scale_lo[cg], sh.scale_hi[cg]);
        const bool fix = block_any<kWaves>((cs.nan_lo | cs.nan_hi) != 0u, sh.vote);   // (also: the scales in LDS free again)
        const uint32_t sh16 = opaque_u32(16u), mhi = opaque_u32(0xFFFF0000u);
        if (lo <= rbase && hi >= rbase + H) {             // all the lane's rows in this group
#pragma unroll
            for (int i = 0; i < H; ++i) {
                const uint2 c = fix ? quantize8<true>(v[i], cs, sh16, mhi) : quantize8<false>(v[i], cs, sh16, mhi);
                if (LAYOUT == 0)
                    buf_store8(c, rq, qoff, (uint32_t)i * (uint32_t)K);
                else
                    out[LAYOUT == 1 ? i : 0] = c;
            }
        } else {
#pragma unroll
            for (int i = 0; i < H; ++i) {
                if (rbase + i >= lo && rbase + i < hi) {
                    const uint2 c = fix ? quantize8<true>(v[i], cs, sh16, mhi) : quantize8<false>(v[i], cs, sh16, mhi);
                    if (LAYOUT == 0)
                        buf_store8(c, rq, qoff, (uint32_t)i * (uint32_t)K);
                    else
                        out[LAYOUT == 1 ? i : 0] = c;
                }
            }
        }
        covered = hi;
    }
    // Empty groups whose start lies in this block (a start at M belongs to the
    // last block) get the scale of amax 0 for this tile's columns.  Wave 0
    // finds them (all its lanes take part); its lanes with rs == 0 own the
    // tile's columns.
    if (threadIdx.x < kWave) {
        const int lane = lane_id();
        int prev = 0;                                     // end of the group before this window
        for (int j = 0; j < gr.nw; ++j) {
            const int en = j == 0 ? gr.e[0] : j == 1 ? gr.e[1] : j == 2 ? gr.e[2] : gr.e[3];
            int st = dpp_prev_lane(en);
            if (lane == 0) st = prev;
            prev = readlane(en, kWave - 1);
            const bool own = 64 * j + lane < G && en == st && st >= row0 && (st < row1 || (st == M && blk == nblk - 1));
            const unsigned long long m = __ballot(own);
            if (m && rs == 0 && k < K) {
                const float se = group_scale_of(0u, pow2);
                const float so = inverse ? 1.0f / se : se;
                const float4 s4 = make_float4(so, so, so, so);
                for (unsigned long long mm = m; mm; mm &= mm - 1) {
                    float* dst = scales_out + (int64_t)(64 * j + __builtin_ctzll(mm)) * K + k;
                    *(float4*)dst = s4;
                    *(float4*)(dst + 4) = s4;
                }
            }
        }
    }

    if (LAYOUT == 0) {
        // rows past the last end: code 0
#pragma unroll
        for (int i = 0; i < H; ++i)
            if (rbase + i >= covered) buf_store8(make_uint2(0, 0), rq, qoff, (uint32_t)i * (uint32_t)K);
        return;
    }
    // column-major: the lane's 8 rows x 8 columns of codes become 8 columns x 8
    // rows (byte transposes), staged as 128 columns x 128 rows, stored as 128-B lines
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int qd = 0; qd < H / 4; ++qd) {
            uint32_t o4[4];
            transpose4x4_bytes(half ? out[4 * qd].y : out[4 * qd].x, half ? out[4 * qd + 1].y : out[4 * qd + 1].x,
                               half ? out[4 * qd + 2].y : out[4 * qd + 2].x, half ? out[4 * qd + 3].y : out[4 * qd + 3].x,
                               o4);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                *(uint32_t*)(sh.stage + col_tile_offset(cg * 8 + half * 4 + c, rbase + 4 * qd)) = o4[c];
        }
    }
    __syncthreads();
    const bool aligned16 = (M & 15) == 0;
    const int64_t col0 = (int64_t)s * kSW;
#pragma unroll
    for (int it = 0; it < (kSW * 8) / kST; ++it) {
        const int sid = (int)threadIdx.x + kST * it;
        const int cc = sid >> 3, seg = sid & 7;
        const int rb = seg * 16;
        if (col0 + cc >= K || rb >= nrows) continue;
        const uint4 val = *(const uint4*)(sh.stage + col_tile_offset(cc, rb));
        uint8_t* dst = q + (col0 + cc) * (int64_t)M + row0 + rb;
        if (aligned16 && rb + 16 <= nrows)
            store_nt(val, (uint4*)dst);
        else
            store_partial16(val, dst, 0, rb + 16 < nrows ? 16 : nrows - rb, aligned16);
    }
}

// With no rows at all: every group is empty and gets the scale of amax 0.
__global__ __launch_bounds__(kST)
void group_split_empty_kernel(int G, int K, float* __restrict__ scales_out, int flags)
{
    const float se = group_scale_of(0u, flags & 1);
    const float so = (flags & 2) ? 1.0f / se : se;
    const int64_t n4 = (int64_t)G * K / 4;
    for (int64_t i = (int64_t)blockIdx.x * kST + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kST)
        ((float4*)scales_out)[i] = make_float4(so, so, so, so);
}

}  // namespace

bool group_split_sizes_ok(int64_t M, int64_t K, int64_t G)
{
    const int64_t lim = ((int64_t)1 << 31) - 1;
    const int64_t nblk = (M + kSR - 1) / kSR;
    const int64_t S = (K + kSW - 1) / kSW;
    return G <= kMaxGroups && nblk * S <= lim && kSR * K * 2 <= lim;
}

size_t group_split_workspace_bytes(int64_t M, int64_t K, int32_t G)
{
    const int64_t nblk = (M + kSR - 1) / kSR;
    return ((size_t)(nblk + G) * (size_t)K * 2 + 255) / 256 * 256;
}

hipError_t launch_group_split(const void* x, int M, int K, const int32_t* offs, int G, int layout, int flags, void* q,
                              float* scales, void* workspace, hipStream_t stream)
{
    if (M == 0) {
        int grid = (int)(((int64_t)G * K / 4 + kST - 1) / kST);
        grid = grid < 1 ? 1 : grid > 1024 ? 1024 : grid;
        hipLaunchKernelGGL(group_split_empty_kernel, dim3(grid), dim3(kST), 0, stream, G, K, scales, flags);
        return hipGetLastError();
    }
    const int nblk = (M + kSR - 1) / kSR;
    const int S = (K + kSW - 1) / kSW;
    uint16_t* partial = (uint16_t*)workspace;
    const unsigned tiles = (unsigned)((int64_t)nblk * S);
    constexpr int AW = kSplitAmaxWidth;
    const int SA = (K + AW - 1) / AW;
    hipLaunchKernelGGL(group_split_amax_kernel<AW>, dim3((unsigned)((int64_t)nblk * SA)), dim3(AmaxCfg<AW>::T), 0,
                       stream, (const uint16_t*)x, M, K, offs, G, SA, partial);
    if (layout == 0)
        hipLaunchKernelGGL(group_split_quant_kernel<0>, dim3(tiles), dim3(kST), 0, stream, (const uint16_t*)x, M, K,
                           offs, G, S, (const uint16_t*)partial, scales, flags, (uint8_t*)q);
    else
        hipLaunchKernelGGL(group_split_quant_kernel<1>, dim3(tiles), dim3(kST), 0, stream, (const uint16_t*)x, M, K,
                           offs, G, S, (const uint16_t*)partial, scales, flags, (uint8_t*)q);
    return hipGetLastError();
}

}  // namespace mxq
