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
// The amax of a (group, column) must be complete before any element of it is
// cast, and a 170 MB input re-read right after it was read comes back from HBM
// at the same rate as a cold read on MI355X (the last-level cache does not turn
// the second pass into a cheap one).  So the input is read ONCE and held on chip:
//
//   plan   build the chunk table, zero the per-(group, strip) arrival counters,
//          ready flags and per-tile "deferred" marks, and write the scales of
//          empty groups.
//   hold   one workgroup per tile (a 128-row chunk of one group x 512 columns).
//          It loads its tile into registers, reduces the column maxima (packed
//          16-bit max of |bf16 bits| -- positive bf16 order is integer order and
//          Inf/NaN sort above every finite value), publishes them as one row of
//          partial maxima, and counts itself in.  The last tile of a (group,
//          strip) to arrive reduces the strip's partial rows, divides, writes
//          the (G, K) scales and raises the strip's ready flag; the others wait
//          for the flag (bounded by a wall-clock limit) and then quantize the
//          tile still in their registers: 2 bytes read + 1 byte written per
//          element, nothing else.  (Folding the maxima with atomic max instead
//          was measured slower: every tile of a strip hits the same addresses.)
//   deferred  tiles of groups too large to hold on chip at once (more tiles than
//          the device can keep resident), and tiles whose wait ran out, are
//          re-read and quantized here after the hold kernel has finished, so the
//          result never depends on how many workgroups are resident.
//
// Cross-workgroup data (partial maxima, scales, counters, flags) crosses XCDs,
// whose L2 caches are not coherent with each other.  An agent-scope fence would
// write back and invalidate the whole L2 at every publish and every wake-up,
// which costs microseconds each on MI355X; instead every such access is a
// relaxed agent-scope atomic (it goes through the caches to the coherence
// point), and ordering between them comes from waiting for the wave's memory
// operations to complete (s_waitcnt vmcnt(0)) with a workgroup-scope fence to
// keep the compiler from moving accesses across.  Ordinary cached accesses are
// used only for data that no other workgroup of the same launch reads.
//
// Row chunks never cross a group boundary and are cut at multiples of the tile
// height, so interior tiles are aligned in both output layouts.  The plan kernel
// writes one table entry per chunk (group, rows, the group's chunk range), so a
// tile learns where it is with one load.  Tiles are 128 rows x 512 columns for
// 512 threads; each lane holds 8 columns of 16 rows.  Row layout: rows 8 apart
// per lane, a wave writes 512 contiguous bytes of one row.  Column layout: 16
// consecutive rows per lane, turned into dwords of 4 consecutive rows per
// column, staged as a 512 x 128-byte transposed tile in LDS, written as 128
// contiguous bytes per output row.
#include <stdlib.h>

#include "device_common.hpp"
#include "internal.hpp"

namespace mxq {

constexpr int kGThreads = 256;      // plan kernel
constexpr int kTThreads = 512;      // hold and deferred kernels
constexpr int kHold = 16;           // rows of 8 columns held per lane

template <int LAYOUT>
struct TileCfg;
template <>
struct TileCfg<0> {                 // row-major output
    static constexpr int R = 128, W = 512;
    static constexpr int CG = W / 8;                  // 8-column groups per strip (lanes per row)
    static constexpr int NS = kTThreads / CG;         // lanes sharing the same columns
    __device__ static int row(int rs, int i) { return rs + NS * i; }
};
template <>
struct TileCfg<1> {                 // column-major output
    static constexpr int R = 128, W = 512;
    static constexpr int CG = W / 8;
    static constexpr int NS = kTThreads / CG;
    __device__ static int row(int rs, int i) { return rs * kHold + i; }
};
static_assert(TileCfg<0>::NS * kHold == TileCfg<0>::R, "row tile shape");
static_assert(TileCfg<1>::NS * kHold == TileCfg<1>::R, "col tile shape");

// ------------------------------------------------------------ workspace ---
struct ChunkEntry {
    int g, r0, r1, first;      // group (G: rows past the last end, -1: unused), rows, first chunk of the group
    int count, gr0, gr1, pad;  // chunks of the group, and the group's rows [gr0, gr1)
};

struct Workspace {
    ChunkEntry* table;    // [slots] one entry per chunk id
    uint16_t* partial;    // [slots][K] column maxima of each chunk (|bf16 bits|)
    uint32_t* count;      // [G][S] arrivals per (group, strip)
    uint32_t* ready;      // [G][S] 1 once the strip's scales are written
    uint32_t* deferred;   // [slots][S] 1 if the tile was left for the deferred kernel
    uint32_t* any;        // [1] 1 if any tile needs the deferred kernel
};

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

static int64_t chunk_slots(int64_t M, int R, int64_t G) { return (M + R - 1) / R + G + 1; }

template <int LAYOUT>
static size_t workspace_layout(int64_t M, int64_t K, int64_t G, size_t off[6])
{
    using C = TileCfg<LAYOUT>;
    const int64_t slots = chunk_slots(M, C::R, G);
    const int64_t S = (K + C::W - 1) / C::W;
    size_t o = 0;
    off[0] = o; o += align256((size_t)(slots * sizeof(ChunkEntry)));
    off[1] = o; o += align256((size_t)(slots * K * 2));
    off[2] = o; o += align256((size_t)(G * S * 4));
    off[3] = o; o += align256((size_t)(G * S * 4));
    off[4] = o; o += align256((size_t)(slots * S * 4));
    off[5] = o; o += 256;
    return o;
}

bool group_scale_sizes_ok(int64_t M, int64_t K, int64_t G)
{
    // every tile id and every (group, strip) index must fit the int arithmetic of the kernels
    const int64_t lim = ((int64_t)1 << 31) - 1;
    const int64_t tiles_row = chunk_slots(M, TileCfg<0>::R, G) * ((K + TileCfg<0>::W - 1) / TileCfg<0>::W);
    const int64_t tiles_col = chunk_slots(M, TileCfg<1>::R, G) * ((K + TileCfg<1>::W - 1) / TileCfg<1>::W);
    return tiles_row <= lim && tiles_col <= lim && (int64_t)M * K / 8 <= lim * 64;
}

size_t group_scale_workspace_bytes(int64_t M, int64_t K, int32_t G)
{
    size_t off[6];
    const size_t a = workspace_layout<0>(M, K, G, off);
    const size_t b = workspace_layout<1>(M, K, G, off);
    return a > b ? a : b;
}

// ------------------------------------------------------------- helpers ----
__device__ __forceinline__ float group_scale_of(uint32_t amax_bits)
{
    if (amax_bits >= 0x7F80u) return __uint_as_float(0x7FC00000u);   // Inf/NaN in the column
    const float amax = __uint_as_float(amax_bits << 16);
    return 448.0f / fmaxf(amax, 1e-12f);                            // correctly rounded divide
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

// Everything a tile needs to know about itself.
struct TileInfo {
    int g, r0, r1;        // group (G = rows past the last end) and its rows [r0, r1)
    int a;                // aligned first row of the tile (r0 rounded down to R)
    int first, count;     // the group's chunks: ids [first, first + count)
    int gr0, gr1;         // the group's rows
    int j, s;             // chunk id and strip
};

template <int R>
__device__ __forceinline__ TileInfo tile_info(const ChunkEntry* __restrict__ table, int j, int s)
{
    const int4 e0 = *(const int4*)(table + j);
    const int4 e1 = *((const int4*)(table + j) + 1);
    TileInfo t;
    t.g = e0.x;
    t.r0 = e0.y;
    t.r1 = e0.z;
    t.first = e0.w;
    t.count = e1.x;
    t.gr0 = e1.y;
    t.gr1 = e1.z;
    t.a = (t.r0 / R) * R;
    t.j = j;
    t.s = s;
    return t;
}

// ---------------------------------------------------- coherent accesses ---
// Relaxed agent-scope atomics: each access reaches the coherence point shared by
// all XCDs.  Ordering between them: order_release() before the access that
// signals, order_acquire() after the access that observed the signal.
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

// vmcnt(0), expcnt and lgkmcnt left at their maxima: wait for this wave's
// outstanding vector memory operations only.
constexpr int kWaitVmem = 0 | (0x7 << 4) | (0xF << 8);

__device__ __forceinline__ void order_release()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(kWaitVmem);
}

__device__ __forceinline__ void order_acquire()
{
    __builtin_amdgcn_s_waitcnt(kWaitVmem);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Load this lane's 16 rows x 8 columns of the tile (zeros outside rows/columns).
template <int LAYOUT>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ x, int K, const TileInfo& t, int k, int rs,
                                          uint4 v[kHold])
{
    using C = TileCfg<LAYOUT>;
    const bool kin = k < K;
#pragma unroll
    for (int i = 0; i < kHold; ++i) {
        const int row = t.a + C::row(rs, i);
        v[i] = (kin && row >= t.r0 && row < t.r1) ? *(const uint4*)(x + (int64_t)row * K + k)
                                                  : make_uint4(0, 0, 0, 0);
    }
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

// Quantize the held rows and store them in the output layout.  `stage` is the
// LDS staging tile (column layout only).
template <int LAYOUT>
__device__ __forceinline__ void quantize_store_tile(const uint4 v[kHold], const ColScales& cs, const TileInfo& t,
                                                    int M, int K, int k, int cg, int rs, uint8_t* __restrict__ q,
                                                    uint8_t* stage, bool zero)
{
    using C = TileCfg<LAYOUT>;
    if (LAYOUT == 0) {
        if (k >= K) return;
#pragma unroll
        for (int i = 0; i < kHold; ++i) {
            const int row = t.a + C::row(rs, i);
            if (row >= t.r0 && row < t.r1) {
                const uint2 out = zero ? make_uint2(0, 0) : group_quantize_chunk(v[i], cs);
                *(uint2*)(q + (int64_t)row * K + k) = out;
            }
        }
    } else {
        // Pair the same column of consecutive rows in each conversion, so that
        // every dword already holds 4 consecutive rows of one column: the lane's
        // 16 rows of a column are one 16-byte unit of the transposed tile.
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float sc = cs.s[c];
            const bool col_nan = (c < 4 ? (cs.nan_lo >> (8 * c)) : (cs.nan_hi >> (8 * (c - 4)))) & 1u;
            uint32_t d[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                float f[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 w = v[4 * b + i];
                    const uint32_t word = c < 2 ? w.x : c < 4 ? w.y : c < 6 ? w.z : w.w;
                    const float xv = (c & 1) ? bf16_hi_to_f32(word) : bf16_lo_to_f32(word);
                    f[i] = __builtin_amdgcn_fmed3f(xv * sc, -448.0f, 448.0f);
                }
                int pk = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
                pk = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], pk, true);
                d[b] = (zero ? 0u : col_nan ? 0x7F7F7F7Fu : (uint32_t)pk);
            }
            *(uint4*)(stage + col_tile_offset(cg * 8 + c, rs * kHold)) = make_uint4(d[0], d[1], d[2], d[3]);
        }
        __syncthreads();
        // column cc of the tile becomes output row (strip * W + cc): rows [lo, hi) of the tile
        const int lo = t.r0 - t.a, hi = t.r1 - t.a;
        const bool aligned16 = (M & 15) == 0;
        const int64_t col0 = (int64_t)t.s * C::W;
        for (int it = 0; it < (C::W * 8) / kTThreads; ++it) {
            const int sid = (int)threadIdx.x + kTThreads * it;
            const int cc = sid >> 3, seg = sid & 7;
            if (col0 + cc >= K) continue;
            const int rb = seg * 16;
            const int a = rb > lo ? rb : lo;
            const int e = rb + 16 < hi ? rb + 16 : hi;
            if (a >= e) continue;
            const uint4 val = *(const uint4*)(stage + col_tile_offset(cc, rb));
            uint8_t* dst = q + (col0 + cc) * (int64_t)M + t.a + rb;
            if (aligned16 && a == rb && e == rb + 16) {
                *(uint4*)dst = val;
            } else {
                store_partial16(val, dst, a - rb, e - rb, aligned16);
            }
        }
    }
}

// ---------------------------------------------------------------- plan ----
// Every block clears counters, ready flags and deferred marks; block 0 also
// writes the chunk table (and marks unused slots) and the scales of empty groups.
template <int R>
__global__ __launch_bounds__(kGThreads)
void group_plan_kernel(const int32_t* __restrict__ offs, int G, int M, int K, Workspace ws, int nGS, int nTiles,
                       int slots, float* __restrict__ scales)
{
    const int tid = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    const int stride = (int)(gridDim.x * blockDim.x);
    for (int i = tid; i < nGS; i += stride) {
        ws.count[i] = 0;
        ws.ready[i] = 0;
    }
    for (int i = tid; i < nTiles; i += stride) ws.deferred[i] = 0;
    if (tid == 0) *ws.any = 0;
    if (blockIdx.x != 0) return;

    __shared__ int sh_st[kWave], sh_en[kWave], sh_first[kWave], sh_cnt[kWave];
    __shared__ int sh_base_chunk, sh_end_chunk;
    __shared__ unsigned long long sh_empty;
    const float s_empty = group_scale_of(0u);
    int carry_end = 0, carry_cnt = 0;      // meaningful in wave 0 only
    for (int base = 0; base < G + 1; base += kWave) {   // groups 0..G-1, then the rows past the last end
        if (threadIdx.x < kWave) {
            const int lane = (int)threadIdx.x;
            const int g = base + lane;
            int e = g < G ? offs[g] : M;
            e = e > 0 ? e : 0;
            e = wave_incl_max(e);
            e = e > carry_end ? e : carry_end;
            e = e < M ? e : M;
            int st = __shfl_up(e, 1, kWave);
            if (lane == 0) st = carry_end;
            const int cnt = (g <= G && e > st) ? ((e + R - 1) / R - st / R) : 0;
            const int incl = wave_incl_sum(cnt) + carry_cnt;
            sh_st[lane] = st;
            sh_en[lane] = e;
            sh_first[lane] = incl - cnt;
            sh_cnt[lane] = cnt;
            const unsigned long long m = __ballot(g < G && e <= st);
            if (lane == 0) {
                sh_empty = m;
                sh_base_chunk = carry_cnt;
            }
            carry_end = readlane(e, kWave - 1);
            carry_cnt = readlane(incl, kWave - 1);
            if (lane == 0) sh_end_chunk = carry_cnt;
        }
        __syncthreads();
        // table entries of this batch's chunks: the owning lane is the last one
        // whose first chunk is at or before c (binary search over non-decreasing firsts)
        for (int c = sh_base_chunk + (int)threadIdx.x; c < sh_end_chunk; c += kGThreads) {
            int l = 0;
#pragma unroll
            for (int step = kWave / 2; step > 0; step >>= 1)
                if (sh_first[l + step] <= c) l += step;
            const int i = c - sh_first[l];
            const int a = (sh_st[l] / R) * R;
            ChunkEntry e;
            e.g = base + l;
            e.r0 = sh_st[l] > a + i * R ? sh_st[l] : a + i * R;
            e.r1 = sh_en[l] < a + (i + 1) * R ? sh_en[l] : a + (i + 1) * R;
            e.first = sh_first[l];
            e.count = sh_cnt[l];
            e.gr0 = sh_st[l];
            e.gr1 = sh_en[l];
            e.pad = 0;
            ws.table[c] = e;
        }
        // scales of this batch's empty groups
        for (unsigned long long mm = sh_empty; mm; mm &= mm - 1) {
            const int g = base + __builtin_ctzll(mm);
            for (int k = (int)threadIdx.x * 4; k < K; k += kGThreads * 4)
                *(float4*)(scales + (int64_t)g * K + k) = make_float4(s_empty, s_empty, s_empty, s_empty);
        }
        __syncthreads();
    }
    for (int c = sh_end_chunk + (int)threadIdx.x; c < slots; c += kGThreads) {
        ChunkEntry e;
        e.g = -1;
        e.r0 = e.r1 = e.first = e.count = 0;
        e.gr0 = e.gr1 = e.pad = 0;
        ws.table[c] = e;
    }
}

__device__ __forceinline__ float4 scales_lo(uint4 a)
{
    return make_float4(group_scale_of(a.x & 0xFFFFu), group_scale_of(a.x >> 16),
                       group_scale_of(a.y & 0xFFFFu), group_scale_of(a.y >> 16));
}
__device__ __forceinline__ float4 scales_hi(uint4 a)
{
    return make_float4(group_scale_of(a.z & 0xFFFFu), group_scale_of(a.z >> 16),
                       group_scale_of(a.w & 0xFFFFu), group_scale_of(a.w >> 16));
}
__device__ __forceinline__ uint4 f4_bits(float4 f)
{
    return make_uint4(__float_as_uint(f.x), __float_as_uint(f.y), __float_as_uint(f.z), __float_as_uint(f.w));
}
__device__ __forceinline__ float4 bits_f4(uint4 u)
{
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}

// ---------------------------------------------------------------- hold ----
template <int LAYOUT>
__global__ __launch_bounds__(kTThreads)
void group_hold_kernel(const uint16_t* __restrict__ x, int M, int K, int G, int S, int SB, int slots, Workspace ws,
                       float* __restrict__ scales, uint8_t* __restrict__ q, int hold_limit,
                       unsigned long long timeout_ticks, int deferred_launched)
{
    using C = TileCfg<LAYOUT>;
    __shared__ __align__(16) uint8_t stage[LAYOUT == 1 ? C::W * C::R : 16];
    __shared__ uint4 red[C::NS][C::CG];
    __shared__ __align__(16) float sh_scale[C::W];
    __shared__ int sh_state;

    // Launch order: blocks of SB strips, chunks within a block, strips within that.
    const int per_block = slots * SB;
    const int sb = (int)blockIdx.x / per_block, rem = (int)blockIdx.x % per_block;
    const int j = rem / SB, s = sb * SB + rem % SB;
    const TileInfo t = tile_info<C::R>(ws.table, j, s);
    if (t.g < 0) return;                                  // unused chunk id (uniform)
    const int cg = (int)threadIdx.x % C::CG, rs = (int)threadIdx.x / C::CG;
    const int k = s * C::W + cg * 8;
    ColScales cs;
    uint4 v[kHold];

    if (t.g == G) {                                       // rows past the last end: zeros
        quantize_store_tile<LAYOUT>(v, cs, t, M, K, k, cg, rs, q, stage, true);
        return;
    }
    // A (group, strip) is one synchronisation domain and its tiles are launched
    // consecutively, so `count` tiles must be resident together.
    const bool streamed = t.count > hold_limit;
    load_tile<LAYOUT>(x, K, t, k, rs, v);

    // Column maxima of this tile, published as one row of the partials by the
    // lanes with rs == 0 -- all in wave 0, like the lane that then counts the
    // tile in, so one wave-wide wait orders the publish before the count.
    uint4 m = abs8(v[0]);
#pragma unroll
    for (int i = 1; i < kHold; ++i) max8(m, abs8(v[i]));
    red[rs][cg] = m;
    __syncthreads();
    if (rs == 0) {
#pragma unroll
        for (int r = 1; r < C::NS; ++r) max8(m, red[r][cg]);
        if (k < K) store_coherent(m, ws.partial + (int64_t)j * K + k);
        order_release();
    }
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(ws.count + (int64_t)t.g * S + s, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (streamed) __hip_atomic_store(ws.any, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        order_acquire();
        sh_state = (old + 1 == (uint32_t)t.count) ? 1 : 0;   // 1: last to arrive
    }
    __syncthreads();

    if (sh_state == 1) {
        // last arrival: reduce the strip's partial rows over the group's chunks, divide
        uint4 a = make_uint4(0, 0, 0, 0);
        if (k < K) {
            const uint16_t* p = ws.partial + (int64_t)t.first * K + k;
            int c = rs;
            for (; c + 3 * C::NS < t.count; c += 4 * C::NS) {
                uint4 b[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) b[u] = load_coherent(p + (int64_t)(c + u * C::NS) * K);
#pragma unroll
                for (int u = 0; u < 4; ++u) max8(a, b[u]);
            }
            for (; c < t.count; c += C::NS) max8(a, load_coherent(p + (int64_t)c * K));
        }
        red[rs][cg] = a;
        __syncthreads();
        if (rs == 0) {
#pragma unroll
            for (int r = 1; r < C::NS; ++r) max8(a, red[r][cg]);
            const float4 lo = scales_lo(a), hi = scales_hi(a);
            *(float4*)(sh_scale + cg * 8) = lo;
            *(float4*)(sh_scale + cg * 8 + 4) = hi;
            if (k < K) {
                store_coherent(f4_bits(lo), scales + (int64_t)t.g * K + k);
                store_coherent(f4_bits(hi), scales + (int64_t)t.g * K + k + 4);
            }
            order_release();                              // scales complete before the flag
        }
        if (threadIdx.x == 0)      // same wave as the scale stores above
            __hip_atomic_store(ws.ready + (int64_t)t.g * S + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (streamed) return;                             // the deferred kernel writes this group
        cs = make_col_scales(*(const float4*)(sh_scale + cg * 8), *(const float4*)(sh_scale + cg * 8 + 4));
    } else {
        if (streamed) return;
        // wait for the strip's scales, bounded in wall-clock time
        if (threadIdx.x == 0) {
            const uint32_t* rdy = ws.ready + (int64_t)t.g * S + s;
            const unsigned long long t0 = wall_clock64();
            int ok = 0;
            while (true) {
                if (__hip_atomic_load(rdy, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                    ok = 1;
                    break;
                }
                if (wall_clock64() - t0 > timeout_ticks) break;
                __builtin_amdgcn_s_sleep(2);
            }
            if (!ok && deferred_launched) {
                __hip_atomic_store(ws.deferred + (int64_t)j * S + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(ws.any, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            order_acquire();
            sh_state = ok ? 2 : deferred_launched ? 3 : 4;
        }
        __syncthreads();
        if (sh_state == 3) return;                        // left for the deferred kernel
        if (sh_state == 4) {
            // The wait ran out and no deferred pass follows: reduce this strip's
            // maxima over all of the group's rows straight from the input (slow,
            // only when the device cannot keep the group's tiles resident).
            uint4 a = make_uint4(0, 0, 0, 0);
            if (k < K)
                for (int r = t.gr0 + rs; r < t.gr1; r += C::NS) max8(a, abs8(*(const uint4*)(x + (int64_t)r * K + k)));
            red[rs][cg] = a;
            __syncthreads();
            if (rs == 0) {
#pragma unroll
                for (int r = 1; r < C::NS; ++r) max8(a, red[r][cg]);
                *(float4*)(sh_scale + cg * 8) = scales_lo(a);
                *(float4*)(sh_scale + cg * 8 + 4) = scales_hi(a);
            }
            __syncthreads();
            cs = make_col_scales(*(const float4*)(sh_scale + cg * 8), *(const float4*)(sh_scale + cg * 8 + 4));
        } else if (k < K) {
            cs = make_col_scales(bits_f4(load_coherent(scales + (int64_t)t.g * K + k)),
                                 bits_f4(load_coherent(scales + (int64_t)t.g * K + k + 4)));
        }
    }
    quantize_store_tile<LAYOUT>(v, cs, t, M, K, k, cg, rs, q, stage, false);
}

// ------------------------------------------------------------ deferred ----
// A small grid walks all tiles; it returns at once when nothing was left over.
// The scales of every group are final (written by the hold kernel's last
// arrivals), so deferred tiles only re-read and quantize.
template <int LAYOUT>
__global__ __launch_bounds__(kTThreads)
void group_deferred_kernel(const uint16_t* __restrict__ x, int M, int K, int G, int S, Workspace ws,
                           const float* __restrict__ scales, uint8_t* __restrict__ q, int hold_limit, int nTiles)
{
    using C = TileCfg<LAYOUT>;
    __shared__ __align__(16) uint8_t stage[LAYOUT == 1 ? C::W * C::R : 16];
    if (*ws.any == 0u) return;                            // nothing was deferred (uniform)
    for (int tile = (int)blockIdx.x; tile < nTiles; tile += (int)gridDim.x) {
        const int j = tile / S, s = tile % S;
        const TileInfo t = tile_info<C::R>(ws.table, j, s);
        if (t.g < 0 || t.g == G) continue;
        const bool streamed = t.count > hold_limit;
        if (!streamed && ws.deferred[(int64_t)j * S + s] == 0u) continue;
        const int cg = (int)threadIdx.x % C::CG, rs = (int)threadIdx.x / C::CG;
        const int k = s * C::W + cg * 8;
        uint4 v[kHold];
        load_tile<LAYOUT>(x, K, t, k, rs, v);
        ColScales cs;
        if (k < K)
            cs = make_col_scales(*(const float4*)(scales + (int64_t)t.g * K + k),
                                 *(const float4*)(scales + (int64_t)t.g * K + k + 4));
        quantize_store_tile<LAYOUT>(v, cs, t, M, K, k, cg, rs, q, stage, false);
        __syncthreads();                                  // the staging tile is reused by the next tile
    }
}

// --------------------------------------------------------------- launch ---
template <int LAYOUT>
static hipError_t launch_layout(const void* x, int M, int K, const int32_t* offs, int G, void* q, float* scales,
                                void* workspace, hipStream_t stream)
{
    using C = TileCfg<LAYOUT>;
    size_t off[6];
    workspace_layout<LAYOUT>(M, K, G, off);
    uint8_t* base = (uint8_t*)workspace;
    Workspace ws;
    ws.table = (ChunkEntry*)(base + off[0]);
    ws.partial = (uint16_t*)(base + off[1]);
    ws.count = (uint32_t*)(base + off[2]);
    ws.ready = (uint32_t*)(base + off[3]);
    ws.deferred = (uint32_t*)(base + off[4]);
    ws.any = (uint32_t*)(base + off[5]);
    const int S = (K + C::W - 1) / C::W;
    const int64_t slots = chunk_slots(M, C::R, G);
    const int nGS = G * S;
    const int64_t nTiles = slots * S;

    // How many tiles of one group may be held at once: the resident capacity of
    // the hold kernel on this device, less a small margin.  Holding more than
    // fits is still correct (waits time out and the tiles are deferred), only slower.
    int dev = 0, cus = 0, per_cu = 0, rate_khz = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, group_hold_kernel<LAYOUT>, kTThreads, 0);
    if (e != hipSuccess) return e;
    // Knobs (read per call): MXQ_GROUP_HOLD_TILES overrides the hold limit (0 sends every
    // group through the deferred kernel); MXQ_GROUP_WAIT_US bounds each wait (default
    // 2000 us; 0 makes every waiting tile defer).  Results are identical either way.
    int hold_limit = cus * per_cu - 16;
    long wait_us = 2000;
    int SB = 1;                                           // chunk-fastest launch order (measured best)
    if (const char* v = getenv("MXQ_GROUP_STRIP_BLOCK")) SB = atoi(v);
    if (SB < 1 || S % SB != 0) SB = S;
    if (const char* v = getenv("MXQ_GROUP_HOLD_TILES")) hold_limit = atoi(v);
    if (const char* v = getenv("MXQ_GROUP_WAIT_US")) wait_us = atol(v);
    if (wait_us < 0) wait_us = 0;
    const unsigned long long timeout_ticks =
        (unsigned long long)(rate_khz > 0 ? rate_khz : 100000) * (unsigned long long)wait_us / 1000ull;

    hipLaunchKernelGGL(group_plan_kernel<C::R>, dim3(64), dim3(kGThreads), 0, stream, offs, G, M, K, ws, nGS,
                       (int)nTiles, (int)slots, scales);
    if (M > 0) {
        // No group spans more than ceil(M/R) + 1 chunks: unless that exceeds the
        // hold limit nothing is streamed, and tiles whose wait runs out finish
        // themselves, so the deferred pass is not launched at all.
        const int deferred = (int64_t)(M + C::R - 1) / C::R + 1 > hold_limit ? 1 : 0;
        hipLaunchKernelGGL(group_hold_kernel<LAYOUT>, dim3((unsigned)nTiles), dim3(kTThreads), 0, stream,
                           (const uint16_t*)x, M, K, G, S, SB, (int)slots, ws, scales, (uint8_t*)q, hold_limit,
                           timeout_ticks, deferred);
        if (!deferred) return hipGetLastError();
        const int dgrid = (int)(nTiles < 512 ? nTiles : 512);
        hipLaunchKernelGGL(group_deferred_kernel<LAYOUT>, dim3((unsigned)dgrid), dim3(kTThreads), 0, stream,
                           (const uint16_t*)x, M, K, G, S, ws, (const float*)scales, (uint8_t*)q, hold_limit,
                           (int)nTiles);
    }
    return hipGetLastError();
}

hipError_t launch_group_scale(const void* x, int M, int K, const int32_t* offs, int G, int layout,
                              void* q, float* scales, void* workspace, hipStream_t stream)
{
    return layout == 0 ? launch_layout<0>(x, M, K, offs, G, q, scales, workspace, stream)
                       : launch_layout<1>(x, M, K, offs, G, q, scales, workspace, stream);
}

}  // namespace mxq
