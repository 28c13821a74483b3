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
// the second pass into a cheap one).  So the hold method reads the input ONCE
// and holds it on chip (the default for row-major output, and for column-major
// output with few groups; with more groups column-major output streams through
// the two-pass method further down, whose kernels never wait):
//
//   plan   build the chunk table and empty-group flags, zero the per-(group,
//          strip) arrival counters and per-tile "deferred" marks, and fill the
//          partial maxima and the scales with values no result takes ("not yet
//          written").
//   hold   one workgroup per tile (a 128-row chunk of one group x 256 columns).
//          It loads its tile into registers, reduces the column maxima (packed
//          16-bit max of |bf16 bits| -- positive bf16 order is integer order and
//          Inf/NaN sort above every finite value) and publishes them as one row
//          of partial maxima.  The group's last chunk, launched after all the
//          others, reduces the strip's partial rows, divides and writes the
//          (G, K) scales; the others poll their scales until written (bounded
//          by a wall-clock limit) and then quantize the tile still in their
//          registers: 2 bytes read + 1 byte written per element, nothing else.
//          (Folding the maxima with atomic max instead was measured slower:
//          every tile of a strip hits the same addresses.)  If a wait runs out
//          (the device, perhaps shared with other work, did not keep the
//          group's tiles resident together), the tiles whose wait ran out
//          compute the missing chunks' maxima from the input between them and
//          the first of them publishes the scales.
//   deferred  tiles of groups too large to hold on chip at once (more tiles than
//          the device can keep resident) are counted in per (group, strip),
//          reduced by the last arrival, and re-read and quantized here after the
//          hold kernel has finished (with this pass launched, tiles whose wait
//          ran out also leave themselves to it), so the result never depends on
//          how many workgroups are resident.
//
// The two-pass method's kernels (amax, finalize, quantize) are here too; the
// split method is in group_split.hip.
//
// Cross-workgroup data (partial maxima, scales, counters) crosses XCDs, whose
// L2 caches are not coherent with each other.  An agent-scope fence would write
// back and invalidate the whole L2 at every publish and every wake-up, which
// costs microseconds each on MI355X; instead every such access is a relaxed
// agent-scope atomic (it goes through the caches to the coherence point), and
// since each partial row and each scale is polled until it holds a written
// value, no ordering between different addresses is needed at all (no fence,
// no flag, no wait for a store to complete).  Ordinary cached accesses are used
// only for data that no other workgroup of the same launch writes.
//
// Row chunks never cross a group boundary and are cut at multiples of the tile
// height, so interior tiles are aligned in both output layouts.  The plan kernel
// writes one table entry per chunk (group, rows, the group's chunk range), so a
// tile learns where it is with one load.  Tiles are 128 rows x 256 columns for
// 256 threads; each lane holds 8 columns of 16 rows.  (128 x 512 tiles for 512
// threads took 67 / 69 / 71 / 78 us at 16 / 32 / 64 / 128 groups, row-major,
// 16640 x 5120, against 65 / 66 / 68 / 73 us; 128 x 128 tiles for 128 threads
// matched the 256-column ones; column-major at 16 groups 78 against 74 us.)
// Row layout: rows 8 apart per lane, a wave writes 256 contiguous bytes of each
// of two rows.  Column layout: 16 consecutive rows per lane, turned into dwords
// of 4 consecutive rows per column, staged as a 256 x 128-byte transposed tile
// in LDS, written as 128 contiguous bytes per output row.
#include <atomic>
#include <mutex>

#include "group_common.hpp"
#include "internal.hpp"

namespace mxq {

constexpr int kGThreads = 256;      // plan kernel
template <int LAYOUT>
struct TileCfg;
template <>
struct TileCfg<0> {                 // row-major output
    static constexpr int T = 256, H = 16, W = 256;
    static constexpr int CG = W / 8;                  // 8-column groups per strip (lanes per row)
    static constexpr int NS = T / CG;                 // lanes sharing the same columns
    static constexpr int R = NS * H;
    __device__ static int row(int rs, int i) { return rs + NS * i; }
};
template <>
struct TileCfg<1> {                 // column-major output
    static constexpr int T = 256, H = 16, W = 256;
    static constexpr int CG = W / 8;
    static constexpr int NS = T / CG;
    static constexpr int R = NS * H;
    __device__ static int row(int rs, int i) { return rs * H + i; }
};
static_assert(TileCfg<1>::R == 128, "col tile shape");
static_assert(TileCfg<0>::R == 128, "row tile shape");

// Values that no finished result takes: a scale is a positive float or the
// canonical NaN 0x7FC00000, a column maximum of |bf16| bits is at most 0x7FFF.
// The plan kernel fills the partial maxima and the scales with them, and a
// reader polls the datum itself until it is written, so no flag and no
// ordering between different addresses is needed.
constexpr uint32_t kScaleUnset = 0xFFFFFFFFu;
constexpr uint16_t kPartialUnset = 0xFFFFu;

// ------------------------------------------------------------ workspace ---
struct ChunkEntry {
    int g, r0, r1, first;      // group (G: rows past the last end, -1: unused), rows, first chunk of the group
    int count, gr0, gr1, pad;  // chunks of the group, and the group's rows [gr0, gr1)
};

struct Workspace {
    ChunkEntry* table;    // [slots] one entry per chunk id
    uint16_t* partial;    // [slots][K] column maxima of each chunk (|bf16 bits|)
    uint32_t* count;      // [G][S] arrivals per (group, strip)
    uint32_t* empty;      // [G] 1 if the group has no rows
    int32_t* gend;        // [G] end row of each group (offsets clamped as documented)
    int32_t* gchunks;     // [G][2] first chunk id and chunk count of each group
    int32_t* bfirst;      // [ceil(M/128)] group containing the first row of each 128-row block (G: none)
    uint32_t* deferred;   // [slots][S] 1 if the tile was left for the deferred kernel
    uint32_t* any;        // [1] 1 if any tile needs the deferred kernel
    uint32_t* stats;      // [2] route counters: tiles whose wait for their scales ran out;
                          // tile-sized pieces (128 rows x one strip) read again from the input
    float* inv_out;       // the caller's (G, K) scales when they hold 1/s (the kernels then keep the
                          // multipliers s in a workspace array); NULL when they hold s itself
    int pow2;             // 1: multipliers rounded down to a power of two
};

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

static int64_t chunk_slots(int64_t M, int R, int64_t G) { return (M + R - 1) / R + G + 1; }

template <int LAYOUT>
static size_t workspace_layout(int64_t M, int64_t K, int64_t G, size_t off[10])
{
    using C = TileCfg<LAYOUT>;
    const int64_t slots = chunk_slots(M, C::R, G);
    const int64_t S = (K + C::W - 1) / C::W;
    size_t o = 0;
    off[0] = o; o += align256((size_t)(slots * sizeof(ChunkEntry)));
    off[1] = o; o += align256((size_t)(slots * K * 2));
    off[2] = o; o += align256((size_t)(G * S * 4));
    off[3] = o; o += align256((size_t)(G * 4));
    off[4] = o; o += align256((size_t)(slots * S * 4));
    off[5] = o; o += 256;
    off[6] = o; o += align256((size_t)(G * 4));
    off[7] = o; o += align256((size_t)(((M + 127) / 128 + 1) * 4));
    off[8] = o; o += align256((size_t)(G * 8));
    off[9] = o; o += align256((size_t)(G * K * 4));       // multipliers when the caller asked for 1/s
    return o;
}

bool group_scale_sizes_ok(int64_t M, int64_t K, int64_t G)
{
    // every tile id and every (group, strip) index must fit the int arithmetic of the kernels
    const int64_t lim = ((int64_t)1 << 31) - 1;
    const int64_t tiles_row = chunk_slots(M, TileCfg<0>::R, G) * ((K + TileCfg<0>::W - 1) / TileCfg<0>::W);
    const int64_t tiles_col = chunk_slots(M, TileCfg<1>::R, G) * ((K + TileCfg<1>::W - 1) / TileCfg<1>::W);
    // (and the plan kernel's fills, counted in 16-byte units)
    const int64_t fill_partial = chunk_slots(M, TileCfg<0>::R, G) * K / 8;
    return tiles_row <= lim && tiles_col <= lim && fill_partial <= lim && G * K / 4 <= lim &&
           (int64_t)M * K / 8 <= lim * 64;
}

size_t group_scale_workspace_bytes(int64_t M, int64_t K, int32_t G)
{
    size_t off[10];
    const size_t a = workspace_layout<0>(M, K, G, off);
    const size_t b = workspace_layout<1>(M, K, G, off);
    const size_t c = group_split_sizes_ok(M, K, G) ? group_split_workspace_bytes(M, K, G) : 0;
    const size_t ab = a > b ? a : b;
    return ab > c ? ab : c;
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

// First index i of this lane's rows (C::row(rs, i), increasing in i) at or past
// tile row `lo`; C::H when the lane's columns are past K.
template <int LAYOUT>
__device__ __forceinline__ int first_held_row(int lo, int rs, bool col_ok)
{
    using C = TileCfg<LAYOUT>;
    int i0 = 0;
    if (LAYOUT == 0)
        i0 = lo > rs ? (lo - rs + C::NS - 1) / C::NS : 0;
    else
        i0 = lo > rs * C::H ? lo - rs * C::H : 0;
    return col_ok ? i0 : C::H;
}

// Load this lane's H rows x 8 columns of the tile (zeros outside rows/columns),
// with the cache policy POLICY.
template <int LAYOUT, int POLICY = kNonTemporal>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ x, int K, const TileInfo& t, int k, int rs,
                                          uint4 (&v)[TileCfg<LAYOUT>::H])
{
    using C = TileCfg<LAYOUT>;
    // Raw buffer loads, one resource per 128 rows of the tile (at most 2^31
    // bytes each) clipped to rows [a, r1): rows past r1 fall outside the
    // resource and rows before r0 or columns past K get an offset outside it,
    // and such loads read zero with no memory traffic.  Masking by offset
    // instead of by branch lets all H loads be in flight at once.
    constexpr int NR = C::R > 128 ? C::R / 128 : 1;      // 128-row resources
    constexpr int PER = C::H / NR;                        // lane rows per resource
    const int i0 = first_held_row<LAYOUT>(t.r0 - t.a, rs, k < K);
    const uint32_t base = ((uint32_t)(C::row(rs, 0)) * (uint32_t)K + (uint32_t)k) * 2u;
    const uint32_t step = (uint32_t)(C::row(0, 1) - C::row(0, 0)) * (uint32_t)K * 2u;
#pragma unroll
    for (int h = 0; h < NR; ++h) {
        const int hi = t.r1 - t.a - 128 * h;
        const uint32_t rows = hi <= 0 ? 0u : hi >= 128 ? 128u : (uint32_t)hi;
        const Rsrc r = make_rsrc(x + (int64_t)(t.a + 128 * h) * K, rows * (uint32_t)K * 2u);
#pragma unroll
        for (int i = h * PER; i < (h + 1) * PER; ++i)
            v[i] = buf_load16<POLICY>(r, i >= i0 ? base + (uint32_t)(i - h * PER) * step : kOOB);
    }
}

// Quantize the held rows and store them in the output layout.  `stage` is the
// LDS staging tile (column layout only).
template <int LAYOUT>
__device__ __forceinline__ void quantize_store_tile(const uint4 (&v)[TileCfg<LAYOUT>::H], const ColScales& cs, const TileInfo& t,
                                                    int M, int K, int k, int cg, int rs, uint8_t* __restrict__ q,
                                                    uint8_t* stage, bool zero)
{
    using C = TileCfg<LAYOUT>;
    if (LAYOUT == 0) {
        // buffer stores over rows [a, r1) (at most 256 x 2^23 bytes): a row before
        // r0 or a column past K gets an offset outside the resource and is dropped
        const Rsrc r = make_rsrc(q + (int64_t)t.a * K, (uint32_t)(t.r1 - t.a) * (uint32_t)K);
        const int i0 = first_held_row<LAYOUT>(t.r0 - t.a, opaque(rs), k < K);
        const uint32_t base = (uint32_t)opaque(rs) * (uint32_t)K + (uint32_t)k;
#pragma unroll
        for (int i = 0; i < C::H; ++i) {
            const uint32_t off = i >= i0 ? base + (uint32_t)(i * C::NS) * (uint32_t)K : kOOB;
            buf_store8(zero ? make_uint2(0, 0) : group_quantize_chunk(v[i], cs), r, off);
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
            *(uint4*)(stage + col_tile_offset(cg * 8 + c, rs * C::H)) = make_uint4(d[0], d[1], d[2], d[3]);
        }
        __syncthreads();
        // column cc of the tile becomes output row (strip * W + cc): rows [lo, hi) of the tile
        const int lo = t.r0 - t.a, hi = t.r1 - t.a;
        const bool aligned16 = (M & 15) == 0;
        const int64_t col0 = (int64_t)t.s * C::W;
        for (int it = 0; it < (C::W * 8) / C::T; ++it) {
            const int sid = (int)threadIdx.x + C::T * it;
            const int cc = sid >> 3, seg = sid & 7;
            if (col0 + cc >= K) continue;
            const int rb = seg * 16;
            const int a = rb > lo ? rb : lo;
            const int e = rb + 16 < hi ? rb + 16 : hi;
            if (a >= e) continue;
            const uint4 val = *(const uint4*)(stage + col_tile_offset(cc, rb));
            uint8_t* dst = q + (col0 + cc) * (int64_t)M + t.a + rb;
            if (aligned16 && a == rb && e == rb + 16) {
                store_nt(val, (uint4*)dst);
            } else {
                store_partial16(val, dst, a - rb, e - rb, aligned16);
            }
        }
    }
}

// ---------------------------------------------------------------- plan ----
// Every block clears counters and deferred marks and fills the partial maxima
// (and, when there are rows, the scales) with their "not yet written" values;
// block 0 writes the chunk table (marking unused slots) and the empty-group
// flags, and when there are no rows at all it writes every group's scales
// (otherwise the hold kernel writes the scales of empty groups).
template <int R>
__global__ __launch_bounds__(kGThreads)
void group_plan_kernel(const int32_t* __restrict__ offs, int G, int M, int K, Workspace ws, int nGS, int nTiles,
                       int slots, float* __restrict__ scales, int nPartial16, int nScale16)
{
    const int tid = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    const int stride = (int)(gridDim.x * blockDim.x);
    const uint32_t pu = (uint32_t)kPartialUnset * 0x10001u;
    const uint4 p_unset = make_uint4(pu, pu, pu, pu);
    const uint4 s_unset = make_uint4(kScaleUnset, kScaleUnset, kScaleUnset, kScaleUnset);
    for (int i = tid; i < nPartial16; i += stride) ((uint4*)ws.partial)[i] = p_unset;
    for (int i = tid; i < nScale16; i += stride) ((uint4*)scales)[i] = s_unset;
    for (int i = tid; i < nGS; i += stride) ws.count[i] = 0;
    for (int i = tid; i < nTiles; i += stride) ws.deferred[i] = 0;
    if (tid == 0) {
        *ws.any = 0;
        ws.stats[0] = 0;
        ws.stats[1] = 0;
    }
    if (blockIdx.x != 0) return;

    __shared__ int sh_st[kWave], sh_en[kWave], sh_first[kWave], sh_cnt[kWave];
    __shared__ int sh_base_chunk, sh_end_chunk;
    __shared__ unsigned long long sh_empty;
    const float s_empty = group_scale_of(0u, ws.pow2);
    const float s_empty_out = ws.inv_out ? 1.0f / s_empty : s_empty;
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
            if (g < G) {
                ws.empty[g] = e <= st ? 1u : 0u;
                ws.gend[g] = e;
                ws.gchunks[2 * g] = incl - cnt;
                ws.gchunks[2 * g + 1] = cnt;
            }
            // 128-row blocks whose first row is in this group (or past the last end)
            if (g <= G)
                for (int c = (st + 127) / 128; c * 128 < e; ++c) ws.bfirst[c] = g;
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
        // with no rows every group is empty and no hold kernel runs: write the scales here
        if (M == 0) {
            for (unsigned long long mm = sh_empty; mm; mm &= mm - 1) {
                const int g = base + __builtin_ctzll(mm);
                float* out = ws.inv_out ? ws.inv_out : scales;
                for (int k = (int)threadIdx.x * 4; k < K; k += kGThreads * 4)
                    *(float4*)(out + (int64_t)g * K + k) = make_float4(s_empty_out, s_empty_out, s_empty_out, s_empty_out);
            }
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

// Size of X from which column-major output holds down to four 128-row blocks
// per group instead of eight (the method choice below).
constexpr int64_t kLargeX = (int64_t)512 << 20;

// The groups' clamped ends and 128-row chunk ranges, computed by one wave from
// the device offsets, for up to kInlineGroups groups (4 per lane: group
// 64 w + l in window w of lane l): the same clamping and chunk numbering as the
// plan kernel's tables, so the two-pass amax kernel can do without that launch
// and leave the tables for the passes after it.
constexpr int kInlineGroups = 256;
struct InlineGroups {
    int e[4], st[4], f[4], n[4];   // end row, start row, first chunk id, chunk count
    int last_end;                  // end of the last group
    __device__ void build(const int32_t* __restrict__ offs, int G, int M)
    {
        const int lane = lane_id();
        const int nw = (G + kWave - 1) / kWave;     // windows in use
        int carry_e = 0, carry_f = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            e[w] = carry_e;
            st[w] = carry_e;
            f[w] = carry_f;
            n[w] = 0;
            if (w >= nw) continue;                  // (uniform)
            const int g = 64 * w + lane;
            int v = g < G ? offs[g] : 0;
            v = dpp_scan_max(v > 0 ? v : 0);
            v = v > carry_e ? v : carry_e;
            v = v < M ? v : M;                      // min(M, .) commutes with the running maximum
            int s0 = dpp_prev_lane(v);
            if (lane == 0) s0 = carry_e;
            const int c = (g < G && v > s0) ? ((v + 127) >> 7) - (s0 >> 7) : 0;   // 128-row chunks
            const int incl = dpp_scan_add(c) + carry_f;
            e[w] = v;
            st[w] = s0;
            n[w] = c;
            f[w] = incl - c;
            carry_e = readlane(v, kWave - 1);
            carry_f = readlane(incl, kWave - 1);
        }
        last_end = carry_e;
    }
    // The plan kernel's tables the finalize and column-block passes read: group
    // ends, chunk ranges, and the group holding the first row of each 128-row
    // block (G past the last end).  One full wave.
    __device__ void write_tables(int G, int M, const Workspace& ws) const
    {
        const int lane = lane_id();
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int g = 64 * w + lane;
            if (g < G) {
                ws.gend[g] = e[w];
                ws.gchunks[2 * g] = f[w];
                ws.gchunks[2 * g + 1] = n[w];
                for (int c = (st[w] + 127) >> 7; (c << 7) < e[w]; ++c) ws.bfirst[c] = g;
            }
        }
        for (int c = ((last_end + 127) >> 7) + lane; (c << 7) < M; c += kWave) ws.bfirst[c] = G;
    }
    // (g is wave-uniform)
    __device__ int pick(const int (&a)[4], int g) const
    {
        const int w = g >> 6, l = g & 63;
        return w == 0 ? readlane(a[0], l) : w == 1 ? readlane(a[1], l) : w == 2 ? readlane(a[2], l) : readlane(a[3], l);
    }
    __device__ int end(int g) const { return pick(e, g); }
    __device__ int start(int g) const { return g == 0 ? 0 : pick(e, g - 1); }
    __device__ int first(int g) const { return pick(f, g); }
    __device__ int count(int g) const { return pick(n, g); }
    // the group whose chunk range holds chunk id j (wave-uniform), G if none
    __device__ int group_of_chunk(int j, int G) const
    {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const unsigned long long m = __ballot(j >= f[w] && j < f[w] + n[w]);
            if (m) return 64 * w + __builtin_ctzll(m);
        }
        return G;
    }
};

// Tile (chunk j, strip s) of a group-ordered chunk numbering, from InlineGroups
// (t.g = G for chunk ids past the last group's chunks).
template <int R>
__device__ __forceinline__ TileInfo tile_info_inline(const InlineGroups& gr, int G, int j, int s)
{
    TileInfo t;
    t.g = gr.group_of_chunk(j, G);
    t.j = j;
    t.s = s;
    if (t.g == G) {
        t.r0 = t.r1 = t.a = t.first = t.count = t.gr0 = t.gr1 = 0;
        return t;
    }
    t.gr0 = gr.start(t.g);
    t.gr1 = gr.end(t.g);
    t.first = gr.first(t.g);
    t.count = gr.count(t.g);
    t.a = (t.gr0 / R + (j - t.first)) * R;
    t.r0 = t.gr0 > t.a ? t.gr0 : t.a;
    t.r1 = t.gr1 < t.a + R ? t.gr1 : t.a + R;
    return t;
}

// (kPartialUnset has the top bit set, which no |bf16| maximum has.)
__device__ __forceinline__ bool partial_written(uint4 w)
{
    static_assert(kPartialUnset & 0x8000u, "unset marker");
    return ((w.x | w.y | w.z | w.w) & 0x80008000u) == 0u;
}
__device__ __forceinline__ bool scales_written(uint4 a, uint4 b)
{
    return a.x != kScaleUnset && a.y != kScaleUnset && a.z != kScaleUnset && a.w != kScaleUnset &&
           b.x != kScaleUnset && b.y != kScaleUnset && b.z != kScaleUnset && b.w != kScaleUnset;
}

// Column maxima of this lane's 8 columns over the group's rows gr0 + rs,
// gr0 + rs + ns, ..., read from the input; only used when a wait ran out.
__device__ __forceinline__ uint4 strip_max_from_x(const uint16_t* __restrict__ x, int K, const TileInfo& t, int k,
                                                  int rs, int ns)
{
    uint4 a = make_uint4(0, 0, 0, 0);
    if (k < K)
        for (int r = t.gr0 + rs; r < t.gr1; r += ns) max8(a, abs8(*(const uint4*)(x + (int64_t)r * K + k)));
    return a;
}

// ------------------------------------------------------- shared pieces ----
template <int LAYOUT, bool STAGE = true>
struct TileShared {
    // (the column-layout staging tile only where a kernel stores q)
    __align__(16) uint8_t stage[LAYOUT == 1 && STAGE ? TileCfg<LAYOUT>::W * TileCfg<LAYOUT>::R : 16];
    uint4 red[TileCfg<LAYOUT>::NS][TileCfg<LAYOUT>::CG];
    // a lane's 8 scales as two float4 indexed by its column group, so that a
    // wave reads 1 KB of consecutive LDS (a 32-byte lane stride put 64 lanes on
    // 8 banks)
    float4 scale_lo[TileCfg<LAYOUT>::CG], scale_hi[TileCfg<LAYOUT>::CG];
    __align__(16) uint32_t vote[TileCfg<LAYOUT>::T / 64];
    int state;
};

// Tile of workgroup `blk`: blocks of SB strips, chunks within a block, strips
// within that (SB = 1: chunk-fastest, so a (group, strip)'s tiles are launched
// back to back).
__device__ __forceinline__ void tile_of_block(int blk, int slots, int SB, int& j, int& s)
{
    const int per_block = slots * SB;
    const int sb = blk / per_block, rem = blk % per_block;
    j = rem / SB;
    s = sb * SB + rem % SB;
}

// The first G workgroups also write the scales of an empty group (nothing
// reads them during the launch).
__device__ __forceinline__ void write_empty_group_scales(int G, int K, const Workspace& ws, float* __restrict__ scales,
                                                         int nthreads)
{
    if ((int)blockIdx.x < G && ws.empty[blockIdx.x] != 0u) {
        const float s_empty = group_scale_of(0u, ws.pow2);
        const float4 e4 = make_float4(s_empty, s_empty, s_empty, s_empty);
        for (int kk = (int)threadIdx.x * 4; kk < K; kk += nthreads * 4) {
            *(float4*)(scales + (int64_t)blockIdx.x * K + kk) = e4;
            if (ws.inv_out) *(float4*)(ws.inv_out + (int64_t)blockIdx.x * K + kk) = inverse4(e4);
        }
    }
}

// Column maxima of the held tile: reduced over the tile's rows through LDS and
// published as the tile's row of the partial maxima by the lanes with rs == 0,
// which return the maxima of their 8 columns (other lanes return zeros).
template <int LAYOUT, class Sh>
__device__ __forceinline__ uint4 publish_tile_max(const uint4 (&v)[TileCfg<LAYOUT>::H], int j, int K, int k, int cg,
                                                  int rs, const Workspace& ws, Sh& sh)
{
    using C = TileCfg<LAYOUT>;
    uint4 m = abs8(v[0]);
#pragma unroll
    for (int i = 1; i < C::H; ++i) max8(m, abs8(v[i]));
    sh.red[rs][cg] = m;
    __syncthreads();
    if (rs == 0) {
        max_rows(m, &sh.red[0][cg], C::NS, C::CG);
        if (k < K) store_coherent(m, ws.partial + (int64_t)j * K + k);
    } else {
        m = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();                                      // sh.red is reused by the strip reduction
    return m;
}

// Streamed groups: publish the tile's maxima, then count the tile in.  Returns 1
// in every lane of the last tile of its (group, strip) to arrive.  No ordering
// between the partial row and the count is needed: the partial row carries its
// own "not yet written" value and the last arrival polls it.
template <int LAYOUT, class Sh>
__device__ __forceinline__ int publish_and_count(const uint4 (&v)[TileCfg<LAYOUT>::H], const TileInfo& t, int j, int s,
                                                 int K, int S, int k, int cg, int rs, const Workspace& ws, Sh& sh)
{
    publish_tile_max<LAYOUT>(v, j, K, k, cg, rs, ws, sh);
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(ws.count + (int64_t)t.g * S + s, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ws.any, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh.state = (old + 1 == (uint32_t)t.count) ? 1 : 0;
    }
    __syncthreads();
    return sh.state;
}

// The strip's scales from its column maxima `a` (rs == 0 lanes: their 8
// columns over their rows; all lanes' values are combined through LDS): divide,
// store them (`publish`: with agent-scope stores, for readers in the same
// launch) and leave this lane's 8 scales in `cs`.
template <int LAYOUT, class Sh>
__device__ __forceinline__ void finish_strip(uint4 a, const TileInfo& t, int K, int k, int cg, int rs,
                                             const Workspace& ws, float* __restrict__ scales, bool publish, Sh& sh,
                                             ColScales& cs)
{
    using C = TileCfg<LAYOUT>;
    sh.red[rs][cg] = a;
    __syncthreads();
    if (rs == 0) {
        max_rows(a, &sh.red[0][cg], C::NS, C::CG);
        const float4 lo = scales_lo(a, ws.pow2), hi = scales_hi(a, ws.pow2);
        sh.scale_lo[cg] = lo;
        sh.scale_hi[cg] = hi;
        if (k < K) {
            float* dst = scales + (int64_t)t.g * K + k;
            if (publish) {
                store_coherent(f4_bits(lo), dst);
                store_coherent(f4_bits(hi), dst + 4);
            } else {
                *(float4*)dst = lo;
                *(float4*)(dst + 4) = hi;
            }
            if (ws.inv_out) {                              // the caller's 1/s (read by no kernel)
                *(float4*)(ws.inv_out + (int64_t)t.g * K + k) = inverse4(lo);
                *(float4*)(ws.inv_out + (int64_t)t.g * K + k + 4) = inverse4(hi);
            }
        }
    }
    __syncthreads();
    cs = make_col_scales(sh.scale_lo[cg], sh.scale_hi[cg]);
}

// The strip's column maxima over all of the group's rows, read from the input
// (only when a wait ran out); counted in the route counters as the group's
// chunk count.
template <int LAYOUT>
__device__ __forceinline__ uint4 strip_max_fallback(const uint16_t* __restrict__ x, const TileInfo& t, int K, int k,
                                                    int rs, const Workspace& ws)
{
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(ws.stats + 1, (uint32_t)t.count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return strip_max_from_x(x, K, t, k, rs, TileCfg<LAYOUT>::NS);
}

// Reduce the strip's partial rows over the group's chunks, except chunk `skip`
// whose maxima the rs == 0 lanes bring in `own` (zeros otherwise), then finish
// the strip.  Each lane polls its rows in batches: every round trip re-reads all
// rows of the batch not yet written, so the batch completes one round trip after
// its last row lands.  If a row does not come within the time limit, the maxima
// are taken from the input instead.
constexpr int kPollBatch = 4;
template <int LAYOUT, class Sh>
__device__ __forceinline__ void reduce_strip(const uint16_t* __restrict__ x, const TileInfo& t, int K, int k, int cg,
                                             int rs, const Workspace& ws, float* __restrict__ scales, int skip,
                                             uint4 own, bool scales_coherent, unsigned long long timeout_ticks,
                                             Sh& sh, ColScales& cs)
{
    using C = TileCfg<LAYOUT>;
    uint4 a = own;
    int ok = 1;
    if (k < K) {
        const uint16_t* p = ws.partial + (int64_t)t.first * K + k;
        const int skip_c = skip - t.first;
        for (int c0 = rs; c0 < t.count && ok; c0 += kPollBatch * C::NS) {
            uint32_t pending = 0;
#pragma unroll
            for (int u = 0; u < kPollBatch; ++u) {
                const int c = c0 + u * C::NS;
                if (c < t.count && c != skip_c) pending |= 1u << u;
            }
            unsigned long long t0 = 0;
            bool timing = false;
            while (pending != 0u) {
                uint4 b[kPollBatch];
#pragma unroll
                for (int u = 0; u < kPollBatch; ++u)
                    b[u] = (pending >> u) & 1u ? load_coherent(p + (int64_t)(c0 + u * C::NS) * K) : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < kPollBatch; ++u) {
                    if (((pending >> u) & 1u) && partial_written(b[u])) {
                        max8(a, b[u]);
                        pending &= ~(1u << u);
                    }
                }
                if (pending == 0u) break;
                if (!timing) {
                    t0 = wall_clock64();
                    timing = true;
                } else if (wall_clock64() - t0 > timeout_ticks) {
                    ok = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
    }
    if (block_any<C::T / 64>(!ok, sh.vote)) a = strip_max_fallback<LAYOUT>(x, t, K, k, rs, ws);   // a partial never came
    finish_strip<LAYOUT>(a, t, K, k, cg, rs, ws, scales, scales_coherent, sh, cs);
}

// The rs == 0 lanes poll their 8 scales until written or until `ticks` have
// passed, and pass them on through LDS.  Returns false (in every lane) if any
// lane's wait ran out.
template <class Sh>
__device__ __forceinline__ bool wait_scales(const float* __restrict__ scales, const TileInfo& t, int K, int k, int cg,
                                            int rs, unsigned long long ticks, Sh& sh)
{
    int ok = 1;
    if (rs == 0 && k < K) {
        const float* sp = scales + (int64_t)t.g * K + k;
        uint4 s0 = load_coherent(sp), s1 = load_coherent(sp + 4);
        if (!scales_written(s0, s1)) {
            const unsigned long long t0 = wall_clock64();
            while (true) {
                __builtin_amdgcn_s_sleep(2);
                s0 = load_coherent(sp);
                s1 = load_coherent(sp + 4);
                if (scales_written(s0, s1)) break;
                if (wall_clock64() - t0 > ticks) {
                    ok = 0;
                    break;
                }
            }
        }
        sh.scale_lo[cg] = bits_f4(s0);
        sh.scale_hi[cg] = bits_f4(s1);
    }
    return !block_any<sizeof(Sh::vote) / sizeof(uint32_t)>(!ok, sh.vote);
}

// Chunk `jc`'s partial row, computed from the input and published (agent
// scope) unless it is written already: the column maxima of the chunk's rows,
// the same values its own tile publishes.  Counted in the route counters.
template <int LAYOUT, class Sh>
__device__ __forceinline__ void publish_chunk_if_missing(const uint16_t* __restrict__ x, const Workspace& ws, int jc,
                                                         int K, int k, int cg, int rs, Sh& sh)
{
    using C = TileCfg<LAYOUT>;
    uint16_t* dst = ws.partial + (int64_t)jc * K + k;
    const bool missing = rs == 0 && k < K && !partial_written(load_coherent(dst));
    if (!block_any<C::T / 64>(missing, sh.vote)) return;
    const int4 e = *(const int4*)(ws.table + jc);         // group, rows [r0, r1) (at most R), first chunk
    uint4 m = make_uint4(0, 0, 0, 0);
    if (k < K) {
        uint4 b[C::H];
#pragma unroll
        for (int i = 0; i < C::H; ++i) {
            const int r = e.y + rs + C::NS * i;
            b[i] = r < e.z ? *(const uint4*)(x + (int64_t)r * K + k) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::H; ++i) max8(m, abs8(b[i]));
    }
    sh.red[rs][cg] = m;
    __syncthreads();
    if (rs == 0) {
        max_rows(m, &sh.red[0][cg], C::NS, C::CG);
        if (k < K) store_coherent(m, dst);
    }
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ws.stats + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
}

// ---------------------------------------------------------------- hold ----
template <int LAYOUT>
__global__ __launch_bounds__(TileCfg<LAYOUT>::T)
void group_hold_kernel(const uint16_t* __restrict__ x, int M, int K, int G, int S, int SB, int slots, Workspace ws,
                       float* __restrict__ scales, uint8_t* __restrict__ q, int hold_limit,
                       unsigned long long timeout_ticks, unsigned long long rescue_ticks, int deferred_launched)
{
    using C = TileCfg<LAYOUT>;
    __shared__ TileShared<LAYOUT> sh;
    int j, s;
    tile_of_block((int)blockIdx.x, slots, SB, j, s);
    write_empty_group_scales(G, K, ws, scales, C::T);
    const TileInfo t = tile_info<C::R>(ws.table, j, s);
    if (t.g < 0) return;                                  // unused chunk id (uniform)
    const int cg = (int)threadIdx.x % C::CG, rs = (int)threadIdx.x / C::CG;
    const int k = s * C::W + cg * 8;
    ColScales cs;
    uint4 v[C::H];

    if (t.g == G) {                                       // rows past the last end: zeros
        quantize_store_tile<LAYOUT>(v, cs, t, M, K, k, cg, rs, q, sh.stage, true);
        return;
    }
    // A (group, strip) is one synchronisation domain and its tiles are launched
    // consecutively, so `count` tiles must be resident together.
    const bool streamed = t.count > hold_limit;
    load_tile<LAYOUT>(x, K, t, k, rs, v);

    if (streamed) {
        // too many tiles to hold: the last arrival reduces the strip and the
        // deferred kernel quantizes the group
        if (publish_and_count<LAYOUT>(v, t, j, s, K, S, k, cg, rs, ws, sh))
            reduce_strip<LAYOUT>(x, t, K, k, cg, rs, ws, scales, -1, make_uint4(0, 0, 0, 0), false, timeout_ticks,
                                 sh, cs);
        return;
    }
    // The group's last chunk, launched after all the others, reduces the strip
    // (its own maxima straight from registers); the others publish and wait.
    const uint4 own = publish_tile_max<LAYOUT>(v, j, K, k, cg, rs, ws, sh);
    if (j == t.first + t.count - 1) {
        reduce_strip<LAYOUT>(x, t, K, k, cg, rs, ws, scales, j, own, true, timeout_ticks, sh, cs);
    } else {
        // wait for the strip's scales (bounded in wall-clock time)
        if (!wait_scales(scales, t, K, k, cg, rs, timeout_ticks, sh)) {
            if (threadIdx.x == 0) __hip_atomic_fetch_add(ws.stats, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (deferred_launched) {
                // left for the deferred kernel, which runs after every strip is reduced
                if (threadIdx.x == 0) {
                    __hip_atomic_store(ws.deferred + (int64_t)j * S + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(ws.any, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                return;
            }
            // The wait ran out and no deferred pass follows: some of the group's
            // tiles are not running (the device, perhaps shared with other work,
            // did not keep them resident together).  The tiles whose wait ran out
            // take the strip's chunks one by one, from the last down, through
            // the strip's arrival counter (unused for held groups); each chunk
            // whose partial row is not written yet is computed from the input and
            // published, as its own tile would.  Then every partial row comes
            // from a running workgroup that waits for nothing, the first of these
            // tiles reduces the strip and publishes the scales, and the others
            // wait for them (the group's last tile, when it runs, publishes the
            // same values).
            bool first_helper = false;
            for (int grab = 0;; ++grab) {
                if (threadIdx.x == 0)
                    sh.state = (int)__hip_atomic_fetch_add(ws.count + (int64_t)t.g * S + s, 1u, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                __syncthreads();
                const int n = sh.state;
                __syncthreads();                          // (sh.state is written again by the next grab)
                if (grab == 0) first_helper = n == 0;
                if (n >= t.count) break;
                publish_chunk_if_missing<LAYOUT>(x, ws, t.first + t.count - 1 - n, K, k, cg, rs, sh);
            }
            if (first_helper)
                reduce_strip<LAYOUT>(x, t, K, k, cg, rs, ws, scales, -1, make_uint4(0, 0, 0, 0), true,
                                     timeout_ticks + rescue_ticks, sh, cs);
            else if (!wait_scales(scales, t, K, k, cg, rs, timeout_ticks + rescue_ticks, sh))
                finish_strip<LAYOUT>(strip_max_fallback<LAYOUT>(x, t, K, k, rs, ws), t, K, k, cg, rs, ws, scales, true,
                                     sh, cs);
            else
                cs = make_col_scales(sh.scale_lo[cg], sh.scale_hi[cg]);
        } else {
            cs = make_col_scales(sh.scale_lo[cg], sh.scale_hi[cg]);
        }
    }
    quantize_store_tile<LAYOUT>(v, cs, t, M, K, k, cg, rs, q, sh.stage, false);
}

// ------------------------------------------------------------ two-pass ----
// The alternative to holding: an amax pass (every tile stores its column maxima
// as one partial row), a finalize pass (one workgroup per (group, strip)
// reduces the group's partial rows and divides), then a quantize pass that
// reads X again.  5 bytes moved per element instead of 3, but no workgroup ever
// waits for another, so every pass streams.
// Amax pass: one workgroup per tile (the hold kernel's tiles); its column
// maxima become the tile's piece of the chunk's partial row.  Its loads keep
// the default cache policy: part of X then still sits in the last-level cache
// when the quantize pass reads it again (measured 52 -> 44 us for that pass at
// 16640 x 5120, for 2 us more here).
// INLINE: the tile comes from the offsets (InlineGroups, G <= kInlineGroups)
// instead of the plan kernel's table, and workgroup 0 writes the tables the
// finalize and quantize passes read.
template <int LAYOUT, bool INLINE>
__global__ __launch_bounds__(TileCfg<LAYOUT>::T)
void group_amax_kernel(const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ offs, int G, int S,
                       Workspace ws)
{
    using C = TileCfg<LAYOUT>;
    __shared__ uint4 red[C::NS][C::CG];
    const int j = (int)blockIdx.x / S, s = (int)blockIdx.x % S;
    TileInfo t;
    if constexpr (INLINE) {
        InlineGroups gr;
        gr.build(offs, G, M);
        if (blockIdx.x == 0 && threadIdx.x < kWave) gr.write_tables(G, M, ws);   // for the next two passes
        t = tile_info_inline<C::R>(gr, G, j, s);
    } else {
        t = tile_info<C::R>(ws.table, j, s);
    }
    if (t.g < 0 || t.g == G) return;                      // unused chunk id or rows past the last end (uniform)
    const int cg = (int)threadIdx.x % C::CG, rs = (int)threadIdx.x / C::CG;
    const int k = s * C::W + cg * 8;
    uint4 v[C::H];
    load_tile<LAYOUT, kCached>(x, K, t, k, rs, v);   // cached: the quantize pass re-reads X
    uint4 m = abs8(v[0]);
#pragma unroll
    for (int i = 1; i < C::H; ++i) max8(m, abs8(v[i]));
    red[rs][cg] = m;
    __syncthreads();
    if (rs == 0 && k < K) {
#pragma unroll
        for (int r = 1; r < C::NS; ++r) max8(m, red[r][cg]);
        *(uint4*)(ws.partial + (int64_t)j * K + k) = m;
    }
}

// One workgroup per (group, strip of 256 columns): lane (cg, rs) reduces
// partial rows rs, rs + 8, ... of the group for columns 8cg..8cg+7.  An empty
// group (no chunks) gets the scale of amax 0.  (128-column strips, 16 row
// slots, ran the G = 128 column-major call about 2 us slower: most groups there
// have one or two chunks, so most row slots were idle; 512 columns measured the
// same as 256.)
constexpr int kFThreads = 256, kFW = 256, kFCG = kFW / 8, kFNS = kFThreads / kFCG;
__global__ __launch_bounds__(kFThreads)
void group_finalize_kernel(int K, int SF, Workspace ws, float* __restrict__ scales)
{
    __shared__ uint4 red[kFNS][kFCG];
    const int g = (int)blockIdx.x / SF, s = (int)blockIdx.x % SF;
    const int first = ws.gchunks[2 * g], count = ws.gchunks[2 * g + 1];
    const int cg = (int)threadIdx.x % kFCG, rs = (int)threadIdx.x / kFCG;
    const int k = s * kFW + cg * 8;
    uint4 a = make_uint4(0, 0, 0, 0);
    if (k < K) {
        const uint16_t* p = ws.partial + (int64_t)first * K + k;
        int c = rs;
        for (; c + 3 * kFNS < count; c += 4 * kFNS) {
            uint4 b[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) b[u] = *(const uint4*)(p + (int64_t)(c + u * kFNS) * K);
#pragma unroll
            for (int u = 0; u < 4; ++u) max8(a, b[u]);
        }
        for (; c < count; c += kFNS) max8(a, *(const uint4*)(p + (int64_t)c * K));
    }
    red[rs][cg] = a;
    __syncthreads();
    if (rs == 0 && k < K) {
#pragma unroll
        for (int r = 1; r < kFNS; ++r) max8(a, red[r][cg]);
        const float4 lo = scales_lo(a, ws.pow2), hi = scales_hi(a, ws.pow2);
        *(float4*)(scales + (int64_t)g * K + k) = lo;
        *(float4*)(scales + (int64_t)g * K + k + 4) = hi;
        if (ws.inv_out) {
            *(float4*)(ws.inv_out + (int64_t)g * K + k) = inverse4(lo);
            *(float4*)(ws.inv_out + (int64_t)g * K + k + 4) = inverse4(hi);
        }
    }
}

template <int LAYOUT>
__global__ __launch_bounds__(TileCfg<LAYOUT>::T)
void group_quant_kernel(const uint16_t* __restrict__ x, int M, int K, int G, int S, Workspace ws,
                        const float* __restrict__ scales, uint8_t* __restrict__ q)
{
    using C = TileCfg<LAYOUT>;
    __shared__ __align__(16) uint8_t stage[LAYOUT == 1 ? C::W * C::R : 16];
    const int j = (int)blockIdx.x / S, s = (int)blockIdx.x % S;
    const TileInfo t = tile_info<C::R>(ws.table, j, s);
    if (t.g < 0) return;                                  // unused chunk id (uniform)
    const int cg = (int)threadIdx.x % C::CG, rs = (int)threadIdx.x / C::CG;
    const int k = s * C::W + cg * 8;
    ColScales cs;
    uint4 v[C::H];
    if (t.g < G) {
        load_tile<LAYOUT>(x, K, t, k, rs, v);
        if (k < K)
            cs = make_col_scales(*(const float4*)(scales + (int64_t)t.g * K + k),
                                 *(const float4*)(scales + (int64_t)t.g * K + k + 4));
    }
    quantize_store_tile<LAYOUT>(v, cs, t, M, K, k, cg, rs, q, stage, t.g == G);
}

// Column-major quantize pass over 128-row blocks that ignore group boundaries,
// so every output row (a column of X) gets whole 128-byte lines, never a
// partial line shared with the neighbouring group's tile.  Each row takes its
// own group's scales: a lane walks its 16 consecutive rows, moving to the next
// group (and loading its 8 scales) whenever a row reaches the group's end.
// Rows are quantized row-wise (8 codes per row) and the lane's 16 x 8 code
// block is transposed in registers (byte permutes) into 8 columns of 16 rows.
__global__ __launch_bounds__(TileCfg<1>::T)
void group_quant_col_blocks_kernel(const uint16_t* __restrict__ x, int M, int K, int G, int S, Workspace ws,
                                   const float* __restrict__ scales, uint8_t* __restrict__ q)
{
    using C = TileCfg<1>;
    __shared__ __align__(16) uint8_t stage[C::W * C::R];
    const int blk = (int)blockIdx.x / S, s = (int)blockIdx.x % S;
    const int a = blk * C::R;
    const int cg = (int)threadIdx.x % C::CG, rs = (int)threadIdx.x / C::CG;
    const int k = s * C::W + cg * 8;
    TileInfo t;
    t.a = a;
    t.r0 = a;
    t.r1 = a + C::R < M ? a + C::R : M;
    t.s = s;
    uint4 v[C::H];
    load_tile<1>(x, K, t, k, rs, v);

    // codes of this lane's 16 rows, row by row, each with its group's scales
    const int row0 = a + rs * C::H;
    int g = ws.bfirst[blk];
    int gend = g < G ? ws.gend[g] : 0x7FFFFFFF;
    ColScales cs;
    bool have = false;
    uint2 out[C::H];
#pragma unroll
    for (int i = 0; i < C::H; ++i) {
        const int row = row0 + i;
        if (row >= gend) {
            do {
                ++g;
                gend = g < G ? ws.gend[g] : 0x7FFFFFFF;
            } while (row >= gend);
            have = false;
        }
        if (!have && g < G && k < K) {
            cs = make_col_scales(*(const float4*)(scales + (int64_t)g * K + k),
                                 *(const float4*)(scales + (int64_t)g * K + k + 4));
            have = true;
        }
        // rows past the last end, and past M, get code 0 (the latter are not stored)
        out[i] = (g < G && row < M) ? group_quantize_chunk(v[i], cs) : make_uint2(0, 0);
    }
    // 16 rows x 8 columns of codes -> 8 columns x 16 rows in the staging tile
#pragma unroll
    for (int half = 0; half < 2; ++half) {           // columns 0..3, then 4..7
        uint32_t col[4][4];                          // [column][row quad]
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            uint32_t o4[4];
            transpose4x4_bytes(half ? out[4 * qd].y : out[4 * qd].x, half ? out[4 * qd + 1].y : out[4 * qd + 1].x,
                               half ? out[4 * qd + 2].y : out[4 * qd + 2].x, half ? out[4 * qd + 3].y : out[4 * qd + 3].x,
                               o4);
#pragma unroll
            for (int c = 0; c < 4; ++c) col[c][qd] = o4[c];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *(uint4*)(stage + col_tile_offset(cg * 8 + half * 4 + c, rs * C::H)) =
                make_uint4(col[c][0], col[c][1], col[c][2], col[c][3]);
    }
    __syncthreads();
    // column cc of the block becomes output row (strip * W + cc): rows [0, r1 - a)
    const int hi = t.r1 - a;
    const bool aligned16 = (M & 15) == 0;
    const int64_t col0 = (int64_t)s * C::W;
    for (int it = 0; it < (C::W * 8) / C::T; ++it) {
        const int sid = (int)threadIdx.x + C::T * it;
        const int cc = sid >> 3, seg = sid & 7;
        if (col0 + cc >= K) continue;
        const int rb = seg * 16;
        if (rb >= hi) continue;
        const uint4 val = *(const uint4*)(stage + col_tile_offset(cc, rb));
        uint8_t* dst = q + (col0 + cc) * (int64_t)M + a + rb;
        if (aligned16 && rb + 16 <= hi) {
            store_nt(val, (uint4*)dst);
        } else {
            store_partial16(val, dst, 0, rb + 16 < hi ? 16 : hi - rb, aligned16);
        }
    }
}

// ------------------------------------------------------------ deferred ----
// A small grid walks all tiles; it returns at once when nothing was left over.
// The scales of every group are final (written by the hold kernel's last
// arrivals), so deferred tiles only re-read and quantize.
template <int LAYOUT>
__global__ __launch_bounds__(TileCfg<LAYOUT>::T)
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
        uint4 v[C::H];
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
// Route and limit overrides (tests and tuning only; the bytes never depend on
// them), set process-wide through mxq_set_group_scale_knobs.
std::atomic<int> g_method{0}, g_hold_tiles{-1}, g_strip_block{0};
std::atomic<long> g_wait_us{-1};

struct GroupKnobs {
    int method, hold_tiles, strip_block;
    long wait_us;
};

static GroupKnobs group_knobs()
{
    return GroupKnobs{g_method.load(std::memory_order_relaxed), g_hold_tiles.load(std::memory_order_relaxed),
                      g_strip_block.load(std::memory_order_relaxed), g_wait_us.load(std::memory_order_relaxed)};
}

void set_group_scale_knobs(int method, int hold_tiles, long wait_us, int strip_block)
{
    g_method.store(method, std::memory_order_relaxed);
    g_hold_tiles.store(hold_tiles, std::memory_order_relaxed);
    g_wait_us.store(wait_us, std::memory_order_relaxed);
    g_strip_block.store(strip_block, std::memory_order_relaxed);
}

// Per-device facts the launcher needs, queried once per device.
struct DeviceInfo {
    int cus, rate_khz, per_cu[2];
    bool ok;
};
constexpr int kMaxDevices = 64;
static DeviceInfo g_dev[kMaxDevices];
static std::once_flag g_dev_once[kMaxDevices];

static const DeviceInfo* device_info()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_dev_once[dev], [dev] {
        DeviceInfo& d = g_dev[dev];
        d.ok = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
               hipDeviceGetAttribute(&d.rate_khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess &&
               hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.per_cu[0], group_hold_kernel<0>, TileCfg<0>::T, 0) ==
                   hipSuccess &&
               hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.per_cu[1], group_hold_kernel<1>, TileCfg<1>::T, 0) ==
                   hipSuccess;
    });
    return g_dev[dev].ok ? &g_dev[dev] : nullptr;
}

template <int LAYOUT>
static hipError_t launch_layout(const void* x, int M, int K, const int32_t* offs, int G, int flags, void* q,
                                float* out_scales, void* workspace, hipStream_t stream)
{
    using C = TileCfg<LAYOUT>;
    size_t off[10];
    workspace_layout<LAYOUT>(M, K, G, off);
    uint8_t* base = (uint8_t*)workspace;
    Workspace ws;
    ws.table = (ChunkEntry*)(base + off[0]);
    ws.partial = (uint16_t*)(base + off[1]);
    ws.count = (uint32_t*)(base + off[2]);
    ws.empty = (uint32_t*)(base + off[3]);
    ws.deferred = (uint32_t*)(base + off[4]);
    ws.any = (uint32_t*)(base + off[5]);
    ws.stats = ws.any + 1;
    ws.gend = (int32_t*)(base + off[6]);
    ws.bfirst = (int32_t*)(base + off[7]);
    ws.gchunks = (int32_t*)(base + off[8]);
    // Every kernel reads and writes the multipliers s through `scales`: the
    // caller's array, or a workspace array when the caller asked for 1/s, which
    // the writers of s then also store in the caller's array.
    const bool inverse = (flags & 2) != 0;
    float* scales = inverse ? (float*)(base + off[9]) : out_scales;
    ws.inv_out = inverse ? out_scales : nullptr;
    ws.pow2 = (flags & 1) ? 1 : 0;
    const int S = (K + C::W - 1) / C::W;
    const int64_t slots = chunk_slots(M, C::R, G);
    const int nGS = G * S;
    const int64_t nTiles = slots * S;

    // How many tiles of one group may be held at once: the resident capacity of
    // the hold kernel on this device, less a small margin.  Holding more than
    // fits is still correct (waits time out and the tiles are deferred), only slower.
    const DeviceInfo* di = device_info();
    if (!di) return hipErrorInvalidDevice;
    const GroupKnobs kn = group_knobs();
    int hold_limit = kn.hold_tiles >= 0 ? kn.hold_tiles : di->cus * di->per_cu[LAYOUT] - 16;
    const long wait_us = kn.wait_us >= 0 ? kn.wait_us : 2000;
    int SB = kn.strip_block > 0 ? kn.strip_block : 1;     // chunk-fastest launch order (measured best)
    if (S % SB != 0) SB = S;
    const unsigned long long ticks_per_ms = (unsigned long long)(di->rate_khz > 0 ? di->rate_khz : 100000);
    const unsigned long long timeout_ticks = ticks_per_ms * (unsigned long long)wait_us / 1000ull;
    // how much longer tiles wait for a strip claimed after a time-out (its
    // claimant reads the group's rows of the strip, one workgroup alone)
    const unsigned long long rescue_ticks = ticks_per_ms * 50ull;
    // The method.  Default, from measurements at 16640 x 5120 (8 to 128 Zipf
    // groups), 16640 x 8192 (4 to 32) and 65536 x 5120 (8 to 256).  Row-major
    // output holds (one read of X; 65-73 us against 75-100 us for the two-read
    // methods at 16640 x 5120).  Column-major output holds while the average
    // group spans at least eight 128-row blocks, and takes the two-pass method
    // with more groups (at 16640 x 5120: 73.5 against 73.7 us at 16 groups,
    // 76.7 against 75.2 at 20, 110 against 81 at 128).  With a larger X the
    // hold method's one read pays off to fewer blocks per group: at 65536 x
    // 5120 (671 MB) it wins down to four (257 against 289 us at 64 groups,
    // 286 against 294 at 128, 335 against 306 at 256), while at 16640 x 8192
    // (272 MB) the crossover is still between 16 and 32 groups (115 against
    // 115, 130 against 116); the threshold of 512 MB lies between the two
    // sizes measured.  The split method (two streaming passes, the
    // second over 128-row blocks; at most 256 groups) is taken only when
    // forced: it was never the fastest, within 1 us of the best at 8 and 16
    // groups at 16640 x 8192 and 2 to 65 us behind at every other point.
    const int64_t nblk = (M + 127) / 128;
    const bool large_x = (int64_t)M * K * 2 >= kLargeX;
    const bool few = 8 * (int64_t)G <= nblk || (large_x && 4 * (int64_t)G <= nblk);
    bool twopass = LAYOUT == 1 && !few;
    bool split = false;
    if (kn.method == 1) twopass = split = false;
    if (kn.method == 2) twopass = true, split = false;
    if (kn.method == 3) split = group_split_sizes_ok(M, K, G);
    if (split) return launch_group_split(x, M, K, offs, G, LAYOUT, flags, q, out_scales, workspace, stream);

    // Column-major two-pass with at most kInlineGroups groups: the amax pass
    // takes the group ends and chunk ranges from the offsets itself, and its
    // first workgroup writes the tables the finalize and quantize passes read,
    // so the plan launch (a kernel boundary) is not needed (84 -> 80 us per call
    // at 16640 x 5120 and 128 groups, measured alternately; every kernel
    // scanning the offsets itself measured 88 us).
    const bool inline_groups = M > 0 && twopass && LAYOUT == 1 && G <= kInlineGroups;
    if (!inline_groups) {
        // the fills are a few MB: give them enough blocks (the scales are polled
        // only by the hold kernel)
        const int nPartial16 = twopass ? 0 : (int)(slots * K / 8);   // (every partial row is written before it is read)
        const int nScale16 = M > 0 && !twopass ? (int)((int64_t)G * K / 4) : 0;
        int pgrid = (int)(((int64_t)nPartial16 + nScale16) / (kGThreads * 8));
        pgrid = pgrid < 64 ? 64 : pgrid > 1024 ? 1024 : pgrid;
        hipLaunchKernelGGL(group_plan_kernel<C::R>, dim3(pgrid), dim3(kGThreads), 0, stream, offs, G, M, K, ws, nGS,
                           (int)nTiles, (int)slots, scales, nPartial16, nScale16);
    }
    if (M > 0 && twopass) {
        if (inline_groups)
            hipLaunchKernelGGL((group_amax_kernel<LAYOUT, true>), dim3((unsigned)nTiles), dim3(C::T), 0, stream,
                               (const uint16_t*)x, M, K, offs, G, S, ws);
        else
            hipLaunchKernelGGL((group_amax_kernel<LAYOUT, false>), dim3((unsigned)nTiles), dim3(C::T), 0, stream,
                               (const uint16_t*)x, M, K, offs, G, S, ws);
        const int SF = (K + kFW - 1) / kFW;
        hipLaunchKernelGGL(group_finalize_kernel, dim3((unsigned)(G * SF)), dim3(kFThreads), 0, stream, K, SF, ws,
                           scales);
        if (LAYOUT == 1) {
            const int nBlk = (M + C::R - 1) / C::R;
            hipLaunchKernelGGL(group_quant_col_blocks_kernel, dim3((unsigned)(nBlk * S)), dim3(TileCfg<1>::T), 0, stream,
                               (const uint16_t*)x, M, K, G, S, ws, (const float*)scales, (uint8_t*)q);
        } else {
            hipLaunchKernelGGL(group_quant_kernel<LAYOUT>, dim3((unsigned)nTiles), dim3(C::T), 0, stream,
                               (const uint16_t*)x, M, K, G, S, ws, (const float*)scales, (uint8_t*)q);
        }
    } else if (M > 0) {
        // No group spans more than ceil(M/R) + 1 chunks: unless that exceeds the
        // hold limit nothing is streamed, and tiles whose wait runs out finish
        // themselves, so the deferred pass is not launched at all.
        const int deferred = (int64_t)(M + C::R - 1) / C::R + 1 > hold_limit ? 1 : 0;
        hipLaunchKernelGGL(group_hold_kernel<LAYOUT>, dim3((unsigned)nTiles), dim3(C::T), 0, stream,
                           (const uint16_t*)x, M, K, G, S, SB, (int)slots, ws, scales, (uint8_t*)q, hold_limit,
                           timeout_ticks, rescue_ticks, deferred);
        if (!deferred) return hipGetLastError();
        const int dgrid = (int)(nTiles < 512 ? nTiles : 512);
        hipLaunchKernelGGL(group_deferred_kernel<LAYOUT>, dim3((unsigned)dgrid), dim3(C::T), 0, stream,
                           (const uint16_t*)x, M, K, G, S, ws, (const float*)scales, (uint8_t*)q, hold_limit,
                           (int)nTiles);
    }
    return hipGetLastError();
}

// ----------------------------------------------------- allocation-free ---
// Scratch for callers that cannot allocate (code under graph capture, serving
// loops, harnesses that forbid hipMalloc): one array per device, alive until
// the process ends.  In host code `scratch` only names the symbol; its device
// address is looked up once per device (with that device current) and used
// everywhere instead.  Every call on a device shares its array, so calls that
// overlap on one device race.  Nothing in it needs to survive a call: the
// plan kernel re-initialises all that the other kernels read.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
static void* g_scratch_ptr[kMaxDevices];
static hipError_t g_scratch_err[kMaxDevices];
static std::once_flag g_scratch_once[kMaxDevices];

hipError_t group_scale_scratch(void** ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t group_scale_route_counters(const void* workspace, int64_t M, int64_t K, int64_t G, int layout,
                                     uint32_t* out, hipStream_t stream)
{
    size_t off[10];
    if (layout == 0)
        workspace_layout<0>(M, K, G, off);
    else
        workspace_layout<1>(M, K, G, off);
    const hipError_t e = hipMemcpyAsync(out, (const uint8_t*)workspace + off[5] + 4, 2 * sizeof(uint32_t),
                                        hipMemcpyDeviceToHost, stream);
    return e != hipSuccess ? e : hipStreamSynchronize(stream);
}

hipError_t launch_group_scale(const void* x, int M, int K, const int32_t* offs, int G, int layout, int flags,
                              void* q, float* scales, void* workspace, hipStream_t stream)
{
    return layout == 0 ? launch_layout<0>(x, M, K, offs, G, flags, q, scales, workspace, stream)
                       : launch_layout<1>(x, M, K, offs, G, flags, q, scales, workspace, stream);
}

}  // namespace mxq
