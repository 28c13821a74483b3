// grouped_mm.hip -- grouped product of MXFP8 operands on gfx950 scaled-fp8 MFMA.
//
// Y[m, :] = X[m, :] W_g^T for the token rows m of group g.  X (M, K) and every
// W_g (N, K) are MXFP8 along K: E4M3 codes plus one E8M0 scale per 32
// consecutive k, exactly the buffers mxq_quantize_mx writes.  The product runs
// on v_mfma_scale_f32_32x32x64_f8f6f4, which takes the two operands' E8M0
// block scales as instruction operands, so the codes are never dequantized in
// software; partial sums are fp32, the output bf16 (or fp32).
//
// Sources: "[moe training] fix uncoalesced global accesses in per group rowwise
// scaling kernel", Summary (the group-scaled tokens are the LHS of a scaled
// grouped GEMM); "[mxfp8 MoE training] Support mxfp8 all to all in expert
// parallel", Summary (the MXFP8 buffers of the token exchange).
//
// Work decomposition
//   Output tiles are 256 token rows x 256 columns.  Row tiles never straddle a
//   group: group g's rows [start, end) are cut into ceil(len/256) tiles from
//   its start, so a tile reads one W_g.  Rows past the last end form one more
//   pseudo-group whose tiles are written with zeros.  A one-workgroup plan
//   kernel turns the device-resident end offsets into this tile list (no host
//   copy), ordered group by group, and inside a group in blocks of kCB column
//   tiles with the row tiles of a block consecutive -- so consecutively
//   numbered tiles share W_g column blocks and X row tiles.  Workgroup b runs
//   list entry (b % 8) * q + b / 8 (q = ceil(count / 8)): the hardware deals
//   workgroups to the 8 XCDs round-robin, so each XCD walks one contiguous
//   stretch of the list and its L2 sees the reuse.
//
// Tile kernel (256 threads = 4 waves in 2 x 2, each wave 128 x 128)
//   K advances 64 bytes (one MFMA k-step) per stage through a 4-slot LDS ring
//   of W_g and X tiles (256 rows x 64 B each; 16-byte chunks XOR-swizzled by
//   row so that the operand reads are free of bank conflicts), filled straight
//   from global memory by buffer-load-to-LDS.  Each stage waits for its own
//   loads, reads the wave's operands into VGPRs, and issues its 16 MFMAs with
//   the loads of the stage three ahead slotted between them.  Global loads use
//   raw buffer resources that end at the tile's last valid row: rows past a
//   group's end or past N read as zero, with no per-row branch.  MFMA operand
//   A is W_g (output columns), B is X (token rows), so each lane ends up holding
//   runs of four consecutive output columns of one row and stores them as one
//   8-byte (bf16) or 16-byte (fp32) write.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <utility>

#include "device_common.hpp"
#include "internal.hpp"

namespace mxq {
namespace {

constexpr int kBM = 256;        // token rows per tile
constexpr int kBN = 256;        // output columns per tile
constexpr int kBK = 64;         // K bytes per LDS stage (one MFMA k-step)
constexpr int kKStep = 128;     // K must be a multiple of this (a scale word covers 128 k)
constexpr int kThreads = 256;
constexpr int kCB = 4;          // column tiles per block of the tile order
constexpr int kXcds = 8;
constexpr int kPlanThreads = 1024;

static_assert(kBM == kBN, "one row count serves both operand tiles");

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Workspace: int header[4] (header[0] = number of tiles), then int4 tiles[].
struct Tile {
    int g, r0, r1, c;           // group, rows [r0, r1), column tile c
};

__host__ __device__ inline int64_t mm_slots(int64_t M, int64_t G)
{
    return (M + kBM - 1) / kBM + G + 1;
}

// ------------------------------------------------------------------ plan ---
// Inclusive block-wide scan over one value per thread (op = max or +).
template <bool MAX>
__device__ int block_scan(int v, int* sh)
{
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int d = 1; d < kPlanThreads; d <<= 1) {
        const int o = t >= d ? sh[t - d] : (MAX ? INT32_MIN : 0);
        __syncthreads();
        v = MAX ? (o > v ? o : v) : v + o;
        sh[t] = v;
        __syncthreads();
    }
    return v;
}

constexpr int kPlanPerThread = 4;
constexpr int kMaxGroups = kPlanThreads * kPlanPerThread - 1;   // + the tail pseudo-group

__global__ __launch_bounds__(kPlanThreads) void mm_plan_kernel(const int32_t* __restrict__ offs, int G, int M,
                                                               int NC, int* __restrict__ ws)
{
    __shared__ int end_sh[kMaxGroups + 1];       // clamped end of group g (g = G: the tail, end = M)
    __shared__ int tile_sh[kMaxGroups + 2];      // first tile of group g; tile_sh[G + 1] = tile count
    __shared__ int scan_sh[kPlanThreads];
    const int t = threadIdx.x;
    const int base = t * kPlanPerThread;

    // clamped ends: running maximum of the offsets, cut to [0, M]
    int e[kPlanPerThread];
    int run = 0;
    for (int i = 0; i < kPlanPerThread; ++i) {
        const int g = base + i;
        int v = g < G ? offs[g] : (g == G ? M : 0);
        run = v > run ? v : run;
        e[i] = run;
    }
    block_scan<true>(run, scan_sh);              // scan_sh: inclusive running maxima
    const int prev = t ? scan_sh[t - 1] : 0;
    __syncthreads();
    for (int i = 0; i < kPlanPerThread; ++i) {
        int v = e[i] > prev ? e[i] : prev;
        v = v < 0 ? 0 : (v > M ? M : v);
        e[i] = v;
        if (base + i <= G) end_sh[base + i] = v;
    }
    __syncthreads();

    // tiles per group and their prefix sum
    int cnt[kPlanPerThread];
    int sum = 0;
    for (int i = 0; i < kPlanPerThread; ++i) {
        const int g = base + i;
        int c = 0;
        if (g <= G) {
            const int st = g ? end_sh[g - 1] : 0;
            c = (e[i] - st + kBM - 1) / kBM;
        }
        cnt[i] = c;
        sum += c;
    }
    const int incl2 = block_scan<false>(sum, scan_sh);
    int run2 = incl2 - sum;
    for (int i = 0; i < kPlanPerThread; ++i) {
        if (base + i <= G) tile_sh[base + i] = run2;
        run2 += cnt[i];
    }
    if (t == kPlanThreads - 1) tile_sh[G + 1] = incl2;
    __syncthreads();
    const int T = tile_sh[G + 1];
    const int V = T * NC;
    if (t == 0) ws[0] = V;

    Tile* tiles = reinterpret_cast<Tile*>(ws + 4);
    for (int L = t; L < V; L += kPlanThreads) {
        // group: last g with tile_sh[g] * NC <= L
        int lo = 0, hi = G;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tile_sh[mid] * NC <= L) lo = mid;
            else hi = mid - 1;
        }
        const int g = lo;
        const int R = tile_sh[g + 1] - tile_sh[g];
        const int local = L - tile_sh[g] * NC;
        const int cb = local / (R * kCB);
        const int rem = local - cb * R * kCB;
        const int w = NC - cb * kCB < kCB ? NC - cb * kCB : kCB;
        const int r = rem / w;
        const int st = g ? end_sh[g - 1] : 0;
        Tile tl;
        tl.g = g;
        tl.r0 = st + r * kBM;
        tl.r1 = tl.r0 + kBM < end_sh[g] ? tl.r0 + kBM : end_sh[g];
        tl.c = cb * kCB + rem % w;
        tiles[L] = tl;
    }
}

// ------------------------------------------------------------ tile kernel ---
// K advances kBK = 64 bytes (one MFMA k-step) per stage.  Stages live in a
// 4-deep LDS ring filled by buffer-load-to-LDS (the data never passes through
// VGPRs), so three stages are in flight while one is multiplied.  Scales
// travel in chunks of 16 bytes per row (16 k-blocks = 8 stages), fetched seven
// stages before their first use into a 2-slot ring.
constexpr int kRing = 4;
constexpr int kChunkStages = 8;                         // stages per scale chunk
constexpr int kTileBytes = kBM * kBK;                   // 16 KB of codes per operand per stage
constexpr int kChunkBytes = kBM * 16;                   // 4 KB of scales per operand per chunk
constexpr int kDataBytes = kRing * 2 * kTileBytes;      // 128 KB
constexpr int kDummyBytes = 4 * 1024;                   // sink for loads that carry nothing
constexpr int kLdsBytes = kDataBytes + 2 * 2 * kChunkBytes + kDummyBytes;   // + 16 KB + 4 KB
static_assert(kBK == 64 && kChunkStages * kBK == 512, "a scale chunk is 16 k-blocks of 32");

typedef __attribute__((address_space(3))) uint8_t* LdsPtr;
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr uint32_t kOOB = 0xFFFFFFF0u;                  // past every buffer resource used here

// Buffer resource in SGPRs for the asm loads below: base, stride 0, size in
// bytes (loads at or past it return zeros), raw-buffer flags.
__device__ __forceinline__ v4i make_srd(const void* base, uint32_t bytes)
{
    const uint64_t b = (uint64_t)(uintptr_t)base;
    v4i r = {(int)(uint32_t)b, (int)(uint32_t)(b >> 32), (int)bytes, 0x00020000};
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p)
{
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(LdsPtr)p);
}

// Buffer load straight into LDS: each lane's `bytes` bytes land at
// lds + lane * bytes (M0 holds the wave-uniform LDS address).  The load has no
// VGPR result; its completion is counted by vmcnt, which the stage barrier waits
// on explicitly.  Written in asm so that the compiler does not add a
// conservative wait for it before every later LDS read.  (M0 is reserved by the
// compiler and set before each of its own uses; nothing else here reads it.)
__device__ __forceinline__ void dma16(const v4i& srd, uint32_t lds, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(srd)
                 : "memory");
}

// Physical 16-byte chunk of logical chunk c in LDS row r (rows of 64 bytes).
// The fragment reads (lane -> row c32 of a 32-row tile, chunks hk and 2 + hk)
// measured conflict-free on gfx950 with this swizzle (4 LDS cycles per
// 128-bit wave read); without it they take 4x as long.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 2) & 3); }

// Loads of stage t, per wave: 2 scale-chunk loads, then 8 data loads into
// ring slot t % 4.  Stage 0 carries chunk 0 and stage 8c + 4 chunk c + 1 (if
// that chunk starts before the last stage); other stages issue the 2 chunk
// loads anyway, out of range and into a sink, and every stage up to the last
// + 3 issues its 8 data loads (past the real K they read zeros into a slot
// nobody reads).  So every stage is exactly 10 loads and no branch splits the
// loop body.
__device__ __forceinline__ int scale_chunk_of(int t, int nk)
{
    if (t == 0) return 0;
    if ((t & 7) == 4 && t + 4 < nk) return (t + 4) >> 3;
    return -1;
}
constexpr int kLoadsPerStage = 10;

// (KB: bytes per row of the weight scales; ldxs: of the token scales.)
__device__ __forceinline__ void issue_chunk(int t, int nk, const v4i& wsr, const v4i& xsr, uint32_t KB,
                                            uint32_t ldxs, uint8_t* lds, int wave, int lane)
{
    const int c = scale_chunk_of(t, nk);
    const uint32_t real = lds_addr(lds + kDataBytes + (c & 1) * 2 * kChunkBytes + 64 * 16 * wave);
    const uint32_t sink = lds_addr(lds + kDataBytes + 2 * 2 * kChunkBytes + 1024 * wave);
    const uint32_t row = (uint32_t)(64 * wave + lane);
    dma16(wsr, c >= 0 ? real : sink, c >= 0 ? row * KB + (uint32_t)c * 16u : kOOB);
    dma16(xsr, c >= 0 ? real + kChunkBytes : sink, c >= 0 ? row * ldxs + (uint32_t)c * 16u : kOOB);
}

// Per-wave state of the data loads: the lane's offset of load i (rows
// 64*wave + 16*i .. +15, its swizzled 16-byte chunk) and the LDS address of
// the wave's first row in slot 0.
struct DataLoads {
    v4i wr, xr;
    uint32_t off[4];          // weight rows (stride K)
    uint32_t offx[4];         // token rows (stride ldx)
    uint32_t lds0;
    int nk;
};

// Data load k (0..7) of stage t: rows of load k/2 of A (k even) or B.
template <int KL>
__device__ __forceinline__ void issue_data(const DataLoads& d, int t)
{
    constexpr int i = KL >> 1, op = KL & 1;
    const uint32_t dst = d.lds0 + (uint32_t)(t & (kRing - 1)) * 2 * kTileBytes + op * kTileBytes + 16 * i * kBK;
    const uint32_t off = t < d.nk ? (op == 0 ? d.off[i] : d.offx[i]) + (uint32_t)t * kBK : kOOB;
    dma16(op == 0 ? d.wr : d.xr, dst, off);
}

__device__ __forceinline__ void issue_stage(int t, int nk, const v4i& wsr, const v4i& xsr, uint32_t KB,
                                            uint32_t ldxs, uint8_t* lds, int wave, int lane, const DataLoads& d)
{
    issue_chunk(t, nk, wsr, xsr, KB, ldxs, lds, wave, lane);
    issue_data<0>(d, t); issue_data<1>(d, t); issue_data<2>(d, t); issue_data<3>(d, t);
    issue_data<4>(d, t); issue_data<5>(d, t); issue_data<6>(d, t); issue_data<7>(d, t);
}

// Wait until at most N of this wave's buffer loads are outstanding and its LDS
// reads are done, then meet the other waves.  (No memory fence: a fence would
// also wait for the loads still meant to be in flight.)
template <int N>
__device__ __forceinline__ void stage_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Top of stage s: its loads (and all older ones) done; stages s+1 and s+2 may
// still be in flight.
__device__ __forceinline__ void stage_wait() { stage_barrier<2 * kLoadsPerStage>(); }

// One lane's MFMA operand: logical 16-byte chunks c0 and c1 of LDS row r.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int r, int c0, int c1)
{
    const uint4 lo = *reinterpret_cast<const uint4*>(tile + r * kBK + (swz(r, c0) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(tile + r * kBK + (swz(r, c1) << 4));
    v8i v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    return v;
}

// acc[tn][tm] += A-tile tn x B-tile tm for all 16 pairs.  Operands are E4M3
// (format code 0 for both); op_sel OPS picks the byte of sa[tn] / sb[tm] that
// holds the E8M0 scale of the lane's row and k-block.
template <int TN, int TM, int OPS>
__device__ __forceinline__ void mma_tiles(v16f (&acc)[4][4], const v8i (&a)[4], const v8i (&b)[4], const int (&sa)[4],
                                          const int (&sb)[4])
{
    acc[TN][TM] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[TN], b[TM], acc[TN][TM], 0, 0, OPS, sa[TN], OPS,
                                                                  sb[TM]);
    if constexpr (TM + 1 < 4) mma_tiles<TN, TM + 1, OPS>(acc, a, b, sa, sb);
    else if constexpr (TN + 1 < 4) mma_tiles<TN + 1, 0, OPS>(acc, a, b, sa, sb);
}

// Stage s = 2p + Q.  Lane (c32, hk) holds, of the 64 k of the stage, the bytes
// k = 16*hk .. +15 and 32 + 16*hk .. +15 (chunks hk and 2 + hk) of its row, and
// its scale byte covers the 32-k block hk: block 4p + 2Q + hk of the row, which
// is byte 2Q of the pair's scale word shifted right by 8*hk.
// MFMA I of the wave's 4 x 4 tiles, then (odd I) data load I/2 of stage t.
template <int Q, int I>
__device__ __forceinline__ void mma_step(v16f (&acc)[4][4], const v8i (&a)[4], const v8i (&b)[4], const int (&sa)[4],
                                         const int (&sb)[4], const DataLoads& d, int t)
{
    constexpr int tn = I >> 2, tm = I & 3;
    acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[tn], b[tm], acc[tn][tm], 0, 0, 2 * Q, sa[tn],
                                                                  2 * Q, sb[tm]);
    if constexpr (I % 2 == 1) issue_data<I / 2>(d, t);
    __builtin_amdgcn_sched_barrier(0);
}

template <int Q, int... Is>
__device__ __forceinline__ void mma_steps(v16f (&acc)[4][4], const v8i (&a)[4], const v8i (&b)[4], const int (&sa)[4],
                                          const int (&sb)[4], const DataLoads& d, int t, std::integer_sequence<int, Is...>)
{
    (mma_step<Q, Is>(acc, a, b, sa, sb, d, t), ...);
}

// Stage s = 2p + Q: read its operands from LDS, then issue its 16 MFMAs with
// the 8 data loads of stage t = s + 3 slotted one after every other MFMA (the
// loads' issue stalls then overlap the matrix core; measured 2 % faster than
// one after each of the first 8, and than all 8 before the MFMAs).
template <int Q>
__device__ __forceinline__ void mma_stage(v16f (&acc)[4][4], const uint8_t* lds, int s, int wn, int wm, int c32,
                                          int hk, const int (&sa)[4], const int (&sb)[4], const DataLoads& d, int t)
{
    const uint8_t* A = lds + (s & (kRing - 1)) * 2 * kTileBytes;
    const uint8_t* B = A + kTileBytes;
    v8i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = read_frag(A, 128 * wn + 32 * i + c32, hk, 2 + hk);
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = read_frag(B, 128 * wm + 32 * i + c32, hk, 2 + hk);
    __builtin_amdgcn_sched_barrier(0);
    mma_steps<Q>(acc, a, b, sa, sb, d, t, std::make_integer_sequence<int, 16>{});
}

// Scale words of the pair of stage s (s even) for the lane's four A and B
// tiles: word (s % 8) / 2 of each row's 16-byte chunk, shifted so that byte 2Q
// is the lane's k-block.
__device__ __forceinline__ void load_scales(int (&sa)[4], int (&sb)[4], const uint8_t* lds, int s, int wn, int wm,
                                            int c32, int hk)
{
    const uint8_t* sl = lds + kDataBytes + ((s >> 3) & 1) * 2 * kChunkBytes + ((s & 7) >> 1) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sa[i] = (int)(*reinterpret_cast<const uint32_t*>(sl + (128 * wn + 32 * i + c32) * 16) >> (8 * hk));
        sb[i] = (int)(*reinterpret_cast<const uint32_t*>(sl + kChunkBytes + (128 * wm + 32 * i + c32) * 16) >>
                      (8 * hk));
    }
}

__device__ __forceinline__ void zero_tile(void* y, int N, int r0, int r1, int n0, bool f32)
{
    const int ncols = N - n0 < kBN ? N - n0 : kBN;
    const int esz = f32 ? 4 : 2;
    const int per_row = ncols * esz / 16;        // 16-byte units per row (N % 8 == 0)
    const int total = (r1 - r0) * per_row;
    for (int i = threadIdx.x; i < total; i += kThreads) {
        const int r = r0 + i / per_row;
        const int u = i % per_row;
        uint8_t* p = static_cast<uint8_t*>(y) + ((int64_t)r * N + n0) * esz + u * 16;
        *reinterpret_cast<uint4*>(p) = make_uint4(0, 0, 0, 0);
    }
}

template <bool F32OUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mm_tile_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, uint32_t ldx, uint32_t ldxs,
                    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc, int N, int K, int G,
                    const int* __restrict__ ws, void* __restrict__ y)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];

    const int V = ws[0];
    const int q = (V + kXcds - 1) / kXcds;
    const int local = blockIdx.x / kXcds;
    const int L = (blockIdx.x % kXcds) * q + local;
    if (local >= q || L >= V) return;
    const Tile tl = reinterpret_cast<const Tile*>(ws + 4)[L];
    const int n0 = tl.c * kBN;
    if (tl.g == G) {                             // rows past the last end: zeros
        zero_tile(y, N, tl.r0, tl.r1, n0, F32OUT);
        return;
    }

    const uint32_t uK = (uint32_t)K;
    const uint32_t KB = uK / 32u;
    const int nrows_w = N - n0 < kBN ? N - n0 : kBN;
    const int nrows_x = tl.r1 - tl.r0;
    const size_t wrow0 = (size_t)tl.g * (size_t)N + (size_t)n0;
    const v4i wr = make_srd(wq + wrow0 * uK, (uint32_t)nrows_w * uK);
    const v4i xr = make_srd(xq + (size_t)tl.r0 * ldx, (uint32_t)nrows_x * ldx);
    const v4i wsr = make_srd(wsc + wrow0 * KB, (uint32_t)nrows_w * KB);
    const v4i xsr = make_srd(xs + (size_t)tl.r0 * ldxs, (uint32_t)nrows_x * ldxs);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wn = wave >> 1;                    // W rows (output columns) 128*wn ..
    const int wm = wave & 1;                     // X rows (tokens) 128*wm ..
    const int c32 = lane & 31;
    const int hk = lane >> 5;

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Pipeline: stages 0..2 in flight before the loop; the top of stage s
    // waits for stage s (loads complete in issue order, and the scale chunk of
    // s was issued with an earlier stage) and frees slot s-1 for stage s+3.
    const int nk = K / kBK;                      // even, >= 2
    DataLoads d;
    d.wr = wr;
    d.xr = xr;
    d.nk = nk;
    d.lds0 = lds_addr(lds + 64 * wave * kBK);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 64 * wave + 16 * i + (lane >> 2);
        d.off[i] = (uint32_t)row * uK + ((uint32_t)swz(row, lane & 3) << 4);
        d.offx[i] = (uint32_t)row * ldx + ((uint32_t)swz(row, lane & 3) << 4);
    }
    int sa[4], sb[4];
    issue_stage(0, nk, wsr, xsr, KB, ldxs, lds, wave, lane, d);
    issue_stage(1, nk, wsr, xsr, KB, ldxs, lds, wave, lane, d);
    issue_stage(2, nk, wsr, xsr, KB, ldxs, lds, wave, lane, d);
    for (int s = 0; s < nk; s += 2) {
        stage_wait();
        issue_chunk(s + 3, nk, wsr, xsr, KB, ldxs, lds, wave, lane);
        load_scales(sa, sb, lds, s, wn, wm, c32, hk);
        mma_stage<0>(acc, lds, s, wn, wm, c32, hk, sa, sb, d, s + 3);
        stage_wait();
        issue_chunk(s + 4, nk, wsr, xsr, KB, ldxs, lds, wave, lane);
        mma_stage<1>(acc, lds, s + 1, wn, wm, c32, hk, sa, sb, d, s + 4);
    }
    // the last three stages' loads read zeros into unused slots; let them land
    // before the workgroup's LDS goes away
    stage_barrier<0>();

    // epilogue: lane holds D[n][m] for m = c32 and n = 8*(e/4) + 4*hk + e%4
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        const int m = tl.r0 + 128 * wm + 32 * tm + c32;
        if (m >= tl.r1) continue;
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int n = n0 + 128 * wn + 32 * tn + 8 * qd + 4 * hk;
                if (n >= N) continue;
                const v16f& v = acc[tn][tm];
                if constexpr (F32OUT) {
                    float4 o = make_float4(v[4 * qd], v[4 * qd + 1], v[4 * qd + 2], v[4 * qd + 3]);
                    *reinterpret_cast<float4*>(static_cast<float*>(y) + (int64_t)m * N + n) = o;
                } else {
                    const v2bf16 lo = {(__bf16)v[4 * qd], (__bf16)v[4 * qd + 1]};
                    const v2bf16 hi = {(__bf16)v[4 * qd + 2], (__bf16)v[4 * qd + 3]};
                    uint2 o = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + (int64_t)m * N + n) = o;
                }
            }
        }
    }
}

}  // namespace

int grouped_mm_max_groups() { return kMaxGroups; }

bool grouped_mm_sizes_ok(int64_t M, int64_t N, int64_t K, int64_t G)
{
    if (M < 0 || N < 0 || K < 0 || G < 1 || G > kMaxGroups) return false;
    if (K % kKStep != 0 || N % 8 != 0) return false;
    // K <= 2^23 keeps a tile's 256 rows of K bytes within a 32-bit buffer resource
    if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31) || K > ((int64_t)1 << 23)) return false;
    const int64_t nc = (N + kBN - 1) / kBN;
    // tile list and grid stay within int32, as does every tile row offset
    if (mm_slots(M, G) * (nc ? nc : 1) >= ((int64_t)1 << 30)) return false;
    return true;
}

size_t grouped_mm_workspace_bytes(int64_t M, int64_t N, int32_t G)
{
    const int64_t nc = (N + kBN - 1) / kBN;
    return (size_t)16 + (size_t)mm_slots(M, G) * (size_t)nc * sizeof(Tile);
}

hipError_t launch_grouped_mm(const void* xq, const void* xs, const void* wq, const void* wsc,
                             const int32_t* offs, int M, int N, int K, int G, void* y, bool f32_out,
                             void* workspace, hipStream_t stream)
{
    return launch_grouped_mm_strided(xq, xs, (uint32_t)K, (uint32_t)K / 32u, wq, wsc, offs, M, N, K, G, y, f32_out,
                                     workspace, stream);
}

hipError_t launch_grouped_mm_strided(const void* xq, const void* xs, uint32_t ldx, uint32_t ldxs, const void* wq,
                                     const void* wsc, const int32_t* offs, int M, int N, int K, int G, void* y,
                                     bool f32_out, void* workspace, hipStream_t stream)
{
    const int NC = (N + kBN - 1) / kBN;
    int* ws = static_cast<int*>(workspace);
    hipLaunchKernelGGL(mm_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, offs, G, M, NC, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t grid = (mm_slots(M, G) * NC + kXcds - 1) / kXcds * kXcds;
    if (f32_out)
        hipLaunchKernelGGL(mm_tile_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           static_cast<const uint8_t*>(xq), static_cast<const uint8_t*>(xs), ldx, ldxs,
                           static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(wsc), N, K, G, ws, y);
    else
        hipLaunchKernelGGL(mm_tile_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           static_cast<const uint8_t*>(xq), static_cast<const uint8_t*>(xs), ldx, ldxs,
                           static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(wsc), N, K, G, ws, y);
    return hipGetLastError();
}

}  // namespace mxq
