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
//   Output tiles are up to 256 token rows x 256 columns.  Row tiles never
//   straddle a group: group g's rows [start, end) are cut into ceil(len/256)
//   tiles from its start, so a tile reads one W_g; the last one runs at the
//   smallest height of 64, 128, 192 or 256 rows that holds its rows.  Rows past the last end form one more
//   pseudo-group whose tiles are written with zeros.  A one-workgroup plan
//   kernel turns the device-resident end offsets into this tile list (no host
//   copy), ordered group by group, and inside a group in blocks of kCB column
//   tiles with the row tiles of a block consecutive -- so consecutively
//   numbered tiles share W_g column blocks and X row tiles.  Workgroup b runs
//   list entry (b % 8) * q + b / 8 (q = ceil(count / 8)): the hardware deals
//   workgroups to the 8 XCDs round-robin, so each XCD walks one contiguous
//   stretch of the list and its L2 sees the reuse.
//
// Tile kernel (256 threads = 4 waves; for 256-row tiles in 2 x 2, each wave
// 128 x 128)
//   K advances 128 bytes (two MFMA k-steps) per pair through a 2-slot LDS ring
//   of W_g and X tiles (up to 256 rows x 128 B each; 16-byte chunks XOR-swizzled
//   by row so that the operand reads are free of bank conflicts), filled
//   straight from global memory by buffer-load-to-LDS in whole 128-byte lines.
//   Each pair waits for its loads, and per k-step reads the wave's operands into
//   VGPRs and issues its MFMAs, with the next pair's loads slotted between the
//   first k-step's MFMAs; the loop body is four pairs, one period of the
//   scale-chunk loads.  Global loads use
//   raw buffer resources that end at the tile's last valid row: rows past a
//   group's end or past N read as zero, with no per-row branch.  MFMA operand
//   A is W_g (output columns), B is X (token rows), so each lane ends up holding
//   runs of four consecutive output columns of one row and stores them as one
//   8-byte (bf16) or 16-byte (fp32) write.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>
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
// K advances 128 bytes per step (a "pair" of MFMA k-steps of 64) through a
// 2-slot LDS ring filled by buffer-load-to-LDS (the data never passes through
// VGPRs): each load instruction brings 8 rows x 128 bytes, whole 128-byte
// lines, and the loads of pair q + 1 go out while pair q is multiplied.  A
// 4-slot ring of single k-steps (three in flight, each load 16 rows x 64
// bytes: half lines) kept more bytes in flight, but its loads alone ran 684 us
// at the MoE configuration against 565 us for the same bytes in whole lines.
// Scales travel in chunks of 16 bytes per row (16 k-blocks = 4 pairs) into a
// 2-slot ring.
constexpr int kPairK = 128;                             // K bytes per ring slot
constexpr int kSlotBytes = kBM * kPairK;                // 32 KB of codes per operand per slot
constexpr int kChunkBytes = kBM * 16;                   // 4 KB of scales per operand per chunk
constexpr int kDataBytes = 2 * 2 * kSlotBytes;          // 128 KB: 2 slots x 2 operands
constexpr int kDummyBytes = 4 * 1024;                   // sink for loads that carry nothing
constexpr int kLdsBytes = kDataBytes + 2 * 2 * kChunkBytes + kDummyBytes;   // + 16 KB + 4 KB
static_assert(kBK == 64 && kPairK == 2 * kBK && 4 * kPairK == 512, "a scale chunk is 16 k-blocks of 32 = 4 pairs");

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
// VGPR result; its completion is counted by vmcnt, which the pair barrier waits
// on explicitly.  Written in asm so that the compiler does not add a
// conservative wait for it before every later LDS read.  (M0 is reserved by the
// compiler and set before each of its own uses; nothing else here reads it.)
// The whole offset is the lane's (VGPR) offset, which the range check covers.
__device__ __forceinline__ void dma16(const v4i& srd, uint32_t lds, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(srd)
                 : "memory");
}

// Physical 16-byte chunk of logical chunk c (0..7) in LDS row r (rows of 128
// bytes).  A 128-bit wave read serves 16 lanes at a time; the fragment reads'
// 16 lanes take 16 consecutive rows at one logical chunk, and with this swizzle
// they hit 16 different 16-byte bank groups (rows 2j and 2j + 1 share a chunk
// index but sit in different halves of a 256-byte bank window).
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// Scale chunks: pair 0 carries chunk 0 and pair 4c + 2 chunk c + 1 (out of
// range into a sink if that chunk does not exist).
__device__ __forceinline__ int scale_chunk_of(int p, int np)
{
    if (p == 0) return 0;
    if ((p & 3) == 2 && p + 2 < np) return (p + 2) >> 2;
    return -1;
}

// (KB: bytes per row of the weight scales; ldxs: of the token scales.)
__device__ __forceinline__ void issue_chunk(int p, int np, const v4i& wsr, const v4i& xsr, uint32_t KB,
                                            uint32_t ldxs, uint8_t* lds, int wave, int lane)
{
    const int c = scale_chunk_of(p, np);
    const uint32_t real = lds_addr(lds + kDataBytes + (c & 1) * 2 * kChunkBytes + 64 * 16 * wave);
    const uint32_t sink = lds_addr(lds + kDataBytes + 2 * 2 * kChunkBytes + 1024 * wave);
    const uint32_t row = (uint32_t)(64 * wave + lane);
    dma16(wsr, c >= 0 ? real : sink, c >= 0 ? row * KB + (uint32_t)c * 16u : kOOB);
    dma16(xsr, c >= 0 ? real + kChunkBytes : sink, c >= 0 ? row * ldxs + (uint32_t)c * 16u : kOOB);
}

// The wave layout of a tile of BM token rows x 256 output columns.  A group's
// rows are cut into 256-row tiles from its start, and its last tile takes the
// smallest height of 64, 128, 192 and 256 that holds its rows, so that a short
// tile does less MFMA work and fewer loads instead of padding to 256 rows with
// zeros.  256 and 192 rows: 4 waves in 2 x 2, each 128 W rows x 128 (96)
// token rows, 4 x 4 (4 x 3) MFMA tiles.  128 and 64 rows: 4 waves side by side
// over the columns, each 64 W rows x 128 (64) token rows, 2 x 4 (2 x 2).
template <int BM>
struct MmShape {
    static_assert(BM == 256 || BM == 192 || BM == 128 || BM == 64, "64- to 256-row tiles");
    static constexpr bool kSquare = BM >= 192;         // 2 x 2 waves (else 4 x 1)
    static constexpr int TN = kSquare ? 4 : 2;         // 32-row W tiles per wave
    static constexpr int TM = kSquare ? BM / 64 : BM / 32;   // 32-row token tiles per wave
    static constexpr int XL = BM / 32;                 // token-row loads (8 rows each) per wave and pair
    static constexpr int NL = 8 + XL;                  // data loads per wave and pair (W: 64 rows, 8)
    static constexpr int NM = TN * TM;                 // MFMAs per wave and k-step
    __device__ static int wn(int wave) { return kSquare ? wave >> 1 : wave; }
    __device__ static int wm(int wave) { return kSquare ? wave & 1 : 0; }
};

// Per-wave state of the data loads.  Load i of an operand covers rows
// base + 8 i .. + 7 (base: 64 wave for W, (BM/4) wave for X), 128 bytes each:
// lane l takes row base + 8 i + l/8 and physical chunk l % 8, whose logical
// chunk depends on the row only through i % 2 (base is a multiple of 16), so
// two lane offsets per operand serve all its loads.
struct DataLoads {
    v4i wr, xr;
    uint32_t offw[2], offx[2];    // lane offsets of the even and odd loads
    uint32_t sw, sx;              // row strides (bytes) of W and X
    uint32_t ldsw, ldsx;          // LDS address of the wave's first W and X rows in slot 0
    int np;
};

// Data load KL of pair p: W and X loads alternate while both last (W0 X0 W1
// X1 ...), then the remaining W loads.
template <int XL, int KL>
__device__ __forceinline__ void issue_data(const DataLoads& d, int p)
{
    constexpr bool alt = KL < 2 * XL;
    constexpr int op = alt ? (KL & 1) : 0;
    constexpr int i = alt ? (KL >> 1) : KL - XL;
    const uint32_t dst = (op == 0 ? d.ldsw : d.ldsx) + (uint32_t)(p & 1) * 2 * kSlotBytes + 8 * i * kPairK;
    const uint32_t off = p < d.np ? (op == 0 ? d.offw[i & 1] : d.offx[i & 1]) + (uint32_t)(8 * i) * (op == 0 ? d.sw : d.sx) +
                                        (uint32_t)p * kPairK
                                  : kOOB;
    dma16(op == 0 ? d.wr : d.xr, dst, off);
}

template <int XL, int... KL>
__device__ __forceinline__ void issue_data_all(const DataLoads& d, int p, std::integer_sequence<int, KL...>)
{
    (issue_data<XL, KL>(d, p), ...);
}

// Wait until at most N of this wave's buffer loads are outstanding and its LDS
// reads are done, then meet the other waves.  (No memory fence: a fence would
// also wait for the loads still meant to be in flight.)
template <int N>
__device__ __forceinline__ void pair_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One lane's MFMA operand: logical 16-byte chunks c0 and c1 of LDS row r.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int r, int c0, int c1)
{
    const uint4 lo = *reinterpret_cast<const uint4*>(tile + r * kPairK + (swz(r, c0) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(tile + r * kPairK + (swz(r, c1) << 4));
    v8i v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    return v;
}

// MFMA I of the wave's TN x TM tiles in k-step H (0, 1) of a pair, then (in
// the first k-step) the data loads of the next pair that fall after it.  Lane
// (c32, hk) holds, of the 64 k of the step, the bytes k = 16*hk .. +15 and
// 32 + 16*hk .. +15 (logical chunks 4H + hk and 4H + 2 + hk of the pair) of its
// row, and its scale byte covers the 32-k block hk of the step: block
// 4p + 2H + hk of the row, which is byte 2H of the pair's scale word shifted
// right by 8*hk.  Load j goes after MFMA (2j + 1) NM / (2 NL) (rounded down).
template <int BM, int J>
__device__ __forceinline__ constexpr int load_slot()
{
    return (2 * J + 1) * MmShape<BM>::NM / (2 * MmShape<BM>::NL);
}

template <int BM, int I, int J>
__device__ __forceinline__ void loads_after(const DataLoads& d, int p)
{
    if constexpr (J < MmShape<BM>::NL) {
        if constexpr (load_slot<BM, J>() == I) issue_data<MmShape<BM>::XL, J>(d, p);
        loads_after<BM, I, J + 1>(d, p);
    }
}

template <int BM, int H, int I>
__device__ __forceinline__ void mma_step(v16f (&acc)[MmShape<BM>::TN][MmShape<BM>::TM],
                                         const v8i (&a)[MmShape<BM>::TN], const v8i (&b)[MmShape<BM>::TM],
                                         const int (&sa)[MmShape<BM>::TN], const int (&sb)[MmShape<BM>::TM],
                                         const DataLoads& d, int p)
{
    constexpr int tn = I / MmShape<BM>::TM, tm = I % MmShape<BM>::TM;
    acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[tn], b[tm], acc[tn][tm], 0, 0, 2 * H, sa[tn],
                                                                  2 * H, sb[tm]);
    if constexpr (H == 0) loads_after<BM, I, 0>(d, p);
    __builtin_amdgcn_sched_barrier(0);
}

template <int BM, int H, int... Is>
__device__ __forceinline__ void mma_steps(v16f (&acc)[MmShape<BM>::TN][MmShape<BM>::TM],
                                          const v8i (&a)[MmShape<BM>::TN], const v8i (&b)[MmShape<BM>::TM],
                                          const int (&sa)[MmShape<BM>::TN], const int (&sb)[MmShape<BM>::TM],
                                          const DataLoads& d, int p, std::integer_sequence<int, Is...>)
{
    (mma_step<BM, H, Is>(acc, a, b, sa, sb, d, p), ...);
}

// K-step H of pair q: read its operands from ring slot q % 2 (the wave's W
// rows from wrow, its token rows from xrow), then issue its MFMAs; in the first
// step, the data loads of pair p = q + 1 are slotted between them.
template <int BM, int H>
__device__ __forceinline__ void mma_kstep(v16f (&acc)[MmShape<BM>::TN][MmShape<BM>::TM], const uint8_t* lds, int q,
                                          int wrow, int xrow, int c32, int hk, const int (&sa)[MmShape<BM>::TN],
                                          const int (&sb)[MmShape<BM>::TM], const DataLoads& d, int p)
{
    using S = MmShape<BM>;
    const uint8_t* A = lds + (q & 1) * 2 * kSlotBytes;
    const uint8_t* B = A + kSlotBytes;
    v8i a[S::TN], b[S::TM];
#pragma unroll
    for (int i = 0; i < S::TN; ++i) a[i] = read_frag(A, wrow + 32 * i + c32, 4 * H + hk, 4 * H + 2 + hk);
#pragma unroll
    for (int i = 0; i < S::TM; ++i) b[i] = read_frag(B, xrow + 32 * i + c32, 4 * H + hk, 4 * H + 2 + hk);
    __builtin_amdgcn_sched_barrier(0);
    mma_steps<BM, H>(acc, a, b, sa, sb, d, p, std::make_integer_sequence<int, S::NM>{});
}

// Scale words of pair q for the lane's W and token tiles: word q % 4 of each
// row's 16-byte chunk, shifted so that byte 2H is the lane's k-block.
template <int BM>
__device__ __forceinline__ void load_scales(int (&sa)[MmShape<BM>::TN], int (&sb)[MmShape<BM>::TM], const uint8_t* lds,
                                            int q, int wrow, int xrow, int c32, int hk)
{
    const uint8_t* sl = lds + kDataBytes + ((q >> 2) & 1) * 2 * kChunkBytes + (q & 3) * 4;
#pragma unroll
    for (int i = 0; i < MmShape<BM>::TN; ++i)
        sa[i] = (int)(*reinterpret_cast<const uint32_t*>(sl + (wrow + 32 * i + c32) * 16) >> (8 * hk));
#pragma unroll
    for (int i = 0; i < MmShape<BM>::TM; ++i)
        sb[i] = (int)(*reinterpret_cast<const uint32_t*>(sl + kChunkBytes + (xrow + 32 * i + c32) * 16) >> (8 * hk));
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

// The K loop and the epilogue of one tile of BM token rows (rows [r0, r1) of
// group g's operand, at most BM of them) x 256 columns from n0.
template <int BM, bool F32OUT>
__device__ __forceinline__ void tile_product(uint8_t* lds, const v4i& wr, const v4i& xr, const v4i& wsr, const v4i& xsr,
                                             uint32_t uK, uint32_t ldx, uint32_t KB, uint32_t ldxs, int N, int K,
                                             int r0, int r1, int n0, void* __restrict__ y)
{
    using S = MmShape<BM>;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wrow = 32 * S::TN * S::wn(wave);   // the wave's first W row (output column) of the tile
    const int xrow = 32 * S::TM * S::wm(wave);   // its first token row
    const int c32 = lane & 31;
    const int hk = lane >> 5;

    v16f acc[S::TN][S::TM];
#pragma unroll
    for (int i = 0; i < S::TN; ++i)
#pragma unroll
        for (int j = 0; j < S::TM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Pipeline: pair 0 is loaded before the loop; the top of pair q waits for
    // every load issued so far (pair q's, and the scale chunk it needs, issued
    // with an earlier pair) and meets the other waves, whose reads of slot
    // (q + 1) % 2 ended with pair q - 1; pair q + 1's loads then go out.
    const int np = K / kPairK;                   // >= 1
    DataLoads d;
    d.wr = wr;
    d.xr = xr;
    d.np = np;
    d.sw = uK;
    d.sx = ldx;
    d.ldsw = lds_addr(lds + 64 * wave * kPairK);
    d.ldsx = lds_addr(lds + kSlotBytes + (BM / 4) * wave * kPairK);
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int pc = lane & 7;                                   // physical chunk
        const int lc = pc ^ ((4 * par + (lane >> 4)) & 7);         // its logical chunk in rows of load parity par
        d.offw[par] = (uint32_t)(64 * wave + (lane >> 3)) * uK + ((uint32_t)lc << 4);
        d.offx[par] = (uint32_t)((BM / 4) * wave + (lane >> 3)) * ldx + ((uint32_t)lc << 4);
    }
    int sa[S::TN], sb[S::TM];
    issue_chunk(0, np, wsr, xsr, KB, ldxs, lds, wave, lane);
    issue_data_all<S::XL>(d, 0, std::make_integer_sequence<int, S::NL>{});
    // Four pairs per iteration, so that which of them fetches a scale chunk
    // (the second, for pair q + 2) is known at compile time: a branch inside
    // the loop body lets the compiler move MFMAs past a barrier.  The pairs of
    // the last partial group of four fetch no chunk (there is none after theirs).
    auto pair = [&](int q, auto chunk) {
        pair_barrier<0>();
        if constexpr (decltype(chunk)::value) issue_chunk(q + 1, np, wsr, xsr, KB, ldxs, lds, wave, lane);
        load_scales<BM>(sa, sb, lds, q, wrow, xrow, c32, hk);
        mma_kstep<BM, 0>(acc, lds, q, wrow, xrow, c32, hk, sa, sb, d, q + 1);
        mma_kstep<BM, 1>(acc, lds, q, wrow, xrow, c32, hk, sa, sb, d, q + 1);
    };
    int q = 0;
    for (; q + 4 <= np; q += 4) {
        pair(q, std::false_type{});
        pair(q + 1, std::true_type{});
        pair(q + 2, std::false_type{});
        pair(q + 3, std::false_type{});
    }
    for (; q < np; ++q) pair(q, std::false_type{});
    // the last pair's loads read zeros into the unused slot; let them land
    // before the workgroup's LDS goes away
    pair_barrier<0>();

    // epilogue: lane holds D[n][m] for m = c32 and n = 8*(e/4) + 4*hk + e%4
    if constexpr (F32OUT) {
        // fp32 (256 KB per 256-row tile, more than the LDS): 16-byte stores straight from the accumulators
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm) {
            const int m = r0 + xrow + 32 * tm + c32;
            if (m >= r1) continue;
#pragma unroll
            for (int tn = 0; tn < S::TN; ++tn) {
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int n = n0 + wrow + 32 * tn + 8 * qd + 4 * hk;
                    if (n >= N) continue;
                    const v16f& v = acc[tn][tm];
                    float4 o = make_float4(v[4 * qd], v[4 * qd + 1], v[4 * qd + 2], v[4 * qd + 3]);
                    *reinterpret_cast<float4*>(static_cast<float*>(y) + (int64_t)m * N + n) = o;
                }
            }
        }
    } else {
        // bf16: the BM x 256 tile (up to 128 KB) goes through the LDS ring, free
        // now, so that each lane stores 16 contiguous bytes and a wave writes
        // two whole 512-byte row segments per instruction (straight from the
        // accumulators, each store instruction touched 32 rows).  A row is 32
        // 16-byte units, XOR-swizzled by the row so that the 8-byte writes of a
        // wave's 32 rows spread over the banks.
        constexpr int kRowBytes = kBN * 2;
        const auto unit_of = [](int m, int u) { return (u ^ m) & 31; };
#pragma unroll
        for (int tm = 0; tm < S::TM; ++tm) {
            const int m = xrow + 32 * tm + c32;
#pragma unroll
            for (int tn = 0; tn < S::TN; ++tn) {
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int u = (wrow + 32 * tn + 8 * qd) / 8;     // 16-byte unit of the row
                    const v16f& v = acc[tn][tm];
                    const v2bf16 lo = {(__bf16)v[4 * qd], (__bf16)v[4 * qd + 1]};
                    const v2bf16 hi = {(__bf16)v[4 * qd + 2], (__bf16)v[4 * qd + 3]};
                    *reinterpret_cast<uint2*>(lds + m * kRowBytes + unit_of(m, u) * 16 + 8 * hk) =
                        make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
                }
            }
        }
        __syncthreads();
        const int nrows = r1 - r0;
        const int u = (int)threadIdx.x & 31;
        const bool col_ok = n0 + 8 * u < N;
#pragma unroll 4
        for (int m = (int)threadIdx.x >> 5; m < BM; m += kThreads / 32) {
            if (m >= nrows || !col_ok) continue;
            const uint4 val = *reinterpret_cast<const uint4*>(lds + m * kRowBytes + unit_of(m, u) * 16);
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + (int64_t)(r0 + m) * N + n0 + 8 * u) = val;
        }
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
    // (uniform per workgroup, outside the K loop)
    if (nrows_x <= 64)
        tile_product<64, F32OUT>(lds, wr, xr, wsr, xsr, uK, ldx, KB, ldxs, N, K, tl.r0, tl.r1, n0, y);
    else if (nrows_x <= 128)
        tile_product<128, F32OUT>(lds, wr, xr, wsr, xsr, uK, ldx, KB, ldxs, N, K, tl.r0, tl.r1, n0, y);
    else if (nrows_x <= 192)
        tile_product<192, F32OUT>(lds, wr, xr, wsr, xsr, uK, ldx, KB, ldxs, N, K, tl.r0, tl.r1, n0, y);
    else
        tile_product<256, F32OUT>(lds, wr, xr, wsr, xsr, uK, ldx, KB, ldxs, N, K, tl.r0, tl.r1, n0, y);
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
