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
//   K advances 128 bytes per stage through a double-buffered LDS (2 x 66 KB):
//   the W_g and X tiles (256 rows x 128 B each; 16-byte chunks XOR-swizzled by
//   row so that fragment reads and tile writes are free of bank conflicts) and
//   their E8M0 scales (transposed so that one 32-bit LDS read gives a lane the
//   scale bytes of its four 32-row MFMA tiles; the instruction's op_sel picks
//   the byte).  Global loads are raw buffer loads whose resource ends at the
//   tile's last valid row: rows past a group's end or past N read as zero, with
//   no per-row branch.  One barrier per stage: the loads of stage s+1 are in
//   flight while the MFMAs of stage s run.  MFMA operand A is W_g (output
//   columns), B is X (token rows), so each lane ends up holding runs of four
//   consecutive output columns of one row and stores them as one 8-byte
//   (bf16) or 16-byte (fp32) write.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.hpp"
#include "internal.hpp"

namespace mxq {
namespace {

constexpr int kBM = 256;        // token rows per tile
constexpr int kBN = 256;        // output columns per tile
constexpr int kBK = 128;        // K bytes per LDS stage
constexpr int kThreads = 256;
constexpr int kCB = 4;          // column tiles per block of the tile order
constexpr int kXcds = 8;
constexpr int kPlanThreads = 1024;

constexpr int kTileBytes = kBM * kBK;                   // 32 KB of codes per operand
constexpr int kScaleBytes = (kBK / 32) * kBM;           // 1 KB of scales per operand
constexpr int kStageBytes = 2 * kTileBytes + 2 * kScaleBytes;
static_assert(kBM == kBN, "one row count serves both operand tiles");

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

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
// Physical 16-byte chunk of logical chunk c in LDS row r (rows of 128 bytes).
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

// Byte offset, in a stage's scale area, of the scale of tile row r for k-block kb:
// rows 128*h + 32*i + c (i = 0..3) of one k-block sit in one 32-bit word.
__device__ __forceinline__ int scale_slot(int r, int kb)
{
    return kb * kBM + (r >> 7) * 128 + (r & 31) * 4 + ((r >> 5) & 3);
}

struct StageRegs {
    uint4 a[8];                  // W_g codes
    uint4 b[8];                  // X codes
    uint32_t sa, sb;             // 4 scale bytes of one W_g row and one X row
};

__device__ __forceinline__ void load_stage(StageRegs& s, Rsrc wr, Rsrc xr, Rsrc wsr, Rsrc xsr, uint32_t K, int k0)
{
    const int t = threadIdx.x;
    const uint32_t chunk = (uint32_t)(t & 7) * 16u + (uint32_t)k0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const uint32_t row = (uint32_t)((t >> 3) + 32 * p);
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, row * K + chunk, 0, 0);
        s.a[p] = make_uint4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const uint32_t row = (uint32_t)((t >> 3) + 32 * p);
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xr, row * K + chunk, 0, 0);
        s.b[p] = make_uint4(v.x, v.y, v.z, v.w);
    }
    const uint32_t soff = (uint32_t)t * (K / 32u) + (uint32_t)(k0 / 32);
    s.sa = __builtin_amdgcn_raw_buffer_load_b32(wsr, soff, 0, 0);
    s.sb = __builtin_amdgcn_raw_buffer_load_b32(xsr, soff, 0, 0);
}

__device__ __forceinline__ void store_stage(const StageRegs& s, uint8_t* stage)
{
    const int t = threadIdx.x;
    uint8_t* A = stage;
    uint8_t* B = stage + kTileBytes;
    uint8_t* SA = stage + 2 * kTileBytes;
    uint8_t* SB = SA + kScaleBytes;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int row = (t >> 3) + 32 * p;
        const int off = row * kBK + (swz(row, t & 7) << 4);
        *reinterpret_cast<uint4*>(A + off) = s.a[p];
        *reinterpret_cast<uint4*>(B + off) = s.b[p];
    }
#pragma unroll
    for (int kb = 0; kb < kBK / 32; ++kb) {
        SA[scale_slot(t, kb)] = (uint8_t)(s.sa >> (8 * kb));
        SB[scale_slot(t, kb)] = (uint8_t)(s.sb >> (8 * kb));
    }
}

// One lane's MFMA operand: logical 16-byte chunks c0 and c1 of LDS row r.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int r, int c0, int c1)
{
    const uint4 lo = *reinterpret_cast<const uint4*>(tile + r * kBK + (swz(r, c0) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(tile + r * kBK + (swz(r, c1) << 4));
    v8i v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    return v;
}

// acc[tn][tm] += A-tile tn x B-tile tm for all 16 pairs.  Operands are E4M3
// (format code 0 for both); op_sel picks byte tn of sa and byte tm of sb, the
// E8M0 scales of the lane's row in those tiles.
template <int TN, int TM>
__device__ __forceinline__ void mma_tiles(v16f (&acc)[4][4], const v8i (&a)[4], const v8i (&b)[4], int sa, int sb)
{
    acc[TN][TM] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[TN], b[TM], acc[TN][TM], 0, 0, TN, sa, TM, sb);
    if constexpr (TM + 1 < 4) mma_tiles<TN, TM + 1>(acc, a, b, sa, sb);
    else if constexpr (TN + 1 < 4) mma_tiles<TN + 1, 0>(acc, a, b, sa, sb);
}

// All MFMAs of one LDS stage: two 64-byte k-steps of the wave's 4 x 4 tiles.
__device__ __forceinline__ void mma_stage(v16f (&acc)[4][4], const uint8_t* stage, int wn, int wm, int c32, int hk)
{
    const uint8_t* A = stage;
    const uint8_t* B = stage + kTileBytes;
    const uint8_t* SA = stage + 2 * kTileBytes;
    const uint8_t* SB = SA + kScaleBytes;
#pragma unroll
    for (int j = 0; j < kBK / 64; ++j) {
        const int kb = 2 * j + hk;
        const int sa = *reinterpret_cast<const int*>(SA + kb * kBM + wn * 128 + c32 * 4);
        const int sb = *reinterpret_cast<const int*>(SB + kb * kBM + wm * 128 + c32 * 4);
        // operand bytes of lane (c32, hk) in the 64-byte k-step j: k = 16*hk .. +15
        // and 32 + 16*hk .. +15, i.e. chunks 4j + hk and 4j + 2 + hk; its scale
        // byte covers the 32-k block hk of the step (block 2j + hk of the stage)
        v8i a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = read_frag(A, 128 * wn + 32 * i + c32, 4 * j + hk, 4 * j + 2 + hk);
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = read_frag(B, 128 * wm + 32 * i + c32, 4 * j + hk, 4 * j + 2 + hk);
        mma_tiles<0, 0>(acc, a, b, sa, sb);
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
void mm_tile_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ wsc, int N, int K, int G,
                    const int* __restrict__ ws, void* __restrict__ y)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];

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
    const Rsrc wr = make_rsrc(wq + wrow0 * uK, (uint32_t)nrows_w * uK);
    const Rsrc xr = make_rsrc(xq + (size_t)tl.r0 * uK, (uint32_t)nrows_x * uK);
    const Rsrc wsr = make_rsrc(wsc + wrow0 * KB, (uint32_t)nrows_w * KB);
    const Rsrc xsr = make_rsrc(xs + (size_t)tl.r0 * KB, (uint32_t)nrows_x * KB);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wn = wave >> 1;                    // W rows (output columns) 128*wn ..
    const int wm = wave & 1;                     // X rows (tokens) 128*wm ..
    const int c32 = lane & 31;
    const int hk = lane >> 5;                    // which 32-byte half of a 64-byte k-step

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int nk = K / kBK;
    StageRegs regs;
    load_stage(regs, wr, xr, wsr, xsr, uK, 0);
    store_stage(regs, lds);
    __syncthreads();

    // every stage but the last: prefetch the next stage while this one multiplies
    for (int kt = 0; kt + 1 < nk; ++kt) {
        // issue order: next stage's global loads, this stage's MFMAs, then the
        // LDS writes (which wait for those loads) -- the loads land while the
        // matrix core is busy.  The scheduling barriers keep that order.
        load_stage(regs, wr, xr, wsr, xsr, uK, (kt + 1) * kBK);
        __builtin_amdgcn_sched_barrier(0);
        mma_stage(acc, lds + (kt & 1) * kStageBytes, wn, wm, c32, hk);
        __builtin_amdgcn_sched_barrier(0);
        store_stage(regs, lds + ((kt + 1) & 1) * kStageBytes);
        __syncthreads();
    }
    mma_stage(acc, lds + ((nk - 1) & 1) * kStageBytes, wn, wm, c32, hk);

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
    if (K % kBK != 0 || N % 8 != 0) return false;
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
    const int NC = (N + kBN - 1) / kBN;
    int* ws = static_cast<int*>(workspace);
    hipLaunchKernelGGL(mm_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, offs, G, M, NC, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t grid = (mm_slots(M, G) * NC + kXcds - 1) / kXcds * kXcds;
    if (f32_out)
        hipLaunchKernelGGL(mm_tile_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           static_cast<const uint8_t*>(xq), static_cast<const uint8_t*>(xs),
                           static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(wsc), N, K, G, ws, y);
    else
        hipLaunchKernelGGL(mm_tile_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           static_cast<const uint8_t*>(xq), static_cast<const uint8_t*>(xs),
                           static_cast<const uint8_t*>(wq), static_cast<const uint8_t*>(wsc), N, K, G, ws, y);
    return hipGetLastError();
}

}  // namespace mxq
