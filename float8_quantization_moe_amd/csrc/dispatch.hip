// dispatch.hip -- the order of the dispatch pack: token-slot pairs sorted by
// expert, stably, on the device (no host synchronisation).
//
// "[mxfp8 MoE training] Support mxfp8 all to all in expert parallel", Summary:
// the all-to-all payload is the MXFP8 encoding of the routed tokens.  Pairs
// p = t*topk + j with expert ids[p] in [0, E) are placed at
//   row(p) = start(e) + #{p' < p : ids[p'] == e},
// a stable counting sort in three passes over 256-pair blocks:
//   count  per-block histograms (LDS atomics) -> bcount[b][e];
//   scan   one workgroup turns them into each block's first row per expert
//          (column prefix sums over blocks, then the experts' starts) and
//          writes the cumulative end offsets group_end[e];
//   place  each pair's rank among the earlier pairs of its block with the same
//          expert gives its row: inside a wave, the lanes holding the same id
//          (one ballot per id bit) below the lane; across waves, per-wave
//          counts in LDS.
// For small count tables the scan is folded into the place pass (every place
// workgroup derives its block's first rows from the whole table), which saves
// the one-workgroup launch.
// The rows themselves (gather + MX quantize + pack) are written by
// mx_dispatch_pack_kernel in mx_codec.hip.
#include "device_common.hpp"
#include "internal.hpp"

namespace mxq {

constexpr int kDpThreads = 256;          // pairs per block
constexpr int kDpScanThreads = 1024;
constexpr int kDpMaxExperts = 1024;
constexpr int kDpWaves = kDpThreads / 64;

// Rank of this lane's pair among the earlier pairs of its workgroup with the
// same expert id e (e < 0: none, rank unused).  wcnt is LDS of kDpWaves x E
// ints; every thread of the workgroup must call this (it has barriers).
// Inside a wave the lanes with the same id are found with one ballot per bit
// of the id (ids are below 2^nbits) and counted below the lane with mbcnt; the
// lowest lane of each id publishes the wave's count of that id, and the ranks
// add the counts of the earlier waves.
__device__ __forceinline__ int rank_in_block(int e, int E, int nbits, int* wcnt)
{
    const int tid = (int)threadIdx.x, wave = tid >> 6;
    for (int i = tid; i < kDpWaves * E; i += kDpThreads) wcnt[i] = 0;
    unsigned long long m = __ballot(e >= 0);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = ((e >> b) & 1) != 0;
        const unsigned long long bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    __syncthreads();
    if (e >= 0 && below == 0) wcnt[wave * E + e] = __builtin_popcountll(m);
    __syncthreads();
    int rank = below;
    for (int w = 0; w < wave; ++w) rank += e >= 0 ? wcnt[w * E + e] : 0;
    return rank;
}

__host__ __device__ inline int id_bits(int E)
{
    int n = 0;
    while ((1 << n) < E) ++n;          // ids 0 .. E-1 fit in n bits
    return n;
}

__global__ __launch_bounds__(kDpThreads)
void dp_count_kernel(const int32_t* __restrict__ ids, int64_t P, int E, int32_t* __restrict__ bcount)
{
    __shared__ int hist[kDpMaxExperts];
    for (int e = (int)threadIdx.x; e < E; e += kDpThreads) hist[e] = 0;
    __syncthreads();
    const int64_t p = (int64_t)blockIdx.x * kDpThreads + threadIdx.x;
    if (p < P) {
        const int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = (int)threadIdx.x; e < E; e += kDpThreads) bcount[(int64_t)blockIdx.x * E + e] = hist[e];
}

// One workgroup.  Thread (e, seg) = (tid % E, tid / E) owns blocks
// [seg*len, seg*len + len) of expert e's column, with S = 1024 / E segments.
__global__ __launch_bounds__(kDpScanThreads)
void dp_scan_kernel(int32_t* __restrict__ bcount, int nblk, int E, int32_t* __restrict__ group_end)
{
    __shared__ int segsum[kDpScanThreads];     // [seg][e], then each segment's start within its column
    __shared__ int start[kDpMaxExperts];
    const int S = kDpScanThreads / E;
    const int len = (nblk + S - 1) / S;
    const int tid = (int)threadIdx.x;
    const int e = tid % E, seg = tid / E;
    const bool mine = seg < S;
    const int b0 = seg * len, b1 = b0 + len < nblk ? b0 + len : nblk;
    int sum = 0;
    if (mine)
#pragma unroll 8
        for (int b = b0; b < b1; ++b) sum += bcount[(int64_t)b * E + e];
    if (mine) segsum[seg * E + e] = sum;
    __syncthreads();
    if (tid < E) {                             // exclusive scan over the segments of column tid
        int run = 0;
        for (int sg = 0; sg < S; ++sg) {
            const int c = segsum[sg * E + tid];
            segsum[sg * E + tid] = run;
            run += c;
        }
        start[tid] = run;                      // the expert's total, scanned below
    }
    __syncthreads();
    // exclusive scan of the totals over the experts (Hillis-Steele on start[0..E))
    for (int d = 1; d < E; d <<= 1) {
        int v = 0;
        if (tid < E && tid >= d) v = start[tid - d];
        __syncthreads();
        if (tid < E) start[tid] += v;
        __syncthreads();
    }
    if (tid < E) group_end[tid] = start[tid];   // inclusive: the end of expert tid
    __syncthreads();
    if (mine) {
        int run = (e > 0 ? start[e - 1] : 0) + segsum[seg * E + e];
        for (int b = b0; b < b1; ++b) {
            const int c = bcount[(int64_t)b * E + e];
            bcount[(int64_t)b * E + e] = run;
            run += c;
        }
    }
}

__global__ __launch_bounds__(kDpThreads)
void dp_place_kernel(const int32_t* __restrict__ ids, int64_t P, int E, const int32_t* __restrict__ bbase,
                     int32_t* __restrict__ src_pair)
{
    __shared__ int wcnt[kDpWaves * kDpMaxExperts];
    const int64_t p = (int64_t)blockIdx.x * kDpThreads + threadIdx.x;
    int e = p < P ? ids[p] : -1;
    e = (e >= 0 && e < E) ? e : -1;
    const int rank = rank_in_block(e, E, id_bits(E), wcnt);
    if (e >= 0) src_pair[bbase[(int64_t)blockIdx.x * E + e] + rank] = (int32_t)p;
}

// Scan folded into the place pass, for small tables (nblk * E <= kDpFoldMax,
// E <= kDpThreads): every workgroup reads the whole (blocks x experts) count
// table from L2 and derives its own block's first row per expert, so the
// one-workgroup scan launch drops out.  Thread (e, seg) = (tid % E, tid / E)
// sums expert e's counts over a segment of the blocks: all of them (the
// expert's total) and those before this block; the totals are then scanned
// over the experts.  Workgroup 0 also writes the end offsets.
constexpr int kDpFoldMax = 16384;
__global__ __launch_bounds__(kDpThreads)
void dp_place_scan_kernel(const int32_t* __restrict__ ids, int64_t P, int E, int nblk,
                          const int32_t* __restrict__ bcount, int32_t* __restrict__ src_pair,
                          int32_t* __restrict__ group_end)
{
    __shared__ int tot[kDpThreads], pre[kDpThreads], start[kDpThreads];
    __shared__ int wcnt[kDpWaves * kDpThreads];
    const int tid = (int)threadIdx.x;
    const int b = (int)blockIdx.x;
    const int S = kDpThreads / E;                        // segments per expert (>= 1)
    const int e0 = tid % E, seg = tid / E;
    if (tid < E) {
        tot[tid] = 0;
        pre[tid] = 0;
    }
    __syncthreads();
    if (seg < S) {
        const int len = (nblk + S - 1) / S;
        const int b0 = seg * len, b1 = b0 + len < nblk ? b0 + len : nblk;
        int t_sum = 0, p_sum = 0;
#pragma unroll 8
        for (int bb = b0; bb < b1; ++bb) {              // (unrolled: the L2 loads go out together)
            const int c = bcount[(int64_t)bb * E + e0];
            t_sum += c;
            p_sum += bb < b ? c : 0;
        }
        atomicAdd(&tot[e0], t_sum);
        atomicAdd(&pre[e0], p_sum);
    }
    __syncthreads();
    // exclusive scan of the totals over the experts (Hillis-Steele on start[0..E))
    if (tid < E) start[tid] = tot[tid];
    __syncthreads();
    for (int d = 1; d < E; d <<= 1) {
        int v = 0;
        if (tid < E && tid >= d) v = start[tid - d];
        __syncthreads();
        if (tid < E) start[tid] += v;
        __syncthreads();
    }
    if (b == 0 && tid < E) group_end[tid] = start[tid];  // inclusive: the end of expert tid
    // the place pass: rank among the earlier pairs of this block with the same expert
    const int64_t p = (int64_t)b * kDpThreads + tid;
    int e = p < P ? ids[p] : -1;
    e = (e >= 0 && e < E) ? e : -1;
    const int rank = rank_in_block(e, E, id_bits(E), wcnt);
    if (e >= 0) src_pair[start[e] - tot[e] + pre[e] + rank] = (int32_t)p;
}

int dispatch_max_experts() { return kDpMaxExperts; }

size_t dispatch_workspace_bytes(int64_t P, int32_t E)
{
    const int64_t nblk = (P + kDpThreads - 1) / kDpThreads;
    return (size_t)(nblk > 0 ? nblk : 1) * (size_t)E * 4u;
}

hipError_t launch_dispatch_order(const int32_t* ids, int64_t P, int E, int32_t* src_pair, int32_t* group_end,
                                 void* workspace, hipStream_t stream)
{
    int32_t* bcount = static_cast<int32_t*>(workspace);
    const int nblk = (int)((P + kDpThreads - 1) / kDpThreads);
    if (nblk > 0) {
        hipLaunchKernelGGL(dp_count_kernel, dim3((unsigned)nblk), dim3(kDpThreads), 0, stream, ids, P, E, bcount);
    }
    if (nblk > 0 && E <= kDpThreads && (int64_t)nblk * E <= kDpFoldMax) {
        hipLaunchKernelGGL(dp_place_scan_kernel, dim3((unsigned)nblk), dim3(kDpThreads), 0, stream, ids, P, E, nblk,
                           (const int32_t*)bcount, src_pair, group_end);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(dp_scan_kernel, dim3(1), dim3(kDpScanThreads), 0, stream, bcount, nblk, E, group_end);
    if (nblk > 0) {
        hipLaunchKernelGGL(dp_place_kernel, dim3((unsigned)nblk), dim3(kDpThreads), 0, stream, ids, P, E,
                           (const int32_t*)bcount, src_pair);
    }
    return hipGetLastError();
}

}  // namespace mxq
