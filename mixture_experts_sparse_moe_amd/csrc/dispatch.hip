// Dispatch: group the T*k (token, slot) pairs by expert, stably.
//
// "What Actually Happens When a Token Hits the Router", Step 3: sort tokens
// by assigned expert into contiguous blocks so each expert runs one dense
// matmul.  Here the grouping is a stable counting sort of pair ids
// p = t*k + j by expert id, done in three small kernels with no float
// atomics, so the result is deterministic:
//   1. count:   one workgroup per chunk of kDispatchChunk pairs builds an LDS
//               histogram (integer LDS atomics) -> chunk_counts[chunk][e].
//   2. scan:    one workgroup: per-expert totals over chunks, exclusive scan
//               over experts -> counts, offsets; chunk_counts becomes each
//               chunk's first grouped row per expert.
//   3. scatter: one workgroup per chunk walks its pairs in order, 256 at a
//               time.  A pair's rank among equal ids in its wave comes from a
//               match mask built with 8 ballots over the id bits (E <= 256);
//               earlier waves' counts come from LDS.  Row = base + rank.
// When all pairs fit one chunk (decode-sized batches) the three steps run in
// one workgroup of one kernel, with the histogram and the bases in LDS.
#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Exclusive scan of `run` (thread e's expert total, 0 past E) over the
// experts: offsets[e] and tot[e] = first grouped row of expert e,
// offsets[E] = P.  Ends with a barrier.
__device__ __forceinline__ void expert_scan(const DispatchArgs& a, int run, int* tot, int* wsum) {
    const int e = threadIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int v = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    int before = 0;
    for (int q = 0; q < w; ++q) before += wsum[q];
    const int incl = v + before;
    const int excl = incl - run;
    tot[e] = excl;
    if (e < a.E) a.offsets[e] = excl;
    if (e == kThreads - 1) a.offsets[a.E] = incl;   // total = P
    __syncthreads();
}

// Pairs [p0, p1) in order: each gets row running[e] + (its rank among the
// earlier pairs of this range with the same expert).  running[] advances.
// wcount[][] must be zero on entry and is zero on exit.
__device__ __forceinline__ void scatter_range(const DispatchArgs& a, int64_t p0, int64_t p1, int* running,
                                              int (*wcount)[256]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t base = p0; base < p1; base += kThreads) {
        const int64_t p = base + threadIdx.x;
        const bool valid = p < p1;
        const int e = valid ? a.ids[p] : 0;
        // lanes of this wave holding the same expert id
        uint64_t same = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint64_t bits = __ballot(valid && ((e >> b) & 1));
            same &= ((e >> b) & 1) ? bits : ~bits;
        }
        const int rank_in_wave = __popcll(same & lt_mask);
        const bool leader = valid && (same & lt_mask) == 0;
        if (leader) wcount[w][e] = __popcll(same);
        __syncthreads();
        if (valid) {
            int r = running[e] + rank_in_wave;
            for (int q = 0; q < w; ++q) r += wcount[q][e];
            a.sorted_pairs[r] = (int32_t)p;
            a.pair_pos[p] = r;
        }
        __syncthreads();
        for (int ee = threadIdx.x; ee < a.E; ee += kThreads) {
            int add = 0;
            for (int q = 0; q < kWaves; ++q) { add += wcount[q][ee]; wcount[q][ee] = 0; }
            running[ee] += add;
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kThreads) void dispatch_count_kernel(DispatchArgs a) {
    __shared__ int hist[256];
    for (int e = threadIdx.x; e < a.E; e += kThreads) hist[e] = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * kDispatchChunk;
    const int64_t p1 = min((int64_t)a.P, p0 + kDispatchChunk);
    for (int64_t p = p0 + threadIdx.x; p < p1; p += kThreads) atomicAdd(&hist[a.ids[p]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < a.E; e += kThreads)
        a.chunk_counts[(int64_t)blockIdx.x * a.E + e] = hist[e];
}

__global__ __launch_bounds__(kThreads) void dispatch_scan_kernel(DispatchArgs a, int nchunks) {
    __shared__ int tot[256];
    __shared__ int wsum[kWaves];
    const int e = threadIdx.x;
    int run = 0;
    if (e < a.E) {
        for (int c = 0; c < nchunks; ++c) {
            int v = a.chunk_counts[(int64_t)c * a.E + e];
            a.chunk_counts[(int64_t)c * a.E + e] = run;   // exclusive within expert
            run += v;
        }
        a.counts[e] = run;
    }
    expert_scan(a, run, tot, wsum);
    if (e < a.E)
        for (int c = 0; c < nchunks; ++c) a.chunk_counts[(int64_t)c * a.E + e] += tot[e];
}

__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(DispatchArgs a) {
    __shared__ int running[256];          // rows handed out so far in this chunk, per expert
    __shared__ int wcount[kWaves][256];   // per-wave counts of the current round
    for (int e = threadIdx.x; e < a.E; e += kThreads) {
        running[e] = a.chunk_counts[(int64_t)blockIdx.x * a.E + e];
        for (int q = 0; q < kWaves; ++q) wcount[q][e] = 0;
    }
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * kDispatchChunk;
    const int64_t p1 = min((int64_t)a.P, p0 + kDispatchChunk);
    scatter_range(a, p0, p1, running, wcount);
}

// All pairs in one chunk: count, scan and scatter in one workgroup.
__global__ __launch_bounds__(kThreads) void dispatch_single_kernel(DispatchArgs a) {
    __shared__ int hist[256];
    __shared__ int wsum[kWaves];
    __shared__ int running[256];
    __shared__ int wcount[kWaves][256];
    const int e = threadIdx.x;
    hist[e] = 0;
    for (int q = 0; q < kWaves; ++q) wcount[q][e] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < a.P; p += kThreads) atomicAdd(&hist[a.ids[p]], 1);
    __syncthreads();
    const int run = e < a.E ? hist[e] : 0;
    if (e < a.E) a.counts[e] = run;
    expert_scan(a, run, running, wsum);
    scatter_range(a, 0, a.P, running, wcount);
}

__global__ void fill_zero_kernel(int32_t* a, int na, int32_t* b, int nb) {
    for (int i = threadIdx.x; i < na; i += blockDim.x) a[i] = 0;
    for (int i = threadIdx.x; i < nb; i += blockDim.x) b[i] = 0;
}

}  // namespace

int dispatch_num_chunks(int P) { return (P + kDispatchChunk - 1) / kDispatchChunk; }

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
    const int nchunks = dispatch_num_chunks(a.P);
    if (a.P == 0) {
        // no pairs: counts and offsets are all zero (a kernel, not a memset,
        // so that the call can be captured into a graph)
        hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(kThreads), 0, s, a.counts, a.E,
                           a.offsets, a.E + 1);
        return hipGetLastError();
    }
    if (nchunks == 1) {
        hipLaunchKernelGGL(dispatch_single_kernel, dim3(1), dim3(kThreads), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(nchunks), dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kThreads), 0, s, a, nchunks);
    hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(nchunks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
