// Dispatch: group the T*k (token, slot) pairs by expert, stably.
//
// "What Actually Happens When a Token Hits the Router", Step 3: sort tokens
// by assigned expert into contiguous blocks so each expert runs one dense
// matmul.  Here the grouping is a stable counting sort of pair ids
// p = t*k + j by expert id, done in three small kernels with no float
// atomics, so the result is deterministic:
//   1. count:   one workgroup per chunk of kScatterChunk pairs builds an LDS
//               histogram (integer LDS atomics) -> chunk_counts[chunk][e].
//   2. scan:    one workgroup: per-expert totals over chunks, exclusive scan
//               over experts -> counts, offsets; chunk_counts becomes each
//               chunk's first rank inside each expert.
// With a capacity C ("8.6 Mixture of Experts", sec. 3.2) an expert keeps its
// first C pairs in pair order: counts and offsets are of the kept pairs, and
// a pair of rank >= C inside its expert gets pair_pos -1.
//   3. scatter: one workgroup per chunk walks its pairs in order, 256 at a
//               time.  A pair's rank among equal ids in its wave comes from a
//               match mask built with 8 ballots over the id bits (E <= 256);
//               earlier waves' counts come from LDS.  Row = base + rank.
// When all pairs fit one chunk (decode-sized batches) the three steps run in
// one workgroup of one kernel, with the histogram and the bases in LDS.
#include "device_util.h"
#include "moe_internal.h"
#include "dispatch_block.h"

namespace moe {

namespace {

constexpr int kThreads = kDispatchThreads;
constexpr int kWaves = kThreads / 64;

__global__ __launch_bounds__(kThreads) void dispatch_count_kernel(DispatchArgs a) {
    __shared__ int hist[256];
    for (int e = threadIdx.x; e < a.E; e += kThreads) hist[e] = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * kScatterChunk;
    const int64_t p1 = min((int64_t)a.P, p0 + kScatterChunk);
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
        // eight chunks' counts loaded together, then rewritten as each
        // chunk's first rank inside the expert
        for (int c0 = 0; c0 < nchunks; c0 += 8) {
            int v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = c0 + i < nchunks ? a.chunk_counts[(int64_t)(c0 + i) * a.E + e] : 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (c0 + i < nchunks) a.chunk_counts[(int64_t)(c0 + i) * a.E + e] = run;   // exclusive within expert
                run += v[i];
            }
        }
        run = min(run, a.cap);
        a.counts[e] = run;
    }
    for (int i = threadIdx.x; i < a.nzero; i += kThreads) a.zero[i] = 0;
    // the trailing group (no capacity, so the experts' pairs end at P)
    for (int i = threadIdx.x; i < a.tail; i += kThreads) a.sorted_pairs[a.P + i] = i * a.tail_mul;
    if (a.tail && threadIdx.x == 0) a.offsets[a.E + 1] = a.P + a.tail;
    expert_scan(a, run, tot, wsum);
}

__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(DispatchArgs a) {
    __shared__ int running[256];          // pairs of each expert before this one (earlier chunks and rounds)
    __shared__ int base[256];             // first grouped row of each expert
    __shared__ int wcount[kWaves][256];   // per-wave counts of the current round
    for (int e = threadIdx.x; e < a.E; e += kThreads) {
        running[e] = a.chunk_counts[(int64_t)blockIdx.x * a.E + e];
        base[e] = a.offsets[e];
        for (int q = 0; q < kWaves; ++q) wcount[q][e] = 0;
    }
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * kScatterChunk;
    const int64_t p1 = min((int64_t)a.P, p0 + kScatterChunk);
    scatter_range(a, p0, p1, running, base, wcount);
}

// All pairs in one chunk: count, scan and scatter in one workgroup.
__global__ __launch_bounds__(kThreads) void dispatch_single_kernel(DispatchArgs a) {
    for (int i = threadIdx.x; i < a.nzero; i += kThreads) a.zero[i] = 0;
    dispatch_in_block(a);
}

__global__ void fill_zero_kernel(int32_t* a, int na, int32_t* b, int nb) {
    for (int i = threadIdx.x; i < na; i += blockDim.x) a[i] = 0;
    for (int i = threadIdx.x; i < nb; i += blockDim.x) b[i] = 0;
}

}  // namespace

// Chunks of 512 pairs: the scatter walks its chunk 256 pairs at a time, with
// barriers between rounds, so smaller chunks spread it over more CUs
// (DeepSeek-V3, 65,536 pairs: 128 workgroups instead of 32).
int dispatch_num_chunks(int P) { return P <= kDispatchChunk ? 1 : (P + kScatterChunk - 1) / kScatterChunk; }

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
    const int nchunks = dispatch_num_chunks(a.P);
    if (a.tail && (nchunks < 2 || a.cap != 0x7FFFFFFF || a.tail < 0)) return hipErrorInvalidValue;
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
