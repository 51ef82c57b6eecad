// Workgroup-level pieces of the stable counting sort of pairs by expert
// (the dispatch), shared by the dispatch kernels and by the router's
// finishing kernel, which runs the whole dispatch of a batch of at most 32
// tokens right after selecting their experts.  256 threads; E <= 256.
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int kDispatchThreads = 256;

// Exclusive scan of `run` (thread e's expert's kept pairs, 0 past E) over
// the experts: offsets[e] and tot[e] = first grouped row of expert e,
// offsets[E] = all kept pairs.  Ends with a barrier.
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
    if (e == kDispatchThreads - 1) a.offsets[a.E] = incl;   // all kept pairs
    __syncthreads();
}

// Pairs [p0, p1) in order.  A pair's rank w inside its expert e is
// running[e] + (its rank among the earlier pairs of this range with expert
// e); it gets row base[e] + w if w < a.cap, else it is dropped (pair_pos
// -1).  running[] advances.  wcount[][] must be zero on entry and is zero on
// exit.
__device__ __forceinline__ void scatter_range(const DispatchArgs& a, int64_t p0, int64_t p1, int* running,
                                              const int* base, int (*wcount)[256]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t q0 = p0; q0 < p1; q0 += kDispatchThreads) {
        const int64_t p = q0 + threadIdx.x;
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
            if (r < a.cap) {
                a.sorted_pairs[base[e] + r] = (int32_t)p;
                a.pair_pos[p] = base[e] + r;
            } else {
                a.pair_pos[p] = -1;
            }
        }
        __syncthreads();
        for (int ee = threadIdx.x; ee < a.E; ee += kDispatchThreads) {
            int add = 0;
            for (int q = 0; q < (kDispatchThreads / 64); ++q) { add += wcount[q][ee]; wcount[q][ee] = 0; }
            running[ee] += add;
        }
        __syncthreads();
    }
}

// The whole dispatch of a.P <= kDispatchChunk pairs in one workgroup: count
// (LDS histogram), exclusive scan over the experts' kept counts, stable
// scatter.  a.ids must be visible to every thread of the workgroup.
__device__ __forceinline__ void dispatch_in_block(const DispatchArgs& a) {
    __shared__ int hist[256];
    __shared__ int wsum[kDispatchThreads / 64];
    __shared__ int base[256];
    __shared__ int wcount[kDispatchThreads / 64][256];
    const int e = threadIdx.x;
    hist[e] = 0;
    for (int q = 0; q < kDispatchThreads / 64; ++q) wcount[q][e] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < a.P; p += kDispatchThreads) atomicAdd(&hist[a.ids[p]], 1);
    __syncthreads();
    const int kept = e < a.E ? min(hist[e], a.cap) : 0;
    if (e < a.E) a.counts[e] = kept;
    expert_scan(a, kept, base, wsum);
    hist[e] = 0;                   // now: rank inside the expert so far
    __syncthreads();
    scatter_range(a, 0, a.P, hist, base, wcount);
}

}  // namespace moe
