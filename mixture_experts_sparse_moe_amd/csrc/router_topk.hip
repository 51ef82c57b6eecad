// Router GEMM + top-k selection + gates, fused in one kernel.
//
// Computes, for each token t ("Mixture-of-Experts Internals" sec. 2.1; "from
// the router to the all-to-all", The router):
//   h[t,e] = sum_i x[t,i] W_r[e,i]         fp32 accumulation
//   I      = the k largest h (ties: lower expert index), listed in order
//   gates  = softmax restricted to I (renormalised softmax; "8.6 Mixture of
//            Experts" sec. 2 writes it as a softmax over the chosen logits,
//            which needs no denominator over all E), or full softmax, or
//            sigmoid (normalised over I or not).
// Selection is taken on the logits: softmax and sigmoid are strictly
// increasing, and fp32 sigmoid saturates to 1.0 for large logits, which would
// make false ties.
//
// Workgroup = 256 threads (4 waves) owns 32 tokens and all E <= 256 experts.
// bf16: the logits tile [32, E] is built with v_mfma_f32_32x32x16_bf16 (bf16
// products are exact in fp32, so this is an fp32-accumulated dot product).
// Each lane streams 64 contiguous bytes of its row per 64-wide K chunk: the
// MFMA's 16 K slots in step s take actual k = 32*half + 8*s + i, a
// permutation of the chunk shared by both operands, so the contraction is
// unchanged while every load is a full 16-byte vector.  When E needs fewer
// than four 32-expert blocks, the K chunks are split over waves and the
// partial tiles are added in a fixed order (deterministic).
// fp32: plain FMA dot products.
// Top-k: one wave per token, 64-bit keys (orderable logit bits, inverted
// expert index) reduced with a butterfly; k rounds.
#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kBT = 32;          // tokens per workgroup
constexpr int kMaxE = 256;
constexpr int kPartStride = 97;  // row stride of a partial tile (E <= 96 when split)
constexpr int kLogitStride = kMaxE + 1;
constexpr int kLdsFloats = (4 * kBT * kPartStride > kBT * kLogitStride) ? 4 * kBT * kPartStride
                                                                         : kBT * kLogitStride;

__device__ __forceinline__ uint32_t ord_bits(float f) {
    f = f + 0.0f;  // -0 -> +0: equal logits compare equal
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        unsigned long long w = __shfl_xor(v, o, 64);
        v = (w > v) ? w : v;
    }
    return v;
}

// Logits of 32 tokens x all experts into lds (bf16 inputs, MFMA).
__device__ void logits_bf16(const RouteArgs& a, int t0, float* lds) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int nb = (a.E + 31) / 32;
    const int KS = nb >= 4 ? 1 : 4 / nb;    // K slices
    const int WPS = 4 / KS;                 // waves per slice
    const int ksl = w % KS, wsub = w / KS;
    const int nchunks = a.d / 64;
    const int half = lane >> 5, r32 = lane & 31;

    const uint16_t* X = static_cast<const uint16_t*>(a.x);
    const uint16_t* W = static_cast<const uint16_t*>(a.w);
    int tok = t0 + r32;
    if (tok >= a.T) tok = a.T - 1;          // clamp; rows past T are discarded
    const uint4* xrow = reinterpret_cast<const uint4*>(X + (int64_t)tok * a.d + 32 * half);

    // this wave's expert blocks: wsub and wsub + WPS (nb <= 8)
    const int blk[2] = {wsub, wsub + WPS};
    const int nmy = (blk[0] < nb) + (blk[1] < nb);
    const uint4* wrow[2];
    bool wvalid[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int e = blk[i] * 32 + r32;
        wvalid[i] = (i < nmy) && (e < a.E);
        if (e >= a.E) e = a.E - 1;
        wrow[i] = reinterpret_cast<const uint4*>(W + (int64_t)e * a.d + 32 * half);
    }

    f32x16_t acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.0f;

    const uint4 z4 = make_uint4(0, 0, 0, 0);
    for (int c = ksl; c < nchunks; c += KS) {
        uint4 av[4], bv[2][4];
#pragma unroll
        for (int s = 0; s < 4; ++s) av[s] = xrow[c * 8 + s];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int s = 0; s < 4; ++s) bv[i][s] = (i < nmy && wvalid[i]) ? wrow[i][c * 8 + s] : z4;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                if (i < nmy)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[s]),
                                                                     as_bf16x8(bv[i][s]), acc[i],
                                                                     0, 0, 0);
        }
    }
    // D element (blk4, r): token row 8*blk4 + 4*half + r, expert col b*32 + r32
    if (KS == 1) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (i >= nmy) continue;
            int e = blk[i] * 32 + r32;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                int row = 8 * (j >> 2) + 4 * half + (j & 3);
                lds[row * kLogitStride + e] = acc[i][j];
            }
        }
        __syncthreads();
    } else {
        float* part = lds + ksl * kBT * kPartStride;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (i >= nmy) continue;
            int e = blk[i] * 32 + r32;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                int row = 8 * (j >> 2) + 4 * half + (j & 3);
                part[row * kPartStride + e] = acc[i][j];
            }
        }
        __syncthreads();
        // sum the K slices in slice order; result replaces slice 0
        const int Epad = nb * 32;            // <= 64 when the K chunks are split
        constexpr int kIt = kBT * 64 / 256;
        float vals[kIt];
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int idx = threadIdx.x + it * 256;
            vals[it] = 0.0f;
            if (idx < kBT * Epad) {
                const int row = idx / Epad, e = idx % Epad;
                float s = lds[row * kPartStride + e];
                for (int q = 1; q < KS; ++q) s += lds[q * kBT * kPartStride + row * kPartStride + e];
                vals[it] = s;
            }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int idx = threadIdx.x + it * 256;
            if (idx < kBT * Epad) {
                const int row = idx / Epad, e = idx % Epad;
                lds[row * kLogitStride + e] = vals[it];
            }
        }
        __syncthreads();
    }
}

// Logits of 32 tokens x all experts into lds (fp32 inputs, FMA).
__device__ void logits_f32(const RouteArgs& a, int t0, float* lds) {
    const float* X = static_cast<const float*>(a.x);
    const float* W = static_cast<const float*>(a.w);
    for (int idx = threadIdx.x; idx < kBT * a.E; idx += 256) {
        int row = idx / a.E, e = idx % a.E;
        int tok = t0 + row;
        if (tok >= a.T) tok = a.T - 1;
        const float* xr = X + (int64_t)tok * a.d;
        const float* wr = W + (int64_t)e * a.d;
        float s = 0.0f;
        for (int i = 0; i < a.d; ++i) s = fmaf(xr[i], wr[i], s);
        lds[row * kLogitStride + e] = s;
    }
    __syncthreads();
}

template <bool BF16>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
    __shared__ float lds[kLdsFloats];
    const int t0 = blockIdx.x * kBT;
    if (BF16) logits_bf16(a, t0, lds);
    else logits_f32(a, t0, lds);

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    for (int row = w; row < kBT; row += 4) {
        const int t = t0 + row;
        if (t >= a.T) break;
        const float* lrow = lds + row * kLogitStride;
        unsigned long long key[4];
        float lv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int e = lane + 64 * q;
            if (e < a.E) {
                lv[q] = lrow[e];
                key[q] = ((unsigned long long)ord_bits(lv[q]) << 32) | (0xFFFFFFFFu - (uint32_t)e);
            } else {
                lv[q] = 0.0f;
                key[q] = 0ull;
            }
        }
        int my_e = 0;
        float my_l = 0.0f, first_l = 0.0f, last_l = 0.0f;
        for (int j = 0; j < a.k; ++j) {
            unsigned long long m = key[0];
#pragma unroll
            for (int q = 1; q < 4; ++q) m = key[q] > m ? key[q] : m;
            m = wave_max_u64(m);
            const int e = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFull));
            const float l = lrow[e];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (key[q] == m) key[q] = 0ull;
            if (lane == j) { my_e = e; my_l = l; }
            if (j == 0) first_l = l;
            last_l = l;
        }
        float gap = __builtin_inff();
        if (a.k < a.E) {
            unsigned long long m = key[0];
#pragma unroll
            for (int q = 1; q < 4; ++q) m = key[q] > m ? key[q] : m;
            m = wave_max_u64(m);
            const int e = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFull));
            gap = last_l - lrow[e];
        }
        const bool mine = lane < a.k;
        float g;
        if (a.score_fn == 0) {
            const float ex = mine ? expf(my_l - first_l) : 0.0f;
            float z;
            if (a.renorm) {
                z = wave_sum(ex);
            } else {
                float part = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (lane + 64 * q < a.E) part += expf(lv[q] - first_l);
                z = wave_sum(part);
            }
            g = ex / z;
        } else {
            const float sg = mine ? 1.0f / (1.0f + expf(-my_l)) : 0.0f;
            g = a.renorm ? sg / wave_sum(sg) : sg;
        }
        if (mine) {
            a.ids[(int64_t)t * a.k + lane] = my_e;
            a.weights[(int64_t)t * a.k + lane] = g;
        }
        if (lane == 0 && a.gap) a.gap[t] = gap;
    }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, bool bf16, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    dim3 grid((a.T + kBT - 1) / kBT), block(256);
    if (bf16) hipLaunchKernelGGL(route_kernel<true>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(route_kernel<false>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
