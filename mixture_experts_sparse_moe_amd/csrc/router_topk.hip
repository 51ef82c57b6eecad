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
// The K dimension streams through LDS in chunks of 64: the chunk of the 32 x
// rows and of the E weight rows (E padded to 32 * NBLK, NBLK in {1, 2, 4, 8})
// is fetched by direct-to-LDS DMA into one of NST stage buffers, NST - 1
// chunks ahead of the MFMAs, one barrier per chunk.  Rows are 128 bytes with
// 16-byte chunks XOR-swizzled.  With NBLK >= 4 each wave owns NBLK / 4
// expert blocks; with fewer blocks 4 / NBLK waves share a block and split
// the four 16-wide K steps of a chunk, their partial tiles added in a fixed
// order (deterministic).
// fp32: plain FMA dot products.
// Top-k: one wave per token, 64-bit keys (orderable logit bits, inverted
// expert index) reduced with DPP lane moves; k rounds.
// Few tokens (moe_forward): the K chunks are split over workgroups, whose
// partial logits a second kernel adds in a fixed order before selecting.
#include <algorithm>

#include "device_util.h"
#include "moe_internal.h"
#include "dispatch_block.h"
#include "skinny.h"

namespace moe {

namespace {

constexpr int kBT = 32;          // tokens per workgroup
// route_partial_wide_kernel: 32-token blocks per workgroup (DeepSeek-V3 route
// 117 us with the fused kernel, 86 us with 2 blocks, 83 us with 4)
constexpr int kWideNA = 4;
constexpr int kMaxE = 256;
constexpr int kLogitStride = kMaxE + 1;
constexpr int kLogitFloats = kBT * kLogitStride;

__device__ __forceinline__ uint32_t ord_bits(float f) {
    f = f + 0.0f;  // -0 -> +0: equal logits compare equal
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave reductions with DPP lane moves inside rows of 16 lanes (quad swaps,
// half-row and row mirrors), then the four row results through scalar
// registers, combined in row order.  No LDS round trips: selecting the top k
// for a token takes k + 1 maxima and one or two sums, one after another.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ unsigned long long max_step(unsigned long long v) {
    const unsigned long long w =
        ((unsigned long long)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
    return w > v ? w : v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
    v = max_step<0xB1>(v);       // quad_perm(1, 0, 3, 2)
    v = max_step<0x4E>(v);       // quad_perm(2, 3, 0, 1)
    v = max_step<0x141>(v);      // row_half_mirror
    v = max_step<0x140>(v);      // row_mirror: every lane holds its row's maximum
    unsigned long long m = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const unsigned long long x =
            ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), 16 * r) << 32) |
            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
        m = x > m ? x : m;
    }
    return m;
}

template <int CTRL>
__device__ __forceinline__ float sum_step(float v) {
    return v + __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

__device__ __forceinline__ float wave_sum(float v) {
    v = sum_step<0xB1>(v);
    v = sum_step<0x4E>(v);
    v = sum_step<0x141>(v);
    v = sum_step<0x140>(v);
    float t = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) t += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
    return t;
}

// Logits of 32 tokens x all experts (E <= 32 NBLK) into lds[32][kLogitStride]
// (bf16 inputs, MFMA, LDS-staged K chunks), over the K chunks [c0, c0 + nc).
template <int NBLK>
__device__ __forceinline__ void logits_bf16(const RouteArgs& a, int t0, int c0, int nc, float* lds,
                                            uint16_t* sX0, uint16_t* sX1, uint16_t* sX2, uint16_t* sX3,
                                            uint16_t* sW0, uint16_t* sW1, uint16_t* sW2, uint16_t* sW3) {
    using Sh = SkinnyShape<NBLK>;
    constexpr int KS = Sh::KS, BPW = Sh::BPW, P = Sh::P;
    static_assert(KS == 1 || BPW == 1, "partial tiles of one block per wave");
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, r32 = lane & 31;
    const int64_t rowb = (int64_t)a.d * 2;               // bytes per row

    // A rows: the 32 tokens (rows past T repeat the last); B rows: the experts
    // (rows past E repeat the last)
    const char* src[P];
    {
        const int64_t kb = (int64_t)c0 * (kSkChunk * 2);
        const int rx = 8 * w + (lane >> 3);
        const int tok = min(t0 + rx, a.T - 1);
        src[0] = static_cast<const char*>(a.x) + tok * rowb + kb + (((lane & 7) ^ swz(rx)) * 16);
#pragma unroll
        for (int j = 1; j < P; ++j) {
            const int rw = 8 * (w + 4 * j - 4) + (lane >> 3);
            const int e = min(rw, a.E - 1);
            src[j] = static_cast<const char*>(a.w) + e * rowb + kb + (((lane & 7) ^ swz(rw)) * 16);
        }
    }
    f32x16_t acc[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.0f;
    skinny_mma<Sh, false, 0>(src, nc, 0, sX0, sX1, sX2, sX3, sW0, sW1, sW2, sW3, acc);
    const int b0 = skinny_block<Sh, false>(w, 0);

    // D element j of block i: token row 8 (j / 4) + 4 half + j % 4, expert r32
    if (KS == 1) {
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            const int e = (b0 + i) * 32 + r32;
#pragma unroll
            for (int j = 0; j < 16; ++j) lds[(8 * (j >> 2) + 4 * half + (j & 3)) * kLogitStride + e] = acc[i][j];
        }
        __syncthreads();
    } else {
        // partial tiles [KS][32][32 NBLK], then their sum in slice order
        constexpr int EP = 32 * NBLK;
        const int q = w / Sh::NG;
        const int e = b0 * 32 + r32;
#pragma unroll
        for (int j = 0; j < 16; ++j) lds[q * kBT * EP + (8 * (j >> 2) + 4 * half + (j & 3)) * EP + e] = acc[0][j];
        __syncthreads();
        constexpr int kIt = kBT * EP / 256;
        float vals[kIt];
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int idx = tid + it * 256;
            float v = lds[idx];
            for (int qq = 1; qq < KS; ++qq) v += lds[qq * kBT * EP + idx];
            vals[it] = v;
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int idx = tid + it * 256;
            lds[(idx / EP) * kLogitStride + idx % EP] = vals[it];
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

// The float whose ord_bits are the upper half of a selection key.
__device__ __forceinline__ float key_value(unsigned long long m) {
    const uint32_t u = (uint32_t)(m >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Largest float over the wave (every lane gets it).
__device__ __forceinline__ float wave_max_f32(float v) {
    return key_value(wave_max_u64((unsigned long long)ord_bits(v) << 32));
}

// Score margin s(a) - s(b) between two experts with logits a >= b, without
// the cancellation of subtracting two rounded scores: softmax
// e^(a - mx) (1 - e^(b - a)) / z with mx the largest logit and z the sum of
// e^(l - mx) over all experts; sigmoid s(a) s(-b) (1 - e^(b - a)), since
// s(a) - s(b) = (e^-b - e^-a) / ((1 + e^-a)(1 + e^-b)).
__device__ __forceinline__ float score_margin(float a, float b, int score_fn, float mx, float z) {
    const float d = -expm1f(b - a);
    if (score_fn == 0) return expf(a - mx) * d / z;
    return d / ((1.0f + expf(-a)) * (1.0f + expf(b)));
}

__device__ __forceinline__ float score_of(float l, int score_fn, float mx, float z) {
    return score_fn == 0 ? expf(l - mx) / z : 1.0f / (1.0f + expf(-l));
}

// Top-k selection and gates of tokens t0 .. t0 + 31 from their logits in
// lds[32][kLogitStride]; one wave per token.  Lane owns experts lane + 64 q.
//   key (what is selected on): the logit; with a bias, logit + bias or
//       score + bias ("Mixture-of-Experts Internals", sec. 3.3; "from the
//       router to the all-to-all", Load balancing).  Ties: lower index.
//   gates: from the unbiased scores, renormalised over the chosen set or not.
//   gap [T, 2]: key_(k) - key_(k+1), and the score margin s_(k) - s_(k+1)
//       of the same two experts (scores unbiased: softmax over all E or
//       sigmoid; with a bias it can be negative).
// With a.stats_part the block's per-expert sums of the chosen count and of
// the router probability (softmax score, or sigmoid score normalised over all
// experts) go to a.stats_part[blockIdx.x][2E], summed over the block's tokens
// in a fixed order.  With s_ids the ids are also kept in LDS,
// s_ids[(t - t0) * k + j].  Every thread of the workgroup must call it.
template <int QN, bool OPT>
__device__ __forceinline__ void topk_rows_q(const RouteArgs& a, int t0, float* lds, int* s_ids) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const bool stats = OPT && a.stats_part != nullptr;
    const float* abias = OPT ? a.bias : nullptr;
    float bias[QN];
#pragma unroll
    for (int q = 0; q < QN; ++q) bias[q] = (abias && lane + 64 * q < a.E) ? abias[lane + 64 * q] : 0.0f;
    float pacc[QN], cacc[QN];
#pragma unroll
    for (int q = 0; q < QN; ++q) pacc[q] = cacc[q] = 0.0f;
    for (int row = w; row < kBT; row += nw) {
        const int t = t0 + row;
        if (t >= a.T) break;
        const float* lrow = lds + row * kLogitStride;
        float lv[QN];
#pragma unroll
        for (int q = 0; q < QN; ++q) lv[q] = lane + 64 * q < a.E ? lrow[lane + 64 * q] : -__builtin_inff();
        // full scores, when the key or the statistics need them
        const bool need_s = (abias && a.bias_on_scores) || stats;
        float sv[QN], mx = 0.0f;
#pragma unroll
        for (int q = 0; q < QN; ++q) sv[q] = 0.0f;
        if (need_s || abias) {
            float m = lv[0];
#pragma unroll
            for (int q = 1; q < QN; ++q) m = fmaxf(m, lv[q]);
            mx = wave_max_f32(m);
        }
        if (need_s) {
            float part = 0.0f;
#pragma unroll
            for (int q = 0; q < QN; ++q) {
                if (lane + 64 * q < a.E) {
                    sv[q] = a.score_fn == 0 ? expf(lv[q] - mx) : 1.0f / (1.0f + expf(-lv[q]));
                    part += sv[q];
                }
            }
            const float z = wave_sum(part);
            if (a.score_fn == 0) {
#pragma unroll
                for (int q = 0; q < QN; ++q) sv[q] /= z;
            }
            if (stats) {
#pragma unroll
                for (int q = 0; q < QN; ++q) pacc[q] += a.score_fn == 0 ? sv[q] : sv[q] / z;
            }
        }
        unsigned long long key[QN];
        float kv[QN];
#pragma unroll
        for (int q = 0; q < QN; ++q) {
            const int e = lane + 64 * q;
            kv[q] = abias ? (a.bias_on_scores ? sv[q] : lv[q]) + bias[q] : lv[q];
            key[q] = e < a.E ? ((unsigned long long)ord_bits(kv[q]) << 32) | (0xFFFFFFFFu - (uint32_t)e) : 0ull;
        }
        int my_e = 0, e_k = 0;
        float my_l = 0.0f, first_l = 0.0f, last_k = 0.0f;
        for (int j = 0; j < a.k; ++j) {
            unsigned long long m = key[0];
#pragma unroll
            for (int q = 1; q < QN; ++q) m = key[q] > m ? key[q] : m;
            m = wave_max_u64(m);
            const int e = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFull));
            const float l = lrow[e];
#pragma unroll
            for (int q = 0; q < QN; ++q)
                if (key[q] == m) {
                    key[q] = 0ull;
                    cacc[q] += 1.0f;
                }
            if (lane == j) { my_e = e; my_l = l; }
            if (j == 0) first_l = l;
            last_k = key_value(m);
            e_k = e;
        }
        float gap = __builtin_inff(), sgap = __builtin_inff();
        if (a.k < a.E) {
            unsigned long long m = key[0];
#pragma unroll
            for (int q = 1; q < QN; ++q) m = key[q] > m ? key[q] : m;
            m = wave_max_u64(m);
            gap = last_k - key_value(m);
            if (a.gap) {
                // score margin of the k-th and (k+1)-th choices
                const int e_k1 = (int)(0xFFFFFFFFu - (uint32_t)(m & 0xFFFFFFFFull));
                const float la = lrow[e_k], lb = lrow[e_k1];
                const float mxs = abias ? mx : first_l;     // the largest logit
                float z = 1.0f;
                if (a.score_fn == 0) {
                    float part = 0.0f;
#pragma unroll
                    for (int q = 0; q < QN; ++q)
                        if (lane + 64 * q < a.E) part += expf(lv[q] - mxs);
                    z = wave_sum(part);
                }
                sgap = abias ? score_of(la, a.score_fn, mxs, z) - score_of(lb, a.score_fn, mxs, z)
                             : score_margin(la, lb, a.score_fn, mxs, z);
            }
        }
        const bool mine = lane < a.k;
        // largest logit among the chosen (the first chosen unless biased)
        const float top = abias ? wave_max_f32(mine ? my_l : -__builtin_inff()) : first_l;
        float g;
        if (a.score_fn == 0) {
            const float ex = mine ? expf(my_l - (a.renorm ? top : (abias ? mx : first_l))) : 0.0f;
            float z;
            if (a.renorm) {
                z = wave_sum(ex);
            } else {
                const float sh = abias ? mx : first_l;
                float part = 0.0f;
#pragma unroll
                for (int q = 0; q < QN; ++q)
                    if (lane + 64 * q < a.E) part += expf(lv[q] - sh);
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
            if (s_ids) s_ids[row * a.k + lane] = my_e;
        }
        if (lane == 0 && a.gap) {
            a.gap[2 * (int64_t)t] = gap;
            a.gap[2 * (int64_t)t + 1] = sgap;
        }
    }
    if (stats) {
        // waves' sums in LDS (the logit tile is no longer read), then added
        // in wave order: [wave][0, E) counts, [wave][E, 2E) probabilities
        __syncthreads();
#pragma unroll
        for (int q = 0; q < QN; ++q) {
            const int e = lane + 64 * q;
            if (e < a.E) {
                lds[w * 2 * a.E + e] = cacc[q];
                lds[w * 2 * a.E + a.E + e] = pacc[q];
            }
        }
        __syncthreads();
        for (int i = threadIdx.x; i < 2 * a.E; i += blockDim.x) {
            float v = 0.0f;
            for (int q = 0; q < nw; ++q) v += lds[q * 2 * a.E + i];
            a.stats_part[(int64_t)blockIdx.x * 2 * a.E + i] = v;
        }
    }
}

// Expert slots per lane QN = ceil(E / 64); the optional bias and statistics
// code only in the variant that needs it (the selection runs once per launch,
// so the instructions it fetches are a large part of its time).
template <int QN>
__device__ __forceinline__ void topk_rows(const RouteArgs& a, int t0, float* lds, int* s_ids = nullptr) {
    if (a.bias || a.stats_part) topk_rows_q<QN, true>(a, t0, lds, s_ids);
    else topk_rows_q<QN, false>(a, t0, lds, s_ids);
}

// Stage buffers of the bf16 logits (NBLK = 0, fp32: none).
#define MOE_ROUTE_LDS(NBLK_)                                                                    \
    constexpr int NB = (NBLK_) ? (NBLK_) : 1;                                                   \
    using St = SkinnyShape<NB>;                                                                 \
    constexpr int XS = (NBLK_) ? St::XS : 8, WS = (NBLK_) ? St::WS : 8;                         \
    constexpr int X3 = St::NST > 3 ? XS : 8, W3 = St::NST > 3 ? WS : 8;                         \
    __shared__ float lds[kLogitFloats];                                                         \
    __shared__ __align__(16) uint16_t sX0[XS], sX1[XS], sX2[XS], sX3[X3];                       \
    __shared__ __align__(16) uint16_t sW0[WS], sW1[WS], sW2[WS], sW3[W3]

// One workgroup per 32 tokens.  NBLK = 0: fp32 inputs; else bf16 with E <= 32 NBLK.
template <int NBLK>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
    MOE_ROUTE_LDS(NBLK);
    const int t0 = blockIdx.x * kBT;
    if (NBLK) logits_bf16<NB>(a, t0, 0, a.d / kSkChunk, lds, sX0, sX1, sX2, sX3, sW0, sW1, sW2, sW3);
    else logits_f32(a, t0, lds);
    topk_rows<NBLK == 0 || NBLK >= 8 ? 4 : (NBLK == 4 ? 2 : 1)>(a, t0, lds);
}

// Few token blocks: the K chunks are cut into ks ranges, one workgroup per
// (token block, range), whose fp32 logits go to part[range][T][E] ...
template <int NBLK>
__global__ __launch_bounds__(256) void route_partial_kernel(RouteArgs a, float* part) {
    MOE_ROUTE_LDS(NBLK);
    const int t0 = blockIdx.x * kBT;
    const int r = blockIdx.y, nr = gridDim.y, n = a.d / kSkChunk;
    const int c0 = (int)((int64_t)r * n / nr), c1 = (int)((int64_t)(r + 1) * n / nr);
    logits_bf16<NB>(a, t0, c0, c1 - c0, lds, sX0, sX1, sX2, sX3, sW0, sW1, sW2, sW3);
    float* out = part + (int64_t)r * a.T * a.E;
    for (int idx = threadIdx.x; idx < kBT * a.E; idx += 256) {
        const int row = idx / a.E, e = idx - row * a.E;
        if (t0 + row < a.T) out[(int64_t)(t0 + row) * a.E + e] = lds[row * kLogitStride + e];
    }
}

// 32 NA tokens per workgroup (NA = kWideNA token blocks of 32) for 129..256
// experts: the W_r chunks a workgroup streams through LDS serve NA times the
// tokens of route_partial_kernel's 32
// (at DeepSeek-V3's shape the router's logits are bound by that stream: every
// workgroup reads all of W_r).  Range r = blockIdx.y of the K chunks; the
// fp32 logits go from the accumulators straight to part[r][T][E].
template <int NA>
__global__ __launch_bounds__(256) void route_partial_wide_kernel(RouteArgs a, float* part) {
    using Sh = SkinnyShape<8, 3, 1, NA>;
    __shared__ __align__(16) uint16_t sX0[Sh::XS], sX1[Sh::XS], sX2[Sh::XS];
    __shared__ __align__(16) uint16_t sW0[Sh::WS], sW1[Sh::WS], sW2[Sh::WS];
    const int t0 = blockIdx.x * (32 * NA);
    const int r = blockIdx.y, nr = gridDim.y, n = a.d / kSkChunk;
    const int c0 = (int)((int64_t)r * n / nr), c1 = (int)((int64_t)(r + 1) * n / nr);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int half = lane >> 5, r32 = lane & 31;
    const int64_t rowb = (int64_t)a.d * 2;
    const int64_t kb = (int64_t)c0 * (kSkChunk * 2);
    // A rows: the 32 NA tokens (rows past T repeat the last); B rows: the experts
    // (rows past E repeat the last)
    const char* src[Sh::P];
#pragma unroll
    for (int ia = 0; ia < Sh::NA; ++ia) {
        const int rx = 32 * ia + 8 * w + (lane >> 3);
        const int tok = min(t0 + rx, a.T - 1);
        src[ia] = static_cast<const char*>(a.x) + tok * rowb + kb + (((lane & 7) ^ swz(rx)) * 16);
    }
#pragma unroll
    for (int j = Sh::NA; j < Sh::P; ++j) {
        const int rw = 8 * (w + 4 * (j - Sh::NA)) + (lane >> 3);
        const int e = min(rw, a.E - 1);
        src[j] = static_cast<const char*>(a.w) + e * rowb + kb + (((lane & 7) ^ swz(rw)) * 16);
    }
    f32x16_t acc[Sh::NA * Sh::BPW];
#pragma unroll
    for (int i = 0; i < Sh::NA * Sh::BPW; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.0f;
    skinny_mma<Sh, false, 0>(src, c1 - c0, 0, sX0, sX1, sX2, sX2, sW0, sW1, sW2, sW2, acc);
    // D element j of tile (ia, i): token row 32 ia + 8 (j / 4) + 4 half + j % 4, expert block w BPW + i
    float* out = part + (int64_t)r * a.T * a.E;
#pragma unroll
    for (int ia = 0; ia < Sh::NA; ++ia)
#pragma unroll
        for (int i = 0; i < Sh::BPW; ++i) {
            const int e = skinny_block<Sh, false>(w, i) * 32 + r32;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int t = t0 + 32 * ia + 8 * (j >> 2) + 4 * half + (j & 3);
                if (t < a.T && e < a.E) out[(int64_t)t * a.E + e] = acc[ia * Sh::BPW + i][j];
            }
        }
}

// ... and one workgroup per token block adds the ranges in order and selects,
// kFinishThreads threads (two tokens per wave: the selection is a chain of
// wave reductions, so few tokens per wave keep it short).  With DISPATCH
// (one token block) the first 256 threads then group the pairs by expert
// (waves that have ended no longer take part in barriers).
constexpr int kFinishThreads = 1024;

template <bool DISPATCH, int QN>
__global__ __launch_bounds__(kFinishThreads) void route_finish_kernel(RouteArgs a, const float* part, int nr,
                                                                      DispatchArgs d) {
    __shared__ float lds[kLogitFloats];
    const int t0 = blockIdx.x * kBT;
    for (int idx = threadIdx.x; idx < kBT * a.E; idx += kFinishThreads) {
        const int row = idx / a.E, e = idx - row * a.E;
        const int t = min(t0 + row, a.T - 1);
        const float* p = part + (int64_t)t * a.E + e;
        const int64_t stride = (int64_t)a.T * a.E;
        // the ranges' values are loaded 8 at a time, then added in range order
        float v = 0.0f;
        for (int r0 = 0; r0 < nr; r0 += 8) {
            float q[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = r0 + i < nr ? p[(r0 + i) * stride] : 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (r0 + i < nr) v += q[i];
        }
        lds[row * kLogitStride + e] = v;
    }
    __syncthreads();
    if (DISPATCH) {
        // the ids of this one block of tokens, from LDS
        __shared__ int s_ids[kBT * 16];
        topk_rows<QN>(a, t0, lds, s_ids);
        __syncthreads();
        if (threadIdx.x >= kDispatchThreads) return;
        DispatchArgs dl = d;
        dl.ids = s_ids;
        dispatch_in_block(dl);
    } else {
        topk_rows<QN>(a, t0, lds);
    }
}

// Statistics of the whole batch from the per-block sums, added in block
// order: f_e = n_e / T, P_e = (sum of probabilities) / T, then (thread 0, in
// expert order) L_aux = alpha E sum_e f_e P_e, max_e n_e / mean_e n_e and the
// capacity overflow sum_e max(0, n_e - cap) ("8.6 Mixture of Experts", sec.
// 3.1; "from the router to the all-to-all", Load balancing; "T2.6 -- What
// Mixture of Experts Changes", In practice).  Counts are whole numbers in
// fp32, exact below 2^24.
__global__ __launch_bounds__(256) void router_stats_kernel(const float* part, int blocks, int E, int T,
                                                           float alpha, int cap, float* out) {
    __shared__ float s_fp[256], s_n[256];
    const int e = threadIdx.x;
    if (e < E) {
        float n = 0.0f, p = 0.0f;
        for (int b = 0; b < blocks; ++b) {
            n += part[(int64_t)b * 2 * E + e];
            p += part[(int64_t)b * 2 * E + E + e];
        }
        const float f = n / (float)T, P = p / (float)T;
        out[e] = f;
        out[E + e] = P;
        s_fp[e] = f * P;
        s_n[e] = n;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float acc = 0.0f, mx = 0.0f, tot = 0.0f, over = 0.0f;
        for (int i = 0; i < E; ++i) {
            acc += s_fp[i];
            mx = fmaxf(mx, s_n[i]);
            tot += s_n[i];
            over += fmaxf(s_n[i] - (float)cap, 0.0f);
        }
        out[2 * E] = alpha * (float)E * acc;
        out[2 * E + 1] = tot > 0.0f ? mx / (tot / (float)E) : 0.0f;
        out[2 * E + 2] = over;
    }
}

}  // namespace

hipError_t launch_router_stats(const float* stats_part, int blocks, int E, int T, float alpha, int cap,
                               float* out, hipStream_t s) {
    if (E < 1 || E > 256 || blocks < 1 || T < 1 || cap < 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(router_stats_kernel, dim3(1), dim3(256), 0, s, stats_part, blocks, E, T, alpha, cap, out);
    return hipGetLastError();
}

int route_ranges(int T, int d, bool bf16) {
    if (!bf16 || T <= 0) return 1;
    const int blocks = (T + kBT - 1) / kBT;
    // about 256 workgroups (one per CU), each range at least 4 chunks of 64
    // (Mixtral prefill, 128 token blocks: 2 ranges, 26 -> 19 us)
    const int r = std::min((256 + blocks - 1) / blocks, d / (4 * kSkChunk));
    return std::max(r, 1);
}

hipError_t launch_route_split(const RouteArgs& a, int ranges, float* part, const DispatchArgs* d,
                              hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    if (ranges < 1 || ranges > a.d / kSkChunk || a.E > 256 || (d && a.T > kBT)) return hipErrorInvalidValue;
    dim3 grid((a.T + kBT - 1) / kBT, ranges), block(256);
    const int nb = (a.E + 31) / 32;
    if (nb <= 1) hipLaunchKernelGGL(route_partial_kernel<1>, grid, block, 0, s, a, part);
    else if (nb <= 2) hipLaunchKernelGGL(route_partial_kernel<2>, grid, block, 0, s, a, part);
    else if (nb <= 4) hipLaunchKernelGGL(route_partial_kernel<4>, grid, block, 0, s, a, part);
    else hipLaunchKernelGGL(route_partial_kernel<8>, grid, block, 0, s, a, part);
    const dim3 fblock(kFinishThreads);
    const DispatchArgs dd = d ? *d : DispatchArgs{};
#define MOE_FINISH(D_, Q_) \
    hipLaunchKernelGGL((route_finish_kernel<D_, Q_>), dim3(grid.x), fblock, 0, s, a, (const float*)part, ranges, dd)
    if (a.E <= 64) {
        if (d) MOE_FINISH(true, 1); else MOE_FINISH(false, 1);
    } else if (a.E <= 128) {
        if (d) MOE_FINISH(true, 2); else MOE_FINISH(false, 2);
    } else {
        if (d) MOE_FINISH(true, 4); else MOE_FINISH(false, 4);
    }
#undef MOE_FINISH
    return hipGetLastError();
}

int route_ranges_wide(int T, int d) {
    if (T <= 0) return 1;
    const int blocks = (T + 32 * kWideNA - 1) / (32 * kWideNA);
    // about 256 workgroups, each range at least 4 chunks of 64 (DeepSeek-V3,
    // 64 blocks of 128 tokens: 4 ranges)
    const int r = std::min((256 + blocks - 1) / blocks, d / (4 * kSkChunk));
    return std::max(r, 1);
}

hipError_t launch_route_split_wide(const RouteArgs& a, int ranges, float* part, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    if (ranges < 1 || ranges > a.d / kSkChunk || a.E > 256 || a.E <= 128 || a.d % kSkChunk)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(route_partial_wide_kernel<kWideNA>, dim3((a.T + 32 * kWideNA - 1) / (32 * kWideNA), ranges),
                       dim3(256), 0, s, a, part);
    hipLaunchKernelGGL((route_finish_kernel<false, 4>), dim3((a.T + kBT - 1) / kBT), dim3(kFinishThreads), 0, s, a,
                       (const float*)part, ranges, DispatchArgs{});
    return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, bool bf16, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    dim3 grid((a.T + kBT - 1) / kBT), block(256);
    const int nb = (a.E + 31) / 32;
    if (!bf16) hipLaunchKernelGGL(route_kernel<0>, grid, block, 0, s, a);
    else if (nb <= 1) hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, a);
    else if (nb <= 2) hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, a);
    else if (nb <= 4) hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
