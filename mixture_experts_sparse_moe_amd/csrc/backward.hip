// Backward pass of the layer for a given routing ("8.6 Mixture of Experts",
// sec. 2: y = sum_i g_i f_i(x); the router learns only through the gates of
// the chosen experts, "Mixture-of-Experts Internals", sec. 2.2).  With dy the
// gradient of the output and the routing (ids, gates) of the forward:
//   pair p (token t, expert e, gate g):  dO_p = g dy_t,  dg_p = <dy_t, f_e(x_t)>
//   dH'_p = dy_t W_down,e        (so dg_p = <dH'_p, h_p> and dH_p = g dH'_p)
//   da = g dH' * u * silu'(a),  du = g dH' * silu(a)   (a, u recomputed)
//   dx_t  = sum over its pairs of (da W_gate,e + du W_up,e) + dl_t W_r (+ shared)
//   dW_down,e = sum_p dO_p h_p^T;  dW_gate,e = sum_p da_p x^T;  dW_up,e likewise
//   dl_t: the gates' Jacobian with respect to the logits times dg; dW_r = dl^T x.
// Gradients are fp32.  Every sum is taken in a fixed order (no atomics).
//
// The GEMMs of the backward are NN (dgrad: the weights are contracted over
// their output dimension) and TN (weight gradients: a sum over each expert's
// rows).  bf16 layers whose widths are multiples of 256 run them on the
// forward's persistent MFMA kernel: the data gradients read the weights as
// they are, through the kernel's N-major B mode (transposed LDS reads), and
// each expert's rows become a range of columns (padded to 128 with zeros) of
// transposed activations, over which the kernel's grouped-K mode sums.  Other shapes use the generic
// grouped GEMMs here (bf16 MFMA with operands transposed on their way into
// LDS, or fp32 FMA), which take any layout.  The recomputation of a and u
// uses the forward's grouped GEMM (on the persistent path one dual-tile
// launch that stores both products).
#include <algorithm>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kGT = 256;                  // threads
constexpr int kGBM = 64, kGBN = 64, kGBK = 16;

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }

template <typename T>
__device__ __forceinline__ void st(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
template <>
__device__ __forceinline__ void st<float>(float* p, int64_t i, float v) { p[i] = v; }

// Output rows of group g in ROWS mode: the M tiles of 64 rows over the groups
// (prefix in LDS, as in the forward GEMM).
template <int BM>
__device__ __forceinline__ bool rows_tile(const GradGemm& a, int mt, int* grp, int* r0, int* nr) {
    if (!a.offsets) {
        *grp = 0;
        *r0 = mt * BM;
        *nr = min(BM, a.M - *r0);
        return *r0 < a.M;
    }
    __shared__ int s_wsum[4], s_res[3];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (threadIdx.x == 0) s_res[0] = -1;
    int nt = 0, cnt = 0, off = 0;
    const int e = threadIdx.x;
    if (e < a.G) {
        off = a.offsets[e];
        cnt = a.offsets[e + 1] - off;
        nt = (cnt + BM - 1) / BM;
    }
    int v = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) s_wsum[w] = v;
    __syncthreads();
    int before = 0;
    for (int q = 0; q < w; ++q) before += s_wsum[q];
    const int incl = v + before, excl = incl - nt;
    if (e < a.G && mt >= excl && mt < incl) {
        s_res[0] = e;
        s_res[1] = off + (mt - excl) * BM;
        s_res[2] = min(BM, cnt - (mt - excl) * BM);
    }
    __syncthreads();
    if (s_res[0] < 0) return false;
    *grp = s_res[0];
    *r0 = s_res[1];
    *nr = s_res[2];
    return true;
}

// C (+)= A B over one 64 x 64 tile; see GradGemm.  Thread (tm, tn) owns a
// 4 x 4 block of outputs; K in steps of 16 through LDS (fp32).
template <typename TA, typename TB, bool KROWS, bool B_KCONT>
__global__ __launch_bounds__(kGT) void grad_gemm_kernel(GradGemm a, int tiles_m, int tiles_n) {
    __shared__ float As[kGBK][kGBM + 4];
    __shared__ float Bs[kGBK][kGBN + 4];
    const int tid = threadIdx.x;
    const int nt = blockIdx.x % tiles_n;
    const int mt = (blockIdx.x / tiles_n) % tiles_m;
    const int gz = blockIdx.x / tiles_n / tiles_m;       // KROWS: the group
    int grp, r0, nr, k0, k1;
    if (KROWS) {
        grp = gz;
        r0 = mt * kGBM;
        nr = min(kGBM, a.M - r0);
        k0 = a.offsets ? a.offsets[grp] : 0;
        k1 = a.offsets ? a.offsets[grp + 1] : a.K;
        if (nr <= 0) return;
    } else {
        if (!rows_tile<kGBM>(a, mt, &grp, &r0, &nr)) return;
        k0 = 0;
        k1 = a.K;
    }
    const int n0 = nt * kGBN;
    const TA* A = static_cast<const TA*>(a.A);
    const TB* B = static_cast<const TB*>(a.B) + (int64_t)grp * a.b_gstride;
    const int tm = tid >> 4, tn = tid & 15;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    for (int kb = k0; kb < k1; kb += kGBK) {
        // A tile -> As[k][m]
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int idx = tid + q * kGT;             // 0 .. 1023
            int m, kk;
            if (KROWS) { kk = idx >> 6; m = idx & 63; }   // M contiguous: consecutive threads, consecutive m
            else { m = idx >> 4; kk = idx & 15; }         // K contiguous
            const int k = kb + kk;
            float v = 0.0f;
            if (m < nr && k < k1) {
                if (KROWS) {
                    v = ld<TA>(A, (int64_t)k * a.lda + r0 + m);
                } else {
                    const int r = r0 + m;
                    const int64_t src = a.a_gather ? a.a_gather[r] / a.a_div : r;
                    v = ld<TA>(A, src * a.lda + k);
                }
            }
            As[kk][m] = v;
        }
        // B tile -> Bs[k][n]
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int idx = tid + q * kGT;
            int n, kk;
            if (B_KCONT) { n = idx >> 4; kk = idx & 15; }
            else { kk = idx >> 6; n = idx & 63; }
            const int k = kb + kk;
            float v = 0.0f;
            if (n0 + n < a.N && k < k1) {
                if (B_KCONT) {
                    v = ld<TB>(B, (int64_t)(n0 + n) * a.ldb + k);
                } else {
                    const int64_t src = (KROWS && a.b_gather) ? a.b_gather[k] / a.b_div : k;
                    v = ld<TB>(B, src * a.ldb + n0 + n);
                }
            }
            Bs[kk][n] = v;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kGBK; ++kk) {
            float x4[4], y4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x4[i] = As[kk][tm * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) y4[j] = Bs[kk][tn * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(x4[i], y4[j], acc[i][j]);
        }
        __syncthreads();
    }
    float* C = a.C + (KROWS ? (int64_t)grp * a.c_gstride : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = tm * 4 + i;
        if (m >= nr) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tn * 4 + j;
            if (n >= a.N) continue;
            float* c = C + (int64_t)(r0 + m) * a.ldc + n;
            *c = a.accumulate ? *c + acc[i][j] : acc[i][j];
        }
    }
}


// The same GEMM on bf16 MFMA for bf16 operands whose contiguous dimension is
// a multiple of 8 elements: 128 x 128 tiles, 4 waves of 64 x 64 (2 x 2 blocks
// of v_mfma_f32_32x32x16_bf16), K in steps of 32.  Operands are loaded 16
// bytes at a time along their contiguous dimension into registers (the next
// K step's loads in flight during this one's MFMAs) and stored to LDS as
// rows of K: directly when K is contiguous, element by element (a transpose)
// when M or N is.  LDS rows are padded to 40 elements against bank conflicts.
constexpr int kMBM = 128, kMBN = 128, kMBK = 32, kMLD = 40;

template <bool KROWS, bool B_KCONT>
__global__ __launch_bounds__(256) void grad_gemm_mfma_kernel(GradGemm a, int tiles_m, int tiles_n) {
    __shared__ __align__(16) uint16_t As[2][kMBM * kMLD];
    __shared__ __align__(16) uint16_t Bs[2][kMBN * kMLD];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int nt = blockIdx.x % tiles_n;
    const int mt = (blockIdx.x / tiles_n) % tiles_m;
    const int gz = blockIdx.x / tiles_n / tiles_m;
    int grp, r0, nr, k0, k1;
    if (KROWS) {
        grp = gz;
        r0 = mt * kMBM;
        nr = min(kMBM, a.M - r0);
        k0 = a.offsets ? a.offsets[grp] : 0;
        k1 = a.offsets ? a.offsets[grp + 1] : a.K;
        if (nr <= 0) return;
    } else {
        if (!rows_tile<kMBM>(a, mt, &grp, &r0, &nr)) return;
        k0 = 0;
        k1 = a.K;
    }
    const int n0 = nt * kMBN;
    const int nn = min(kMBN, a.N - n0);
    const uint16_t* A = static_cast<const uint16_t*>(a.A);
    const uint16_t* B = static_cast<const uint16_t*>(a.B) + (int64_t)grp * a.b_gstride;

    // this thread's two 16-byte pieces of each operand per K step
    uint4 ra0, ra1, rb0, rb1;
    const uint4 zero = make_uint4(0, 0, 0, 0);
#define MOE_G_LOAD_A(ra_, i_, kb_)                                                                  \
    do {                                                                                           \
        if (KROWS) {        /* A(m, k) = A[k lda + m]: 8 m at one k */                             \
            const int k_ = (kb_) + (tid >> 4) + 16 * (i_), m_ = (tid & 15) * 8;                    \
            ra_ = zero;                                                                            \
            if (k_ < k1 && m_ < nr) ra_ = *reinterpret_cast<const uint4*>(A + (int64_t)k_ * a.lda + r0 + m_); \
        } else {            /* A(m, k) = A[src(m) lda + k]: 8 k at one m */                        \
            const int m_ = (tid >> 2) + 64 * (i_), k_ = (kb_) + (tid & 3) * 8;                     \
            ra_ = zero;                                                                            \
            if (m_ < nr && k_ < k1) {                                                              \
                const int r_ = r0 + m_;                                                            \
                const int64_t src_ = a.a_gather ? a.a_gather[r_] / a.a_div : r_;                   \
                ra_ = *reinterpret_cast<const uint4*>(A + src_ * a.lda + k_);                      \
            }                                                                                      \
        }                                                                                          \
    } while (0)
#define MOE_G_LOAD_B(rb_, i_, kb_)                                                                  \
    do {                                                                                           \
        if (B_KCONT) {      /* B(n, k) = B[n ldb + k] */                                           \
            const int n_ = (tid >> 2) + 64 * (i_), k_ = (kb_) + (tid & 3) * 8;                     \
            rb_ = zero;                                                                            \
            if (n_ < nn && k_ < k1) rb_ = *reinterpret_cast<const uint4*>(B + (int64_t)(n0 + n_) * a.ldb + k_); \
        } else {            /* B(n, k) = B[src(k) ldb + n]: 8 n at one k */                        \
            const int k_ = (kb_) + (tid >> 4) + 16 * (i_), n_ = (tid & 15) * 8;                    \
            rb_ = zero;                                                                            \
            if (k_ < k1 && n_ < nn) {                                                              \
                const int64_t src_ = (KROWS && a.b_gather) ? a.b_gather[k_] / a.b_div : k_;        \
                rb_ = *reinterpret_cast<const uint4*>(B + src_ * a.ldb + n0 + n_);                 \
            }                                                                                      \
        }                                                                                          \
    } while (0)
// 8 elements of a 16-byte piece to 8 LDS rows (one column of K)
#define MOE_G_SCATTER(dst_, row_, kk_, v_)                                                          \
    do {                                                                                           \
        uint16_t* d_ = (dst_) + (row_) * kMLD + (kk_);                                             \
        d_[0 * kMLD] = (uint16_t)(v_).x; d_[1 * kMLD] = (uint16_t)((v_).x >> 16);                  \
        d_[2 * kMLD] = (uint16_t)(v_).y; d_[3 * kMLD] = (uint16_t)((v_).y >> 16);                  \
        d_[4 * kMLD] = (uint16_t)(v_).z; d_[5 * kMLD] = (uint16_t)((v_).z >> 16);                  \
        d_[6 * kMLD] = (uint16_t)(v_).w; d_[7 * kMLD] = (uint16_t)((v_).w >> 16);                  \
    } while (0)
#define MOE_G_STORE_A(ra_, i_, buf_)                                                                \
    do {                                                                                           \
        if (KROWS) MOE_G_SCATTER(As[buf_], (tid & 15) * 8, (tid >> 4) + 16 * (i_), ra_);            \
        else *reinterpret_cast<uint4*>(&As[buf_][((tid >> 2) + 64 * (i_)) * kMLD + (tid & 3) * 8]) = ra_; \
    } while (0)
#define MOE_G_STORE_B(rb_, i_, buf_)                                                                \
    do {                                                                                           \
        if (B_KCONT) *reinterpret_cast<uint4*>(&Bs[buf_][((tid >> 2) + 64 * (i_)) * kMLD + (tid & 3) * 8]) = rb_; \
        else MOE_G_SCATTER(Bs[buf_], (tid & 15) * 8, (tid >> 4) + 16 * (i_), rb_);                  \
    } while (0)
#define MOE_G_LOAD(kb_)                                                                             \
    do {                                                                                           \
        MOE_G_LOAD_A(ra0, 0, kb_); MOE_G_LOAD_A(ra1, 1, kb_);                                     \
        MOE_G_LOAD_B(rb0, 0, kb_); MOE_G_LOAD_B(rb1, 1, kb_);                                     \
    } while (0)
#define MOE_G_STORE(buf_)                                                                           \
    do {                                                                                           \
        MOE_G_STORE_A(ra0, 0, buf_); MOE_G_STORE_A(ra1, 1, buf_);                                 \
        MOE_G_STORE_B(rb0, 0, buf_); MOE_G_STORE_B(rb1, 1, buf_);                                 \
    } while (0)

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    const int half = lane >> 5, r32 = lane & 31;
    int buf = 0;
    MOE_G_LOAD(k0);
    MOE_G_STORE(0);
    __syncthreads();
    for (int kb = k0; kb < k1; kb += kMBK) {
        const bool more = kb + kMBK < k1;
        if (more) MOE_G_LOAD(kb + kMBK);
#pragma unroll
        for (int st = 0; st < kMBK / 16; ++st) {
            const int c = (2 * st + half) * 8;
            bf16x8_t af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&As[buf][(wm * 64 + i * 32 + r32) * kMLD + c]));
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = as_bf16x8(*reinterpret_cast<const uint4*>(&Bs[buf][(wn * 64 + j * 32 + r32) * kMLD + c]));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (more) MOE_G_STORE(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
#undef MOE_G_LOAD_A
#undef MOE_G_LOAD_B
#undef MOE_G_SCATTER
#undef MOE_G_STORE_A
#undef MOE_G_STORE_B
#undef MOE_G_LOAD
#undef MOE_G_STORE
    float* C = a.C + (KROWS ? (int64_t)grp * a.c_gstride : 0);
    // element q of block (i, j): row 8 (q / 4) + 4 half + q % 4, column r32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = wn * 64 + j * 32 + r32;
            if (n >= nn) continue;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int m = wm * 64 + i * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
                if (m >= nr) continue;
                float* cp = C + (int64_t)(r0 + m) * a.ldc + n0 + n;
                *cp = a.accumulate ? *cp + acc[i][j][q] : acc[i][j][q];
            }
        }
}

// One workgroup per grouped row r (pair p = sorted[r], or token r when there
// is no grouping): h = silu(a) u; dg = <dH', h>; da, du; dO = g dy.
template <typename T>
__global__ __launch_bounds__(256) void bwd_pair_kernel(BwdPairArgs b) {
    const int r = blockIdx.x;
    if (b.offsets && r >= b.offsets[b.G]) return;
    const int p = b.sorted ? b.sorted[r] : r;
    const int t = b.sorted ? p / b.k : r;
    const float g = b.gates ? b.gates[p] : 1.0f;
    const T* A = static_cast<const T*>(b.a) + (int64_t)r * b.f;
    const T* U = static_cast<const T*>(b.u) + (int64_t)r * b.f;
    const float* dHp = b.dhp + (int64_t)r * b.f;
    T* H = static_cast<T*>(b.h) + (int64_t)r * b.f;
    const int64_t ldd = b.ld_dadu ? b.ld_dadu : b.f;
    T* DA = static_cast<T*>(b.da) + (int64_t)r * ldd;
    T* DU = static_cast<T*>(b.du) + (int64_t)r * ldd;
    float part = 0.0f;
    for (int i = threadIdx.x; i < b.f; i += 256) {
        const float av = ld<T>(A, i), uv = ld<T>(U, i), d = dHp[i];
        const float sg = 1.0f / (1.0f + expf(-av));
        const float hv = av * sg * uv;
        st<T>(H, i, hv);
        part = fmaf(d, hv, part);
        const float dh = g * d;
        st<T>(DA, i, dh * uv * (sg * (1.0f + av * (1.0f - sg))));
        st<T>(DU, i, dh * av * sg);
    }
    if (b.dgate) {
        // fixed-order sum: per thread, then threads in index order
        __shared__ float s_part[256];
        s_part[threadIdx.x] = part;
        __syncthreads();
        if (threadIdx.x == 0) {
            float v = 0.0f;
            for (int i = 0; i < 256; ++i) v += s_part[i];
            b.dgate[p] = v;
        }
    }
    if (b.d_o) {
        const T* dy = static_cast<const T*>(b.dy) + (int64_t)t * b.dm;
        T* dO = static_cast<T*>(b.d_o) + (int64_t)r * b.dm;
        for (int i = threadIdx.x; i < b.dm; i += 256) st<T>(dO, i, g * ld<T>(dy, i));
    }
}

// One wave per token: dl[t, :] from dg of its k pairs (pair p = t k + j) and,
// when needed, the recomputed logits.
__global__ __launch_bounds__(256) void bwd_router_kernel(BwdRouterArgs b) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= b.T) return;
    float* dl = b.dl + (int64_t)t * b.E;
    const int32_t* id = b.ids + (int64_t)t * b.k;
    const float* gate = b.gates + (int64_t)t * b.k;
    const float* dg = b.dgate + (int64_t)t * b.k;
    const float* l = b.logits ? b.logits + (int64_t)t * b.E : nullptr;
    // sum_j g_j dg_j over the chosen (the gates as the forward computed them)
    float gdg = 0.0f;
    for (int j = 0; j < b.k; ++j) gdg = fmaf(gate[j], dg[j], gdg);
    // each lane writes its own experts' entries (0 for experts not chosen,
    // except for softmax without renormalisation, where every logit matters)
    float mx = 0.0f, z = 1.0f, ssum = 0.0f;
    if (b.score_fn == 0 && !b.renorm) {
        mx = -__builtin_inff();
        for (int e = 0; e < b.E; ++e) mx = fmaxf(mx, l[e]);
        z = 0.0f;
        for (int e = 0; e < b.E; ++e) z += expf(l[e] - mx);
    }
    if (b.score_fn == 1)
        for (int j = 0; j < b.k; ++j) ssum += 1.0f / (1.0f + expf(-l[id[j]]));
    // load-balancing loss: the token's router probabilities p (softmax) or
    // q = s / sum s (sigmoid s), and their mean fraction fbar = <f, p>
    float amx = 0.0f, anorm = 1.0f, fbar = 0.0f;
    if (b.aux_coef != 0.0f) {
        if (b.score_fn == 0) {
            amx = -__builtin_inff();
            for (int m = 0; m < b.E; ++m) amx = fmaxf(amx, l[m]);
            anorm = 0.0f;
            for (int m = 0; m < b.E; ++m) anorm += expf(l[m] - amx);
            for (int m = 0; m < b.E; ++m) fbar += (float)b.aux_counts[m] * b.inv_T * (expf(l[m] - amx) / anorm);
        } else {
            anorm = 0.0f;
            for (int m = 0; m < b.E; ++m) anorm += 1.0f / (1.0f + expf(-l[m]));
            for (int m = 0; m < b.E; ++m)
                fbar += (float)b.aux_counts[m] * b.inv_T * (1.0f / (1.0f + expf(-l[m])) / anorm);
        }
    }
    for (int e = lane; e < b.E; e += 64) {
        int j = -1;
        for (int q = 0; q < b.k; ++q)
            if (id[q] == e) j = q;
        float v = 0.0f;
        if (b.score_fn == 0 && b.renorm) {
            // g = softmax over the chosen logits: dl_i = g_i (dg_i - sum_j g_j dg_j)
            if (j >= 0) v = gate[j] * (dg[j] - gdg);
        } else if (b.score_fn == 0) {
            // g_i = s_i, the softmax over all E: dl_e = s_e (dg_e - sum_j s_{e_j} dg_j)
            v = expf(l[e] - mx) / z * ((j >= 0 ? dg[j] : 0.0f) - gdg);
        } else if (j >= 0) {
            // sigmoid s_i; renormalised: g_i = s_i / S, ds_i = (dg_i - sum_j g_j dg_j) / S
            const float sg = 1.0f / (1.0f + expf(-l[e]));
            const float ds = b.renorm ? (dg[j] - gdg) / ssum : dg[j];
            v = ds * sg * (1.0f - sg);
        }
        if (b.aux_coef != 0.0f) {
            // dL_aux/dl_e = aux_coef p_e (f_e - fbar); for the normalised sigmoid
            // the Jacobian adds the factor (1 - s_e)
            float pe;
            if (b.score_fn == 0) {
                pe = expf(l[e] - amx) / anorm;
            } else {
                const float sg = 1.0f / (1.0f + expf(-l[e]));
                pe = sg / anorm * (1.0f - sg);
            }
            v += b.aux_coef * pe * ((float)b.aux_counts[e] * b.inv_T - fbar);
        }
        dl[e] = v;
    }
}

__global__ __launch_bounds__(1024) void count_ids_kernel(const int32_t* ids, int64_t P, int E, int32_t* counts) {
    __shared__ int hist[256];
    for (int e = threadIdx.x; e < E; e += 1024) hist[e] = 0;
    __syncthreads();
    for (int64_t p = threadIdx.x; p < P; p += 1024) {
        const int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 1024) counts[e] = hist[e];
}

// dx[t, :] = sum over the token's pairs, in slot order, of dXp[pair_pos].
// dx[t] = sum over the token's slots j (and K slices s, in that order) of
// dxp[s][pair_pos[t k + j]].
__global__ __launch_bounds__(256) void bwd_token_sum_kernel(const float* dxp, const int32_t* pair_pos, int k, int d,
                                                            float* dx, int splitk, int64_t part_stride) {
    const int t = blockIdx.x;
    int pos[16];                     // k <= 16
#pragma unroll
    for (int j = 0; j < 16; ++j) pos[j] = j < k ? pair_pos[(int64_t)t * k + j] : -1;
    // 4 columns per thread (d % 4 == 0, slices and rows 16-byte aligned); each
    // column still sums slots in order, slices in order
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
        float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (pos[j] < 0) continue;
            for (int sl = 0; sl < splitk; ++sl) {
                const float4 q = *reinterpret_cast<const float4*>(dxp + sl * part_stride + (int64_t)pos[j] * d + c);
                v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
            }
        }
        *reinterpret_cast<float4*>(dx + (int64_t)t * d + c) = v;
    }
}

// Router weight gradient dW_r[e][i] = sum_t dl[t][e] x[t][i] (E rows only, so a
// GEMM tile would sit mostly idle): workgroup (column block, token chunk)
// gives each thread one column and 16 experts at a time in registers, the
// chunk's dl rows staged 32 tokens at a time in LDS.  out: the chunk's
// partial sums [chunk][E][d] (or dW_r itself with one chunk).
constexpr int kRwE = 16, kRwTok = 32;
template <typename TX>
__global__ __launch_bounds__(256) void router_wgrad_kernel(const float* dl, const TX* x, int T, int E, int d,
                                                           int chunk_tokens, float* out) {
    __shared__ float s_dl[kRwTok][kRwE];
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int c = blockIdx.y;
    const int t0 = c * chunk_tokens, t1 = min(T, t0 + chunk_tokens);
    for (int eg = 0; eg < E; eg += kRwE) {
        float acc[kRwE];
#pragma unroll
        for (int j = 0; j < kRwE; ++j) acc[j] = 0.0f;
        for (int tb = t0; tb < t1; tb += kRwTok) {
            for (int q = threadIdx.x; q < kRwTok * kRwE; q += 256) {
                const int tt = q / kRwE, j = q % kRwE;
                s_dl[tt][j] = (tb + tt < t1 && eg + j < E) ? dl[(int64_t)(tb + tt) * E + eg + j] : 0.0f;
            }
            __syncthreads();
            const int nt = min(kRwTok, t1 - tb);
            if (i < d) {
                for (int tt = 0; tt < nt; ++tt) {
                    const float xv = ld<TX>(x, (int64_t)(tb + tt) * d + i);
#pragma unroll
                    for (int j = 0; j < kRwE; ++j) acc[j] = fmaf(s_dl[tt][j], xv, acc[j]);
                }
            }
            __syncthreads();
        }
        if (i < d) {
#pragma unroll
            for (int j = 0; j < kRwE; ++j)
                if (eg + j < E) out[((int64_t)c * E + eg + j) * d + i] = acc[j];
        }
    }
}

// The router weight gradient as one bf16 product on the persistent kernel:
// out [E, 2 Tr] gets out[e][t] = hi and out[e][Tr + t] = lo, where hi is dl[t][e]
// rounded to bf16 and lo the rest rounded to bf16 (zero for T <= t < Tr), so
// that hi x + lo x carries about 16 bits of dl.  64 x 64 tiles through LDS:
// reads along E, writes along t.
__global__ __launch_bounds__(256) void dl_split_kernel(const float* dl, int T, int E, int Tr, uint16_t* out) {
    __shared__ float tile[64][65];
    const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int tt = i >> 6, ee = i & 63;
        tile[tt][ee] = (t0 + tt < T && e0 + ee < E) ? dl[(int64_t)(t0 + tt) * E + e0 + ee] : 0.0f;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int ee = i >> 6, tt = i & 63;
        if (e0 + ee >= E) continue;
        const float v = tile[tt][ee];
        const uint16_t hi = f32_to_bf16(v);
        uint16_t* row = out + (int64_t)(e0 + ee) * 2 * Tr + t0 + tt;
        row[0] = hi;
        row[Tr] = f32_to_bf16(v - bf16_to_f32(hi));
    }
}

// out [T, 2 E] bf16: out[t][e] = dl[t][e] rounded to bf16, out[t][E + e] the
// rest rounded to bf16 (the router's part of dx, dl W_r, as one bf16 product
// over 2 E columns against W_r read twice).
__global__ __launch_bounds__(256) void dl_rows_kernel(const float* dl, int64_t n, int E, uint16_t* out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t t = i / E, e = i - t * E;
    const float v = dl[i];
    const uint16_t hi = f32_to_bf16(v);
    out[t * 2 * E + e] = hi;
    out[t * 2 * E + E + e] = f32_to_bf16(v - bf16_to_f32(hi));
}

// p[0 .. n) = 0 (a fill kernel rather than a memset, so the call stays capturable).
__global__ __launch_bounds__(256) void fill_zero_f32_kernel(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}

// dst[j] = sum over chunks c (in order) of part[c * n + j].
__global__ __launch_bounds__(256) void sum_chunks_kernel(const float* part, int chunks, int64_t n, float* dst) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= n) return;
    float v = 0.0f;
    for (int c = 0; c < chunks; ++c) v += part[c * n + j];
    dst[j] = v;
}

// ---- transposes feeding the backward's weight gradients on the forward kernel ----------
// Its grouped-K mode reads both operands along K, and the weight gradients
// sum over rows, so the pairs' activations are transposed first (HBM-bound
// copies, 64 x 64 tiles through LDS).

constexpr int kTT = 64;   // transpose tile edge

// Rows of each group as columns: for q < kofs[G] (one group: q < kpad), in the
// group e with kofs[e] <= q < kofs[e + 1] and j = q - kofs[e]:
//   dst[c][q] = scale(p) src[row][c] if j < n_e (grouped row r = off[e] + j,
//   p = gather[r] or r, row = p / div or r), else 0.
// kofs values are multiples of 128, so a 64-column tile lies in one group.
__global__ __launch_bounds__(256) void transpose_rows_kernel(TransposeRowsArgs a) {
    __shared__ uint16_t tile[kTT][kTT + 2];
    const int q0 = blockIdx.x * kTT, c0 = blockIdx.y * kTT;
    const int total = a.offsets ? a.kofs[a.G] : a.kpad;
    if (q0 >= total) return;
    int e = 0;
    if (a.offsets) {
        int lo = 0, hi = a.G;                        // kofs[lo] <= q0 < kofs[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.kofs[mid] <= q0) lo = mid; else hi = mid;
        }
        e = lo;
    }
    const int kbeg = a.offsets ? a.kofs[e] : 0;
    const int roff = a.offsets ? a.offsets[e] : 0;
    const int n = a.offsets ? a.offsets[e + 1] - roff : a.M;
    const int t = threadIdx.x, cc = (t & 7) * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int ql = (t >> 3) + 32 * h;
        const int j = q0 + ql - kbeg;
        uint32_t w4[4] = {0u, 0u, 0u, 0u};
        if (j < n) {
            const int r = roff + j;
            const int p = a.gather ? a.gather[r] : r;
            const int row = a.gather ? p / a.div : r;
            const uint4 v = *reinterpret_cast<const uint4*>(a.src + (int64_t)row * a.ld_src + c0 + cc);
            w4[0] = v.x; w4[1] = v.y; w4[2] = v.z; w4[3] = v.w;
            if (a.scale) {
                const float g = a.scale[p];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    w4[i] = pack_bf16x2(g * bf16_to_f32((uint16_t)(w4[i] & 0xFFFFu)),
                                        g * bf16_to_f32((uint16_t)(w4[i] >> 16)));
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            tile[ql][cc + 2 * i] = (uint16_t)(w4[i] & 0xFFFFu);
            tile[ql][cc + 2 * i + 1] = (uint16_t)(w4[i] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = (t >> 3) + 32 * h;
        uint32_t w4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w4[i] = (uint32_t)tile[cc + 2 * i][c] | ((uint32_t)tile[cc + 2 * i + 1][c] << 16);
        *reinterpret_cast<uint4*>(a.dst + (int64_t)(c0 + c) * a.ld_dst + q0 + cc) =
            make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
}

// kofs[e] = sum over e' < e of n_e' rounded up to 128 (an expert with no rows
// takes 128 zero columns, so its weight gradients come out zero).  One block.
__global__ __launch_bounds__(256) void kgroup_offsets_kernel(const int32_t* offsets, int G, int32_t* kofs) {
    __shared__ int s_w[4];
    const int e = threadIdx.x, lane = e & 63, w = e >> 6;
    int v = 0;
    if (e < G) {
        const int n = offsets[e + 1] - offsets[e];
        v = n > 0 ? (n + 127) / 128 * 128 : 128;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) s_w[w] = v;
    __syncthreads();
    for (int q = 0; q < w; ++q) v += s_w[q];
    if (e < G) kofs[e + 1] = v;
    if (e == 0) kofs[0] = 0;
}

template <typename TA, typename TB>
hipError_t launch_grad_gemm_t(const GradGemm& a, bool krows, bool b_kcont, hipStream_t s) {
    const int tiles_n = (a.N + kGBN - 1) / kGBN;
    int tiles_m, groups;
    if (krows) {
        tiles_m = (a.M + kGBM - 1) / kGBM;
        groups = a.offsets ? a.G : 1;
    } else {
        tiles_m = (int)(a.offsets ? grouped_m_tiles_upper(a.M, a.G, kGBM) : (a.M + kGBM - 1) / kGBM);
        groups = 1;
    }
    const int64_t grid = (int64_t)tiles_m * tiles_n * groups;
    if (grid == 0) return hipSuccess;
    if (grid > INT32_MAX || (krows && b_kcont)) return hipErrorInvalidValue;
    const dim3 g3((unsigned)grid), b3(kGT);
    if (krows) hipLaunchKernelGGL((grad_gemm_kernel<TA, TB, true, false>), g3, b3, 0, s, a, tiles_m, tiles_n);
    else if (b_kcont) hipLaunchKernelGGL((grad_gemm_kernel<TA, TB, false, true>), g3, b3, 0, s, a, tiles_m, tiles_n);
    else hipLaunchKernelGGL((grad_gemm_kernel<TA, TB, false, false>), g3, b3, 0, s, a, tiles_m, tiles_n);
    return hipGetLastError();
}

// bf16 operands whose contiguous dimensions and strides are multiples of 8
// elements (16-byte pieces) go to the MFMA kernel.
bool mfma_fits(const GradGemm& a, bool krows, bool b_kcont) {
    auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (!al(a.A) || !al(a.B) || a.lda % 8 || a.ldb % 8 || a.b_gstride % 8) return false;
    const bool a_ok = krows ? a.M % 8 == 0 : a.K % 8 == 0;
    const bool b_ok = b_kcont ? a.K % 8 == 0 : a.N % 8 == 0;
    return a_ok && b_ok;
}

hipError_t launch_grad_gemm_mfma(const GradGemm& a, bool krows, bool b_kcont, hipStream_t s) {
    const int tiles_n = (a.N + kMBN - 1) / kMBN;
    int tiles_m, groups;
    if (krows) {
        tiles_m = (a.M + kMBM - 1) / kMBM;
        groups = a.offsets ? a.G : 1;
    } else {
        tiles_m = (int)(a.offsets ? grouped_m_tiles_upper(a.M, a.G, kMBM) : (a.M + kMBM - 1) / kMBM);
        groups = 1;
    }
    const int64_t grid = (int64_t)tiles_m * tiles_n * groups;
    if (grid == 0) return hipSuccess;
    if (grid > INT32_MAX || (krows && b_kcont)) return hipErrorInvalidValue;
    const dim3 g3((unsigned)grid), b3(256);
    if (krows) hipLaunchKernelGGL((grad_gemm_mfma_kernel<true, false>), g3, b3, 0, s, a, tiles_m, tiles_n);
    else if (b_kcont) hipLaunchKernelGGL((grad_gemm_mfma_kernel<false, true>), g3, b3, 0, s, a, tiles_m, tiles_n);
    else hipLaunchKernelGGL((grad_gemm_mfma_kernel<false, false>), g3, b3, 0, s, a, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grad_gemm(const GradGemm& a, bool krows, bool b_kcont, bool a_bf16, bool b_bf16, hipStream_t s) {
    if (a.G > 256) return hipErrorInvalidValue;
    if (a_bf16 && b_bf16 && mfma_fits(a, krows, b_kcont)) return launch_grad_gemm_mfma(a, krows, b_kcont, s);
    if (a_bf16 && b_bf16) return launch_grad_gemm_t<uint16_t, uint16_t>(a, krows, b_kcont, s);
    if (!a_bf16 && b_bf16) return launch_grad_gemm_t<float, uint16_t>(a, krows, b_kcont, s);
    if (!a_bf16 && !b_bf16) return launch_grad_gemm_t<float, float>(a, krows, b_kcont, s);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_pair(const BwdPairArgs& b, int rows, bool bf16, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (bf16) hipLaunchKernelGGL(bwd_pair_kernel<uint16_t>, dim3(rows), dim3(256), 0, s, b);
    else hipLaunchKernelGGL(bwd_pair_kernel<float>, dim3(rows), dim3(256), 0, s, b);
    return hipGetLastError();
}

hipError_t launch_bwd_router(const BwdRouterArgs& b, hipStream_t s) {
    if (b.T <= 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_router_kernel, dim3((b.T + 3) / 4), dim3(256), 0, s, b);
    return hipGetLastError();
}

hipError_t launch_bwd_token_sum(const float* dxp, const int32_t* pair_pos, int T, int k, int d, float* dx,
                                hipStream_t s, int splitk, int64_t part_stride) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_token_sum_kernel, dim3(T), dim3(256), 0, s, dxp, pair_pos, k, d, dx, splitk, part_stride);
    return hipGetLastError();
}

hipError_t launch_count_ids(const int32_t* ids, int64_t P, int E, int32_t* counts, hipStream_t s) {
    if (E < 1 || E > 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL(count_ids_kernel, dim3(1), dim3(1024), 0, s, ids, P, E, counts);
    return hipGetLastError();
}

hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(fill_zero_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

int router_wgrad_chunks(int T, int d, int E) {
    const int col_blocks = (d + 255) / 256;
    const int want = (1024 + col_blocks - 1) / col_blocks;       // about 1024 workgroups
    const int most = std::max(1, (T + 31) / 32);                 // at least 32 tokens a chunk
    const int64_t cap = std::max<int64_t>(1, (int64_t(64) << 20) / ((int64_t)E * d * 4));   // partials <= 64 MB
    return (int)std::max<int64_t>(1, std::min<int64_t>(std::min(want, most), cap));
}

hipError_t launch_router_wgrad(const float* dl, const void* x, bool x_bf16, int T, int E, int d, float* part,
                               float* dwr, hipStream_t s) {
    if (E <= 0 || d <= 0) return hipSuccess;
    const int chunks = router_wgrad_chunks(T, d, E);
    const int per = chunks > 1 ? ((T + chunks - 1) / chunks + kRwTok - 1) / kRwTok * kRwTok : std::max(T, 1);
    const int used = std::max(1, (T + per - 1) / per);            // chunks that hold tokens
    float* out = used > 1 ? part : dwr;
    const dim3 grid((d + 255) / 256, used);
    if (x_bf16)
        hipLaunchKernelGGL(router_wgrad_kernel<uint16_t>, grid, dim3(256), 0, s, dl,
                           static_cast<const uint16_t*>(x), T, E, d, per, out);
    else
        hipLaunchKernelGGL(router_wgrad_kernel<float>, grid, dim3(256), 0, s, dl, static_cast<const float*>(x), T, E,
                           d, per, out);
    if (used > 1) {
        const int64_t n = (int64_t)E * d;
        hipLaunchKernelGGL(sum_chunks_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, used, n, dwr);
    }
    return hipGetLastError();
}

hipError_t launch_dl_split(const float* dl, int T, int E, int Tr, uint16_t* out, hipStream_t s) {
    if (T < 0 || E <= 0 || Tr < T || Tr % 64) return hipErrorInvalidValue;
    if (Tr == 0) return hipSuccess;
    hipLaunchKernelGGL(dl_split_kernel, dim3(Tr / 64, (E + 63) / 64), dim3(256), 0, s, dl, T, E, Tr, out);
    return hipGetLastError();
}

hipError_t launch_dl_rows(const float* dl, int T, int E, uint16_t* out, hipStream_t s) {
    const int64_t n = (int64_t)T * E;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(dl_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dl, n, E, out);
    return hipGetLastError();
}

hipError_t launch_sum_chunks(const float* part, int chunks, int64_t n, float* dst, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(sum_chunks_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, chunks, n, dst);
    return hipGetLastError();
}

hipError_t launch_transpose_rows(const TransposeRowsArgs& a, int64_t cols_upper, hipStream_t s) {
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (a.C % kTT || a.ld_src % 8 || a.ld_dst % 8 || !al16(a.src) || !al16(a.dst) || cols_upper % 128 ||
        cols_upper > a.ld_dst || (a.offsets && (!a.kofs || a.G < 1 || a.G > 256)) ||
        (!a.offsets && (a.kpad % 128 || a.kpad < a.M || a.kpad > cols_upper)))
        return hipErrorInvalidValue;
    if (a.C == 0 || cols_upper == 0) return hipSuccess;
    hipLaunchKernelGGL(transpose_rows_kernel, dim3((unsigned)(cols_upper / kTT), a.C / kTT), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_kgroup_offsets(const int32_t* offsets, int G, int32_t* kofs, hipStream_t s) {
    if (G < 1 || G > 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kgroup_offsets_kernel, dim3(1), dim3(256), 0, s, offsets, G, kofs);
    return hipGetLastError();
}

}  // namespace moe
