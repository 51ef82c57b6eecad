// Grouped GEMMs of the expert SwiGLU FFNs ("8.6 Mixture of Experts" sec. 2;
// "What Actually Happens When a Token Hits the Router", Step 4).
//
// For each group (expert) e with grouped rows [off[e], off[e+1]):
//   dual:   C[r, n] = silu(sum_k A[src(r), k] B0[e, n, k]) * (sum_k A[src(r), k] B1[e, n, k])
//   single: C[r, n] = sum_k A[src(r), k] B0[e, n, k]
// src(r) = gather[r] / gather_div (token of the pair) when gathering, else r.
// Both operands are K-contiguous ("NT"), the natural MFMA operand layout.
//
// bf16 kernel (gfx950):
//   - v_mfma_f32_32x32x16_bf16, fp32 accumulation.
//   - Workgroup 256 threads = 2x2 waves on a BM x BN output tile (x2 weight
//     matrices in dual mode: the gate and up tiles of the same columns sit
//     in the same lanes, so silu(g)*u is a register-only epilogue).
//   - BK = 64.  Global -> registers -> LDS, double-buffered: the next K tile
//     is in flight while the MFMAs consume the current one; one barrier per
//     K tile.  A rows are gathered on load (no permuted copy of x).
//   - LDS rows are 64 bf16 = 8 chunks of 16 B; chunk c of row r is stored at
//     c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1), so the 16-byte fragment reads
//     of 32 consecutive rows hit distinct banks.
//   - M tiles are data dependent: tile mt of the flattened list maps to
//     (expert, row range) by a prefix sum of ceil(count_e / BM) done in the
//     workgroup, so no host sync is needed; the grid is sized by the upper
//     bound ceil(rows / BM) + G and surplus tiles exit at once.
//   - Workgroup ids are remapped so that the 8 XCDs (ids dealt round-robin)
//     each run a contiguous range of logical tiles; logical tiles run WMW
//     M-tiles at a time per N column, so tiles sharing a weight panel are
//     resident in the same XCD's L2 together.
// fp32 kernel: LDS-tiled FMA (the tiny fp32 layer only).
#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kWMW = 4;   // M tiles per window (share one weight panel)

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Block-wide: map flattened M tile `mt` to (group, first row, rows).  Returns
// false if mt is past the last real tile.
template <int BM>
__device__ bool locate_tile(const GemmGroup& g, int mt, int* grp, int* row0, int* nrows) {
    if (g.offsets == nullptr) {
        const int r0 = mt * BM;
        if (r0 >= g.M) return false;
        *grp = 0;
        *row0 = r0;
        *nrows = min(BM, g.M - r0);
        return true;
    }
    __shared__ int s_wsum[8];      // one slot per wave, up to 512 threads
    __shared__ int s_res[3];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (threadIdx.x == 0) s_res[0] = -1;
    int nt = 0, cnt = 0, off = 0;
    const int e = threadIdx.x;
    if (e < g.G) {
        off = g.offsets[e];
        cnt = g.offsets[e + 1] - off;
        nt = (cnt + BM - 1) / BM;
    }
    int v = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) s_wsum[w] = v;
    __syncthreads();
    int before = 0;
    for (int q = 0; q < w; ++q) before += s_wsum[q];
    const int incl = v + before, excl = incl - nt;
    if (e < g.G && mt >= excl && mt < incl) {
        s_res[0] = e;
        s_res[1] = off + (mt - excl) * BM;
        s_res[2] = min(BM, cnt - (mt - excl) * BM);
    }
    __syncthreads();
    if (s_res[0] < 0) return false;
    *grp = s_res[0];
    *row0 = s_res[1];
    *nrows = s_res[2];
    return true;
}

// Logical tile of this workgroup: XCD-contiguous, then windows of kWMW M tiles
// per N column.
__device__ __forceinline__ void logical_tile(int tiles_n, int mt_upper, int* mt, int* nt) {
    const int grid = gridDim.x;              // multiple of 8
    const int wid = blockIdx.x;
    const int L = (wid & 7) * (grid >> 3) + (wid >> 3);
    const int per_win = tiles_n * kWMW;
    const int win = L / per_win;
    const int rem = L - win * per_win;
    const int wm = min(kWMW, mt_upper - win * kWMW);
    if (wm <= 0) { *mt = mt_upper; *nt = 0; return; }
    *nt = rem / wm;
    *mt = win * kWMW + rem % wm;
}

template <int BM, int BN, bool DUAL>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(GemmGroup g, int tiles_n, int mt_upper) {
    constexpr int NMAT = DUAL ? 2 : 1;
    constexpr int WM = BM / 2, WN = BN / 2;       // per-wave tile
    constexpr int FM = WM / 32, FN = WN / 32;     // 32x32 MFMA blocks per wave
    constexpr int A_CHUNKS = BM * 8 / kThreads;   // 16-byte chunks per thread per K tile
    constexpr int B_CHUNKS = BN * 8 / kThreads;
    static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small");

    extern __shared__ __align__(16) uint16_t lds[];
    uint16_t* As = lds;                                 // [2][BM][64]
    uint16_t* Bs = lds + 2 * BM * kBK;                  // [2][NMAT][BN][64]

    int mt, ntile;
    logical_tile(tiles_n, mt_upper, &mt, &ntile);
    if (mt >= mt_upper || ntile >= tiles_n) return;
    int grp, row0, nrows;
    if (!locate_tile<BM>(g, mt, &grp, &row0, &nrows)) return;
    const int n0 = ntile * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int K = g.K;
    const int KT = K / kBK;

    // global source pointers of this thread's chunks
    const uint16_t* A = static_cast<const uint16_t*>(g.A);
    const int kc = tid & 7;
    const uint16_t* a_src[A_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        int r = (tid >> 3) + i * (kThreads / 8);
        int rr = min(r, nrows - 1);
        int src = g.gather ? g.gather[row0 + rr] / g.gather_div : row0 + rr;
        a_src[i] = A + (int64_t)src * K + kc * 8;
    }
    const uint16_t* b_src[NMAT][B_CHUNKS];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        const uint16_t* B = static_cast<const uint16_t*>(m == 0 ? g.B0 : g.B1);
        B += (int64_t)grp * g.N * K;
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) {
            int n = (tid >> 3) + i * (kThreads / 8);
            b_src[m][i] = B + (int64_t)(n0 + n) * K + kc * 8;
        }
    }

    uint4 ra[A_CHUNKS], rb[NMAT][B_CHUNKS];
#define MOE_LOAD_REGS(kt_)                                                                   \
    do {                                                                                     \
        _Pragma("unroll") for (int i = 0; i < A_CHUNKS; ++i) ra[i] =                         \
            *reinterpret_cast<const uint4*>(a_src[i] + (kt_) * kBK);                         \
        _Pragma("unroll") for (int m = 0; m < NMAT; ++m)                                     \
            _Pragma("unroll") for (int i = 0; i < B_CHUNKS; ++i) rb[m][i] =                  \
                *reinterpret_cast<const uint4*>(b_src[m][i] + (kt_) * kBK);                  \
    } while (0)
#define MOE_STORE_LDS(buf_)                                                                  \
    do {                                                                                     \
        _Pragma("unroll") for (int i = 0; i < A_CHUNKS; ++i) {                               \
            const int r = (tid >> 3) + i * (kThreads / 8);                                   \
            *reinterpret_cast<uint4*>(As + (buf_) * BM * kBK + r * kBK + ((kc ^ swz(r)) * 8)) = \
                ra[i];                                                                       \
        }                                                                                    \
        _Pragma("unroll") for (int m = 0; m < NMAT; ++m)                                     \
            _Pragma("unroll") for (int i = 0; i < B_CHUNKS; ++i) {                           \
                const int n = (tid >> 3) + i * (kThreads / 8);                               \
                *reinterpret_cast<uint4*>(Bs + ((buf_) * NMAT + m) * BN * kBK + n * kBK +    \
                                          ((kc ^ swz(n)) * 8)) = rb[m][i];                   \
            }                                                                                \
    } while (0)

    f32x16_t acc[NMAT][FM][FN];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[m][i][j][q] = 0.0f;

    const int half = lane >> 5, r32 = lane & 31;
    MOE_LOAD_REGS(0);
    MOE_STORE_LDS(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        // prefetch the next K tile (the last iteration reloads its own tile;
        // keeping the load unconditional keeps the staging in registers)
        const int kn = kt + 1 < KT ? kt + 1 : kt;
        MOE_LOAD_REGS(kn);
        const uint16_t* Ab = As + cur * BM * kBK;
        const uint16_t* Bb = Bs + cur * NMAT * BN * kBK;
#pragma unroll
        for (int s = 0; s < kBK / 16; ++s) {
            const int c = 2 * s + half;
            bf16x8_t af[FM], bfr[NMAT][FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * WM + i * 32 + r32;
                af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(Ab + r * kBK + ((c ^ swz(r)) * 8)));
            }
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = wn * WN + j * 32 + r32;
                    bfr[m][j] = as_bf16x8(*reinterpret_cast<const uint4*>(
                        Bb + m * BN * kBK + n * kBK + ((c ^ swz(n)) * 8)));
                }
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[m][j],
                                                                               acc[m][i][j], 0, 0, 0);
        }
        MOE_STORE_LDS(cur ^ 1);   // unused after the last iteration
        __syncthreads();
    }

#undef MOE_LOAD_REGS
#undef MOE_STORE_LDS
    // epilogue: D element q of block (i, j): row 8*(q/4) + 4*half + q%4, col r32
    uint16_t* C = static_cast<uint16_t*>(g.C);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WN + j * 32 + r32;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int r = wm * WM + i * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
                if (r < nrows) {
                    float v = acc[0][i][j][q];
                    if (DUAL) v = silu_f32(v) * acc[NMAT - 1][i][j][q];
                    C[(int64_t)(row0 + r) * g.N + col] = f32_to_bf16(v);
                }
            }
        }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kBKs = 32;   // K elements per pipeline stage of the 256 kernel
// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]).  The builtin, unlike inline asm, is seen by the
// compiler's own wait insertion, so it adds no waits of its own after these.
constexpr int kWaitVm16Lgkm0 = (1 << 14) | (7 << 4) | (0 << 8);   // vmcnt(16) lgkmcnt(0)
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);                     // vmcnt(0)
constexpr int kWaitVm0Lgkm0 = (7 << 4);                            // vmcnt(0) lgkmcnt(0)

// ---- persistent tile schedule shared by the 256-tile kernels -------------
// s_tb[e] = M tiles (of BM rows) before group e, s_tb[G] = all of them.
template <int BM>
__device__ __forceinline__ int tile_prefix(const GemmGroup& g, int* s_tb, int* s_wsum) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (g.offsets) {
        int nt = 0;
        if (tid < g.G) nt = (g.offsets[tid + 1] - g.offsets[tid] + BM - 1) / BM;
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
        if (tid < g.G) s_tb[tid] = v + before - nt;
        if (tid == g.G - 1) s_tb[g.G] = v + before;     // all M tiles (G <= 256 threads)
    } else if (tid == 0) {
        s_tb[0] = 0;
        s_tb[1] = (g.M + BM - 1) / BM;
    }
    __syncthreads();
    return g.offsets ? g.G : 1;
}

struct TileRef {
    int grp, row0, nrows, n0;
};

// Logical tile L -> (group, rows, first column).  Bands of kWMW M tiles; in a
// band, windows of wn_win N tiles; inside a window, M-tile-fastest order.
template <int BM, int BN>
__device__ __forceinline__ TileRef tile_at(const GemmGroup& g, const int* s_tb, int G, int mt_total,
                                           int tiles_n, int wn_win, int L) {
    const int band = L / (kWMW * tiles_n);
    const int mb0 = band * kWMW;
    const int mh = min(kWMW, mt_total - mb0);
    const int rem = L - band * kWMW * tiles_n;
    const int nwin = rem / (mh * wn_win);
    const int r2 = rem - nwin * mh * wn_win;
    const int mt = mb0 + r2 % mh;
    const int ntile = nwin * wn_win + r2 / mh;
    int lo = 0, hi = G;                              // s_tb[lo] <= mt < s_tb[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_tb[mid] <= mt) lo = mid; else hi = mid;
    }
    TileRef t;
    t.grp = lo;
    const int base_row = g.offsets ? g.offsets[lo] : 0;
    const int end_row = g.offsets ? g.offsets[lo + 1] : g.M;
    t.row0 = base_row + (mt - s_tb[lo]) * BM;
    t.nrows = min(BM, end_row - t.row0);
    t.n0 = ntile * BN;
    return t;
}

// Swizzle of 64-byte LDS rows (4 chunks of 16 B): chunk c of row r sits at
// c ^ f(r).  32 lanes reading rows r..r+31 at one logical chunk then hit
// distinct bank groups whether the LDS serves 8 or 16 lanes per cycle.
__device__ __forceinline__ int swz4(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// Main bf16 kernel, persistent: one workgroup per CU walks a list of
// 256 x 256 tiles of MFMA work.
//   single: C tile 256 rows x 256 cols of one weight matrix;
//   dual:   C tile 256 rows x 128 cols, computed for the gate and the up
//           matrix (B rows 0..127 = gate, 128..255 = up, same columns).
// Tile schedule: the real M tiles (ceil(count_e / 256) per expert, prefix sums
// in LDS) times the N tiles form a list of logical tiles, cut into 8 equal
// ranges, one per XCD (workgroup ids are dealt to the XCDs round-robin).
// Inside a range the XCD's workgroups take consecutive tiles in rounds; a
// round is a window of 4 M tiles x (workgroups / 4) N tiles, so its A and B
// panels are shared in the XCD's L2 while all its tiles advance through K in
// step (same work per tile, all resident at once).
// 4 waves in 2 x 2; each wave owns 128 rows x 4 blocks of 32 B-rows, i.e.
// 4 x 4 MFMA 32x32 blocks = 256 fp32 accumulators (AGPRs).
// Global -> LDS by direct 16-byte DMA (global_load_lds_dwordx4): lane i of
// an instruction fills bytes [16 i, 16 i + 16) of a 1 KB block = 16 LDS rows
// of 32 bf16, so each lane fetches the chunk the swizzle places there.
// Four LDS stages of 32 K-elements (separate arrays, so the compiler can see
// that a DMA into one stage does not alias fragment reads of another), DMA
// issued three stages ahead.  One barrier per stage, in the middle of the
// stage: after it, the next stage's first fragments are read while the
// current stage's last MFMAs run.
template <bool DUAL>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_256_kernel(GemmGroup g, int tiles_n) {
    constexpr int BM = 256;
    constexpr int BN = DUAL ? 128 : 256;
    constexpr int STG = 256 * kBKs;   // elements of one A or B stage
    __shared__ __align__(16) uint16_t sA0[STG], sA1[STG], sA2[STG], sA3[STG];
    __shared__ __align__(16) uint16_t sB0[STG], sB1[STG], sB2[STG], sB3[STG];
    __shared__ int s_tb[257];          // M tiles before group e; s_tb[G] = all M tiles
    __shared__ int s_wsum[kThreads / 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int K = g.K;
    const int KT = K / kBKs;          // multiple of 4

    const int G = tile_prefix<BM>(g, s_tb, s_wsum);
    const int mt_total = s_tb[G];
    const int TL = mt_total * tiles_n;
    const int nslot = gridDim.x >> 3;             // workgroups per XCD
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    // per-XCD range: a whole number of rounds, so every round is one window
    const int per = ((TL + 7) / 8 + nslot - 1) / nslot * nslot;
    const int Lend = min(TL, (xcd + 1) * per);
    const int wn_win = max(nslot / kWMW, 1);      // N tiles per round window

    const int half = lane >> 5, r32 = lane & 31;
    int a_row[4], b_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a_row[i] = wm * 128 + i * 32 + r32;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        b_row[b] = DUAL ? (b >> 1) * 128 + wn * 64 + (b & 1) * 32 + r32 : wn * 128 + b * 32 + r32;

    for (int L = xcd * per + slot; L < Lend; L += nslot) {
        const TileRef tr = tile_at<BM, BN>(g, s_tb, G, mt_total, tiles_n, wn_win, L);
        const int grp = tr.grp, row0 = tr.row0, nrows = tr.nrows, n0 = tr.n0;

        // DMA sources: instruction j of wave w fills LDS rows 64 w + 16 j + lane / 4
        // at physical chunk lane % 4, which holds logical chunk (lane % 4) ^ swz4(row).
        // Addresses are a wave-uniform base plus a 32-bit per-lane byte offset.
        const char* a_base = static_cast<const char*>(g.A);
        // B rows 64 w .. 64 w + 63: dual -> gate (w < 2) or up (w >= 2) matrix,
        // column n0 + row % 128; single -> column n0 + row.
        const char* b_base = static_cast<const char*>(DUAL ? (w < 2 ? g.B0 : g.B1) : g.B0) +
                             ((int64_t)grp * g.N + n0) * K * 2;
        uint32_t a_off[4], b_off[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = w * 64 + j * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz4(r);
            const int rr = min(r, nrows - 1);
            const int src = g.gather ? g.gather[row0 + rr] / g.gather_div : row0 + rr;
            a_off[j] = (uint32_t)src * (uint32_t)(K * 2) + c * 16;
            b_off[j] = (uint32_t)(DUAL ? (r & 127) : r) * (uint32_t)(K * 2) + c * 16;
        }

        f32x16_t acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
        bf16x8_t fa0[4], fb0[4], fa1[4], fb1[4];

#define MOE_DMA(sA_, sB_, kt_)                                                                  \
    do {                                                                                        \
        const char* ab_ = a_base + (kt_) * (kBKs * 2);                                          \
        const char* bb_ = b_base + (kt_) * (kBKs * 2);                                          \
        _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                         \
            __builtin_amdgcn_global_load_lds(ab_ + a_off[j],                                    \
                                             (lds_ptr_t)((sA_) + (w * 64 + j * 16) * kBKs), 16, 0, 0); \
            __builtin_amdgcn_global_load_lds(bb_ + b_off[j],                                    \
                                             (lds_ptr_t)((sB_) + (w * 64 + j * 16) * kBKs), 16, 0, 0); \
        }                                                                                       \
    } while (0)
#define MOE_LOAD_FRAGS(sA_, sB_, s_, af_, bf_)                                                  \
    do {                                                                                        \
        const int c_ = 2 * (s_) + half;                                                        \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) af_[i] = as_bf16x8(                       \
            *reinterpret_cast<const uint4*>((sA_) + a_row[i] * kBKs + ((c_ ^ swz4(a_row[i])) * 8))); \
        _Pragma("unroll") for (int b = 0; b < 4; ++b) bf_[b] = as_bf16x8(                       \
            *reinterpret_cast<const uint4*>((sB_) + b_row[b] * kBKs + ((c_ ^ swz4(b_row[b])) * 8))); \
    } while (0)
#define MOE_MFMAS(af_, bf_)                                                                     \
    do {                                                                                        \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                           \
            _Pragma("unroll") for (int b = 0; b < 4; ++b) acc[i][b] =                           \
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af_[i], bf_[b], acc[i][b], 0, 0, 0);    \
    } while (0)
// 16 MFMAs with the 8 fragment reads of the following step between the first 8
#define MOE_INTERLEAVE()                                                                        \
    do {                                                                                        \
        _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {                                      \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                  \
        }                                                                                       \
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);                                      \
    } while (0)
// Stage kt in buffers (sAc, sBc); next stage in (sAn, sBn); DMA target of
// stage kt + 3 in (sAp, sBp).  On entry fa0/fb0 hold step 0 of stage kt.
// Branch-free, so each half is one scheduling region: past the last K tile
// the DMA re-fetches the last tile into the free buffer (never read), so
// exactly 8 DMAs are always issued per stage and vmcnt(16) always means
// "stage kt + 1 has landed"; the fragment prefetch past the end is unused.
#define MOE_STAGE(sAc, sBc, sAn, sBn, sAp, sBp, kt_)                                            \
    do {                                                                                        \
        const int st_ = (kt_);                                                                  \
        MOE_DMA(sAp, sBp, min(st_ + 3, KT - 1));                                                \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAc, sBc, 1, fa1, fb1);                                                  \
        MOE_MFMAS(fa0, fb0);                                                                    \
        MOE_INTERLEAVE();                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        /* stage kt + 1 landed (own DMAs) and this wave's reads of stage kt are done */        \
        __builtin_amdgcn_s_waitcnt(kWaitVm16Lgkm0);                                             \
        __builtin_amdgcn_s_barrier();                                                           \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAn, sBn, 0, fa0, fb0);                                                  \
        MOE_MFMAS(fa1, fb1);                                                                    \
        MOE_INTERLEAVE();                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                      \
    } while (0)

        // every wave is past its reads of the previous tile's buffers
        __syncthreads();
        MOE_DMA(sA0, sB0, 0);
        MOE_DMA(sA1, sB1, 1);
        MOE_DMA(sA2, sB2, 2);
        __builtin_amdgcn_s_waitcnt(kWaitVm16Lgkm0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        MOE_LOAD_FRAGS(sA0, sB0, 0, fa0, fb0);
        for (int kt = 0; kt < KT; kt += 4) {
            MOE_STAGE(sA0, sB0, sA1, sB1, sA3, sB3, kt);
            MOE_STAGE(sA1, sB1, sA2, sB2, sA0, sB0, kt + 1);
            MOE_STAGE(sA2, sB2, sA3, sB3, sA1, sB1, kt + 2);
            MOE_STAGE(sA3, sB3, sA0, sB0, sA2, sB2, kt + 3);
        }
#undef MOE_DMA
#undef MOE_LOAD_FRAGS
#undef MOE_MFMAS
#undef MOE_INTERLEAVE
#undef MOE_STAGE
        // the trailing (re-fetch) DMAs land before the buffers are reused
        __builtin_amdgcn_s_waitcnt(kWaitVm0);

        // epilogue: D element q of block (i, b): row 8 (q / 4) + 4 half + q % 4, col r32
        uint16_t* C = static_cast<uint16_t*>(g.C);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int bo = 0; bo < (DUAL ? 2 : 4); ++bo) {
                const int col = DUAL ? n0 + wn * 64 + bo * 32 + r32 : n0 + wn * 128 + bo * 32 + r32;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int r = wm * 128 + i * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
                    if (r < nrows) {
                        float v = acc[i][bo][q];
                        if (DUAL) v = silu_f32(v) * acc[i][bo + 2][q];
                        C[(int64_t)(row0 + r) * g.N + col] = f32_to_bf16(v);
                    }
                }
            }
        }
    }
}

// Variant of the persistent 256-tile kernel with 64-element K stages: every
// LDS row is a full 128-byte line (8 chunks, swizzle swz), so each row's DMA
// is one 128-byte request; two LDS stages, the DMA one stage ahead.
template <bool DUAL>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_256w_kernel(GemmGroup g, int tiles_n) {
    constexpr int BM = 256;
    constexpr int BN = DUAL ? 128 : 256;
    constexpr int STG = 256 * kBK;    // elements of one A or B stage (32 KB)
    __shared__ __align__(16) uint16_t sA0[STG], sA1[STG];
    __shared__ __align__(16) uint16_t sB0[STG], sB1[STG];
    __shared__ int s_tb[257];
    __shared__ int s_wsum[kThreads / 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int K = g.K;
    const int KT = K / kBK;            // even

    const int G = tile_prefix<BM>(g, s_tb, s_wsum);
    const int mt_total = s_tb[G];
    const int TL = mt_total * tiles_n;
    const int nslot = gridDim.x >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    // per-XCD range: a whole number of rounds, so every round is one window
    const int per = ((TL + 7) / 8 + nslot - 1) / nslot * nslot;
    const int Lend = min(TL, (xcd + 1) * per);
    const int wn_win = max(nslot / kWMW, 1);

    const int half = lane >> 5, r32 = lane & 31;
    int a_row[4], b_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a_row[i] = wm * 128 + i * 32 + r32;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        b_row[b] = DUAL ? (b >> 1) * 128 + wn * 64 + (b & 1) * 32 + r32 : wn * 128 + b * 32 + r32;

    for (int L = xcd * per + slot; L < Lend; L += nslot) {
        const TileRef tr = tile_at<BM, BN>(g, s_tb, G, mt_total, tiles_n, wn_win, L);
        const int grp = tr.grp, row0 = tr.row0, nrows = tr.nrows, n0 = tr.n0;

        // instruction j of wave w fills LDS rows 64 w + 8 j + lane / 8 at physical
        // chunk lane % 8, which holds logical chunk (lane % 8) ^ swz(row)
        const char* a_base = static_cast<const char*>(g.A);
        const char* b_base = static_cast<const char*>(DUAL ? (w < 2 ? g.B0 : g.B1) : g.B0) +
                             ((int64_t)grp * g.N + n0) * K * 2;
        uint32_t a_off[8], b_off[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = w * 64 + j * 8 + (lane >> 3);
            const int c = (lane & 7) ^ swz(r);
            const int rr = min(r, nrows - 1);
            const int src = g.gather ? g.gather[row0 + rr] / g.gather_div : row0 + rr;
            a_off[j] = (uint32_t)src * (uint32_t)(K * 2) + c * 16;
            b_off[j] = (uint32_t)(DUAL ? (r & 127) : r) * (uint32_t)(K * 2) + c * 16;
        }

        f32x16_t acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
        bf16x8_t fa0[4], fb0[4], fa1[4], fb1[4];

#define MOE_DMA(sA_, sB_, kt_)                                                                  \
    do {                                                                                        \
        const char* ab_ = a_base + (kt_) * (kBK * 2);                                           \
        const char* bb_ = b_base + (kt_) * (kBK * 2);                                           \
        _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                         \
            __builtin_amdgcn_global_load_lds(ab_ + a_off[j],                                    \
                                             (lds_ptr_t)((sA_) + (w * 64 + j * 8) * kBK), 16, 0, 0); \
            __builtin_amdgcn_global_load_lds(bb_ + b_off[j],                                    \
                                             (lds_ptr_t)((sB_) + (w * 64 + j * 8) * kBK), 16, 0, 0); \
        }                                                                                       \
    } while (0)
#define MOE_LOAD_FRAGS(sA_, sB_, s_, af_, bf_)                                                  \
    do {                                                                                        \
        const int c_ = 2 * (s_) + half;                                                         \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) af_[i] = as_bf16x8(                       \
            *reinterpret_cast<const uint4*>((sA_) + a_row[i] * kBK + ((c_ ^ swz(a_row[i])) * 8))); \
        _Pragma("unroll") for (int b = 0; b < 4; ++b) bf_[b] = as_bf16x8(                       \
            *reinterpret_cast<const uint4*>((sB_) + b_row[b] * kBK + ((c_ ^ swz(b_row[b])) * 8))); \
    } while (0)
#define MOE_MFMAS(af_, bf_)                                                                     \
    do {                                                                                        \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                           \
            _Pragma("unroll") for (int b = 0; b < 4; ++b) acc[i][b] =                           \
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af_[i], bf_[b], acc[i][b], 0, 0, 0);    \
    } while (0)
#define MOE_INTERLEAVE()                                                                        \
    do {                                                                                        \
        _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {                                      \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                  \
        }                                                                                       \
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);                                      \
    } while (0)
// Stage kt in (sAc, sBc), stage kt + 1 DMA'd into (sAn, sBn); fa0/fb0 hold
// step 0 on entry.  Past the end the DMA re-fetches the last tile (unread).
#define MOE_STAGE(sAc, sBc, sAn, sBn, kt_)                                                      \
    do {                                                                                        \
        MOE_DMA(sAn, sBn, min((kt_) + 1, KT - 1));                                              \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAc, sBc, 1, fa1, fb1);                                                  \
        MOE_MFMAS(fa0, fb0);                                                                    \
        MOE_INTERLEAVE();                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAc, sBc, 2, fa0, fb0);                                                  \
        MOE_MFMAS(fa1, fb1);                                                                    \
        MOE_INTERLEAVE();                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAc, sBc, 3, fa1, fb1);                                                  \
        MOE_MFMAS(fa0, fb0);                                                                    \
        MOE_INTERLEAVE();                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);                                              \
        __builtin_amdgcn_s_barrier();                                                           \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAn, sBn, 0, fa0, fb0);                                                  \
        MOE_MFMAS(fa1, fb1);                                                                    \
        MOE_INTERLEAVE();                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                      \
    } while (0)

        __syncthreads();
        MOE_DMA(sA0, sB0, 0);
        __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        MOE_LOAD_FRAGS(sA0, sB0, 0, fa0, fb0);
        for (int kt = 0; kt < KT; kt += 2) {
            MOE_STAGE(sA0, sB0, sA1, sB1, kt);
            MOE_STAGE(sA1, sB1, sA0, sB0, kt + 1);
        }
#undef MOE_DMA
#undef MOE_LOAD_FRAGS
#undef MOE_MFMAS
#undef MOE_INTERLEAVE
#undef MOE_STAGE
        __builtin_amdgcn_s_waitcnt(kWaitVm0);

        uint16_t* C = static_cast<uint16_t*>(g.C);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int bo = 0; bo < (DUAL ? 2 : 4); ++bo) {
                const int col = DUAL ? n0 + wn * 64 + bo * 32 + r32 : n0 + wn * 128 + bo * 32 + r32;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int r = wm * 128 + i * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
                    if (r < nrows) {
                        float v = acc[i][bo][q];
                        if (DUAL) v = silu_f32(v) * acc[i][bo + 2][q];
                        C[(int64_t)(row0 + r) * g.N + col] = f32_to_bf16(v);
                    }
                }
            }
        }
    }
}

// 8-wave variant (512 threads, two waves per SIMD) of the persistent
// 256-tile kernel with 64-element K stages.  Eight waves keep twice as many
// DMA requests in flight per CU as four, which the load path needs to feed
// the MFMAs.  Waves form a 2 x 4 grid: wave (wm, wn) owns 128 rows and two
// 32-row blocks of B (dual: gate columns 32 wn .. 32 wn + 31 and the same up
// columns, so silu(g)*u stays in registers; single: B rows 64 wn .. 64 wn +
// 63), i.e. 4 x 2 MFMA blocks = 128 accumulators.
template <bool DUAL>
__global__ __launch_bounds__(512, 1) void gemm_bf16_256x8_kernel(GemmGroup g, int tiles_n) {
    constexpr int BM = 256;
    constexpr int BN = DUAL ? 128 : 256;
    constexpr int STG = 256 * kBK;    // elements of one A or B stage (32 KB)
    __shared__ __align__(16) uint16_t sA0[STG], sA1[STG];
    __shared__ __align__(16) uint16_t sB0[STG], sB1[STG];
    __shared__ int s_tb[257];
    __shared__ int s_wsum[8];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3;
    const int K = g.K;
    const int KT = K / kBK;            // even

    const int G = tile_prefix<BM>(g, s_tb, s_wsum);
    const int mt_total = s_tb[G];
    const int TL = mt_total * tiles_n;
    const int nslot = gridDim.x >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    // per-XCD range: a whole number of rounds, so every round is one window
    const int per = ((TL + 7) / 8 + nslot - 1) / nslot * nslot;
    const int Lend = min(TL, (xcd + 1) * per);
    const int wn_win = max(nslot / kWMW, 1);

    const int half = lane >> 5, r32 = lane & 31;
    int a_row[4], b_row[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a_row[i] = wm * 128 + i * 32 + r32;
#pragma unroll
    for (int b = 0; b < 2; ++b) b_row[b] = DUAL ? b * 128 + wn * 32 + r32 : wn * 64 + b * 32 + r32;

    for (int L = xcd * per + slot; L < Lend; L += nslot) {
        const TileRef tr = tile_at<BM, BN>(g, s_tb, G, mt_total, tiles_n, wn_win, L);
        const int grp = tr.grp, row0 = tr.row0, nrows = tr.nrows, n0 = tr.n0;

        // instruction j (0..3) of wave w fills LDS rows 32 w + 8 j + lane / 8 at
        // physical chunk lane % 8, which holds logical chunk (lane % 8) ^ swz(row)
        const char* a_base = static_cast<const char*>(g.A);
        const char* b_base = static_cast<const char*>(DUAL ? (w < 4 ? g.B0 : g.B1) : g.B0) +
                             ((int64_t)grp * g.N + n0) * K * 2;
        uint32_t a_off[4], b_off[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = w * 32 + j * 8 + (lane >> 3);
            const int c = (lane & 7) ^ swz(r);
            const int rr = min(r, nrows - 1);
            const int src = g.gather ? g.gather[row0 + rr] / g.gather_div : row0 + rr;
            a_off[j] = (uint32_t)src * (uint32_t)(K * 2) + c * 16;
            b_off[j] = (uint32_t)(DUAL ? (r & 127) : r) * (uint32_t)(K * 2) + c * 16;
        }

        f32x16_t acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
        bf16x8_t fa0[4], fb0[2], fa1[4], fb1[2];

#define MOE_DMA(sA_, sB_, kt_)                                                                  \
    do {                                                                                        \
        const char* ab_ = a_base + (kt_) * (kBK * 2);                                           \
        const char* bb_ = b_base + (kt_) * (kBK * 2);                                           \
        _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                         \
            __builtin_amdgcn_global_load_lds(ab_ + a_off[j],                                    \
                                             (lds_ptr_t)((sA_) + (w * 32 + j * 8) * kBK), 16, 0, 0); \
            __builtin_amdgcn_global_load_lds(bb_ + b_off[j],                                    \
                                             (lds_ptr_t)((sB_) + (w * 32 + j * 8) * kBK), 16, 0, 0); \
        }                                                                                       \
    } while (0)
#define MOE_LOAD_FRAGS(sA_, sB_, s_, af_, bf_)                                                  \
    do {                                                                                        \
        const int c_ = 2 * (s_) + half;                                                         \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) af_[i] = as_bf16x8(                       \
            *reinterpret_cast<const uint4*>((sA_) + a_row[i] * kBK + ((c_ ^ swz(a_row[i])) * 8))); \
        _Pragma("unroll") for (int b = 0; b < 2; ++b) bf_[b] = as_bf16x8(                       \
            *reinterpret_cast<const uint4*>((sB_) + b_row[b] * kBK + ((c_ ^ swz(b_row[b])) * 8))); \
    } while (0)
#define MOE_MFMAS(af_, bf_)                                                                     \
    do {                                                                                        \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                           \
            _Pragma("unroll") for (int b = 0; b < 2; ++b) acc[i][b] =                           \
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af_[i], bf_[b], acc[i][b], 0, 0, 0);    \
    } while (0)
// 8 MFMAs with the 6 fragment reads of the following step between them
#define MOE_INTERLEAVE()                                                                        \
    do {                                                                                        \
        _Pragma("unroll") for (int i_ = 0; i_ < 6; ++i_) {                                      \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                  \
        }                                                                                       \
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                      \
    } while (0)
#define MOE_STAGE(sAc, sBc, sAn, sBn, kt_)                                                      \
    do {                                                                                        \
        MOE_DMA(sAn, sBn, min((kt_) + 1, KT - 1));                                              \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAc, sBc, 1, fa1, fb1);                                                  \
        MOE_MFMAS(fa0, fb0);                                                                    \
        MOE_INTERLEAVE();                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAc, sBc, 2, fa0, fb0);                                                  \
        MOE_MFMAS(fa1, fb1);                                                                    \
        MOE_INTERLEAVE();                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAc, sBc, 3, fa1, fb1);                                                  \
        MOE_MFMAS(fa0, fb0);                                                                    \
        MOE_INTERLEAVE();                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);                                              \
        __builtin_amdgcn_s_barrier();                                                           \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAn, sBn, 0, fa0, fb0);                                                  \
        MOE_MFMAS(fa1, fb1);                                                                    \
        MOE_INTERLEAVE();                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                      \
    } while (0)

        __syncthreads();
        MOE_DMA(sA0, sB0, 0);
        __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        MOE_LOAD_FRAGS(sA0, sB0, 0, fa0, fb0);
        for (int kt = 0; kt < KT; kt += 2) {
            MOE_STAGE(sA0, sB0, sA1, sB1, kt);
            MOE_STAGE(sA1, sB1, sA0, sB0, kt + 1);
        }
#undef MOE_DMA
#undef MOE_LOAD_FRAGS
#undef MOE_MFMAS
#undef MOE_INTERLEAVE
#undef MOE_STAGE
        __builtin_amdgcn_s_waitcnt(kWaitVm0);

        uint16_t* C = static_cast<uint16_t*>(g.C);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int bo = 0; bo < (DUAL ? 1 : 2); ++bo) {
                const int col = DUAL ? n0 + wn * 32 + r32 : n0 + wn * 64 + bo * 32 + r32;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int r = wm * 128 + i * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
                    if (r < nrows) {
                        float v = acc[i][bo][q];
                        if (DUAL) v = silu_f32(v) * acc[i][1][q];
                        C[(int64_t)(row0 + r) * g.N + col] = f32_to_bf16(v);
                    }
                }
            }
        }
    }
}

// fp32 grouped GEMM: 64x64 tiles, BK 16, 4x4 outputs per thread.
template <bool DUAL>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmGroup g, int tiles_n, int mt_upper) {
    constexpr int BM = 64, BN = 64, BK = 16;
    constexpr int NMAT = DUAL ? 2 : 1;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[NMAT][BK][BN + 4];
    const int mt = blockIdx.x / tiles_n, ntile = blockIdx.x % tiles_n;
    if (mt >= mt_upper) return;
    int grp, row0, nrows;
    if (!locate_tile<BM>(g, mt, &grp, &row0, &nrows)) return;
    const int n0 = ntile * BN;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const float* A = static_cast<const float*>(g.A);
    const int K = g.K;
    // loader: 64 rows x 16 k = 1024 elements, 4 per thread: row = tid/4 , k4 = (tid%4)*4
    const int lr = tid >> 2, lk = (tid & 3) * 4;
    const int rr = min(lr, nrows - 1);
    const int src = g.gather ? g.gather[row0 + rr] / g.gather_div : row0 + rr;
    const float* a_src = A + (int64_t)src * K + lk;
    const float* b_src[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
        b_src[m] = static_cast<const float*>(m == 0 ? g.B0 : g.B1) + (int64_t)grp * g.N * K +
                   (int64_t)(n0 + lr) * K + lk;
    float acc[NMAT][4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
        float4 av = *reinterpret_cast<const float4*>(a_src + k0);
        As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            float4 bv = *reinterpret_cast<const float4*>(b_src[m] + k0);
            Bs[m][lk + 0][lr] = bv.x; Bs[m][lk + 1][lr] = bv.y;
            Bs[m][lk + 2][lr] = bv.z; Bs[m][lk + 3][lr] = bv.w;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[NMAT][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j) b[m][j] = Bs[m][kk][tx * 4 + j];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[m][i][j] = fmaf(a[i], b[m][j], acc[m][i][j]);
        }
        __syncthreads();
    }
    float* C = static_cast<float*>(g.C);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = ty * 4 + i;
        if (r >= nrows) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v = acc[0][i][j];
            if (DUAL) v = silu_f32(v) * acc[NMAT - 1][i][j];
            C[(int64_t)(row0 + r) * g.N + n0 + tx * 4 + j] = v;
        }
    }
}

template <int BM, int BN, bool DUAL>
hipError_t launch_bf16(const GemmGroup& g, hipStream_t s) {
    const int tiles_n = g.N / BN;
    const int64_t mtu = g.offsets ? grouped_m_tiles_upper(g.M, g.G, BM) : (g.M + BM - 1) / BM;
    if (mtu == 0) return hipSuccess;
    int64_t nwg = mtu * tiles_n;
    nwg = (nwg + 7) / 8 * 8;
    constexpr int NMAT = DUAL ? 2 : 1;
    const size_t lds = (size_t)2 * (BM + NMAT * BN) * kBK * sizeof(uint16_t);
    auto kern = gemm_bf16_kernel<BM, BN, DUAL>;
    static bool attr_set = false;   // same value on every device; set once per process
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(kThreads), lds, s, g, tiles_n, (int)mtu);
    return hipGetLastError();
}

int persistent_grid() {
    static int cus = 0;   // CUs of the current device, read once
    if (cus == 0) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
            cus = prop.multiProcessorCount;
        if (cus < 8) cus = 256;
    }
    return cus / 8 * 8;
}

#ifndef MOE_GEMM_WIDE_STAGES
#define MOE_GEMM_WIDE_STAGES 1
#endif
#ifndef MOE_GEMM_EIGHT_WAVES
#define MOE_GEMM_EIGHT_WAVES 1
#endif

template <bool DUAL>
hipError_t launch_bf16_256(const GemmGroup& g, hipStream_t s) {
    constexpr int BN = DUAL ? 128 : 256;
    const int tiles_n = g.N / BN;
    if (MOE_GEMM_EIGHT_WAVES)
        hipLaunchKernelGGL((gemm_bf16_256x8_kernel<DUAL>), dim3(persistent_grid()), dim3(512), 0, s,
                           g, tiles_n);
    else if (MOE_GEMM_WIDE_STAGES)
        hipLaunchKernelGGL((gemm_bf16_256w_kernel<DUAL>), dim3(persistent_grid()), dim3(kThreads), 0,
                           s, g, tiles_n);
    else
        hipLaunchKernelGGL((gemm_bf16_256_kernel<DUAL>), dim3(persistent_grid()), dim3(kThreads), 0, s,
                           g, tiles_n);
    return hipGetLastError();
}

template <bool DUAL>
hipError_t launch_f32(const GemmGroup& g, hipStream_t s) {
    const int tiles_n = g.N / 64;
    const int64_t mtu = g.offsets ? grouped_m_tiles_upper(g.M, g.G, 64) : (g.M + 63) / 64;
    if (mtu == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_f32_kernel<DUAL>, dim3((unsigned)(mtu * tiles_n)), dim3(kThreads), 0, s,
                       g, tiles_n, (int)mtu);
    return hipGetLastError();
}

}  // namespace

int64_t grouped_m_tiles_upper(int64_t rows, int G, int bm) {
    // sum_e ceil(n_e / bm) <= floor((sum_e n_e + G*(bm-1)) / bm)
    return (rows + (int64_t)G * (bm - 1)) / bm;
}

hipError_t launch_grouped_gemm(const GemmGroup& g, bool dual, bool bf16, hipStream_t s) {
    if (g.M == 0) return hipSuccess;
    if (!bf16) return dual ? launch_f32<true>(g, s) : launch_f32<false>(g, s);
    // the 256-tile kernel takes K tiles in pairs: K % 128 == 0
    if (g.K % 128 == 0 && dual && g.N % 128 == 0) return launch_bf16_256<true>(g, s);
    if (g.K % 128 == 0 && !dual && g.N % 256 == 0) return launch_bf16_256<false>(g, s);
    if (g.N % 128 == 0) return dual ? launch_bf16<128, 128, true>(g, s) : launch_bf16<128, 128, false>(g, s);
    return dual ? launch_bf16<128, 64, true>(g, s) : launch_bf16<128, 64, false>(g, s);
}

}  // namespace moe
