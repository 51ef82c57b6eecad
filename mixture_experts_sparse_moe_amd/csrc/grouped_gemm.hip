// Grouped GEMMs of the expert SwiGLU FFNs ("8.6 Mixture of Experts" sec. 2;
// "What Actually Happens When a Token Hits the Router", Step 4).
//
// For each group (expert) e with grouped rows [off[e], off[e+1]):
//   dual:   C[r, n] = silu(sum_k A[src(r), k] B0[e, n, k]) * (sum_k A[src(r), k] B1[e, n, k])
//   single: C[r, n] = sum_k A[src(r), k] B0[e, n, k]
// src(r) = gather[r] / gather_div (token of the pair) when gathering, else r.
// Both operands are K-contiguous ("NT"), the natural MFMA operand layout.
//
// bf16 kernels (gfx950), fp32 accumulation on v_mfma_f32_32x32x16_bf16:
//   - gemm_bf16_persistent_kernel: the main path.  One workgroup of 8 waves
//     per CU walks 256 x 256 tiles of MFMA work with a direct-to-LDS DMA
//     pipeline that runs on across tiles; described at the kernel.  Two more
//     modes serve the backward pass: fp32 products over the grouped rows, and
//     grouped K (each group sums over its own range of K columns: the weight
//     gradients, over transposed activations).
//   - gemm_bf16_kernel: the general fallback for N or K that the persistent
//     kernel does not take (N % 128, K % 128 != 0): 4 waves, BM x BN tiles,
//     global -> registers -> LDS, double-buffered, one workgroup per tile.
//   - LDS rows are 64 bf16 = 8 chunks of 16 B; chunk c of row r is stored at
//     c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1), so the 16-byte fragment reads
//     of 32 consecutive rows hit distinct banks.
//   - M tiles are data dependent: the flattened M-tile list maps to
//     (expert, row range) by a prefix sum of ceil(count_e / BM) done in the
//     workgroup from the device-side offsets, so no host sync is needed.
//   - A rows are gathered on load (no permuted copy of x).
// fp32 kernel: LDS-tiled FMA (the tiny fp32 layer only).
#include "device_util.h"
#include "moe_internal.h"
#include "skinny.h"

#include <hip/hip_ext.h>

namespace moe {

namespace {

constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kWMW = 4;   // M tiles per window (share one weight panel)
constexpr int kMaxBand = 6;   // most M tiles in one band of the expert-aligned order


// Block-wide: map flattened M tile `mt` to (group, first row, rows).  Returns
// false if mt is past the last real tile.  scratch: 11 ints of LDS.
template <int BM>
__device__ bool locate_tile_in(const GemmGroup& g, int mt, int* grp, int* row0, int* nrows, int* scratch) {
    if (g.offsets == nullptr) {
        const int r0 = mt * BM;
        if (r0 >= g.M) return false;
        *grp = 0;
        *row0 = r0;
        *nrows = min(BM, g.M - r0);
        return true;
    }
    int* s_wsum = scratch;         // one slot per wave, up to 512 threads
    int* s_res = scratch + 8;
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

template <int BM>
__device__ bool locate_tile(const GemmGroup& g, int mt, int* grp, int* row0, int* nrows) {
    __shared__ int s_scratch[11];
    return locate_tile_in<BM>(g, mt, grp, row0, nrows, s_scratch);
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

// ---- persistent 256 x 256 kernel ---------------------------------------------
// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]).  The builtin, unlike inline asm, is seen by the
// compiler's own wait insertion, so it adds no waits of its own after these.
constexpr int kWaitVm0Lgkm0 = (7 << 4);                 // vmcnt(0) lgkmcnt(0)

// A-row offset of a row past the tile's end: at or past the record count of
// the buffer the A rows are loaded through, so the bounds check drops its
// load (no request leaves the CU; the LDS row gets zeros, never stored).
constexpr uint32_t kDeadOff = 0xFFFFFFF0u;

// Cache policy operand of a load or store: nt (non-temporal, for data read
// once)
constexpr int kCacheNT = 2;

// Rows of M tile `local` of a group of n rows in m tiles of at most bm rows:
// first row (relative) and count.  BAL: the tiles share the rows evenly
// (height ceil(n / m)), else full tiles and a short last one.  With about
// one tile per group, a short last tile runs ahead of the full one beside it
// and streams the same weight panel from HBM a second time; two equal tiles
// run in step and the second read hits L2 (DeepSeek-V3 gate/up: 27.7 ->
// 18.6 GB read from the fabric per launch, 15.4 GB algorithmic).
template <bool BAL>
__device__ __forceinline__ void group_tile_rows(int n, int m, int local, int bm, int* r0, int* nr) {
    const int h = BAL ? (n + m - 1) / m : bm;
    *r0 = local * h;
    *nr = min(h, n - local * h);
}

// Per-workgroup tile table in LDS: s_tb[e] = M tiles (of BM rows) before
// group e, s_tb[G] = all of them; s_off[e] = first grouped row of group e.
template <int BM>
__device__ __forceinline__ int tile_prefix(const GemmGroup& g, int* s_tb, int* s_off, int* s_wsum) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (g.offsets) {
        int nt = 0, off = 0;
        if (tid < g.G) {
            off = g.offsets[tid];
            nt = (g.offsets[tid + 1] - off + BM - 1) / BM;
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
        if (tid < g.G) {
            s_tb[tid] = v + before - nt;
            s_off[tid] = off;
        }
        if (tid == g.G - 1) {           // G <= 257 < threads
            s_tb[g.G] = v + before;
            s_off[g.G] = g.offsets[g.G];
        }
    } else if (tid == 0) {
        s_tb[0] = 0;
        s_tb[1] = (g.M + BM - 1) / BM;
        s_off[0] = 0;
        s_off[1] = g.M;
    }
    __syncthreads();
    return g.offsets ? g.G : 1;
}

struct TileRef {
    int grp, row0, nrows, n0, ks;
    int kbeg, kt;   // grouped K: first K column and K stages of the tile
};

// Logical tile L -> (M tile, N tile).  Bands of kWMW M tiles; in a band,
// windows of wn_win N tiles; inside a window, M-tile-fastest order.
__device__ __forceinline__ void band_window(int mt_total, int tiles_n, int wn_win, int L, int& mt, int& ntile) {
    const int band = L / (kWMW * tiles_n);
    const int mb0 = band * kWMW;
    const int mh = min(kWMW, mt_total - mb0);
    const int rem = L - band * kWMW * tiles_n;
    const int nwin = rem / (mh * wn_win);
    const int r2 = rem - nwin * mh * wn_win;
    mt = mb0 + r2 % mh;
    ntile = nwin * wn_win + r2 / mh;
}

// Logical tile L -> (group, rows, first column), in band_window order.
template <int BM, int BN, bool BAL = false>
__device__ __forceinline__ TileRef tile_at(const int* s_tb, const int* s_off, int G, int mt_total,
                                           int tiles_n, int wn_win, int L) {
    int mt, ntile;
    band_window(mt_total, tiles_n, wn_win, L, mt, ntile);
    int lo = 0, hi = G;                              // s_tb[lo] <= mt < s_tb[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_tb[mid] <= mt) lo = mid; else hi = mid;
    }
    TileRef t;
    t.grp = lo;
    int r0, nr;
    group_tile_rows<BAL>(s_off[lo + 1] - s_off[lo], s_tb[lo + 1] - s_tb[lo], mt - s_tb[lo], BM, &r0, &nr);
    t.row0 = s_off[lo] + r0;
    t.nrows = nr;
    t.n0 = ntile * BN;
    t.ks = 0;
    return t;
}

// Expert-aligned order: the M tiles of each group form bands of near-equal
// height, at most kMaxBand; a band's tiles come in windows of (nslot /
// height) N tiles, M tile fastest, so a round's tiles share a few A panels
// and the B panels of one group, and each group's weights are streamed about
// once.  Band b covers logical tiles [first M tile * tiles_n, (first M tile +
// height) * tiles_n), so the band holding L holds M tile L / tiles_n.
template <int BM, int BN, bool BAL = false>
__device__ __forceinline__ TileRef tile_at_aligned(const int* s_tb, const int* s_off, int G, int tiles_n,
                                                   int nslot, int L) {
    const int mt0 = L / tiles_n;
    int lo = 0, hi = G;                              // s_tb[lo] <= mt0 < s_tb[lo + 1]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_tb[mid] <= mt0) lo = mid; else hi = mid;
    }
    const int gbase = s_tb[lo], m = s_tb[lo + 1] - gbase;   // the group's M tiles (>= 1)
    const int nb = (m + kMaxBand - 1) / kMaxBand;           // its bands: r of q + 1, then q
    const int q = m / nb, r = m - nb * q;
    const int local = mt0 - gbase;
    int j, start;
    if (local < r * (q + 1)) {
        j = local / (q + 1);
        start = j * (q + 1);
    } else {
        j = r + (local - r * (q + 1)) / q;
        start = r * (q + 1) + (j - r) * q;
    }
    const int mh = j < r ? q + 1 : q;
    const int wn = max(1, min(tiles_n, nslot / mh));
    const int rem = L - (gbase + start) * tiles_n;
    const int nwin = rem / (mh * wn);
    const int r2 = rem - nwin * mh * wn;             // the last window may be narrower
    const int mt = gbase + start + r2 % mh;
    TileRef t;
    t.grp = lo;
    int r0, nr;
    group_tile_rows<BAL>(s_off[lo + 1] - s_off[lo], m, mt - gbase, BM, &r0, &nr);
    t.row0 = s_off[lo] + r0;
    t.nrows = nr;
    t.n0 = (nwin * wn + r2 / mh) * BN;
    t.ks = 0;
    return t;
}

// Logical tile L of a K-split GEMM: the split index is the slowest, so each
// split walks the same windows of M x N tiles.
template <int BM, int BN, bool ALIGNED, bool BAL = false>
__device__ __forceinline__ TileRef split_tile_at(const int* s_tb, const int* s_off, int G, int mt_total,
                                                 int tiles_n, int wn_win, int L) {
    const int per_split = mt_total * tiles_n;
    const int ks = L / per_split;
    TileRef t = ALIGNED ? tile_at_aligned<BM, BN, BAL>(s_tb, s_off, G, tiles_n, wn_win * kWMW, L - ks * per_split)
                        : tile_at<BM, BN, BAL>(s_tb, s_off, G, mt_total, tiles_n, wn_win, L - ks * per_split);
    // the same in every lane (read from LDS at uniform addresses): scalar registers
    t.grp = __builtin_amdgcn_readfirstlane(t.grp);
    t.row0 = __builtin_amdgcn_readfirstlane(t.row0);
    t.nrows = __builtin_amdgcn_readfirstlane(t.nrows);
    t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
    t.ks = __builtin_amdgcn_readfirstlane(ks);
    return t;
}

// Grouped K: group g owns M tiles [g mtiles, (g + 1) mtiles) of the
// band_window order, all N tiles, and K columns [s_off[g], s_off[g + 1]).
template <int BM, int BN>
__device__ __forceinline__ TileRef kgroup_tile_at(const int* s_off, int mtiles, int mt_total, int tiles_n,
                                                  int wn_win, int L) {
    int mt, ntile;
    band_window(mt_total, tiles_n, wn_win, L, mt, ntile);
    TileRef t;
    t.grp = __builtin_amdgcn_readfirstlane(mt / mtiles);
    t.row0 = __builtin_amdgcn_readfirstlane((mt - t.grp * mtiles) * BM);
    t.nrows = BM;
    t.n0 = __builtin_amdgcn_readfirstlane(ntile * BN);
    t.ks = 0;
    t.kbeg = __builtin_amdgcn_readfirstlane(s_off[t.grp]);
    t.kt = __builtin_amdgcn_readfirstlane((s_off[t.grp + 1] - t.kbeg) / kBK);
    return t;
}

// Grouped K: s_off[g] = first K column of group g, g <= G.  Returns G.
__device__ __forceinline__ int kgroup_prefix(const GemmGroup& g, int* s_off) {
    const int G = g.kofs ? g.G : 1;
    const int tid = threadIdx.x;
    if (tid <= G) s_off[tid] = g.kofs ? g.kofs[tid] : (tid ? g.K : 0);
    __syncthreads();
    return G;
}

// DMA sources of one tile for one wave: wave-uniform bases and 32-bit per-lane
// byte offsets.  Instruction j (0..3) of wave w fills LDS rows 32 w + 8 j +
// lane / 8 at physical 16-byte chunk lane % 8, which holds logical chunk
// (lane % 8) ^ swz(row).  Gathered A rows are addressed from the start of A
// (the host keeps A under 4 GiB for that case); other A rows from the tile.
template <int J>
struct DmaSrc {
    const char* a;
    const char* b;
    uint32_t ao[J], bo[J];
    int rot;        // first K stage of the walk (stage s reads stage (s + rot) mod stages)
    int kt;         // grouped K: stages of the tile
    // B stored [K, N] (N contiguous): K stage s (counted from the start of K)
    // at b + s bstage, or from stage khalf on at b1 + (s - khalf) bstage;
    // kbase: the first stage of the tile's K split
    const char* b1;
    uint32_t bstage;
    int khalf, kbase;
};

// NW waves; wave w stages rows (256 / NW) w .. (256 / NW)(w + 1) - 1 of the A
// and the B tile, J = 32 / NW instructions of 8 rows each per operand.
// gather_rows() issues the loads of the gathered pair ids of those rows (rows
// past the tile's end repeat its last row); dma_src() turns them into the
// tile's DMA sources.  Kept apart so the loads can be in flight long before
// their values are needed.
template <int NW>
__device__ __forceinline__ void gather_rows(const GemmGroup& g, const TileRef& t, int w, int lane,
                                            int* src) {
    constexpr int J = 32 / NW;
    if (g.gather) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int r = w * (256 / NW) + j * 8 + (lane >> 3);
            src[j] = g.gather[t.row0 + min(r, t.nrows - 1)];
        }
    } else {
#pragma unroll
        for (int j = 0; j < J; ++j) src[j] = min(w * (256 / NW) + j * 8 + (lane >> 3), t.nrows - 1);
    }
}

// LAST: a last group with weights of its own is possible (B0_last); only the
// tile-queue instantiations take it, which leaves the others' code as it was
// (the extra pointer choice moved the register allocation of the fixed-order
// dual kernel and put waits for all loads into its K loop: +6 % there).
template <bool DUAL, int NW, bool KG = false, bool LAST = false>
__device__ __forceinline__ DmaSrc<32 / NW> dma_src(const GemmGroup& g, const TileRef& t, const int* src,
                                                  int w, int lane, int k_split) {
    constexpr int J = 32 / NW;
    if constexpr (KG) {
        // A rows t.row0 .., B rows t.n0 .., both from K column t.kbeg, strides lda / ldb
        static_assert(!DUAL, "grouped K is a single GEMM");
        const uint32_t A2 = (uint32_t)g.lda * 2, B2 = (uint32_t)g.ldb * 2;
        DmaSrc<J> s;
        s.kt = t.kt;
        s.rot = __builtin_amdgcn_readfirstlane((t.n0 / 256 + 17 * t.grp) % t.kt);
        s.a = static_cast<const char*>(g.A) + ((int64_t)t.row0 * g.lda + t.kbeg) * 2;
        s.b = static_cast<const char*>(g.B0) + ((int64_t)t.n0 * g.ldb + t.kbeg) * 2;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int r = w * (256 / NW) + j * 8 + (lane >> 3);
            const int c = (lane & 7) ^ swz(r);
            s.ao[j] = (uint32_t)src[j] * A2 + c * 16;
            s.bo[j] = (uint32_t)r * B2 + c * 16;
        }
        return s;
    }
    const uint32_t K2 = (uint32_t)g.K * 2;
    const int64_t k0 = (int64_t)t.ks * k_split * 2;    // first byte of the tile's K range
    DmaSrc<J> s;
    // Tiles that run at the same time start their K walks at different
    // stages: every workgroup reading the same offset of its 8 KB-strided
    // weight rows at once crowds a few HBM channels.  Tiles of one group and
    // N tile (the same weight panel) start together; N tiles of a window,
    // which share an A panel, are a few stages apart.
    s.rot = __builtin_amdgcn_readfirstlane((t.n0 / (DUAL ? 128 : 256) + 17 * t.grp) % (k_split / kBK));
    s.a = static_cast<const char*>(g.A) + (g.gather ? 0 : (int64_t)t.row0 * K2) + k0;
    // dual: the first half of the waves stage gate rows n0 .. n0 + 127, the
    // second half the same up rows; a last group with weights of its own
    // (the shared expert) reads them from B0_last / B1_last
    const bool own = LAST && g.B0_last != nullptr && t.grp == g.G - 1;
    const void* b0 = own ? g.B0_last : g.B0;
    const void* b1 = own ? g.B1_last : g.B1;
    s.b = static_cast<const char*>(DUAL ? (w < NW / 2 ? b0 : b1) : b0) +
          ((int64_t)(own ? 0 : t.grp) * g.N + t.n0) * K2 + k0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int r = w * (256 / NW) + j * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        const int a_row = g.gather ? src[j] / g.gather_div : src[j];   // token row, or tile row
        s.ao[j] = r >= t.nrows ? kDeadOff : (uint32_t)a_row * K2 + c * 16;
        s.bo[j] = (uint32_t)(DUAL ? (r & 127) : r) * K2 + c * 16;
    }
    return s;
}

// B stored [K, N] with N contiguous (the backward's data gradients read the
// weights as they are).  A stage holds 64 K rows of 256 columns (512 bytes);
// each DMA instruction fills two rows, lane i row i / 32 and 16-byte chunk
// i % 32, which holds logical chunk (i % 32) ^ 4 bt_swz(row): the 64-byte
// granules are permuted per row so that the eight rows one transposed read
// touches sit in different granules.
__device__ __forceinline__ int bt_swz(int kr) { return (kr & 3) | ((kr & 8) >> 1); }

template <int NW>
__device__ __forceinline__ DmaSrc<32 / NW> dma_src_bt(const GemmGroup& g, const TileRef& t, const int* src, int w,
                                                     int lane, int k_split) {
    constexpr int J = 32 / NW;
    static_assert(NW == 8, "two B rows per instruction and wave");
    const uint32_t K2 = (uint32_t)g.K * 2;
    const int64_t k0 = (int64_t)t.ks * k_split * 2;
    DmaSrc<J> s;
    s.rot = __builtin_amdgcn_readfirstlane((t.n0 / 256 + 17 * t.grp) % (k_split / kBK));
    s.kt = 0;
    s.a = static_cast<const char*>(g.A) + (g.gather ? 0 : (int64_t)t.row0 * K2) + k0;
    const int64_t kb = g.b_khalf ? g.b_khalf : g.K;       // K rows of one source per group
    const int64_t bofs = ((int64_t)t.grp * kb * g.N + t.n0) * 2;
    s.b = static_cast<const char*>(g.B0) + bofs;
    s.b1 = static_cast<const char*>(g.b_khalf ? g.B1 : g.B0) + bofs;
    s.bstage = (uint32_t)kBK * (uint32_t)g.N * 2;
    s.khalf = g.b_khalf ? (int)(g.b_khalf / kBK) : 0x7FFFFFFF;
    s.kbase = t.ks * (k_split / kBK);
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int r = w * (256 / NW) + j * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        const int a_row = g.gather ? src[j] / g.gather_div : src[j];
        s.ao[j] = r >= t.nrows ? kDeadOff : (uint32_t)a_row * K2 + c * 16;
        const int kr = 2 * (J * w + j) + (lane >> 5);     // K row of the stage
        const int cb = (lane & 31) ^ (4 * bt_swz(kr));
        s.bo[j] = ((uint32_t)kr * (uint32_t)g.N + 8u * cb) * 2;
    }
    return s;
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// The B fragment of one MFMA step from an N-major stage: two transposed LDS
// reads (ds_read_b64_tr_b16).  In each group of 16 lanes the read hands lane
// i element i % 4 of the 8-byte pieces read by lanes i / 4, 4 + i / 4,
// 8 + i / 4 and 12 + i / 4; source lane a of group q points at K row
// 8 (q / 2) + a / 4 (+ 4 for the second read) and columns 16 (q % 2) + 4 (a % 4)
// of the 32-column block, so lane l receives K rows 8 (l / 32) .. + 7 of
// column l % 32, the layout the MFMA expects.  off: the lane's element
// offset for step 0 (steps are 16 rows apart).
__device__ __forceinline__ int bt_frag_offset(int n_blk, int lane) {
    const int q = lane >> 4, a = lane & 15;
    const int kr = 8 * (q >> 1) + (a >> 2);
    const int col = n_blk + 16 * (q & 1) + 4 * (a & 3);
    return kr * 256 + 8 * ((col >> 3) ^ (4 * bt_swz(kr))) + (col & 7);
}

__device__ __forceinline__ bf16x8_t load_b_tr(const uint16_t* sB, int off) {
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(sB + off));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(sB + off + 4 * 256));
    const v8i16_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// store_block_bf16 with every store issued: the block's rows go through a
// buffer resource of rows_left rows (none if rows_left <= 0), whose bounds
// check drops the stores of rows past the end.  A block thus issues exactly
// four stores per lane, whatever its rows, so a later wait can leave a known
// number of them in flight.
__device__ __forceinline__ void store_block_bf16_all(uint16_t* Cb, int64_t ldc, int rows_left, const float* v,
                                                     int lane) {
    const int half = lane >> 5, r32 = lane & 31, j = r32 & 3;
    const uint32_t sel = (j & 1) ? 0x03020706u : 0x05040100u;
    const int recs = rows_left > 0 ? (int)((int64_t)rows_left * ldc * 2) : 0;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc((void*)Cb, (short)0, recs, 0x00020000);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const uint32_t d0 = pack_bf16x2(v[4 * a + 0], v[4 * a + 1]);
        const uint32_t d1 = pack_bf16x2(v[4 * a + 2], v[4 * a + 3]);
        const uint32_t n0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d0, 0xB1, 0xF, 0xF, true);
        const uint32_t n1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d1, 0xB1, 0xF, 0xF, true);
        const uint32_t e0 = __builtin_amdgcn_perm(n0, d0, sel);
        const uint32_t e1 = __builtin_amdgcn_perm(n1, d1, sel);
        const uint32_t s = (j & 2) ? e0 : e1;
        const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)s, 0x4E, 0xF, 0xF, true);
        u32x2_t out;
        out.x = (j & 2) ? r : e0;
        out.y = (j & 2) ? e1 : r;
        const int row = 8 * a + 4 * half + j;
        __builtin_amdgcn_raw_buffer_store_b64(out, rc, (int)((row * ldc + (r32 - j)) * 2), 0, 0);
    }
}

// Two adjacent 32 x 32 blocks of MFMA results (columns 0..31 and 32..63 of a
// 64-column span) as bf16, in whole 128-byte row pieces.  After the 4 x 4
// quad transpose of each block (lane j = r32 % 4 of quad q = r32 / 4 holds
// row 8 a + 4 half + j, columns 4 q .. 4 q + 3), the lanes of quads q and
// q ^ 1 swap halves (DPP row shifts by 4 lanes): an even quad ends with
// columns 4 q .. 4 q + 7 of block 0, an odd quad columns 4 (q - 1) ..
// 4 (q - 1) + 7 of block 1.  One 16-byte store per lane and a then writes 8
// rows of 128 bytes: half the store instructions of an 8-byte store per block
// and no half-written cache lines (DeepSeek-V3 down GEMM: its stores, left
// out altogether in a timing-only build, cost 12 % of it).  ALL: every lane
// issues its 4 stores through a buffer resource of rows_left rows, whose bounds
// check drops the rows past the end; else rows past the end are not stored.
template <bool ALL>
__device__ __forceinline__ void store_pair_bf16(uint16_t* Cb, int64_t ldc, int rows_left, const float* v0,
                                                const float* v1, int lane) {
    const int half = lane >> 5, r32 = lane & 31, j = r32 & 3;
    const bool odd = (r32 >> 2) & 1;
    const uint32_t sel = (j & 1) ? 0x03020706u : 0x05040100u;
    const int col = odd ? 32 + (r32 - j) - 4 : r32 - j;
    const int recs = rows_left > 0 ? (int)((int64_t)rows_left * ldc * 2) : 0;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc((void*)Cb, (short)0, recs, 0x00020000);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        uint32_t q0[2], q1[2];   // this lane's row, 4 columns, of block 0 and of block 1
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const float* v = b ? v1 : v0;
            uint32_t* o = b ? q1 : q0;
            const uint32_t d0 = pack_bf16x2(v[4 * a + 0], v[4 * a + 1]);
            const uint32_t d1 = pack_bf16x2(v[4 * a + 2], v[4 * a + 3]);
            const uint32_t n0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d0, 0xB1, 0xF, 0xF, true);
            const uint32_t n1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d1, 0xB1, 0xF, 0xF, true);
            const uint32_t e0 = __builtin_amdgcn_perm(n0, d0, sel);
            const uint32_t e1 = __builtin_amdgcn_perm(n1, d1, sel);
            const uint32_t sq = (j & 2) ? e0 : e1;
            const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)sq, 0x4E, 0xF, 0xF, true);
            o[0] = (j & 2) ? r : e0;
            o[1] = (j & 2) ? e1 : r;
        }
        // an even quad passes its block-1 piece to the odd quad 4 lanes up and
        // takes that quad's block-0 piece (row_shl:4: lane i reads lane i + 4;
        // row_shr:4: lane i reads lane i - 4; both stay inside a row of 16 lanes)
        const uint32_t s0 = odd ? q0[0] : q1[0], s1 = odd ? q0[1] : q1[1];
        const uint32_t up0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0x104, 0xF, 0xF, true);
        const uint32_t up1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0x104, 0xF, 0xF, true);
        const uint32_t dn0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0x114, 0xF, 0xF, true);
        const uint32_t dn1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0x114, 0xF, 0xF, true);
        u32x4_t out;
        out.x = odd ? dn0 : q0[0];
        out.y = odd ? dn1 : q0[1];
        out.z = odd ? q1[0] : up0;
        out.w = odd ? q1[1] : up1;
        const int row = 8 * a + 4 * half + j;
        if constexpr (ALL) {
            __builtin_amdgcn_raw_buffer_store_b128(out, rc, (int)((row * ldc + col) * 2), 0, 0);
        } else {
            if (row < rows_left) *reinterpret_cast<u32x4_t*>(Cb + row * ldc + col) = out;
        }
        // one row group at a time: interleaving them raised the register use
        // of the 288-row down kernel past its budget (spills)
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Stores one 32 x 32 block of MFMA results as bf16.  Lane (half, r32) holds
// column r32 of block rows 8 a + 4 half + b in v[4 a + b].  Inside each quad
// of lanes a 4 x 4 transpose (two DPP exchanges and byte permutes) gives lane
// j = r32 % 4 row 8 a + 4 half + j, columns r32 - j .. r32 - j + 3, written as
// one 8-byte store per a.  Rows at or past rows_left are not written.
__device__ __forceinline__ void store_block_bf16(uint16_t* Cb, int64_t ldc, int rows_left,
                                                 const float* v, int lane) {
    const int half = lane >> 5, r32 = lane & 31, j = r32 & 3;
    const uint32_t sel = (j & 1) ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const uint32_t d0 = pack_bf16x2(v[4 * a + 0], v[4 * a + 1]);   // rows b = 0, 1
        const uint32_t d1 = pack_bf16x2(v[4 * a + 2], v[4 * a + 3]);   // rows b = 2, 3
        // exchange with lane j ^ 1: even lanes keep rows 0 and 2, odd lanes rows 1 and 3
        const uint32_t n0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d0, 0xB1, 0xF, 0xF, true);
        const uint32_t n1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d1, 0xB1, 0xF, 0xF, true);
        const uint32_t e0 = __builtin_amdgcn_perm(n0, d0, sel);
        const uint32_t e1 = __builtin_amdgcn_perm(n1, d1, sel);
        // exchange with lane j ^ 2: lane j ends with row j, all four columns
        const uint32_t s = (j & 2) ? e0 : e1;
        const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)s, 0x4E, 0xF, 0xF, true);
        uint2 out;
        out.x = (j & 2) ? r : e0;
        out.y = (j & 2) ? e1 : r;
        const int row = 8 * a + 4 * half + j;
        if (row < rows_left) *reinterpret_cast<uint2*>(Cb + row * ldc + (r32 - j)) = out;
    }
}

// Stores (or adds to) one 32 x 32 block of MFMA results as fp32.  Lane (half,
// r32) holds column r32 of block rows 8 a + 4 half + b in v[4 a + b].
// VEC: inside each quad of lanes a 4 x 4 transpose (exchanges with lane j ^ 1,
// then j ^ 2) gives lane j = r32 % 4 row 8 a + 4 half + j, columns r32 - j ..
// r32 - j + 3, written as one 16-byte store per a.  Otherwise each store
// instruction writes two 128-byte row pieces (measured faster for the short
// tiles of the grouped-K mode).  Rows at or past rows_left are not written.
template <bool VEC>
__device__ __forceinline__ void store_block_f32(float* Cf, int64_t ldc, int rows_left, const f32x16_t& v,
                                                int lane, bool accumulate) {
    if constexpr (!VEC) {
        const int half = lane >> 5, r32 = lane & 31;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int row = 8 * (q >> 2) + 4 * half + (q & 3);
            if (row < rows_left) {
                float* p = Cf + row * ldc + r32;
                *p = accumulate ? *p + v[q] : v[q];
            }
        }
        return;
    }
    const int half = lane >> 5, r32 = lane & 31, j = r32 & 3;
    const bool odd = j & 1, upper = j & 2;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const float c0 = v[4 * a + 0], c1 = v[4 * a + 1], c2 = v[4 * a + 2], c3 = v[4 * a + 3];
        // j ^ 1: even lanes keep rows 0 and 2 of columns (j, j + 1), odd lanes rows 1 and 3 of (j - 1, j)
        const float r0 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(odd ? c0 : c1), 0xB1, 0xF, 0xF, true));
        const float r1 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(odd ? c2 : c3), 0xB1, 0xF, 0xF, true));
        const float p0 = odd ? r0 : c0, p1 = odd ? c1 : r0;   // row j & 1, column pair of the lane
        const float q0 = odd ? r1 : c2, q1 = odd ? c3 : r1;   // row 2 + (j & 1), same columns
        // j ^ 2: lanes 0, 1 keep their first row and take columns 2, 3 of it; lanes 2, 3 the second row
        const float t0 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(upper ? p0 : q0), 0x4E, 0xF, 0xF, true));
        const float t1 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(upper ? p1 : q1), 0x4E, 0xF, 0xF, true));
        float4 out = upper ? make_float4(t0, t1, q0, q1) : make_float4(p0, p1, t0, t1);
        const int row = 8 * a + 4 * half + j;
        if (row < rows_left) {
            float4* p = reinterpret_cast<float4*>(Cf + row * ldc + (r32 - j));
            if (accumulate) {
                const float4 o = *p;
                out.x += o.x; out.y += o.y; out.z += o.z; out.w += o.w;
            }
            *p = out;
        }
    }
}

// Tile queue of a persistent workgroup (GEMMs over ragged expert groups: the
// forward's, and the backward's recomputation, dH' and dx).
// Each XCD's range [xcd per, end) of logical tiles is walked in rounds as
// without the queue, but only the first three rounds are fixed (tile
// xcd per + r nslot + slot for round r); later tiles are claimed through
// counter q[32 xcd] (zeroed before the launch), and a workgroup whose range
// is used up claims the next tiles of the other XCDs' ranges.  Nearly empty
// tiles, of which an expert with a few rows past a multiple of 256 has one,
// then even out between workgroups.  Kept in LDS for thread 0.
struct TileQueue {
    int* q;
    int per, TL, nslot, xcd;
    int lo, end;    // the own range's claimed part
};

// Claims from counter c (a global address: a flat atomic would also hold up
// the LDS waits of the next K stage).  An atomic increment, unlike an atomic
// add, is not combined across the wave by the compiler, which would wait for
// its result at once.
__device__ __forceinline__ int claim_next(int* c) {
    using gu32 = __attribute__((address_space(1))) unsigned;
    return (int)__builtin_amdgcn_atomic_inc32((volatile gu32*)c, 0x7FFFFFFFu, __ATOMIC_RELAXED, "agent");
}

// The next unclaimed tile of another XCD's range, or -1.
__device__ __forceinline__ int steal_tile(const TileQueue& t) {
    for (int k = 1; k < 8; ++k) {
        const int y = (t.xcd + k) & 7;
        const int lo = y * t.per + 3 * t.nslot, hi = min(t.TL, (y + 1) * t.per);
        if (lo >= hi) continue;
        const int c = lo + claim_next(t.q + 32 * y);
        if (c < hi) return c;
    }
    return -1;
}

// Thread 0 at the start of tile it (it > 0): publishes tile it + 2 in
// next[(it + 1) & 1] from the claim made at the start of tile it - 1, then
// claims the tile after it (tiles 1 and 2 are fixed, and tile 3 is claimed
// at the start of tile 0).  Returns the claim in flight (-1: none), whose
// value is first needed at the start of tile it + 1, so the K loop's waits
// cover its latency.
__device__ __forceinline__ int next_tile_step(const TileQueue& ts, int* next, int it, int claim) {
    const TileQueue t = ts;
    int pub = next[1];
    if (it > 0) {
        pub = claim < 0 ? -1 : (t.lo + claim < t.end ? t.lo + claim : steal_tile(t));
        next[(it + 1) & 1] = pub;
    }
    return pub >= 0 ? claim_next(t.q + 32 * t.xcd) : -1;
}

// Kernel modes: forward (bf16 C), fp32 C over grouped rows, fp32 C over grouped K.
constexpr int kModeFwd = 0, kModeF32 = 1, kModeKgroup = 2;
// fp32 C over grouped rows with B stored [K, N], N contiguous (B0, and B1 for
// K rows from b_khalf on)
constexpr int kModeF32BT = 4;
// dual only: both products stored as bf16, A B0^T to C and A B1^T to C2 (the
// backward's recomputed pre-activations)
constexpr int kModeDualOut = 3;

// Main bf16 kernel, persistent: one workgroup of 8 waves per CU walks a list
// of 256 x 256 tiles of MFMA work.
//   single: C tile 256 rows x 256 cols of one weight matrix;
//   dual:   C tile 256 rows x 128 cols, computed for the gate and the up
//           matrix (B rows 0..127 = gate, 128..255 = up, same columns).
// Tile schedule: the real M tiles (ceil(count_e / 256) per expert, prefix sums
// in LDS) times the N tiles form a list of logical tiles, cut into 8 ranges of
// whole rounds, one per XCD (workgroup ids are dealt to the XCDs round-robin).
// Inside a range the XCD's workgroups take consecutive tiles in rounds; a
// round is a window of 4 M tiles x (workgroups / 4) N tiles, so its A and B
// panels are shared in the XCD's L2 while its tiles advance through K together.
// With ALIGNED the bands follow the groups instead (up to 6 M tiles of one
// expert, whose weights are then streamed about once).  With QUEUE only the
// first three rounds are fixed and later tiles are claimed (TileQueue above).
// Waves form a 2 x 4 grid: wave (wm, wn) owns 128 rows and two 32-row blocks
// of B (dual: gate columns 32 wn .. 32 wn + 31 and the same up columns, so
// silu(g)*u stays in registers; single: B rows 64 wn .. 64 wn + 63), i.e.
// 4 x 2 MFMA blocks = 128 fp32 accumulators per lane.
// Global -> LDS by direct 16-byte DMA (global_load_lds_dwordx4), two LDS
// buffers of 64 K-elements (separate arrays, so the compiler can see that a
// DMA into one does not alias fragment reads of the other).  Each K stage is
// four MFMA steps; one barrier per stage, before the last step.  Right after
// the barrier the buffer just consumed is refilled with the stage after next,
// so every DMA has a whole stage of MFMA work to land behind.  The stream of
// stages runs on across tiles: the last two stages of a tile fetch the first
// two of the workgroup's next tile, whose loads are in flight during the
// epilogue.
// MODE kModeF32 (single): the same tiles, C stored as fp32 (or added to C).
// MODE kModeKgroup (single): every group has all M x N tiles and walks its own
// K columns (the weight gradients of the backward: sums over each expert's
// rows, with both operands transposed so that K is contiguous).
template <bool DUAL, bool ALIGNED, int MODE = kModeFwd, bool QUEUE = false>
__global__ __launch_bounds__(512, 1) void gemm_bf16_persistent_kernel(GemmGroup g, int tiles_n) {
    constexpr int BM = 256;
    constexpr int BN = DUAL ? 128 : 256;
    constexpr bool KG = MODE == kModeKgroup;
    constexpr bool BT = MODE == kModeF32BT;
    static_assert(MODE == kModeFwd || !DUAL || MODE == kModeDualOut, "fp32 products are single GEMMs");
    static_assert(MODE != kModeDualOut || DUAL, "two outputs need the dual tile");
    static_assert(!QUEUE || (MODE != kModeKgroup && MODE != kModeF32), "no tile queue in these modes");
    constexpr int STG = 256 * kBK;    // elements of one A or B stage (32 KB)
    // A tile's first K-stage wait: with every epilogue store issued (forward
    // dual mode: 4 per block, 4 blocks), vmcnt(kEpiStores) covers the stage
    // DMA issued before them and leaves the stores in flight (vector memory
    // operations complete in issue order for this counter).  Gate/up GEMMs
    // -0.3 to -0.9 %; for the single GEMMs the stores of dead blocks cost more
    // than the wait (DeepSeek-V3 down +0.8 %), so they keep skipping them.
    constexpr bool kAllStores = MODE == kModeFwd && DUAL;
    constexpr int kEpiStores = kAllStores ? 16 : 0;
    constexpr int kWaitFirst = (7 << 4) | (kEpiStores & 15) | ((kEpiStores >> 4) << 14);
    // even M split for the gate/up tiles claimed through the queue (about one
    // M tile per expert)
    constexpr bool BAL = DUAL && QUEUE;
    __shared__ __align__(16) uint16_t sA0[STG], sA1[STG];
    __shared__ __align__(16) uint16_t sB0[STG], sB1[STG];
    __shared__ int s_tb[258], s_off[258];     // up to 257 groups (256 experts + a shared one)
    __shared__ int s_wsum[8];

    // launched beside the 288-row kernel: run only if the 256-row tiles are chosen
    if constexpr (MODE == kModeFwd)
        if (g.choice.offsets &&
            tall_tiles_chosen(g.choice.offsets, g.choice.E, g.choice.tiles_n, g.choice.slots) != (g.choice.rows == 288))
            return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 2, wn = w & 3;
    const int S = DUAL || KG ? 1 : g.splitk;  // K ranges (single GEMM only)
    const int KT = g.K / kBK / S;       // stages per tile: even, >= 2 (grouped K: per tile)

    int G, mt_total;
    if constexpr (KG) {
        G = kgroup_prefix(g, s_off);
        mt_total = G * (g.M / BM);
    } else {
        G = tile_prefix<BM>(g, s_tb, s_off, s_wsum);
        mt_total = s_tb[G];
    }
    const int TL = mt_total * tiles_n * S;
    const int nslot = gridDim.x >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    // per-XCD range: a whole number of rounds, so every round is one window
    const int per = ((TL + 7) / 8 + nslot - 1) / nslot * nslot;
    const int Lend = min(TL, (xcd + 1) * per);
    const int wn_win = max(nslot / kWMW, 1);
    int L = xcd * per + slot;
    if (L >= Lend) return;
    // queue: at the start of tile i, s_next[i & 1] holds tile i + 1 (or -1)
    __shared__ int s_next[2];
    __shared__ TileQueue s_tq;
    int claim = -1;         // thread 0: counter value of the claim in flight, or -1
    if (QUEUE && tid == 0) {
        s_tq = TileQueue{g.queue, per, TL, nslot, xcd, xcd * per + 3 * nslot, Lend};
        s_next[0] = L + nslot < Lend ? L + nslot : -1;
        s_next[1] = s_next[0] >= 0 && L + 2 * nslot < Lend ? L + 2 * nslot : -1;
    }

    const int half = lane >> 5, r32 = lane & 31;
    int a_row[4], b_row[2], bt_off[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a_row[i] = wm * 128 + i * 32 + r32;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        b_row[b] = DUAL ? b * 128 + wn * 32 + r32 : wn * 64 + b * 32 + r32;
        bt_off[b] = BT ? bt_frag_offset(wn * 64 + b * 32, lane) : 0;
    }

// Refill of a stage buffer: every A and B instruction, unconditionally (control
// flow among the DMA instructions makes the compiler wait for them before the
// next fragment reads).  A rows go through a bounds-checked buffer resource
// (record count kDeadOff), so the lanes of rows past the tile's end, whose
// offset is kDeadOff (kept there by the saturating add of the stage offset),
// issue no load: a nearly empty tile fetches little more than its B rows
// (measured -1.1 % on the DeepSeek-V3 layer, -0.5 % on Mixtral prefill).
// Grouped-K tiles have no such rows and keep plain loads.
#define MOE_DMA(sA_, sB_, src_, kt_)                                                            \
    do {                                                                                        \
        const int kr_ = (kt_) + (src_).rot;                                                     \
        const int kw_ = KG ? (src_).kt : KT;                                                    \
        const int kp_ = kr_ >= kw_ ? kr_ - kw_ : kr_;                                           \
        const char* ab_ = (src_).a + kp_ * (kBK * 2);                                           \
        const char* bb_;                                                                        \
        if constexpr (BT) {                                                                     \
            const int gs_ = (src_).kbase + kp_;                                                 \
            const bool hi_ = gs_ >= (src_).khalf;                                               \
            bb_ = (hi_ ? (src_).b1 : (src_).b) + (size_t)(hi_ ? gs_ - (src_).khalf : gs_) * (src_).bstage; \
        } else {                                                                                \
            bb_ = (src_).b + kp_ * (kBK * 2);                                                   \
        }                                                                                       \
        _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                         \
            if constexpr (!KG) {                                                                \
                /* bounds-checked: a row past the tile's end (offset kDeadOff, which the */      \
                /* saturating add keeps at or past the record count) loads nothing */            \
                const __amdgpu_buffer_rsrc_t ra_ =                                              \
                    __builtin_amdgcn_make_buffer_rsrc((void*)(src_).a, (short)0, (int)kDeadOff, 0x00020000); \
                __builtin_amdgcn_raw_ptr_buffer_load_lds(                                       \
                    ra_, (lds_ptr_t)((sA_) + (w * 32 + j * 8) * kBK), 16,                       \
                    (int)__builtin_elementwise_add_sat((src_).ao[j], (uint32_t)kp_ * (kBK * 2u)), 0, 0, 0); \
            } else {                                                                            \
                __builtin_amdgcn_global_load_lds(ab_ + (src_).ao[j],                            \
                                                 (lds_ptr_t)((sA_) + (w * 32 + j * 8) * kBK), 16, 0, 0); \
            }                                                                                   \
            __builtin_amdgcn_global_load_lds(bb_ + (src_).bo[j],                                \
                                             (lds_ptr_t)((sB_) + (w * 32 + j * 8) * kBK), 16, 0, 0); \
        }                                                                                       \
    } while (0)
// Fragments of step s_ for the first NA_ row blocks (and B, if NA_ > 0).
#define MOE_LOAD_FRAGS(sA_, sB_, s_, af_, bf_, NA_)                                             \
    do {                                                                                        \
        const int c_ = 2 * (s_) + half;                                                         \
        _Pragma("unroll") for (int i = 0; i < (NA_); ++i) af_[i] = as_bf16x8(                   \
            *reinterpret_cast<const uint4*>((sA_) + a_row[i] * kBK + ((c_ ^ swz(a_row[i])) * 8))); \
        _Pragma("unroll") for (int b = 0; b < ((NA_) ? 2 : 0); ++b) bf_[b] = BT                 \
            ? load_b_tr((sB_), bt_off[b] + (s_) * (16 * 256))                                   \
            : as_bf16x8(*reinterpret_cast<const uint4*>((sB_) + b_row[b] * kBK + ((c_ ^ swz(b_row[b])) * 8))); \
    } while (0)
#define MOE_MFMAS(af_, bf_, NA_)                                                                \
    do {                                                                                        \
        _Pragma("unroll") for (int i = 0; i < (NA_); ++i)                                       \
            _Pragma("unroll") for (int b = 0; b < 2; ++b) acc[i][b] =                           \
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af_[i], bf_[b], acc[i][b], 0, 0, 0);    \
    } while (0)
// The MFMAs of a step with the fragment reads of the following step between
// them: 2 NA MFMAs and NA + 2 reads for NA live row blocks.
#define MOE_INTERLEAVE(NA_)                                                                     \
    do {                                                                                        \
        if ((NA_) == 4) {                                                                       \
            _Pragma("unroll") for (int i_ = 0; i_ < 6; ++i_) {                                  \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                              \
            }                                                                                   \
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                  \
        } else if ((NA_) == 3) {                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < 5; ++i_) {                                  \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                              \
            }                                                                                   \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  \
        } else if ((NA_) == 2) {                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                  \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                              \
            }                                                                                   \
        } else if ((NA_) == 1) {                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < 2; ++i_) {                                  \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                              \
            }                                                                                   \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                  \
        }                                                                                       \
    } while (0)
// One K stage from buffer (sAc, sBc) for NA_ row blocks; after the barrier
// that buffer is refilled with stage kd_ of src_ (if fetch_) and the first
// fragments of (sAn, sBn) are read for NN_ row blocks (at a tile boundary,
// all 4: the next tile may have more live rows).
#define MOE_STAGE_W(NA_, NN_, sAc, sBc, sAn, sBn, src_, kd_, fetch_, wait_)                     \
    do {                                                                                        \
        MOE_LOAD_FRAGS(sAc, sBc, 1, fa1, fb1, NA_);                                             \
        MOE_MFMAS(fa0, fb0, NA_);                                                               \
        MOE_INTERLEAVE(NA_);                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAc, sBc, 2, fa0, fb0, NA_);                                             \
        MOE_MFMAS(fa1, fb1, NA_);                                                               \
        MOE_INTERLEAVE(NA_);                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAc, sBc, 3, fa1, fb1, NA_);                                             \
        MOE_MFMAS(fa0, fb0, NA_);                                                               \
        MOE_INTERLEAVE(NA_);                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        __builtin_amdgcn_s_waitcnt(wait_);                                                      \
        __builtin_amdgcn_s_barrier();                                                           \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        if (fetch_) MOE_DMA(sAc, sBc, src_, kd_);                                               \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        MOE_LOAD_FRAGS(sAn, sBn, 0, fa0, fb0, NN_);                                             \
        MOE_MFMAS(fa1, fb1, NA_);                                                               \
        MOE_INTERLEAVE((NN_) < (NA_) ? (NN_) : (NA_));                                          \
        __builtin_amdgcn_sched_barrier(0);                                                      \
    } while (0)
#define MOE_STAGE(NA_, NN_, sAc, sBc, sAn, sBn, src_, kd_, fetch_)                              \
    MOE_STAGE_W(NA_, NN_, sAc, sBc, sAn, sBn, src_, kd_, fetch_, kWaitVm0Lgkm0)
// The K stages of one tile for a wave with NA_ live row blocks.  The first
// stage's wait leaves the previous tile's epilogue stores in flight (kWaitFirst).
#define MOE_KLOOP(NA_)                                                                          \
    do {                                                                                        \
        const int kl_ = KG ? cur.kt : KT;                                                       \
        if (kl_ > 2) {                                                                          \
            MOE_STAGE_W(NA_, NA_, sA0, sB0, sA1, sB1, cur, 2, true, kWaitFirst);                \
            gather_rows<8>(g, tn, w, lane, gsrc);                                               \
            MOE_STAGE(NA_, NA_, sA1, sB1, sA0, sB0, cur, 3, true);                              \
        } else {                                                                                \
            gather_rows<8>(g, tn, w, lane, gsrc);                                               \
        }                                                                                       \
        for (int kt = 2; kt < kl_ - 2; kt += 2) {                                               \
            MOE_STAGE(NA_, NA_, sA0, sB0, sA1, sB1, cur, kt + 2, true);                         \
            MOE_STAGE(NA_, NA_, sA1, sB1, sA0, sB0, cur, kt + 3, true);                         \
        }                                                                                       \
        nxt = make_src(tn);                                                                     \
        MOE_STAGE(NA_, NA_, sA0, sB0, sA1, sB1, nxt, 0, more);                                  \
        MOE_STAGE(NA_, 4, sA1, sB1, sA0, sB0, nxt, 1, more);                                    \
    } while (0)

    const int mtiles = KG ? g.M / BM : 0;
    auto tile_of = [&](int Lt) {
        if constexpr (KG) return kgroup_tile_at<BM, BN>(s_off, mtiles, mt_total, tiles_n, wn_win, Lt);
        else return split_tile_at<BM, BN, ALIGNED, BAL>(s_tb, s_off, G, mt_total, tiles_n, wn_win, Lt);
    };
    TileRef tr = tile_of(L);
    int gsrc[4];
    gather_rows<8>(g, tr, w, lane, gsrc);
    auto make_src = [&](const TileRef& t) {
        if constexpr (BT) return dma_src_bt<8>(g, t, gsrc, w, lane, KT * kBK);
        else return dma_src<DUAL, 8, KG, QUEUE>(g, t, gsrc, w, lane, KT * kBK);
    };
    DmaSrc<4> cur = make_src(tr);
    bf16x8_t fa0[4], fb0[2], fa1[4], fb1[2];
    // prologue: the first tile's stages 0 and 1
    MOE_DMA(sA0, sB0, cur, 0);
    MOE_DMA(sA1, sB1, cur, 1);
    __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    MOE_LOAD_FRAGS(sA0, sB0, 0, fa0, fb0, 4);

    uint16_t* C = static_cast<uint16_t*>(g.C);
    for (int it = 0;; ++it) {
        int Ln;
        bool more;
        if constexpr (QUEUE) {
            Ln = __builtin_amdgcn_readfirstlane(s_next[it & 1]);
            more = Ln >= 0;
            if (tid == 0) claim = next_tile_step(s_tq, s_next, it, claim);
        } else {
            Ln = L + nslot;
            more = Ln < Lend;
        }
        const TileRef tn = tile_of(more ? Ln : L);
        // the next tile's gathered rows load after the K loop's first stage
        // (behind the previous epilogue's stores and that stage's wait); their
        // values are used at the end of the K loop
        DmaSrc<4> nxt;

        f32x16_t acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

        // live row blocks of this wave (32 rows each, from its first row): the
        // K loop runs the MFMAs and fragment reads of those blocks only
        // (one loop per count: with two counts, 2 and 4, the DeepSeek-V3
        // gate/up GEMM ran 24 % more MFMA work than its rows, with one per
        // count 11 %; layer -0.3 %, Mixtral prefill -0.5 %)
        const int blocks = min(4, max(0, (tr.nrows - wm * 128 + 31) >> 5));
        if (blocks == 4) MOE_KLOOP(4);
        else if (blocks == 3) MOE_KLOOP(3);
        else if (blocks == 2) MOE_KLOOP(2);
        else if (blocks == 1) MOE_KLOOP(1);
        else MOE_KLOOP(0);

        // epilogue: the next tile's first two stages are in flight meanwhile.
        // kAllStores: every store is issued (kEpiStores per lane; those of rows
        // past the tile's end are dropped by their bounds), so the next tile's
        // first wait leaves them in flight instead of waiting for all of them.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rb = wm * 128 + i * 32;
            if (!kAllStores && rb >= tr.nrows) break;
#pragma unroll
            for (int bo = 0; bo < (DUAL ? 1 : 2); ++bo) {
                const int cb = DUAL ? wn * 32 : wn * 64 + bo * 32;
                if constexpr (MODE == kModeDualOut) {
                    const int64_t at = (int64_t)(tr.row0 + rb) * g.N + tr.n0 + cb;
                    float v[16];
#pragma unroll
                    for (int q = 0; q < 16; ++q) v[q] = acc[i][0][q];
                    store_block_bf16(C + at, g.N, tr.nrows - rb, v, lane);
#pragma unroll
                    for (int q = 0; q < 16; ++q) v[q] = acc[i][1][q];
                    store_block_bf16(static_cast<uint16_t*>(g.C2) + at, g.N, tr.nrows - rb, v, lane);
                } else if constexpr (MODE == kModeFwd && DUAL) {
                    float v[16];
#pragma unroll
                    for (int q = 0; q < 16; ++q) v[q] = silu_f32(acc[i][0][q]) * acc[i][1][q];
                    uint16_t* Cb = C + tr.ks * g.part_stride + (int64_t)(tr.row0 + rb) * g.N + tr.n0 + cb;
                    store_block_bf16_all(Cb, g.N, tr.nrows - rb, v, lane);
                } else if constexpr (MODE == kModeFwd) {
                    // both 32-column blocks of the wave at once, as whole 128-byte rows
                    if (bo == 0) {
                        float v0[16], v1[16];
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            v0[q] = acc[i][0][q];
                            v1[q] = acc[i][1][q];
                        }
                        uint16_t* Cb = C + tr.ks * g.part_stride + (int64_t)(tr.row0 + rb) * g.N + tr.n0 + cb;
                        store_pair_bf16<false>(Cb, g.N, tr.nrows - rb, v0, v1, lane);
                    }
                } else {
                    float* Cf = static_cast<float*>(g.C) +
                                (KG ? (int64_t)tr.grp * g.c_gstride : (int64_t)tr.ks * g.part_stride) +
                                (int64_t)(tr.row0 + rb) * g.ldc + tr.n0 + cb;
                    store_block_f32<!KG>(Cf, g.ldc, tr.nrows - rb, acc[i][bo], lane, g.accumulate);
                }
            }
        }
        if (!more) break;
        L = Ln;
        tr = tn;
        cur = nxt;
    }
#undef MOE_DMA
#undef MOE_LOAD_FRAGS
#undef MOE_MFMAS
#undef MOE_INTERLEAVE
#undef MOE_STAGE
#undef MOE_STAGE_W
#undef MOE_KLOOP
}

// Tall tiles for layers with about one M tile per expert (the tile-queue
// regime): 288 rows x 256 B rows on 12 waves, for the forward's routed
// GEMMs (and the shared expert as their last group).  With 256-row tiles an
// expert of 257..288 rows takes two tiles of about 140 rows, and such a tile
// costs 85 % of a full one (it streams the whole weight panel through the DMA
// path for half the rows); with 288-row tiles nearly every expert of a
// DeepSeek-V3-sized layer (about 256 rows each) is one tile.
// Waves form a 3 x 4 grid: wave (wm, wn) owns rows 96 wm .. 96 wm + 95 (three
// 32-row blocks) and the same two 32-row blocks of B as in the 256-row kernel,
// so 96 fp32 accumulators per lane, within the 168 registers that three waves
// per SIMD leave.  Per K stage each wave issues three A and three B DMA
// instructions of 8 rows: A blocks 3 w .. 3 w + 2 (36 blocks = 288 rows), B
// blocks 3 w .. 3 w + 2, of which blocks 32..35 are spare (their lanes issue
// no request, through the bounds check of their buffer resource) and land
// in LDS rows 256..287 of the B buffer, which no fragment reads.  The K stage
// loop, the stream of stages across tiles, the tile order (expert-aligned
// bands) and the queue are those of the 256-row kernel; the epilogue issues
// every store of both the dual and the single tile, and the next tile's
// first fragments are read after it.
struct TallSrc {
    const char* a;      // A: the start of A (gathered rows) or of the tile's rows
    const char* b0;     // B panel: gate rows (dual) or the weight rows
    const char* b1;     // dual: the up rows of the same columns
    uint32_t ao[3];     // A offsets of this lane's three instructions (kDeadOff: row past the end)
    int rot;            // first K stage of the walk
};

template <bool DUAL, bool QUEUE>
__global__ __launch_bounds__(768, 1) void gemm_bf16_tall_kernel(GemmGroup g, int tiles_n) {
    constexpr int NB = 3;                  // 32-row blocks per wave
    constexpr int BM = 3 * NB * 32;        // 288
    constexpr int BN = DUAL ? 128 : 256;   // output columns of a tile
    constexpr int STG = BM * kBK;          // elements of one A or B stage buffer (36 KB)
    constexpr bool BAL = DUAL;             // even M split for the gate/up tiles
    // every epilogue store is issued (4 per 32 x 32 block; rows past the end
    // are dropped by the bounds check), so the next tile's first wait leaves
    // them in flight (the down GEMM at DeepSeek-V3: -1.9 %, where the 256-row
    // kernel, with more dead blocks, measured +0.8 %)
    constexpr int kEpiStores = 4 * NB;
    constexpr int kWaitFirst = (7 << 4) | (kEpiStores & 15) | ((kEpiStores >> 4) << 14);
    __shared__ __align__(16) uint16_t sA0[STG], sA1[STG];
    __shared__ __align__(16) uint16_t sB0[STG], sB1[STG];
    __shared__ int s_tb[258], s_off[258];
    __shared__ int s_wsum[12];
    __shared__ int s_next[2];
    __shared__ TileQueue s_tq;

    // launched beside the 256-row kernel: run only if the 288-row tiles are chosen
    if (g.choice.offsets &&
        tall_tiles_chosen(g.choice.offsets, g.choice.E, g.choice.tiles_n, g.choice.slots) != (g.choice.rows == 288))
        return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 2, wn = w & 3;
    const int KT = g.K / kBK;

    const int G = tile_prefix<BM>(g, s_tb, s_off, s_wsum);
    const int mt_total = s_tb[G];
    const int TL = mt_total * tiles_n;
    const int nslot = gridDim.x >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = ((TL + 7) / 8 + nslot - 1) / nslot * nslot;
    const int Lend = min(TL, (xcd + 1) * per);
    const int wn_win = max(nslot / kWMW, 1);
    int L = xcd * per + slot;
    if (L >= Lend) return;
    // queue: at the start of tile i, s_next[i & 1] holds tile i + 1 (or -1);
    // fixed schedule: every nslot-th tile of the XCD's range
    int claim = -1;
    if (QUEUE && tid == 0) {
        s_tq = TileQueue{g.queue, per, TL, nslot, xcd, xcd * per + 3 * nslot, Lend};
        s_next[0] = L + nslot < Lend ? L + nslot : -1;
        s_next[1] = s_next[0] >= 0 && L + 2 * nslot < Lend ? L + 2 * nslot : -1;
    }

    const int half = lane >> 5, r32 = lane & 31;
    int a_row[NB], b_row[2];
#pragma unroll
    for (int i = 0; i < NB; ++i) a_row[i] = wm * (NB * 32) + i * 32 + r32;
#pragma unroll
    for (int b = 0; b < 2; ++b) b_row[b] = DUAL ? b * 128 + wn * 32 + r32 : wn * 64 + b * 32 + r32;

    // B offsets of this lane's three instructions: the same for every tile
    const uint32_t K2 = (uint32_t)g.K * 2;
    uint32_t bo[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int r = (3 * w + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        bo[j] = r >= 256 ? kDeadOff : (uint32_t)(DUAL ? (r & 127) : r) * K2 + c * 16;
    }
    // gathered pair ids of this lane's A rows (rows past the end repeat the last)
    auto gather = [&](const TileRef& t, int* src) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int r = min((3 * w + j) * 8 + (lane >> 3), t.nrows - 1);
            src[j] = g.gather ? g.gather[t.row0 + r] : r;
        }
    };
    auto make_src = [&](const TileRef& t, const int* src) {
        TallSrc s;
        s.rot = __builtin_amdgcn_readfirstlane((t.n0 / BN + 17 * t.grp) % KT);
        s.a = static_cast<const char*>(g.A) + (g.gather ? 0 : (int64_t)t.row0 * K2);
        const bool own = g.B0_last != nullptr && t.grp == g.G - 1;
        const int64_t pan = ((int64_t)(own ? 0 : t.grp) * g.N + t.n0) * K2;
        s.b0 = static_cast<const char*>(own ? g.B0_last : g.B0) + pan;
        s.b1 = DUAL ? static_cast<const char*>(own ? g.B1_last : g.B1) + pan : s.b0;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int r = (3 * w + j) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ swz(r);
            const int arow = g.gather ? src[j] / g.gather_div : src[j];
            s.ao[j] = r >= t.nrows ? kDeadOff : (uint32_t)arow * K2 + c * 16;
        }
        return s;
    };

// Refill of a stage buffer: three A and three B instructions per wave, all
// through bounds-checked buffer resources, unconditionally.  With the tile
// queue (about one M tile per expert) the weight rows, read by one M tile,
// are loaded with the non-temporal cache policy (nt), which leaves the L2 to
// the gathered x rows that the N tiles of an expert share (DeepSeek-V3
// gate/up 4.40 -> 4.26 ms, layer -2.2 %); on the fixed schedule several M
// tiles of an expert share each weight panel, which the plain policy keeps
// in L2 for them.
#define TALL_DMA(sA_, sB_, src_, kt_)                                                           \
    do {                                                                                        \
        const int kr_ = (kt_) + (src_).rot;                                                     \
        const uint32_t ko_ = (uint32_t)(kr_ >= KT ? kr_ - KT : kr_) * (kBK * 2u);               \
        const __amdgpu_buffer_rsrc_t ra_ =                                                      \
            __builtin_amdgcn_make_buffer_rsrc((void*)(src_).a, (short)0, (int)kDeadOff, 0x00020000); \
        _Pragma("unroll") for (int j = 0; j < 3; ++j)                                           \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(                                           \
                ra_, (lds_ptr_t)((sA_) + (3 * w + j) * 8 * kBK), 16,                            \
                (int)__builtin_elementwise_add_sat((src_).ao[j], ko_), 0, 0, 0);                \
        _Pragma("unroll") for (int j = 0; j < 3; ++j) {                                         \
            const char* bp_ = DUAL && 3 * w + j >= 16 ? (src_).b1 : (src_).b0;                  \
            const __amdgpu_buffer_rsrc_t rb_ =                                                  \
                __builtin_amdgcn_make_buffer_rsrc((void*)bp_, (short)0, (int)kDeadOff, 0x00020000); \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(                                           \
                rb_, (lds_ptr_t)((sB_) + (3 * w + j) * 8 * kBK), 16,                            \
                (int)__builtin_elementwise_add_sat(bo[j], ko_), 0, 0, QUEUE ? kCacheNT : 0);    \
        }                                                                                       \
    } while (0)
#define TALL_FRAGS(sA_, sB_, s_, af_, bf_, NA_)                                                 \
    do {                                                                                        \
        const int c_ = 2 * (s_) + half;                                                         \
        _Pragma("unroll") for (int i = 0; i < (NA_); ++i) af_[i] = as_bf16x8(                   \
            *reinterpret_cast<const uint4*>((sA_) + a_row[i] * kBK + ((c_ ^ swz(a_row[i])) * 8))); \
        _Pragma("unroll") for (int b = 0; b < ((NA_) ? 2 : 0); ++b) bf_[b] = as_bf16x8(         \
            *reinterpret_cast<const uint4*>((sB_) + b_row[b] * kBK + ((c_ ^ swz(b_row[b])) * 8))); \
    } while (0)
#define TALL_MFMAS(af_, bf_, NA_)                                                               \
    do {                                                                                        \
        _Pragma("unroll") for (int i = 0; i < (NA_); ++i)                                       \
            _Pragma("unroll") for (int b = 0; b < 2; ++b) acc[i][b] =                           \
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af_[i], bf_[b], acc[i][b], 0, 0, 0);    \
    } while (0)
// MFMAs of a step with the next step's fragment reads between them
#define TALL_INTERLEAVE(NA_)                                                                    \
    do {                                                                                        \
        if ((NA_) == 3) {                                                                       \
            _Pragma("unroll") for (int i_ = 0; i_ < 5; ++i_) {                                  \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                              \
            }                                                                                   \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  \
        } else if ((NA_) == 2) {                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                  \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                              \
            }                                                                                   \
        } else if ((NA_) == 1) {                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < 2; ++i_) {                                  \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                              \
            }                                                                                   \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                  \
        }                                                                                       \
    } while (0)
#define TALL_STAGE_W(NA_, NN_, sAc, sBc, sAn, sBn, src_, kd_, fetch_, wait_)                    \
    do {                                                                                        \
        TALL_FRAGS(sAc, sBc, 1, fa1, fb1, NA_);                                                 \
        TALL_MFMAS(fa0, fb0, NA_);                                                              \
        TALL_INTERLEAVE(NA_);                                                                   \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        TALL_FRAGS(sAc, sBc, 2, fa0, fb0, NA_);                                                 \
        TALL_MFMAS(fa1, fb1, NA_);                                                              \
        TALL_INTERLEAVE(NA_);                                                                   \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        TALL_FRAGS(sAc, sBc, 3, fa1, fb1, NA_);                                                 \
        TALL_MFMAS(fa0, fb0, NA_);                                                              \
        TALL_INTERLEAVE(NA_);                                                                   \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        __builtin_amdgcn_s_waitcnt(wait_);                                                      \
        __builtin_amdgcn_s_barrier();                                                           \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        if (fetch_) TALL_DMA(sAc, sBc, src_, kd_);                                              \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        TALL_FRAGS(sAn, sBn, 0, fa0, fb0, NN_);                                                 \
        TALL_MFMAS(fa1, fb1, NA_);                                                              \
        TALL_INTERLEAVE((NN_) < (NA_) ? (NN_) : (NA_));                                         \
        __builtin_amdgcn_sched_barrier(0);                                                      \
    } while (0)
#define TALL_STAGE(NA_, NN_, sAc, sBc, sAn, sBn, src_, kd_, fetch_)                             \
    TALL_STAGE_W(NA_, NN_, sAc, sBc, sAn, sBn, src_, kd_, fetch_, kWaitVm0Lgkm0)
#define TALL_KLOOP(NA_)                                                                         \
    do {                                                                                        \
        if (KT > 2) {                                                                           \
            TALL_STAGE_W(NA_, NA_, sA0, sB0, sA1, sB1, cur, 2, true, kWaitFirst);               \
            gather(tn, gsrc);                                                                   \
            TALL_STAGE(NA_, NA_, sA1, sB1, sA0, sB0, cur, 3, true);                             \
        } else {                                                                                \
            gather(tn, gsrc);                                                                   \
        }                                                                                       \
        for (int kt = 2; kt < KT - 2; kt += 2) {                                                \
            TALL_STAGE(NA_, NA_, sA0, sB0, sA1, sB1, cur, kt + 2, true);                        \
            TALL_STAGE(NA_, NA_, sA1, sB1, sA0, sB0, cur, kt + 3, true);                        \
        }                                                                                       \
        nxt = make_src(tn, gsrc);                                                               \
        TALL_STAGE(NA_, NA_, sA0, sB0, sA1, sB1, nxt, 0, more);                                 \
        TALL_STAGE(NA_, 0, sA1, sB1, sA0, sB0, nxt, 1, more);                                   \
    } while (0)

    auto tile_of = [&](int Lt) {
        return split_tile_at<BM, BN, true, BAL>(s_tb, s_off, G, mt_total, tiles_n, wn_win, Lt);
    };
    TileRef tr = tile_of(L);
    int gsrc[3];
    gather(tr, gsrc);
    TallSrc cur = make_src(tr, gsrc);
    bf16x8_t fa0[NB], fb0[2], fa1[NB], fb1[2];
    TALL_DMA(sA0, sB0, cur, 0);
    TALL_DMA(sA1, sB1, cur, 1);
    __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    TALL_FRAGS(sA0, sB0, 0, fa0, fb0, NB);

    uint16_t* C = static_cast<uint16_t*>(g.C);
    for (int it = 0;; ++it) {
        int Ln;
        bool more;
        if constexpr (QUEUE) {
            Ln = __builtin_amdgcn_readfirstlane(s_next[it & 1]);
            more = Ln >= 0;
            if (tid == 0) claim = next_tile_step(s_tq, s_next, it, claim);
        } else {
            Ln = L + nslot;
            more = Ln < Lend;
        }
        const TileRef tn = tile_of(more ? Ln : L);
        TallSrc nxt;

        f32x16_t acc[NB][2];
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

        // live row blocks of this wave; a wave with one runs the two-block loop
        // (a third K loop variant made the compiler spill 90 registers per lane
        // around the loops)
        const int blocks = min(NB, max(0, (tr.nrows - wm * (NB * 32) + 31) >> 5));
        if (blocks == 3) TALL_KLOOP(3);
        else if (blocks > 0) TALL_KLOOP(2);
        else TALL_KLOOP(0);

#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int rb = wm * (NB * 32) + i * 32;
            if constexpr (DUAL) {
                float v[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) v[q] = silu_f32(acc[i][0][q]) * acc[i][1][q];
                store_block_bf16_all(C + (int64_t)(tr.row0 + rb) * g.N + tr.n0 + wn * 32, g.N, tr.nrows - rb, v,
                                     lane);
            } else {
                float v0[16], v1[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    v0[q] = acc[i][0][q];
                    v1[q] = acc[i][1][q];
                }
                store_pair_bf16<true>(C + (int64_t)(tr.row0 + rb) * g.N + tr.n0 + wn * 64, g.N, tr.nrows - rb, v0,
                                      v1, lane);
            }
        }
        if (!more) break;
        // the next tile's first fragments (its stage 0 landed before the last
        // barrier): read after the epilogue, so that they do not hold registers
        // through it
        TALL_FRAGS(sA0, sB0, 0, fa0, fb0, NB);
        L = Ln;
        tr = tn;
        cur = nxt;
    }
#undef TALL_DMA
#undef TALL_FRAGS
#undef TALL_MFMAS
#undef TALL_INTERLEAVE
#undef TALL_STAGE
#undef TALL_STAGE_W
#undef TALL_KLOOP
}

// Few rows per group (decode): the weights are the stream and the MFMA work
// is small, so the tile is 32 rows of one group x NBLK blocks of 32 weight
// rows (dual: NBLK / 2 gate blocks and the same up blocks, so a tile yields
// 16 NBLK columns of silu(g) * u; single: 32 NBLK columns) over one K range.
// One workgroup of 4 waves per tile; the K chunks stream through LDS (the
// shared 32-row product above).  With NST = 4 and NBLK = 4 a workgroup takes
// 80 KB of LDS (four 20 KB stages; the tile lookup borrows the last one before
// the stream starts), so two run on a CU and one's set-up and epilogue overlap
// the other's stream.  Logical tile L: N tile fastest, then the M tile (of 32
// rows, by the prefix over the groups), then the K range.  The K walk of a
// tile starts at a chunk that depends on its N tile and group, so tiles that
// run together read different offsets of their weight rows.
template <bool DUAL, int NBLK, int NST>
__global__ __launch_bounds__(256, NBLK * NST <= 16 ? 2 : 1) void gemm_bf16_skinny_kernel(GemmGroup g, int tiles_n,
                                                                                        int mt_upper) {
    constexpr int KS = (DUAL && NBLK == 4) ? 2 : 1;
    using Sh = SkinnyShape<NBLK, NST, KS>;
    constexpr int COLS = DUAL ? 16 * NBLK : 32 * NBLK;   // output columns per tile
    constexpr int X3 = NST > 3 ? Sh::XS : 8, W3 = NST > 3 ? Sh::WS : 8;
    __shared__ __align__(16) uint16_t sX0[Sh::XS], sX1[Sh::XS], sX2[Sh::XS], sX3[X3];
    __shared__ __align__(16) uint16_t sW0[Sh::WS], sW1[Sh::WS], sW2[Sh::WS], sW3[W3];

    const int L = blockIdx.x;
    const int nt = L % tiles_n;
    const int mt = (L / tiles_n) % mt_upper;
    const int ks = L / tiles_n / mt_upper;
    int grp, row0, nrows;
    // the tile lookup's scratch: the last stage buffer, first written after
    // the first barrier of the K loop
    if (!locate_tile_in<32>(g, mt, &grp, &row0, &nrows, reinterpret_cast<int*>(NST > 3 ? sX3 : sX2)))
        return;   // uniform over the workgroup
    grp = __builtin_amdgcn_readfirstlane(grp);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    nrows = __builtin_amdgcn_readfirstlane(nrows);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int S = DUAL ? 1 : g.splitk;
    const int nchunks = g.K / kSkChunk / S;
    const int64_t rowb = (int64_t)g.K * 2;
    const int64_t k0b = (int64_t)ks * nchunks * (kSkChunk * 2);
    const int n0 = nt * COLS;

    const char* src[Sh::P];
    {
        const int r = 8 * w + (lane >> 3);
        const int rr = row0 + min(r, nrows - 1);       // rows past the tile's end repeat its last row
        const int64_t arow = g.gather ? g.gather[rr] / g.gather_div : rr;
        src[0] = static_cast<const char*>(g.A) + arow * rowb + k0b + (((lane & 7) ^ swz(r)) * 16);
#pragma unroll
        for (int j = 1; j < Sh::P; ++j) {
            const int rb = 8 * (w + 4 * j - 4) + (lane >> 3);          // B row of the tile
            const char* base;
            int n;
            if (DUAL) {
                base = static_cast<const char*>(rb < 16 * NBLK ? g.B0 : g.B1);
                n = n0 + (rb < 16 * NBLK ? rb : rb - 16 * NBLK);
            } else {
                base = static_cast<const char*>(g.B0);
                n = n0 + rb;
            }
            src[j] = base + ((int64_t)grp * g.N + n) * rowb + k0b + (((lane & 7) ^ swz(rb)) * 16);
        }
    }
    const int rot = __builtin_amdgcn_readfirstlane((nt + 17 * grp) % nchunks);

    f32x16_t acc[Sh::BPW];
#pragma unroll
    for (int i = 0; i < Sh::BPW; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.0f;
    skinny_mma<Sh, DUAL, kCacheNT>(src, nchunks, rot, sX0, sX1, sX2, sX3, sW0, sW1, sW2, sW3, acc);

    const int gi = w % Sh::NG;
    if (KS == 2) {
        // waves 2, 3 hold the partial sums of K steps 2, 3 of groups 0, 1:
        // handed to waves 0, 1 through LDS (after every wave's last reads
        // and DMAs), added in that order
        float* red = reinterpret_cast<float*>(sW0);
        static_assert(KS != 2 || Sh::WS * 2 >= 2 * Sh::BPW * 16 * 64 * 4, "reduction space");
        __syncthreads();
        if (w >= 2) {
#pragma unroll
            for (int i = 0; i < Sh::BPW; ++i)
#pragma unroll
                for (int j = 0; j < 16; ++j) red[((gi * Sh::BPW + i) * 16 + j) * 64 + lane] = acc[i][j];
        }
        __syncthreads();
        if (w >= 2) return;
#pragma unroll
        for (int i = 0; i < Sh::BPW; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][j] += red[((gi * Sh::BPW + i) * 16 + j) * 64 + lane];
    }
    uint16_t* C = static_cast<uint16_t*>(g.C) + (int64_t)ks * g.part_stride + (int64_t)row0 * g.N + n0;
    if (DUAL) {
        // this wave: gate block gi (acc[0]) and up block gi + NG (acc[1]), columns 32 gi ..
        static_assert(!DUAL || Sh::BPW == 2, "dual pairs one gate and one up block per wave");
        float v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = silu_f32(acc[0][q]) * acc[1][q];
        store_block_bf16(C + 32 * gi, g.N, nrows, v, lane);
    } else {
#pragma unroll
        for (int i = 0; i < Sh::BPW; ++i) {
            float v[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = acc[i][q];
            store_block_bf16(C + 32 * skinny_block<Sh, false>(w, i), g.N, nrows, v, lane);
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
    hipExtLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(kThreads), lds, s, g.t_start, g.t_stop, 0, g, tiles_n,
                          (int)mtu);
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

template <bool DUAL>
hipError_t launch_bf16_persistent(const GemmGroup& g, hipStream_t s) {
    constexpr int BN = DUAL ? 128 : 256;
    // one instantiation per tile order: a runtime choice inside the kernel
    // costs the K loop a compiler-inserted wait on the loads in flight
    const dim3 grid(persistent_grid()), block(512);
    if (g.tall) {
        // 288-row tiles on 12 waves: the expert-aligned order, no K split; the
        // fixed schedule only as one side of a device-side choice
        if (!g.aligned_bands || g.splitk != 1 || !(g.queue || g.choice.offsets)) return hipErrorInvalidValue;
        if (g.queue)
            hipExtLaunchKernelGGL((gemm_bf16_tall_kernel<DUAL, true>), grid, dim3(768), 0, s, g.t_start, g.t_stop,
                                  0, g, g.N / BN);
        else
            hipExtLaunchKernelGGL((gemm_bf16_tall_kernel<DUAL, false>), grid, dim3(768), 0, s, g.t_start,
                                  g.t_stop, 0, g, g.N / BN);
        return hipGetLastError();
    }
    if (g.queue) {
        if (g.aligned_bands)
            hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<DUAL, true, kModeFwd, true>), grid, block, 0, s,
                                  g.t_start, g.t_stop, 0, g, g.N / BN);
        else
            hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<DUAL, false, kModeFwd, true>), grid, block, 0, s,
                                  g.t_start, g.t_stop, 0, g, g.N / BN);
        return hipGetLastError();
    }
    if (g.aligned_bands) {
        hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<DUAL, true>), grid, block, 0, s, g.t_start, g.t_stop,
                              0, g, g.N / BN);
        return hipGetLastError();
    }
    hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<DUAL, false>), grid, block, 0, s, g.t_start, g.t_stop, 0,
                          g, g.N / BN);
    return hipGetLastError();
}

// fp32 products on the persistent kernel (the backward's GEMMs).
hipError_t launch_bf16_f32out(const GemmGroup& g, hipStream_t s) {
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    // 16-byte fp32 stores: C, its row stride and slice / group strides in whole 4-float pieces
    if (!al16(g.A) || !al16(g.B0) || !al16(g.C) || g.ldc < g.N || g.ldc % 4 || g.part_stride % 4 ||
        g.c_gstride % 4 || g.N % 256 || g.N <= 0)
        return hipErrorInvalidValue;
    const dim3 grid(persistent_grid()), block(512);
    if (g.kgrouped) {
        const int G = g.kofs ? g.G : 1;
        // 32-bit DMA offsets: 256 rows of A or B from the tile's first row
        const bool ok = g.M > 0 && g.M % 256 == 0 && G >= 1 && G <= 256 && g.splitk == 1 && !g.accumulate &&
                        !g.gather && g.lda % 8 == 0 && g.ldb % 8 == 0 && (int64_t)256 * g.lda * 2 < (int64_t(1) << 32) &&
                        (int64_t)256 * g.ldb * 2 < (int64_t(1) << 32) && (g.kofs || (g.K % 128 == 0 && g.K >= 128));
        if (!ok) return hipErrorInvalidValue;
        hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<false, false, kModeKgroup>), grid, block, 0, s,
                              g.t_start, g.t_stop, 0, g, g.N / 256);
        return hipGetLastError();
    }
    const int64_t a_rows = g.gather ? ((int64_t)g.M + g.gather_div - 1) / g.gather_div : 0;
    if (g.splitk < 1 || g.K % (128 * g.splitk) || (g.accumulate && g.splitk != 1) ||
        a_rows * g.K * 2 >= (int64_t(1) << 32))
        return hipErrorInvalidValue;
    if (g.b_nmajor) {
        // 32-bit offsets inside one B stage (64 rows of N); two sources split at a stage boundary
        if ((int64_t)kBK * g.N * 2 >= (int64_t(1) << 32) || (g.b_khalf && (g.K != 2 * g.b_khalf ||
            g.b_khalf % kBK || !g.B1 || !al16(g.B1))))
            return hipErrorInvalidValue;
        if (g.queue && !g.aligned_bands) return hipErrorInvalidValue;
        if (g.queue)
            hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<false, true, kModeF32BT, true>), grid, block, 0, s,
                                  g.t_start, g.t_stop, 0, g, g.N / 256);
        else if (g.aligned_bands)
            hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<false, true, kModeF32BT>), grid, block, 0, s,
                                  g.t_start, g.t_stop, 0, g, g.N / 256);
        else
            hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<false, false, kModeF32BT>), grid, block, 0, s,
                                  g.t_start, g.t_stop, 0, g, g.N / 256);
        return hipGetLastError();
    }
    if (g.aligned_bands)
        hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<false, true, kModeF32>), grid, block, 0, s, g.t_start,
                              g.t_stop, 0, g, g.N / 256);
    else
        hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<false, false, kModeF32>), grid, block, 0, s, g.t_start,
                              g.t_stop, 0, g, g.N / 256);
    return hipGetLastError();
}

constexpr int kSkNblk = 4, kSkNst = 4;

template <bool DUAL>
hipError_t launch_bf16_skinny(const GemmGroup& g, hipStream_t s) {
    constexpr int COLS = DUAL ? 16 * kSkNblk : 32 * kSkNblk;
    const int tiles_n = g.N / COLS;
    const int64_t mtu = g.offsets ? grouped_m_tiles_upper(g.M, g.G, 32) : (g.M + 31) / 32;
    const int S = DUAL ? 1 : g.splitk;
    const int64_t grid = mtu * tiles_n * S;
    if (grid == 0) return hipSuccess;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL((gemm_bf16_skinny_kernel<DUAL, kSkNblk, kSkNst>), dim3((unsigned)grid), dim3(256), 0, s,
                          g.t_start, g.t_stop, 0,
                       g, tiles_n, (int)mtu);
    return hipGetLastError();
}

template <bool DUAL>
hipError_t launch_f32(const GemmGroup& g, hipStream_t s) {
    const int tiles_n = g.N / 64;
    const int64_t mtu = g.offsets ? grouped_m_tiles_upper(g.M, g.G, 64) : (g.M + 63) / 64;
    if (mtu == 0) return hipSuccess;
    hipExtLaunchKernelGGL(gemm_f32_kernel<DUAL>, dim3((unsigned)(mtu * tiles_n)), dim3(kThreads), 0, s,
                          g.t_start, g.t_stop, 0,
                       g, tiles_n, (int)mtu);
    return hipGetLastError();
}

}  // namespace

int persistent_slots() { return persistent_grid(); }

int64_t grouped_m_tiles_upper(int64_t rows, int G, int bm) {
    // sum_e ceil(n_e / bm) <= floor((sum_e n_e + G*(bm-1)) / bm)
    return (rows + (int64_t)G * (bm - 1)) / bm;
}

int choose_splitk(int64_t mt_expected, int N, int K) {
    constexpr int kCUs = 256;                  // MI355X; only the choice depends on it
    if (N % 256 || K % 128 || mt_expected <= 0) return 1;
    const int64_t tiles = mt_expected * (N / 256);
    int best = 1;
    double best_cost = (double)((tiles + kCUs - 1) / kCUs);
    for (int sk = 2; sk <= 8; sk *= 2) {
        // at least 24 K stages of 64 per split, or the tile set-up dominates
        if (K % (128 * sk) || K / (64 * sk) < 24) break;
        // rounds of tiles, each 1/sk of a whole tile; a split must save 5 %
        const double cost = (double)((tiles * sk + kCUs - 1) / kCUs) / sk;
        if (cost < best_cost * 0.95) { best = sk; best_cost = cost; }
    }
    return best;
}

bool skinny_rows(int64_t rows, int G) { return rows <= (int64_t)32 * G; }

bool skinny_fits(int N, int K, bool dual, int splitk) {
    const int cols = dual ? 16 * kSkNblk : 32 * kSkNblk;
    return N % cols == 0 && splitk >= 1 && K % (kSkChunk * splitk) == 0 && (!dual || splitk == 1);
}

int choose_splitk_skinny(int64_t mt_expected, int N, int K) {
    constexpr int kSlots = 2 * 256;            // workgroups in flight: two per CU
    const int cols = 32 * kSkNblk;
    if (N % cols || mt_expected <= 0) return 1;
    const int64_t tiles = mt_expected * (N / cols);
    int best = 1;
    double best_cost = (double)((tiles + kSlots - 1) / kSlots);
    for (int sk = 2; sk <= 8; sk *= 2) {
        // at least 32 chunks of 64 per split
        if (K % (kSkChunk * sk) || K / (kSkChunk * sk) < 32) break;
        const double cost = (double)((tiles * sk + kSlots - 1) / kSlots) / sk;
        if (cost < best_cost * 0.95) { best = sk; best_cost = cost; }
    }
    return best;
}

hipError_t launch_grouped_gemm(const GemmGroup& g, bool dual, bool bf16, hipStream_t s) {
    if (g.M == 0) return hipSuccess;
    if (g.B0_last) {
        // a last group with weights of its own: the forward's persistent kernels
        // with the tile queue only
        const int64_t a_rows = g.gather ? ((int64_t)g.M + g.gather_div - 1) / g.gather_div : 0;
        const bool persistent = bf16 && !g.skinny && !g.f32_out && !g.kgrouped && !g.C2 && g.splitk == 1 &&
                                g.K % 128 == 0 && a_rows * g.K * 2 < (int64_t(1) << 32) && g.offsets &&
                                g.queue && g.aligned_bands && !g.b_nmajor && g.G >= 2 && g.G <= 257 &&
                                (dual ? (g.N % 128 == 0 && g.B1_last) : g.N % 256 == 0);
        if (!persistent) return hipErrorInvalidValue;
    } else if (g.G > 256) {
        return hipErrorInvalidValue;
    }
    if (g.C2) {
        // both products of the dual tile: the persistent kernel only
        const int64_t a_rows = g.gather ? ((int64_t)g.M + g.gather_div - 1) / g.gather_div : 0;
        if (!dual || !bf16 || g.skinny || g.splitk != 1 || g.f32_out || g.kgrouped || g.K % 128 ||
            g.N % 128 || a_rows * g.K * 2 >= (int64_t(1) << 32))
            return hipErrorInvalidValue;
        const dim3 grid(persistent_grid()), block(512);
        if (g.queue && !g.aligned_bands) return hipErrorInvalidValue;
        if (g.queue)
            hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<true, true, kModeDualOut, true>), grid, block, 0, s,
                                  g.t_start, g.t_stop, 0, g, g.N / 128);
        else if (g.aligned_bands)
            hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<true, true, kModeDualOut>), grid, block, 0, s,
                                  g.t_start, g.t_stop, 0, g, g.N / 128);
        else
            hipExtLaunchKernelGGL((gemm_bf16_persistent_kernel<true, false, kModeDualOut>), grid, block, 0, s,
                                  g.t_start, g.t_stop, 0, g, g.N / 128);
        return hipGetLastError();
    }
    if (g.f32_out || g.kgrouped) {
        if (dual || !bf16 || g.skinny) return hipErrorInvalidValue;
        return launch_bf16_f32out(g, s);
    }
    if (g.skinny) {
        if (!bf16 || !skinny_fits(g.N, g.K, dual, g.splitk)) return hipErrorInvalidValue;
        return dual ? launch_bf16_skinny<true>(g, s) : launch_bf16_skinny<false>(g, s);
    }
    if (g.splitk != 1 && (dual || !bf16 || g.splitk < 1 || g.K % (128 * g.splitk) || g.N % 256))
        return hipErrorInvalidValue;
    if (!bf16) return dual ? launch_f32<true>(g, s) : launch_f32<false>(g, s);
    // The persistent kernel takes K stages in pairs (K % 128 == 0) and
    // addresses gathered A rows with 32-bit byte offsets from the start of A.
    const int64_t a_rows = g.gather ? ((int64_t)g.M + g.gather_div - 1) / g.gather_div : 0;
    const bool fits = g.K % 128 == 0 && a_rows * g.K * 2 < (int64_t(1) << 32);
    if (fits && dual && g.N % 128 == 0) return launch_bf16_persistent<true>(g, s);
    if (fits && !dual && g.N % 256 == 0) return launch_bf16_persistent<false>(g, s);
    if (g.splitk != 1) return hipErrorInvalidValue;
    if (g.N % 128 == 0) return dual ? launch_bf16<128, 128, true>(g, s) : launch_bf16<128, 128, false>(g, s);
    return dual ? launch_bf16<128, 64, true>(g, s) : launch_bf16<128, 64, false>(g, s);
}

}  // namespace moe
