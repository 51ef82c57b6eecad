// Internal declarations shared by the HIP kernels and the C-ABI host code.
// gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct moe_config;

namespace moe {

using bf16_t = uint16_t;  // bf16 storage: upper half of an IEEE fp32

// The C ABI's check of a moe_config: MOE_OK or the negative status the entry
// points return for it (host only).
int validate_config(const moe_config* cfg);

// ---- dispatch: histogram, scan, stable scatter ------------------------------
constexpr int kDispatchChunk = 2048;   // at most this many pairs: one workgroup does the whole dispatch
constexpr int kScatterChunk = 512;     // more pairs: chunks of this many, one workgroup each
struct DispatchArgs {
    const int32_t* ids;     // [P]
    int32_t* counts;        // [E]
    int32_t* offsets;       // [E+1]
    int32_t* sorted_pairs;  // [P]
    int32_t* pair_pos;      // [P]
    int32_t* chunk_counts;  // [nchunks, E] scratch
    int P, E;
    int cap = 0x7FFFFFFF;   // pairs kept per expert (the first ones); the rest get pair_pos -1
    int32_t* zero = nullptr;  // P > 0: nzero ints set to 0 on the way (the GEMMs' tile-queue counters)
    int nzero = 0;
    // tail > 0 (no capacity; several chunks): one more group of `tail` rows
    // after the experts' pairs, sorted_pairs[P + i] = i * tail_mul and
    // offsets[E + 1] = P + tail (the shared expert's tokens as a group of the
    // routed GEMMs)
    int tail = 0;
    int tail_mul = 1;
};
// 1 for P <= kDispatchChunk (one workgroup), else chunks of kScatterChunk pairs.
int dispatch_num_chunks(int P);
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);

// ---- router + top-k ---------------------------------------------------------
struct RouteArgs {
    const void* x;          // [T, d]
    const void* w;          // [E, d]
    int32_t* ids;           // [T, k]
    float* weights;         // [T, k]
    float* gap;             // [T, 2] (key margin, score margin) or nullptr
    int T, d, E, k;
    int score_fn;           // 0 softmax, 1 sigmoid
    int renorm;
    const float* bias = nullptr;  // [E] selection-only bias, or nullptr
    int bias_on_scores = 0;       // 0: key = logit + bias; 1: key = score + bias
    float* stats_part = nullptr;  // [token blocks of 32][2E] per-block sums, or nullptr
};
hipError_t launch_route(const RouteArgs& a, bool bf16, hipStream_t s);
// Router statistics from the per-block sums of a routing call:
// out [2E + 3] = f_e (E), P_e (E), L_aux = alpha E sum_e f_e P_e, max_e n_e / mean_e n_e,
// sum_e max(0, n_e - cap) (cap = INT32_MAX: no capacity, 0).
hipError_t launch_router_stats(const float* stats_part, int blocks, int E, int T, float alpha, int cap,
                               float* out, hipStream_t s);
// bf16 only: the K chunks in `ranges` ranges, one workgroup per (32 tokens,
// range), partial logits in part [ranges, T, E] fp32, then a second kernel
// adds them in range order and selects.  For batches of fewer than 256 token
// blocks (route_ranges: about 256 workgroups).
// With d (T <= 32 only; d->ids == a.ids) the second kernel also runs the
// dispatch of the pairs.
int route_ranges(int T, int d, bool bf16);
hipError_t launch_route_split(const RouteArgs& a, int ranges, float* part, const DispatchArgs* d,
                              hipStream_t s);
// bf16, 129..256 experts: 128 tokens per workgroup (the W_r stream serves
// four times the tokens), ranges of K chunks (route_ranges_wide: about 256
// workgroups), partial logits in part [ranges, T, E] fp32, then the same
// selection kernel.
int route_ranges_wide(int T, int d);
hipError_t launch_route_split_wide(const RouteArgs& a, int ranges, float* part, hipStream_t s);

// ---- tile height chosen on the device ---------------------------------------
// With several M tiles per expert (the routed GEMMs' fixed schedule) the
// expert counts decide whether 256-row tiles (8 waves) or 288-row tiles (12
// waves; the down GEMM unsplit) take less time, and only the device holds
// them.  moe_forward then launches both kernels of each GEMM (and, when the
// K splits differ, a combine for each), and a kernel given a TileChoice runs
// only if the choice is its tile height (tall_tiles_chosen, device_util.h).
struct TileChoice {
    const int32_t* offsets = nullptr;  // [E + 1] grouped rows per expert; nullptr: no choice
    int E = 0;
    int tiles_n = 0;    // N tiles of 256 columns of the gate/up GEMM (2 d_ff / 256)
    int slots = 0;      // workgroups of the persistent grid
    int rows = 0;       // the tile height this kernel stands for: 256 or 288
};

// ---- grouped GEMMs ----------------------------------------------------------
// One "problem group" of the grouped GEMM: rows of A (optionally gathered)
// times per-group weight matrices.  Row r of group g spans
// [offsets[g], offsets[g+1]) (or [0, M) when offsets == nullptr).
struct GemmGroup {
    const void* A;          // activation source [*, K]
    const int32_t* gather;  // grouped row -> pair id (nullptr: identity rows)
    int gather_div;         // source row = pair id / gather_div
    const int32_t* offsets; // [G+1] or nullptr
    int G;                  // number of groups (experts)
    int M;                  // rows when offsets == nullptr; upper bound otherwise
    const void* B0;         // [G, N, K]   (gate weights, or down weights)
    const void* B1;         // [G, N, K]   (up weights; dual mode only)
    void* C;                // [rows, N]; split K: [splitk][part_stride]
    int N, K;
    int splitk = 1;         // single bf16 only: K cut into splitk ranges, one C slice each
    int64_t part_stride = 0;// elements between C slices when splitk > 1
    bool aligned_bands = false; // bf16 persistent kernel: tile bands follow group boundaries
    bool skinny = false;    // bf16, few rows per group: 32-row tiles streaming the weights
    hipEvent_t t_start = nullptr, t_stop = nullptr;  // recorded when the kernel starts / ends
    // fp32 products (single bf16 GEMM on the persistent kernel):
    //   f32_out: C fp32 [rows, ldc] (split K: slices part_stride apart);
    //     accumulate (splitk 1): C += product.
    //   kgrouped: every group has the whole M x N output and sums over its own
    //     K columns [kofs[g], kofs[g+1]) (multiples of 128, at least 128;
    //     kofs == nullptr: one group over [0, K)): A(m, k) = A[m lda + k],
    //     B(n, k) = B0[n ldb + k], C(g, m, n) = C[g c_gstride + m ldc + n];
    //     M and N multiples of 256.
    bool f32_out = false;
    bool accumulate = false;
    //   b_nmajor (f32_out, persistent kernel): B stored [G][K][N] with N
    //     contiguous instead of [G][N][K]; with b_khalf > 0 (K == 2 b_khalf)
    //     K rows from b_khalf on come from B1 [G][b_khalf][N] (the weights as
    //     they are: no transposed copies for the data gradients)
    bool b_nmajor = false;
    int64_t b_khalf = 0;
    // dual, bf16, persistent kernel only: C = A B0^T and C2 = A B1^T, both
    // [rows, N] bf16 (no SiLU product)
    void* C2 = nullptr;
    bool kgrouped = false;
    const int32_t* kofs = nullptr;
    int64_t lda = 0, ldb = 0, ldc = 0, c_gstride = 0;
    // bf16 persistent kernel, forward mode: 256 ints, zeroed before the
    // launch, through which the workgroups claim tiles past their first three
    // rounds and take other XCDs' tiles once their own run out (nullptr: each
    // workgroup walks a fixed list)
    int* queue = nullptr;
    // bf16 persistent kernel, forward mode, non-null: the last group (G - 1)
    // takes its weights from B0_last [N, K] (and B1_last, dual) instead of
    // B0 + (G - 1) N K
    const void* B0_last = nullptr;
    const void* B1_last = nullptr;
    // bf16 persistent kernel, forward mode with the tile queue and the
    // expert-aligned order: 288-row tiles on 12 waves instead of 256-row ones
    // (also on the fixed schedule, when launched with a choice)
    bool tall = false;
    // bf16 persistent kernel, forward mode: run only if the device-side choice
    // of tile height is choice.rows (choice.offsets nullptr: always run)
    TileChoice choice;
};
// Dual mode: C = silu(A B0^T) * (A B1^T).  Single: C = A B0^T, or with
// splitk > 1 the partial products of the K ranges, C slice s = A[:, Ks] B0[:, Ks]^T.
hipError_t launch_grouped_gemm(const GemmGroup& g, bool dual, bool bf16, hipStream_t s);
// K split for a single bf16 GEMM with about mt_expected M tiles of 256 rows
// and N / 256 N tiles: the split in {1, 2, 4, 8} (K % (128 split) == 0, at
// least 24 stages of 64 per split) whose rounds of tiles over 256 CUs waste
// the least.  Depends only on its arguments.
int choose_splitk(int64_t mt_expected, int N, int K);
// The 32-row kernel suits groups of about 32 rows or fewer on average.
bool skinny_rows(int64_t rows, int G);
// Shapes it takes: N a multiple of its tile width, K of 64 per range; dual unsplit.
bool skinny_fits(int N, int K, bool dual, int splitk);
// K split for its single GEMM with about mt_expected M tiles of 32 rows.
int choose_splitk_skinny(int64_t mt_expected, int N, int K);
// Upper bound of M-tiles over all groups for tile height bm.
int64_t grouped_m_tiles_upper(int64_t rows, int G, int bm);
// Workgroups of the persistent GEMM grid on the current device (CUs, a multiple of 8).
int persistent_slots();

// ---- backward -------------------------------------------------------------------
// Generic grouped GEMM for the backward (any operand layout; bf16 MFMA when both
// operands are bf16 in 16-byte pieces, else fp32 FMA), C fp32:
//   C(m, n) (+)= sum_k A(m, k) B(n, k)
// rows mode (krows = false): group g owns output rows [offsets[g], offsets[g+1])
//   (or [0, M) without offsets); A(m, k) = A[src(m) lda + k] with src(m) =
//   a_gather[m] / a_div (or m); B(n, k) = Bg[k ldb + n], or Bg[n ldb + k]
//   with b_kcont; Bg = B + g b_gstride; C(m, n) at C[m ldc + n].
// krows mode: group g sums over k in [offsets[g], offsets[g+1]) (or [0, K));
//   A(m, k) = A[k lda + m]; B(n, k) = B[src(k) ldb + n] with src(k) =
//   b_gather[k] / b_div (or k); C(m, n) at C[g c_gstride + m ldc + n].
struct GradGemm {
    const void* A;
    int64_t lda;
    const int32_t* a_gather;
    int a_div;
    const void* B;
    int64_t ldb, b_gstride;
    const int32_t* b_gather;
    int b_div;
    float* C;
    int64_t ldc, c_gstride;
    bool accumulate;
    const int32_t* offsets;
    int G, M, N, K;
};
// a_bf16 / b_bf16: element type of A / B (bf16, or fp32); bf16 A needs bf16 B.
hipError_t launch_grad_gemm(const GradGemm& a, bool krows, bool b_kcont, bool a_bf16, bool b_bf16, hipStream_t s);

// Per grouped row r: h = silu(a) u, dg = <dH', h> (to dgate[pair], nullable),
// da = g dH' u silu'(a), du = g dH' silu(a), dO = g dy[token] (nullable).
struct BwdPairArgs {
    const int32_t* sorted;  // grouped row -> pair (nullptr: rows are tokens)
    const int32_t* offsets; // [G+1] or nullptr
    int G, k;
    const float* gates;     // [P] by pair, or nullptr (gate 1)
    const void* a;          // [rows, f]
    const void* u;          // [rows, f]
    const float* dhp;       // [rows, f] dy W_down
    void* h;                // [rows, f] out
    void* da;               // [rows, f] out
    void* du;               // [rows, f] out
    float* dgate;           // [P] out, or nullptr
    const void* dy;         // [T, dm]
    void* d_o;              // [rows, dm] out, or nullptr
    int f, dm;
    int64_t ld_dadu = 0;    // row stride of da and du (0: f)
};
hipError_t launch_bwd_pair(const BwdPairArgs& b, int rows, bool bf16, hipStream_t s);

// dl [T, E] from the pairs' dg, the forward's gates and (sigmoid or softmax
// without renormalisation) the logits.
struct BwdRouterArgs {
    const int32_t* ids;     // [T, k]
    const float* gates;     // [T, k]
    const float* dgate;     // [T, k] by pair
    const float* logits;    // [T, E] or nullptr (softmax + renormalise, no aux loss)
    float* dl;              // [T, E] out
    int T, E, k, score_fn, renorm;
    // load-balancing loss L_aux = alpha E sum_e f_e P_e: with aux_coef = alpha E / T
    // (0: none), dl += aux_coef p (f - <f, p>) (softmax) or aux_coef q (1 - s) (f - <f, q>)
    // (normalised sigmoid), f_e = aux_counts[e] inv_T
    const int32_t* aux_counts = nullptr;  // [E] pairs per expert before any capacity drop
    float aux_coef = 0.0f, inv_T = 0.0f;
};
// counts[e] = #{p < P : ids[p] = e}, E <= 256 (one workgroup).
hipError_t launch_count_ids(const int32_t* ids, int64_t P, int E, int32_t* counts, hipStream_t s);
hipError_t launch_bwd_router(const BwdRouterArgs& b, hipStream_t s);
// dx[t] = sum over slots j, then K slices, of dxp[slice][pair_pos[t k + j]] (pos -1 skipped).
hipError_t launch_bwd_token_sum(const float* dxp, const int32_t* pair_pos, int T, int k, int d, float* dx,
                                hipStream_t s, int splitk = 1, int64_t part_stride = 0);

hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t s);
// dW_r [E, d] = dl^T x (x bf16 or fp32) over token chunks; part holds
// router_wgrad_chunks(T, d, E) x E x d floats.
int router_wgrad_chunks(int T, int d, int E);
// out [E, 2 Tr] bf16 from dl [T, E] fp32: columns t < Tr hold dl rounded to
// bf16, columns Tr + t the rest rounded to bf16 (zero for t >= T); Tr % 64 == 0.
hipError_t launch_dl_split(const float* dl, int T, int E, int Tr, uint16_t* out, hipStream_t s);
// out [T, 2 E] bf16: dl rounded to bf16 in columns e < E, the rest rounded to
// bf16 in columns E + e.
hipError_t launch_dl_rows(const float* dl, int T, int E, uint16_t* out, hipStream_t s);
// dst[j] = sum over c < chunks, in order, of part[c n + j].
hipError_t launch_sum_chunks(const float* part, int chunks, int64_t n, float* dst, hipStream_t s);
hipError_t launch_router_wgrad(const float* dl, const void* x, bool x_bf16, int T, int E, int d, float* part,
                               float* dwr, hipStream_t s);

// Grouped rows as columns, each group's columns starting at kofs[g] (zero past its rows).
struct TransposeRowsArgs {
    const uint16_t* src;    // source rows [*, ld_src], columns c < C (C multiple of 64)
    int64_t ld_src;
    int C;
    const int32_t* gather;  // grouped row -> pair id, or nullptr (source row = grouped row)
    int div;                // source row = pair id / div
    const float* scale;     // [pairs] factor by pair id, or nullptr
    const int32_t* offsets; // [G+1] grouped rows per group, or nullptr (one group of M rows)
    const int32_t* kofs;    // [G+1] first column of each group (multiples of 128)
    int G, M, kpad;         // one group: M rows, kpad columns (multiple of 128)
    uint16_t* dst;          // [C, ld_dst]
    int64_t ld_dst;
};
// cols_upper: a multiple of 128 at least the columns written (kofs[G] or kpad).
hipError_t launch_transpose_rows(const TransposeRowsArgs& a, int64_t cols_upper, hipStream_t s);
// kofs[0..G] from offsets: each group's rows rounded up to 128 (empty: 128).
hipError_t launch_kgroup_offsets(const int32_t* offsets, int G, int32_t* kofs, hipStream_t s);

// ---- combine ------------------------------------------------------------------
struct CombineArgs {
    const void* expert_out; // [P, d]
    const float* weights;   // [T, k]
    const int32_t* pair_pos;// [P]
    const void* shared;     // [T, d] or nullptr
    void* y;                // [T, d]
    int T, d, k;
    int splitk = 1;         // bf16: expert_out holds splitk slices, summed in slice order
    int64_t part_stride = 0;// elements between expert_out slices
    int shared_splitk = 1;  // the same for the shared rows
    int64_t shared_stride = 0;
    TileChoice choice;      // bf16: run only if the device-side choice is choice.rows
};
hipError_t launch_combine(const CombineArgs& a, bool bf16, hipStream_t s);

}  // namespace moe
