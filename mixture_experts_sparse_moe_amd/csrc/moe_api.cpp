// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace layout and the launch sequence.  Everything is validated before
// the first launch; nothing here synchronises or copies to the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "moe.h"
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;
// tile-queue counters of the routed persistent GEMMs: 256 per launch
// (gate/up, down)
constexpr int kQueueInts = 2 * 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int validate_cfg(const moe_config* c) {
    if (!c) return MOE_ERR_NULL;
    if (c->num_tokens < 0 || c->d_model <= 0 || c->num_experts <= 0 || c->top_k <= 0 ||
        c->d_ff <= 0)
        return MOE_ERR_SHAPE;
    if (c->num_shared < 0 || c->num_shared > 1) return MOE_ERR_SHAPE;
    if (c->num_shared == 1 && c->d_ff_shared <= 0) return MOE_ERR_SHAPE;
    if (c->top_k > c->num_experts) return MOE_ERR_SHAPE;
    if (c->num_experts > 256 || c->top_k > 16) return MOE_ERR_UNSUPPORTED;
    if (c->d_model % 64 || c->d_ff % 64 || (c->num_shared && c->d_ff_shared % 64))
        return MOE_ERR_UNSUPPORTED;
    if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID)
        return MOE_ERR_UNSUPPORTED;
    if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_UNSUPPORTED;
    if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)c->num_tokens * c->top_k >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

size_t elem(const moe_config* c) { return c->dtype == MOE_BF16 ? 2 : 4; }

bool misaligned(const void* p);

// Options: NULL or all fields zero is the plain layer.
int validate_opts(const moe_options* o) {
    if (!o) return MOE_OK;
    if (o->bias_on_scores != 0 && o->bias_on_scores != 1) return MOE_ERR_UNSUPPORTED;
    if (o->expert_bias && misaligned(o->expert_bias)) return MOE_ERR_ALIGN;
    if (o->router_stats && misaligned(o->router_stats)) return MOE_ERR_ALIGN;
    if (!(o->aux_alpha == o->aux_alpha)) return MOE_ERR_SHAPE;      // NaN
    return MOE_OK;
}

int capacity_of(const moe_options* o) {
    return (o && o->expert_capacity > 0) ? o->expert_capacity : 0x7FFFFFFF;
}

// Which bf16 GEMM kernel the routed and the shared expert GEMMs use: the
// 32-row streaming kernel when groups hold about 32 rows or fewer on average
// (decode), else the 256 x 256 tile kernel.
struct Paths {
    bool routed_skinny, shared_skinny;
};

Paths paths(const moe_config* c) {
    const bool bf16 = c->dtype == MOE_BF16;
    const int64_t P = (int64_t)c->num_tokens * c->top_k;
    Paths p{bf16 && skinny_rows(P, c->num_experts) && skinny_fits(c->d_ff, c->d_model, true, 1) &&
                skinny_fits(c->d_model, c->d_ff, false, 1),
            bf16 && c->num_shared && skinny_rows(c->num_tokens, 1) &&
                skinny_fits(c->d_ff_shared, c->d_model, true, 1) && skinny_fits(c->d_model, c->d_ff_shared, false, 1)};
    return p;
}

// K splits of the down projections inside moe_forward (moe_expert_ffn never
// splits: its expert_out is the finished product).  For the 256-row kernel the
// routed GEMM has about P / 256 + min(E, P) / 2 M tiles (each expert's last
// tile is partial), the shared one T / 256; for the 32-row kernel about
// P / 32 + min(E, P) / 2 and T / 32.  Only bf16 layers split.
struct Splits {
    int routed, shared;
};

Splits splits(const moe_config* c) {
    Splits sp{1, 1};
    if (c->dtype != MOE_BF16 || c->num_tokens == 0) return sp;
    const Paths pa = paths(c);
    const int64_t P = (int64_t)c->num_tokens * c->top_k, E = c->num_experts, T = c->num_tokens;
    if (pa.routed_skinny) {
        const int64_t mt_exp = std::min<int64_t>(grouped_m_tiles_upper(P, (int)E, 32),
                                                 (P + 31) / 32 + std::min<int64_t>(E, P) / 2);
        sp.routed = choose_splitk_skinny(mt_exp, c->d_model, c->d_ff);
    } else {
        const int64_t mt_upper = grouped_m_tiles_upper(P, (int)E, 256);
        const int64_t mt_exp = std::min<int64_t>(mt_upper, (P + 255) / 256 + std::min<int64_t>(E, P) / 2);
        sp.routed = choose_splitk(mt_exp, c->d_model, c->d_ff);
    }
    if (c->num_shared) {
        sp.shared = pa.shared_skinny ? choose_splitk_skinny((T + 31) / 32, c->d_model, c->d_ff_shared)
                                     : choose_splitk((T + 255) / 256, c->d_model, c->d_ff_shared);
    }
    return sp;
}

// How moe_forward's router runs (bf16, with the workspace's partial logits).
// ranges 0: the fused kernel (fp32 layers).  Else logits and selection as
// two kernels over `ranges` K ranges: fewer than 256 blocks of 32 tokens (K
// split so that about 256 workgroups run) or at most 128 experts (one range:
// the selection then has 16 waves per workgroup where the fused kernel's 4
// waves walk 8 tokens each after the MFMA loop, alone on their SIMDs;
// Hunyuan-A13B, 64 experts: 47 -> 40 us); or, for 129..256 experts (wide),
// tiles of 128 tokens so that the W_r stream every workgroup reads serves
// four times the tokens, K split to about 256 workgroups (DeepSeek-V3).  One
// range adds nothing to the logits: the same values as the fused kernel's.
struct RoutePlan {
    int ranges;
    bool wide;
};

RoutePlan route_plan(const moe_config* c) {
    if (c->dtype != MOE_BF16 || c->num_tokens <= 0) return RoutePlan{0, false};
    const int rr = route_ranges(c->num_tokens, c->d_model, true);
    if (rr > 1 || c->num_experts <= 128) return RoutePlan{rr, false};
    return RoutePlan{route_ranges_wide(c->num_tokens, c->d_model), true};
}

// Device workspace layout.  Every region starts on a 256-byte boundary.
struct Layout {
    size_t ids, wts, counts, offsets, chunk, sorted, pos, H, O, Hs, S, rpart, spart, total, queue;
    size_t dispatch_need, ffn_need;   // bytes used by moe_dispatch / moe_expert_ffn (from 0)
};

Layout layout(const moe_config* c) {
    const size_t T = (size_t)c->num_tokens, P = T * c->top_k, E = c->num_experts;
    const size_t nchunks = (size_t)dispatch_num_chunks((int)P);
    Layout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
    // moe_expert_ffn's scratch first, so it can start at offset 0
    L.H = take(P * c->d_ff * elem(c));
    L.Hs = take(c->num_shared ? T * c->d_ff_shared * elem(c) : 0);
    L.queue = take(T > 0 ? kQueueInts * sizeof(int32_t) : 0);
    L.ffn_need = o;
    L.chunk = take(nchunks * E * sizeof(int32_t));
    L.ids = take(P * sizeof(int32_t));
    L.wts = take(P * sizeof(float));
    L.counts = take(E * sizeof(int32_t));
    L.offsets = take((E + 2) * sizeof(int32_t));
    // room for the shared expert's tokens as a trailing group (merged_shared)
    L.sorted = take((P + (c->num_shared ? T : 0)) * sizeof(int32_t));
    L.pos = take(P * sizeof(int32_t));
    const Splits sp = splits(c);
    L.O = take(sp.routed * P * c->d_model * elem(c));
    L.S = take(c->num_shared ? sp.shared * T * c->d_model * elem(c) : 0);
    const RoutePlan rp = route_plan(c);
    L.rpart = take((size_t)rp.ranges * T * E * sizeof(float));
    L.spart = take(((T + 31) / 32) * 2 * E * sizeof(float));
    L.total = o;
    L.dispatch_need = align_up(nchunks * E * sizeof(int32_t));
    return L;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

// The routed GEMMs claim their tiles through counters when there is about one
// M tile per expert (fewer than 640 rows per expert on average).
bool routed_queue(const moe_config* c) {
    return c->dtype == MOE_BF16 && !paths(c).routed_skinny &&
           (int64_t)c->num_tokens * c->top_k < (int64_t)640 * c->num_experts;
}

// The routed GEMMs of the tile-queue regime take 288-row tiles on 12 waves
// (gemm_bf16_tall_kernel) when the experts hold 224 to 287 rows on average.
// With 256-row tiles an expert of 257..288 rows takes two tiles of about 140
// rows, and such a tile costs 85 % of a full one: it streams the whole
// weight panel for half the rows.  At DeepSeek-V3's shape (256 rows per
// expert on average, 212..315 with its routing) about half the experts are
// such; gate/up 5.05 -> 4.34 ms, down 2.64 -> 2.58 ms.  Outside that range
// most experts take the same number of tiles either way, and the 12-wave
// tiles measured 1-5 % slower.
bool routed_tall(const moe_config* c) {
    if (!routed_queue(c)) return false;
    const int64_t P = (int64_t)c->num_tokens * c->top_k, E = c->num_experts;
    return P >= 224 * E && P < 288 * E;
}

// With several M tiles per expert (the fixed schedule) the routed GEMMs'
// tile height is chosen on the device from the expert counts
// (tall_tiles_chosen): moe_forward launches the 256-row and the 288-row
// kernel of each GEMM, and the one not chosen exits at once.  Whole layers,
// same session, each height forced: Mixtral prefill (experts of 982-1068
// rows) 2.83 ms on 256-row tiles, 2.64 ms on 288-row ones (35 -> 32 M tiles,
// the down GEMM unsplit); Hunyuan-A13B (Zipf-skewed, 199-6363 rows) 4.81 ms
// against 4.90 ms.  The average rows per expert, which the host knows, is
// 1024 for both.  bf16 layers whose GEMMs both fit the persistent kernels
// (d a multiple of 256, d_ff of 128, gathered rows under 4 GiB).
bool routed_choice(const moe_config* c) {
    if (c->dtype != MOE_BF16 || c->num_tokens == 0 || paths(c).routed_skinny || routed_queue(c)) return false;
    const int64_t T = c->num_tokens, P = T * c->top_k, d = c->d_model, f = c->d_ff;
    return d % 256 == 0 && f % 128 == 0 && T * d * 2 < (int64_t(1) << 32) && P * f * 2 < (int64_t(1) << 32) &&
           c->num_experts <= 256;
}

// moe_forward computes the shared expert in the routed GEMMs' launches, as one
// more group (its T tokens after the T k pairs; its weights through the
// GEMMs' last-group pointers), when it is as wide as the routed experts, the
// layer is bf16 on the 256-row persistent kernels with the tile queue, without
// K splits and with no capacity, and the workspace holds its rows right after
// the routed ones (H then H_s, O then S).  The two short dense GEMMs of the
// shared expert then fill the routed GEMMs' last rounds instead of running
// after them, each with its own last round (DeepSeek-V3: 8.27 -> 8.19 ms).
// Stages 4 and 5 of moe_forward_staged are then empty.
bool merged_shared(const moe_config* c, int cap) {
    if (c->dtype != MOE_BF16 || c->num_shared != 1 || c->d_ff_shared != c->d_ff || c->num_tokens == 0 ||
        cap != 0x7FFFFFFF || !routed_queue(c))
        return false;
    const Paths pa = paths(c);
    const Splits sp = splits(c);
    if (pa.routed_skinny || pa.shared_skinny || sp.routed != 1 || sp.shared != 1) return false;
    const int64_t T = c->num_tokens, P = T * c->top_k, d = c->d_model, f = c->d_ff;
    // the persistent kernels take both GEMMs (N % 128 dual, N % 256 single,
    // K % 128, gathered rows of x under 4 GiB); the scan kernel writes the tail
    if (f % 128 || d % 256 || T * d * 2 >= (int64_t(1) << 32) || dispatch_num_chunks((int)P) < 2) return false;
    const Layout L = layout(c);
    return L.Hs == L.H + (size_t)(P * f * 2) && L.S == L.O + (size_t)(P * d * 2);
}

// A tensor pointer must be non-null unless its size is zero, and 16-byte aligned.
int check_ptr(const void* p, bool empty_ok) {
    if (!p) return empty_ok ? MOE_OK : MOE_ERR_NULL;
    return misaligned(p) ? MOE_ERR_ALIGN : MOE_OK;
}

#define MOE_TRY(expr)                  \
    do {                               \
        int rc_ = (expr);              \
        if (rc_ != MOE_OK) return rc_; \
    } while (0)

#define MOE_HIP(expr)                                  \
    do {                                               \
        if ((expr) != hipSuccess) return MOE_ERR_HIP;  \
    } while (0)

// part: scratch for the partial logits of a K-split router (moe_forward,
// batches of few token blocks), or nullptr for the one-kernel router.
// disp (with part): the dispatch of these ids, run by the router's second
// kernel when the batch is one block of at most 32 tokens.  Returns in
// *dispatched whether it did.
// opts (nullable): selection bias; router statistics into opts->router_stats,
// with per-block sums in spart (required then).
int run_route(const moe_config* c, const void* x, const void* w_router, int32_t* ids, float* wts,
              float* gap, hipStream_t s, float* part = nullptr, const DispatchArgs* disp = nullptr,
              bool* dispatched = nullptr, const moe_options* opts = nullptr, float* spart = nullptr) {
    RouteArgs a{x, w_router, ids, wts, gap, c->num_tokens, c->d_model, c->num_experts,
                c->top_k, c->score_fn, c->renormalize};
    const bool stats = opts && opts->router_stats;
    if (opts) {
        a.bias = opts->expert_bias;
        a.bias_on_scores = opts->bias_on_scores;
        a.stats_part = stats ? spart : nullptr;
    }
    const bool bf16 = c->dtype == MOE_BF16;
    const RoutePlan rp = route_plan(c);
    const bool fuse = part && rp.ranges > 1 && !rp.wide && disp && c->num_tokens <= 32;
    if (dispatched) *dispatched = fuse;
    if (part && rp.wide) MOE_HIP(launch_route_split_wide(a, rp.ranges, part, s));
    else if (part && rp.ranges > 0) MOE_HIP(launch_route_split(a, rp.ranges, part, fuse ? disp : nullptr, s));
    else MOE_HIP(launch_route(a, bf16, s));
    if (stats)
        MOE_HIP(launch_router_stats(spart, (c->num_tokens + 31) / 32, c->num_experts, c->num_tokens,
                                    opts->aux_alpha, capacity_of(opts), opts->router_stats, s));
    return MOE_OK;
}

int run_dispatch(const moe_config* c, const int32_t* ids, int32_t* counts, int32_t* offsets,
                 int32_t* sorted, int32_t* pos, int32_t* chunk, hipStream_t s, int cap = 0x7FFFFFFF,
                 int32_t* zero = nullptr, int nzero = 0, int tail = 0) {
    DispatchArgs a{ids, counts, offsets, sorted, pos, chunk, c->num_tokens * c->top_k,
                   c->num_experts, cap, zero, nzero, tail, c->top_k};
    MOE_HIP(launch_dispatch(a, s));
    return MOE_OK;
}

// Record stage event i if events were given.
int mark(void* const* ev, int i, hipStream_t s) {
    if (ev && ev[i]) MOE_HIP(hipEventRecord(static_cast<hipEvent_t>(ev[i]), s));
    return MOE_OK;
}

// out / shared_out receive sp.routed / sp.shared slices of [P, d] / [T, d].
int run_ffn(const moe_config* c, const void* x, const int32_t* sorted, const int32_t* offsets,
            const void* wg, const void* wu, const void* wd, const void* sg, const void* su,
            const void* sd, void* out, void* shared_out, void* H, void* Hs, int32_t* queue,
            bool queue_zeroed, hipStream_t s, void* const* ev = nullptr, Splits sp = Splits{1, 1},
            bool merged = false) {
    const bool bf16 = c->dtype == MOE_BF16;
    const int P = c->num_tokens * c->top_k;
    const Paths pa = paths(c);
    if (P > 0) {
        // Tile order of the routed persistent GEMMs: expert-aligned bands, so
        // that each expert's weights stream about once.  With several M tiles
        // per expert (640 rows or more) the tiles follow a fixed schedule
        // (aligned bands measured -6 % on the down GEMM and -5 % on gate/up
        // at ~4 tiles per expert, with 16 % less HBM traffic).  With about
        // one tile per expert, about half the experts add a nearly empty
        // tile: the GEMMs then claim tiles through counters (zeroed by
        // moe_forward's dispatch, else here by a kernel, not a memset, so that
        // a captured graph replays it), which evens those tiles out between
        // workgroups (DeepSeek-V3 prefill: 9.36 -> 8.35 ms with both, where
        // the aligned order alone was 2 % slower than the plain one).  At
        // several tiles per expert the queue did not speed the GEMMs up and
        // its windows read 26 % more bytes.
        const bool use_queue = routed_queue(c);
        if (use_queue && !queue_zeroed)
            MOE_HIP(launch_fill_zero_f32(reinterpret_cast<float*>(queue), kQueueInts, s));
        // merged: the shared expert's T tokens are group E (rows P .. P + T)
        const int G = c->num_experts + (merged ? 1 : 0), rows = P + (merged ? c->num_tokens : 0);
        // tile height chosen on the device: the 256-row kernels (down split
        // in sp.routed K ranges) and the 288-row ones (unsplit) both launch
        const bool choose = routed_choice(c);
        TileChoice tc;
        if (choose) tc = TileChoice{offsets, c->num_experts, 2 * c->d_ff / 256, persistent_slots(), 256};
        GemmGroup up{x, sorted, c->top_k, offsets, G, rows, wg, wu, H, c->d_ff, c->d_model};
        up.skinny = pa.routed_skinny;
        up.aligned_bands = true;
        up.queue = use_queue ? queue : nullptr;
        up.tall = routed_tall(c);
        up.choice = tc;
        if (merged) {
            up.B0_last = sg;
            up.B1_last = su;
        }
        // stage events 1 and 2 are the routed gate/up kernel's own start and
        // end timestamps (with a choice, the first launch's start and the
        // second's end): no separate records around the dominant kernel
        hipEvent_t e1 = ev ? static_cast<hipEvent_t>(ev[1]) : nullptr;
        hipEvent_t e2 = ev ? static_cast<hipEvent_t>(ev[2]) : nullptr;
        up.t_start = e1;
        up.t_stop = choose ? nullptr : e2;
        MOE_HIP(launch_grouped_gemm(up, true, bf16, s));
        if (choose) {
            GemmGroup up288 = up;
            up288.tall = true;
            up288.choice.rows = 288;
            up288.t_start = nullptr;
            up288.t_stop = e2;
            MOE_HIP(launch_grouped_gemm(up288, true, bf16, s));
        }
        GemmGroup down{H, nullptr, 1, offsets, G, rows, wd, nullptr, out, c->d_model,
                       c->d_ff, sp.routed, (int64_t)P * c->d_model, true};
        down.skinny = pa.routed_skinny;
        down.queue = use_queue ? queue + 256 : nullptr;
        down.tall = routed_tall(c) && sp.routed == 1;
        down.choice = tc;
        if (merged) down.B0_last = sd;
        MOE_HIP(launch_grouped_gemm(down, false, bf16, s));
        if (choose) {
            GemmGroup down288 = down;
            down288.tall = true;
            down288.splitk = 1;
            down288.choice.rows = 288;
            MOE_HIP(launch_grouped_gemm(down288, false, bf16, s));
        }
        MOE_TRY(mark(ev, 3, s));
    } else {
        MOE_TRY(mark(ev, 1, s));
        MOE_TRY(mark(ev, 2, s));
        MOE_TRY(mark(ev, 3, s));
    }
    if (c->num_shared && c->num_tokens > 0 && !merged) {
        GemmGroup up{x, nullptr, 1, nullptr, 1, c->num_tokens, sg, su, Hs, c->d_ff_shared,
                     c->d_model};
        up.skinny = pa.shared_skinny;
        MOE_HIP(launch_grouped_gemm(up, true, bf16, s));
        MOE_TRY(mark(ev, 4, s));
        GemmGroup down{Hs, nullptr, 1, nullptr, 1, c->num_tokens, sd, nullptr, shared_out,
                       c->d_model, c->d_ff_shared, sp.shared, (int64_t)c->num_tokens * c->d_model};
        down.skinny = pa.shared_skinny;
        MOE_HIP(launch_grouped_gemm(down, false, bf16, s));
        MOE_TRY(mark(ev, 5, s));
    } else {
        MOE_TRY(mark(ev, 4, s));
        MOE_TRY(mark(ev, 5, s));
    }
    return MOE_OK;
}

// offsets (moe_forward, when routed_choice): the routed down GEMM wrote
// sp.routed slices on 256-row tiles or one on 288-row tiles, as the device
// chose; with sp.routed > 1 a combine for each launches and one exits.
int run_combine(const moe_config* c, const void* out, const float* wts, const int32_t* pos,
                const void* shared_out, void* y, hipStream_t s, Splits sp = Splits{1, 1},
                const int32_t* offsets = nullptr) {
    const int64_t P = (int64_t)c->num_tokens * c->top_k;
    CombineArgs a{out, wts, pos, shared_out, y, c->num_tokens, c->d_model, c->top_k,
                  sp.routed, P * c->d_model, sp.shared, (int64_t)c->num_tokens * c->d_model};
    const bool choose = offsets && sp.routed > 1 && routed_choice(c);
    if (choose) a.choice = TileChoice{offsets, c->num_experts, 2 * c->d_ff / 256, persistent_slots(), 256};
    MOE_HIP(launch_combine(a, c->dtype == MOE_BF16, s));
    if (choose) {
        a.splitk = 1;
        a.choice.rows = 288;
        MOE_HIP(launch_combine(a, c->dtype == MOE_BF16, s));
    }
    return MOE_OK;
}

int forward_impl(const moe_config* cfg, const moe_options* opts, const void* x, const void* w_router,
                 const void* w_gate, const void* w_up, const void* w_down, const void* ws_gate,
                 const void* ws_up, const void* ws_down, void* y, int32_t* topk_ids_out,
                 float* topk_weights_out, int32_t* expert_counts_out, float* topk_gap_out, void* ws,
                 size_t ws_bytes, void* start_event, void* const* ev, void* stream) {
    MOE_TRY(validate_cfg(cfg));
    MOE_TRY(validate_opts(opts));
    const bool empty = cfg->num_tokens == 0;
    MOE_TRY(check_ptr(x, empty));
    MOE_TRY(check_ptr(w_router, false));
    MOE_TRY(check_ptr(w_gate, false));
    MOE_TRY(check_ptr(w_up, false));
    MOE_TRY(check_ptr(w_down, false));
    if (cfg->num_shared) {
        MOE_TRY(check_ptr(ws_gate, false));
        MOE_TRY(check_ptr(ws_up, false));
        MOE_TRY(check_ptr(ws_down, false));
    }
    MOE_TRY(check_ptr(y, empty));
    if (topk_ids_out) MOE_TRY(check_ptr(topk_ids_out, true));
    if (topk_weights_out) MOE_TRY(check_ptr(topk_weights_out, true));
    if (expert_counts_out) MOE_TRY(check_ptr(expert_counts_out, true));
    if (topk_gap_out) MOE_TRY(check_ptr(topk_gap_out, true));
    const Layout L = layout(cfg);
    if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    MOE_TRY(check_ptr(ws, false));
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
    float* wts = topk_weights_out ? topk_weights_out : at<float>(ws, L.wts);
    int32_t* counts = expert_counts_out ? expert_counts_out : at<int32_t>(ws, L.counts);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* sorted = at<int32_t>(ws, L.sorted);
    int32_t* pos = at<int32_t>(ws, L.pos);
    if (start_event) MOE_HIP(hipEventRecord(static_cast<hipEvent_t>(start_event), s));
    const int cap = capacity_of(opts);
    if (empty) {
        // routing outputs are empty; expert counts are all zero
        MOE_TRY(mark(ev, 0, s));
        MOE_TRY(run_dispatch(cfg, ids, counts, offsets, sorted, pos, at<int32_t>(ws, L.chunk), s, cap));
        for (int i = 1; i < MOE_NUM_STAGES; ++i) MOE_TRY(mark(ev, i, s));
        return MOE_OK;
    }
    const DispatchArgs disp{ids, counts, offsets, sorted, pos, at<int32_t>(ws, L.chunk),
                            cfg->num_tokens * cfg->top_k, cfg->num_experts, cap};
    bool dispatched = false;
    MOE_TRY(run_route(cfg, x, w_router, ids, wts, topk_gap_out, s, at<float>(ws, L.rpart), &disp, &dispatched,
                      opts, at<float>(ws, L.spart)));
    MOE_TRY(mark(ev, 0, s));
    int32_t* queue = at<int32_t>(ws, L.queue);
    const bool merged = !dispatched && merged_shared(cfg, cap);
    if (!dispatched)
        MOE_TRY(run_dispatch(cfg, ids, counts, offsets, sorted, pos, at<int32_t>(ws, L.chunk), s, cap, queue,
                             cfg->num_tokens > 0 ? kQueueInts : 0, merged ? cfg->num_tokens : 0));
    void* O = at<void>(ws, L.O);
    void* S = cfg->num_shared ? at<void>(ws, L.S) : nullptr;
    const Splits sp = splits(cfg);
    MOE_TRY(run_ffn(cfg, x, sorted, offsets, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, O, S,
                    at<void>(ws, L.H), at<void>(ws, L.Hs), queue, !dispatched, s, ev, sp, merged));
    MOE_TRY(run_combine(cfg, O, wts, pos, S, y, s, sp, offsets));
    return mark(ev, 6, s);
}


// Backward workspace, 256-byte aligned regions.
// The backward's bf16 GEMMs run on the forward's persistent kernel when the
// widths are multiples of its 256-wide tiles (fast); otherwise, and for fp32
// layers, on the generic grouped GEMM.
struct BwdPlan {
    bool fast = false;          // routed experts on the persistent kernel
    bool shared_fast = false;   // shared expert likewise
    int64_t Q = 0;              // columns of the transposed pair operands (rows padded per expert)
    int64_t Tq = 0;             // columns of the transposed token operands
    int xsplit = 1;             // K split of dx per pair (dXp slices)
    // dW_r = dl^T x on the persistent kernel (bf16, 32 or more experts): one
    // product over 2 Tr columns, dl split into bf16 high and low parts and x
    // transposed twice, its K split into rsplit fp32 slices
    bool router_mfma = false;
    int64_t Tr = 0;
    int rsplit = 1;
    // dx += dl W_r likewise (E a multiple of 64): dl split into [T, 2 E], W_r
    // [E, d] read as stored (N-major) for both halves
    bool router_dx_mfma = false;
};

BwdPlan bwd_plan(const moe_config* c) {
    BwdPlan p;
    if (c->dtype != MOE_BF16) return p;
    const int64_t T = c->num_tokens, P = T * c->top_k, E = c->num_experts;
    const int64_t d = c->d_model, f = c->d_ff;
    auto round128 = [](int64_t v) { return (v + 127) / 128 * 128; };
    p.Q = round128(P + 128 * E);
    p.Tq = std::max<int64_t>(128, round128(T));
    const int64_t lim = int64_t(1) << 32;
    // 32-bit DMA offsets: gathered rows of dy from its start; 256 rows of a transposed operand
    p.fast = d % 256 == 0 && f % 256 == 0 && T * d * 2 < lim && 256 * p.Q * 2 < lim;
    if (p.fast) {
        const int64_t mt_upper = grouped_m_tiles_upper(P, (int)E, 256);
        const int64_t mt_exp = std::min<int64_t>(mt_upper, (P + 255) / 256 + std::min<int64_t>(E, P) / 2);
        p.xsplit = choose_splitk(mt_exp, (int)d, (int)(2 * f));
    }
    if (c->num_shared) {
        const int64_t fs = c->d_ff_shared;
        p.shared_fast = d % 256 == 0 && fs % 256 == 0 && 256 * p.Tq * 2 < lim;
    }
    // the FMA kernel reads x E / 16 times (DeepSeek-V3 prefill: 4.7 ms); the
    // product takes ~0.2 ms.  Few experts keep the FMA kernel (Mixtral: 45 us).
    p.Tr = (T + 511) / 512 * 512;
    p.router_mfma = E >= 32 && T > 0 && d % 256 == 0 && 256 * 2 * p.Tr * 2 < lim;
    if (p.router_mfma) p.rsplit = choose_splitk(1, (int)d, (int)(2 * p.Tr));
    p.router_dx_mfma = p.router_mfma && E % 64 == 0;
    return p;
}

struct BwdLayout {
    size_t counts, offsets, sorted, pos, chunk, A, U, H, DA, DU, dHp, dO, dXp, dgate, logits, dl, rw, auxcnt, DLT, XT2;
    size_t queue;   // fast path: tile-queue counters of the three routed GEMMs over the pairs
    size_t DLR;     // router_dx_mfma: dl split into bf16 parts, [T, 2 E]
    size_t As, Us, Hs, DAs, DUs, dHs;
    // fast path: DA and DU share rows [da | du] (DA), transposed operands
    size_t kofs, dOT, HT, DADUT, XgT, dyT, HsT, DADUsT, xT;
    size_t total;
};

BwdLayout bwd_layout(const moe_config* c) {
    const BwdPlan pl = bwd_plan(c);
    const size_t T = (size_t)c->num_tokens, P = T * c->top_k, E = c->num_experts;
    const size_t d = c->d_model, f = c->d_ff, fs = c->num_shared ? c->d_ff_shared : 0, w = elem(c);
    const size_t Q = (size_t)pl.Q, Tq = (size_t)pl.Tq;
    BwdLayout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
    L.chunk = take((size_t)dispatch_num_chunks((int)P) * E * 4);
    L.counts = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.sorted = take(P * 4);
    L.pos = take(P * 4);
    L.A = take(P * f * w);
    L.U = take(P * f * w);
    L.H = take(P * f * w);
    L.dHp = take(P * f * 4);
    L.dgate = take(P * 4);
    L.logits = take(T * E * 4);
    L.dl = take(T * E * 4);
    if (pl.router_mfma) {
        L.rw = take((size_t)pl.rsplit * E * d * 4);
        L.DLT = take(E * 2 * (size_t)pl.Tr * w);
        L.XT2 = take(d * 2 * (size_t)pl.Tr * w);
        if (pl.router_dx_mfma) L.DLR = take(T * 2 * E * w);
    } else {
        L.rw = take((size_t)router_wgrad_chunks((int)T, (int)d, (int)E) * E * d * 4);
    }
    L.auxcnt = take(E * 4);
    if (pl.fast) {
        L.queue = take(3 * 256 * 4);
        L.DA = take(P * 2 * f * w);
        L.dXp = take((size_t)pl.xsplit * P * d * 4);
        L.kofs = take((E + 1) * 4);
        L.dOT = take(d * Q * w);
        L.HT = take(f * Q * w);
        L.DADUT = take(2 * f * Q * w);
        L.XgT = take(d * Q * w);
    } else {
        L.DA = take(P * f * w);
        L.DU = take(P * f * w);
        L.dO = take(P * d * w);
        L.dXp = take(P * d * 4);
    }
    L.As = take(T * fs * w);
    L.Us = take(T * fs * w);
    L.Hs = take(T * fs * w);
    L.dHs = take(T * fs * 4);
    if (pl.shared_fast) {
        L.DAs = take(T * 2 * fs * w);
        L.dyT = take(d * Tq * w);
        L.HsT = take(fs * Tq * w);
        L.DADUsT = take(2 * fs * Tq * w);
        L.xT = take(d * Tq * w);
    } else {
        L.DAs = take(T * fs * w);
        L.DUs = take(T * fs * w);
    }
    L.total = o;
    return L;
}

GradGemm grad_gemm(const void* A, int64_t lda, const void* B, int64_t ldb, float* C, int64_t ldc, int M, int N,
                   int K) {
    GradGemm g{};
    g.A = A; g.lda = lda; g.a_div = 1;
    g.B = B; g.ldb = ldb; g.b_div = 1;
    g.C = C; g.ldc = ldc;
    g.G = 1; g.M = M; g.N = N; g.K = K;
    return g;
}

// fp32 product on the persistent kernel: C [rows, ldc] = A B0^T over grouped rows.
GemmGroup f32_gemm(const void* A, const int32_t* gather, int div, const int32_t* offsets, int G, int M,
                   const void* B0, float* C, int64_t ldc, int N, int K) {
    GemmGroup g{A, gather, div, offsets, G, M, B0, nullptr, C, N, K};
    g.f32_out = true;
    g.ldc = ldc;
    return g;
}

// Weight gradients on the persistent kernel: C[g] (M x N) = sum over group g's
// columns of A (M rows, stride lda) times B (N rows, stride ldb).
GemmGroup kgroup_gemm(const void* A, int64_t lda, const void* B, int64_t ldb, const int32_t* kofs, int G, int M,
                      int N, int K, float* C, int64_t ldc, int64_t c_gstride) {
    GemmGroup g{A, nullptr, 1, nullptr, G, M, B, nullptr, C, N, K};
    g.kgrouped = true;
    g.kofs = kofs;
    g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.c_gstride = c_gstride;
    return g;
}

TransposeRowsArgs rows_t(const void* src, int64_t ld_src, int C, const int32_t* gather, int div, const float* scale,
                         const int32_t* offsets, const int32_t* kofs, int G, int M, int kpad, void* dst,
                         int64_t ld_dst) {
    return TransposeRowsArgs{static_cast<const uint16_t*>(src), ld_src, C, gather, div, scale, offsets, kofs,
                             G, M, kpad, static_cast<uint16_t*>(dst), ld_dst};
}

int run_backward(const moe_config* c, const void* x, const void* wr, const void* wg, const void* wu,
                 const void* wd, const void* sg, const void* su, const void* sd, const void* dy,
                 const int32_t* ids, const float* gates, float* dx, float* dwr, float* dwg, float* dwu,
                 float* dwd, float* dsg, float* dsu, float* dsd, void* ws, hipStream_t s,
                 int cap = 0x7FFFFFFF, float aux_alpha = 0.0f) {
    const BwdPlan pl = bwd_plan(c);
    const BwdLayout L = bwd_layout(c);
    const bool bf16 = c->dtype == MOE_BF16;
    const int T = c->num_tokens, k = c->top_k, E = c->num_experts, P = T * k;
    const int d = c->d_model, f = c->d_ff;
    const size_t w = elem(c);
    int32_t* counts = at<int32_t>(ws, L.counts);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* sorted = at<int32_t>(ws, L.sorted);
    int32_t* pos = at<int32_t>(ws, L.pos);
    void *A = at<void>(ws, L.A), *U = at<void>(ws, L.U), *H = at<void>(ws, L.H);
    void* DA = at<void>(ws, L.DA);
    float *dHp = at<float>(ws, L.dHp), *dXp = at<float>(ws, L.dXp), *dgate = at<float>(ws, L.dgate);
    float *logits = at<float>(ws, L.logits), *dl = at<float>(ws, L.dl);

    // routing groups of the forward's ids; pairs past an expert's capacity are
    // left out of the groups (pair_pos -1), as in the forward
    // The routed GEMMs over the pairs take the forward's tile orders: expert-
    // aligned bands, and with about one M tile per expert (fewer than 640 rows)
    // tiles claimed through counters, which the dispatch zeroes on its way.
    const bool aligned = (int64_t)P >= (int64_t)640 * E;
    int32_t* q = pl.fast && !aligned && P > 0 ? at<int32_t>(ws, L.queue) : nullptr;
    MOE_TRY(run_dispatch(c, ids, counts, offsets, sorted, pos, at<int32_t>(ws, L.chunk), s, cap, q,
                         q ? 3 * 256 : 0));
    // a dropped pair's gate gets no gradient (the pair kernel writes kept pairs only)
    if ((int64_t)cap < P) MOE_HIP(launch_fill_zero_f32(dgate, P, s));
    // a = x W_gate^T, u = x W_up^T on the grouped rows (the forward's GEMM)
    if (pl.fast) {
        // both from one dual-tile GEMM (the gathered x rows are read once)
        GemmGroup gau{x, sorted, k, offsets, E, P, wg, wu, A, f, d};
        gau.C2 = U;
        gau.aligned_bands = aligned || q;
        gau.queue = q;
        MOE_HIP(launch_grouped_gemm(gau, true, true, s));
    } else {
        GemmGroup ga{x, sorted, k, offsets, E, P, wg, nullptr, A, f, d};
        ga.aligned_bands = aligned;
        MOE_HIP(launch_grouped_gemm(ga, false, bf16, s));
        GemmGroup gu{x, sorted, k, offsets, E, P, wu, nullptr, U, f, d};
        gu.aligned_bands = aligned;
        MOE_HIP(launch_grouped_gemm(gu, false, bf16, s));
    }
    if (pl.fast) {
        const int64_t Q = pl.Q;
        int32_t* kofs = at<int32_t>(ws, L.kofs);
        void *dOT = at<void>(ws, L.dOT), *HT = at<void>(ws, L.HT), *DADUT = at<void>(ws, L.DADUT);
        void* XgT = at<void>(ws, L.XgT);
        // dH' = dy W_down, reading W_down [E, d, f] as it is (K = d rows of N = f)
        GemmGroup g1 = f32_gemm(dy, sorted, k, offsets, E, P, wd, dHp, f, f, d);
        g1.b_nmajor = true;
        g1.aligned_bands = aligned || q;
        g1.queue = q ? q + 256 : nullptr;
        MOE_HIP(launch_grouped_gemm(g1, false, true, s));
        // h, dg, [da | du] per pair
        BwdPairArgs pa{sorted, offsets, E, k, gates, A, U, dHp, H, DA, static_cast<char*>(DA) + f * w, dgate,
                       dy, nullptr, f, d};
        pa.ld_dadu = 2 * (int64_t)f;
        MOE_HIP(launch_bwd_pair(pa, P, true, s));
        // dx of each pair = [da | du] [W_gate ; W_up] (one K walk of 2 f: rows of
        // W_gate [E, f, d], then of W_up, read as they are)
        GemmGroup g2 = f32_gemm(DA, nullptr, 1, offsets, E, P, wg, dXp, d, d, 2 * f);
        g2.B1 = wu;
        g2.b_nmajor = true;
        g2.b_khalf = f;
        g2.splitk = pl.xsplit;
        g2.part_stride = (int64_t)P * d;
        g2.aligned_bands = true;
        g2.queue = q ? q + 512 : nullptr;
        MOE_HIP(launch_grouped_gemm(g2, false, true, s));
        MOE_HIP(launch_bwd_token_sum(dXp, pos, T, k, d, dx, s, pl.xsplit, (int64_t)P * d));
        // weight gradients: each expert's rows as a K range of transposed operands
        MOE_HIP(launch_kgroup_offsets(offsets, E, kofs, s));
        MOE_HIP(launch_transpose_rows(rows_t(dy, d, d, sorted, k, gates, offsets, kofs, E, P, 0, dOT, Q), Q, s));
        MOE_HIP(launch_transpose_rows(rows_t(H, f, f, nullptr, 1, nullptr, offsets, kofs, E, P, 0, HT, Q), Q, s));
        MOE_HIP(launch_transpose_rows(
            rows_t(DA, 2 * (int64_t)f, 2 * f, nullptr, 1, nullptr, offsets, kofs, E, P, 0, DADUT, Q), Q, s));
        MOE_HIP(launch_transpose_rows(rows_t(x, d, d, sorted, k, nullptr, offsets, kofs, E, P, 0, XgT, Q), Q, s));
        GemmGroup w1 = kgroup_gemm(dOT, Q, HT, Q, kofs, E, d, f, 0, dwd, f, (int64_t)d * f);
        MOE_HIP(launch_grouped_gemm(w1, false, true, s));
        GemmGroup w2 = kgroup_gemm(DADUT, Q, XgT, Q, kofs, E, f, d, 0, dwg, d, (int64_t)f * d);
        MOE_HIP(launch_grouped_gemm(w2, false, true, s));
        w2.A = static_cast<const char*>(DADUT) + (size_t)f * Q * w;
        w2.C = dwu;
        MOE_HIP(launch_grouped_gemm(w2, false, true, s));
    } else {
        void *DU = at<void>(ws, L.DU), *dO = at<void>(ws, L.dO);
        // dH' = dy W_down (rows gathered by pair)
        GradGemm g1 = grad_gemm(dy, d, wd, f, dHp, f, P, f, d);
        g1.a_gather = sorted; g1.a_div = k; g1.b_gstride = (int64_t)d * f; g1.offsets = offsets; g1.G = E;
        MOE_HIP(launch_grad_gemm(g1, false, false, bf16, bf16, s));
        // h, dg, da, du, dO per pair
        BwdPairArgs pa{sorted, offsets, E, k, gates, A, U, dHp, H, DA, DU, dgate, dy, dO, f, d};
        MOE_HIP(launch_bwd_pair(pa, P, bf16, s));
        // dx of each pair = da W_gate + du W_up, then summed per token in slot order
        GradGemm g2 = grad_gemm(DA, f, wg, d, dXp, d, P, d, f);
        g2.b_gstride = (int64_t)f * d; g2.offsets = offsets; g2.G = E;
        MOE_HIP(launch_grad_gemm(g2, false, false, bf16, bf16, s));
        g2.A = DU; g2.B = wu; g2.accumulate = true;
        MOE_HIP(launch_grad_gemm(g2, false, false, bf16, bf16, s));
        MOE_HIP(launch_bwd_token_sum(dXp, pos, T, k, d, dx, s));
        // weight gradients: sums over each expert's rows
        GradGemm w1 = grad_gemm(dO, d, H, f, dwd, f, d, f, P);
        w1.c_gstride = (int64_t)d * f; w1.offsets = offsets; w1.G = E;
        MOE_HIP(launch_grad_gemm(w1, true, false, bf16, bf16, s));
        GradGemm w2 = grad_gemm(DA, f, x, d, dwg, d, f, d, P);
        w2.b_gather = sorted; w2.b_div = k; w2.c_gstride = (int64_t)f * d; w2.offsets = offsets; w2.G = E;
        MOE_HIP(launch_grad_gemm(w2, true, false, bf16, bf16, s));
        w2.A = DU; w2.C = dwu;
        MOE_HIP(launch_grad_gemm(w2, true, false, bf16, bf16, s));
    }
    // router: dl from dg (logits recomputed when the gates or the
    // load-balancing loss need them)
    const bool aux = aux_alpha != 0.0f && T > 0;
    const bool need_logits = !(c->score_fn == MOE_SCORE_SOFTMAX && c->renormalize) || aux;
    if (need_logits) {
        GradGemm gl = grad_gemm(x, d, wr, d, logits, E, T, E, d);
        MOE_HIP(launch_grad_gemm(gl, false, true, bf16, bf16, s));
    }
    BwdRouterArgs ra{ids, gates, dgate, need_logits ? logits : nullptr, dl, T, E, k, c->score_fn, c->renormalize};
    if (aux) {
        int32_t* cnt = at<int32_t>(ws, L.auxcnt);
        MOE_HIP(launch_count_ids(ids, P, E, cnt, s));
        ra.aux_counts = cnt;
        ra.aux_coef = aux_alpha * (float)E / (float)T;
        ra.inv_T = 1.0f / (float)T;
    }
    MOE_HIP(launch_bwd_router(ra, s));
    if (pl.router_mfma) {
        const int tr = (int)pl.Tr;
        char* XT2 = at<char>(ws, L.XT2);
        MOE_HIP(launch_dl_split(dl, T, E, tr, at<uint16_t>(ws, L.DLT), s));
        for (int half = 0; half < 2; ++half)
            MOE_HIP(launch_transpose_rows(rows_t(x, d, d, nullptr, 1, nullptr, nullptr, nullptr, 1, T, tr,
                                                 XT2 + (size_t)half * pl.Tr * w, 2 * pl.Tr),
                                          pl.Tr, s));
        float* rw = at<float>(ws, L.rw);
        GemmGroup gr = f32_gemm(at<void>(ws, L.DLT), nullptr, 1, nullptr, 1, E, XT2, pl.rsplit > 1 ? rw : dwr, d, d,
                                2 * tr);
        gr.splitk = pl.rsplit;
        gr.part_stride = (int64_t)E * d;
        MOE_HIP(launch_grouped_gemm(gr, false, true, s));
        if (pl.rsplit > 1) MOE_HIP(launch_sum_chunks(rw, pl.rsplit, (int64_t)E * d, dwr, s));
    } else {
        MOE_HIP(launch_router_wgrad(dl, x, bf16, T, E, d, at<float>(ws, L.rw), dwr, s));
    }
    if (pl.router_dx_mfma) {
        // the FMA kernel below took 0.59 ms at DeepSeek-V3 prefill (E = 256)
        uint16_t* DLR = at<uint16_t>(ws, L.DLR);
        MOE_HIP(launch_dl_rows(dl, T, E, DLR, s));
        GemmGroup gx = f32_gemm(DLR, nullptr, 1, nullptr, 1, T, wr, dx, d, d, 2 * E);
        gx.B1 = wr;
        gx.b_nmajor = true;
        gx.b_khalf = E;
        gx.accumulate = true;
        MOE_HIP(launch_grouped_gemm(gx, false, true, s));
    } else {
        GradGemm gx = grad_gemm(dl, E, wr, d, dx, d, T, d, E);
        gx.accumulate = true;
        MOE_HIP(launch_grad_gemm(gx, false, false, false, bf16, s));
    }
    // shared expert: a pair per token with gate 1
    if (c->num_shared) {
        const int fs = c->d_ff_shared;
        void *As = at<void>(ws, L.As), *Us = at<void>(ws, L.Us), *Hs = at<void>(ws, L.Hs);
        void* DAs = at<void>(ws, L.DAs);
        float* dHs = at<float>(ws, L.dHs);
        GemmGroup sa{x, nullptr, 1, nullptr, 1, T, sg, nullptr, As, fs, d};
        MOE_HIP(launch_grouped_gemm(sa, false, bf16, s));
        GemmGroup su_{x, nullptr, 1, nullptr, 1, T, su, nullptr, Us, fs, d};
        MOE_HIP(launch_grouped_gemm(su_, false, bf16, s));
        if (pl.shared_fast) {
            const int64_t Tq = pl.Tq;
            void* dyT = at<void>(ws, L.dyT);
            void *HsT = at<void>(ws, L.HsT), *DADUsT = at<void>(ws, L.DADUsT), *xT = at<void>(ws, L.xT);
            GemmGroup s1 = f32_gemm(dy, nullptr, 1, nullptr, 1, T, sd, dHs, fs, fs, d);
            s1.b_nmajor = true;
            MOE_HIP(launch_grouped_gemm(s1, false, true, s));
            BwdPairArgs sp{nullptr, nullptr, 1, 1, nullptr, As, Us, dHs, Hs, DAs, static_cast<char*>(DAs) + fs * w,
                           nullptr, dy, nullptr, fs, d};
            sp.ld_dadu = 2 * (int64_t)fs;
            MOE_HIP(launch_bwd_pair(sp, T, true, s));
            GemmGroup s2 = f32_gemm(DAs, nullptr, 1, nullptr, 1, T, sg, dx, d, d, 2 * fs);
            s2.B1 = su;
            s2.b_nmajor = true;
            s2.b_khalf = fs;
            s2.accumulate = true;
            MOE_HIP(launch_grouped_gemm(s2, false, true, s));
            const int tq = (int)Tq;
            MOE_HIP(launch_transpose_rows(rows_t(dy, d, d, nullptr, 1, nullptr, nullptr, nullptr, 1, T, tq, dyT, Tq),
                                          Tq, s));
            MOE_HIP(launch_transpose_rows(rows_t(Hs, fs, fs, nullptr, 1, nullptr, nullptr, nullptr, 1, T, tq, HsT, Tq),
                                          Tq, s));
            MOE_HIP(launch_transpose_rows(
                rows_t(DAs, 2 * (int64_t)fs, 2 * fs, nullptr, 1, nullptr, nullptr, nullptr, 1, T, tq, DADUsT, Tq), Tq,
                s));
            MOE_HIP(launch_transpose_rows(rows_t(x, d, d, nullptr, 1, nullptr, nullptr, nullptr, 1, T, tq, xT, Tq),
                                          Tq, s));
            GemmGroup s3 = kgroup_gemm(dyT, Tq, HsT, Tq, nullptr, 1, d, fs, tq, dsd, fs, 0);
            MOE_HIP(launch_grouped_gemm(s3, false, true, s));
            GemmGroup s4 = kgroup_gemm(DADUsT, Tq, xT, Tq, nullptr, 1, fs, d, tq, dsg, d, 0);
            MOE_HIP(launch_grouped_gemm(s4, false, true, s));
            s4.A = static_cast<const char*>(DADUsT) + (size_t)fs * Tq * w;
            s4.C = dsu;
            MOE_HIP(launch_grouped_gemm(s4, false, true, s));
        } else {
            void* DUs = at<void>(ws, L.DUs);
            GradGemm s1 = grad_gemm(dy, d, sd, fs, dHs, fs, T, fs, d);
            MOE_HIP(launch_grad_gemm(s1, false, false, bf16, bf16, s));
            BwdPairArgs sp{nullptr, nullptr, 1, 1, nullptr, As, Us, dHs, Hs, DAs, DUs, nullptr, dy, nullptr, fs, d};
            MOE_HIP(launch_bwd_pair(sp, T, bf16, s));
            GradGemm s2 = grad_gemm(DAs, fs, sg, d, dx, d, T, d, fs);
            s2.accumulate = true;
            MOE_HIP(launch_grad_gemm(s2, false, false, bf16, bf16, s));
            s2.A = DUs; s2.B = su;
            MOE_HIP(launch_grad_gemm(s2, false, false, bf16, bf16, s));
            GradGemm s3 = grad_gemm(dy, d, Hs, fs, dsd, fs, d, fs, T);
            MOE_HIP(launch_grad_gemm(s3, true, false, bf16, bf16, s));
            GradGemm s4 = grad_gemm(DAs, fs, x, d, dsg, d, fs, d, T);
            MOE_HIP(launch_grad_gemm(s4, true, false, bf16, bf16, s));
            s4.A = DUs; s4.C = dsu;
            MOE_HIP(launch_grad_gemm(s4, true, false, bf16, bf16, s));
        }
    }
    return MOE_OK;
}

}  // namespace

int moe::validate_config(const moe_config* cfg) { return validate_cfg(cfg); }

extern "C" {

size_t moe_workspace_bytes(const moe_config* cfg) {
    if (validate_cfg(cfg) != MOE_OK) return 0;
    return layout(cfg).total;
}

const char* moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size is out of range or inconsistent";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside the supported limits";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a pointer is not 16-byte aligned";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
        default: return "unknown moe_status";
    }
}

int moe_route(const moe_config* cfg, const void* x, const void* w_router, int32_t* topk_ids,
              float* topk_weights, float* topk_gap, void* stream) {
    return moe_route_ex(cfg, nullptr, x, w_router, topk_ids, topk_weights, topk_gap, nullptr, 0, stream);
}

int moe_route_ex(const moe_config* cfg, const moe_options* opts, const void* x, const void* w_router,
                 int32_t* topk_ids, float* topk_weights, float* topk_gap, void* ws, size_t ws_bytes,
                 void* stream) {
    MOE_TRY(validate_cfg(cfg));
    MOE_TRY(validate_opts(opts));
    const bool empty = cfg->num_tokens == 0;
    MOE_TRY(check_ptr(x, empty));
    MOE_TRY(check_ptr(w_router, false));
    MOE_TRY(check_ptr(topk_ids, empty));
    MOE_TRY(check_ptr(topk_weights, empty));
    if (topk_gap) MOE_TRY(check_ptr(topk_gap, true));
    const bool stats = opts && opts->router_stats;
    const Layout L = layout(cfg);
    if (stats) {
        if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
        MOE_TRY(check_ptr(ws, false));
    }
    if (empty) return MOE_OK;
    return run_route(cfg, x, w_router, topk_ids, topk_weights, topk_gap,
                     static_cast<hipStream_t>(stream), nullptr, nullptr, nullptr, opts,
                     stats ? at<float>(ws, L.spart) : nullptr);
}

int moe_dispatch(const moe_config* cfg, const int32_t* topk_ids, int32_t* expert_counts,
                 int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos, void* ws,
                 size_t ws_bytes, void* stream) {
    return moe_dispatch_ex(cfg, nullptr, topk_ids, expert_counts, expert_offsets, sorted_pairs, pair_pos,
                           ws, ws_bytes, stream);
}

int moe_dispatch_ex(const moe_config* cfg, const moe_options* opts, const int32_t* topk_ids,
                    int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_pairs,
                    int32_t* pair_pos, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(validate_cfg(cfg));
    MOE_TRY(validate_opts(opts));
    const bool empty = cfg->num_tokens == 0;
    MOE_TRY(check_ptr(topk_ids, empty));
    MOE_TRY(check_ptr(expert_counts, false));
    MOE_TRY(check_ptr(expert_offsets, false));
    MOE_TRY(check_ptr(sorted_pairs, empty));
    MOE_TRY(check_ptr(pair_pos, empty));
    const Layout L = layout(cfg);
    if (L.dispatch_need > 0) {
        if (!ws || ws_bytes < L.dispatch_need) return MOE_ERR_WORKSPACE;
        MOE_TRY(check_ptr(ws, false));
    }
    return run_dispatch(cfg, topk_ids, expert_counts, expert_offsets, sorted_pairs, pair_pos,
                        static_cast<int32_t*>(ws), static_cast<hipStream_t>(stream), capacity_of(opts));
}

int moe_expert_ffn(const moe_config* cfg, const void* x, const int32_t* sorted_pairs,
                   const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                   const void* w_down, const void* ws_gate, const void* ws_up,
                   const void* ws_down, void* expert_out, void* shared_out, void* ws,
                   size_t ws_bytes, void* stream) {
    MOE_TRY(validate_cfg(cfg));
    const bool empty = cfg->num_tokens == 0;
    MOE_TRY(check_ptr(x, empty));
    MOE_TRY(check_ptr(sorted_pairs, empty));
    MOE_TRY(check_ptr(expert_offsets, false));
    MOE_TRY(check_ptr(w_gate, false));
    MOE_TRY(check_ptr(w_up, false));
    MOE_TRY(check_ptr(w_down, false));
    MOE_TRY(check_ptr(expert_out, empty));
    if (cfg->num_shared) {
        MOE_TRY(check_ptr(ws_gate, false));
        MOE_TRY(check_ptr(ws_up, false));
        MOE_TRY(check_ptr(ws_down, false));
        MOE_TRY(check_ptr(shared_out, empty));
    }
    const Layout L = layout(cfg);
    if (L.ffn_need > 0) {
        if (!ws || ws_bytes < L.ffn_need) return MOE_ERR_WORKSPACE;
        MOE_TRY(check_ptr(ws, false));
    }
    if (empty) return MOE_OK;
    return run_ffn(cfg, x, sorted_pairs, expert_offsets, w_gate, w_up, w_down, ws_gate, ws_up,
                   ws_down, expert_out, shared_out, at<void>(ws, L.H), at<void>(ws, L.Hs),
                   at<int32_t>(ws, L.queue), false, static_cast<hipStream_t>(stream));
}

int moe_combine(const moe_config* cfg, const void* expert_out, const float* topk_weights,
                const int32_t* pair_pos, const void* shared_out, void* y, void* stream) {
    MOE_TRY(validate_cfg(cfg));
    const bool empty = cfg->num_tokens == 0;
    MOE_TRY(check_ptr(expert_out, empty));
    MOE_TRY(check_ptr(topk_weights, empty));
    MOE_TRY(check_ptr(pair_pos, empty));
    MOE_TRY(check_ptr(y, empty));
    if (cfg->num_shared) MOE_TRY(check_ptr(shared_out, empty));
    if (empty) return MOE_OK;
    return run_combine(cfg, expert_out, topk_weights, pair_pos,
                       cfg->num_shared ? shared_out : nullptr, y, static_cast<hipStream_t>(stream));
}

int moe_forward_staged(const moe_config* cfg, const void* x, const void* w_router,
                       const void* w_gate, const void* w_up, const void* w_down,
                       const void* ws_gate, const void* ws_up, const void* ws_down, void* y,
                       int32_t* topk_ids_out, float* topk_weights_out,
                       int32_t* expert_counts_out, float* topk_gap_out, void* ws, size_t ws_bytes,
                       void* start_event, void* const* ev, void* stream) {
    return forward_impl(cfg, nullptr, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y,
                        topk_ids_out, topk_weights_out, expert_counts_out, topk_gap_out, ws, ws_bytes,
                        start_event, ev, stream);
}

int moe_forward_ex(const moe_config* cfg, const moe_options* opts, const void* x, const void* w_router,
                   const void* w_gate, const void* w_up, const void* w_down, const void* ws_gate,
                   const void* ws_up, const void* ws_down, void* y, int32_t* topk_ids_out,
                   float* topk_weights_out, int32_t* expert_counts_out, float* topk_gap_out, void* ws,
                   size_t ws_bytes, void* stream) {
    return forward_impl(cfg, opts, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y,
                        topk_ids_out, topk_weights_out, expert_counts_out, topk_gap_out, ws, ws_bytes, nullptr,
                        nullptr, stream);
}

size_t moe_backward_workspace_bytes(const moe_config* cfg) {
    if (validate_cfg(cfg) != MOE_OK) return 0;
    return bwd_layout(cfg).total;
}

int moe_backward(const moe_config* cfg, const void* x, const void* w_router, const void* w_gate,
                 const void* w_up, const void* w_down, const void* ws_gate, const void* ws_up,
                 const void* ws_down, const void* dy, const int32_t* topk_ids, const float* topk_weights,
                 float* dx, float* dw_router, float* dw_gate, float* dw_up, float* dw_down, float* dws_gate,
                 float* dws_up, float* dws_down, void* ws, size_t ws_bytes, void* stream) {
    return moe_backward_ex(cfg, nullptr, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, dy, topk_ids,
                           topk_weights, dx, dw_router, dw_gate, dw_up, dw_down, dws_gate, dws_up, dws_down, ws,
                           ws_bytes, stream);
}

int moe_backward_ex(const moe_config* cfg, const moe_options* opts, const void* x, const void* w_router,
                    const void* w_gate, const void* w_up, const void* w_down, const void* ws_gate,
                    const void* ws_up, const void* ws_down, const void* dy, const int32_t* topk_ids,
                    const float* topk_weights, float* dx, float* dw_router, float* dw_gate, float* dw_up,
                    float* dw_down, float* dws_gate, float* dws_up, float* dws_down, void* ws, size_t ws_bytes,
                    void* stream) {
    MOE_TRY(validate_cfg(cfg));
    MOE_TRY(validate_opts(opts));
    if (opts && opts->router_stats) return MOE_ERR_UNSUPPORTED;     // the backward computes no statistics
    if (opts && !std::isfinite(opts->aux_alpha)) return MOE_ERR_SHAPE;
    const bool empty = cfg->num_tokens == 0;
    for (const void* p : {x, dy, (const void*)topk_ids, (const void*)topk_weights, (const void*)dx})
        MOE_TRY(check_ptr(p, empty));
    for (const void* p : {w_router, w_gate, w_up, w_down, (const void*)dw_router, (const void*)dw_gate,
                          (const void*)dw_up, (const void*)dw_down})
        MOE_TRY(check_ptr(p, false));
    if (cfg->num_shared)
        for (const void* p : {ws_gate, ws_up, ws_down, (const void*)dws_gate, (const void*)dws_up,
                              (const void*)dws_down})
            MOE_TRY(check_ptr(p, false));
    const BwdLayout L = bwd_layout(cfg);
    if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    MOE_TRY(check_ptr(ws, false));
    // T = 0 still runs: the weight gradients are written as zeros
    return run_backward(cfg, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, dy, topk_ids,
                        topk_weights, dx, dw_router, dw_gate, dw_up, dw_down, dws_gate, dws_up, dws_down, ws,
                        static_cast<hipStream_t>(stream), capacity_of(opts), opts ? opts->aux_alpha : 0.0f);
}

int moe_forward(const moe_config* cfg, const void* x, const void* w_router, const void* w_gate,
                const void* w_up, const void* w_down, const void* ws_gate, const void* ws_up,
                const void* ws_down, void* y, int32_t* topk_ids_out, float* topk_weights_out,
                int32_t* expert_counts_out, float* topk_gap_out, void* ws, size_t ws_bytes, void* stream) {
    return moe_forward_staged(cfg, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y,
                              topk_ids_out, topk_weights_out, expert_counts_out, topk_gap_out, ws, ws_bytes,
                              nullptr, nullptr, stream);
}

int moe_capacity(const moe_config* cfg, double capacity_factor) {
    MOE_TRY(validate_cfg(cfg));
    if (!(capacity_factor > 0.0) || !std::isfinite(capacity_factor)) return MOE_ERR_SHAPE;
    const double q = (double)cfg->num_tokens * cfg->top_k / cfg->num_experts * capacity_factor;
    // The factor is a decimal the caller wrote (1.1, 1.25), which a double
    // holds only to about 1e-16: a product that close to a whole number is
    // that number (640 * 8 / 8 * 1.1 is 704.0000000000001 in doubles: 704 slots).
    const double r = std::nearbyint(q);
    const double c = std::fabs(q - r) <= 1e-12 * std::max(1.0, q) ? r : std::ceil(q);
    if (c > 2147483647.0) return MOE_ERR_UNSUPPORTED;
    return (int)c;
}

int moe_forward_plan(const moe_config* cfg, int32_t* plan_out) {
    MOE_TRY(validate_cfg(cfg));
    if (plan_out == nullptr) return MOE_ERR_NULL;
    const Paths pa = paths(cfg);
    const Splits sp = splits(cfg);
    plan_out[0] = pa.routed_skinny ? 32 : routed_tall(cfg) ? 288 : routed_choice(cfg) ? 0 : 256;
    plan_out[1] = sp.routed;
    plan_out[2] = cfg->num_shared ? sp.shared : 0;
    plan_out[3] = merged_shared(cfg, 0x7FFFFFFF) ? 1 : 0;
    return MOE_OK;
}

}  // extern "C"
