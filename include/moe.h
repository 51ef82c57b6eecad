/*
 * moe.h -- C ABI of the MI355X (gfx950) top-k Mixture-of-Experts FFN layer:
 * the forward pass (whole, or step by step), its optional routing features
 * (selection bias, expert capacity, load statistics) and the backward pass.
 *
 * The layer (pages: "Mixture-of-Experts Internals: A Systems Engineer's Field
 * Manual" sec. 2.1; "8.6 -- Mixture of Experts (MoE)" sec. 2 and 4.1;
 * "Mixture-of-Experts, from the router to the all-to-all", The router;
 * "Mixture of Experts: What Actually Happens When a Token Hits the Router",
 * Steps 1-4):
 *
 *   h = W_r x                              router logits, fp32
 *   s = softmax(h) | sigmoid(h)            scores
 *   I = top-k of h (ties: lower index)     selection
 *   g_i = s_i / sum_{j in I} s_j           gates (or g_i = s_i unrenormalised)
 *   y = sum_{i in I} g_i f_i(x) + f_s(x)   f(x) = W_down(silu(W_gate x) * W_up x)
 *
 * Conventions shared by every entry point:
 *   - Ownership: the caller owns every buffer.  The library never allocates
 *     or frees device memory and keeps no state between calls (beyond the
 *     device's compute-unit count, read once); calls are thread-safe.  A
 *     workspace is scratch for one call at a time (each call sets up what it
 *     needs in it, tile counters included): calls that may run together on
 *     different streams need workspaces of their own.
 *   - Pointers: every tensor pointer is a DEVICE pointer (HBM of the current
 *     HIP device).  `cfg` is a HOST pointer read during the call only.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Every call only enqueues work on it: no host synchronisation,
 *     no device-to-host copy.  Results are valid once the stream reaches them.
 *   - Layouts, row-major, C order:
 *       x, y [T, d]; w_router [E, d]
 *       w_gate, w_up [E, d_ff, d]; w_down [E, d, d_ff]
 *       ws_gate, ws_up [d_ff_s, d]; ws_down [d, d_ff_s]
 *       topk_ids, topk_weights [T, k]
 *       expert_out [T*k, d] in expert-grouped order; shared_out [T, d]
 *   - Types: x, y, weights, expert_out, shared_out use cfg->dtype (fp32 or
 *     bf16).  Gates, gaps and logits are fp32; indices and counts int32.
 *   - Pairs: the T*k (token, slot) assignments are numbered p = t*k + j.
 *   - Limits: 1 <= E <= 256, 1 <= k <= min(E, 16), d, d_ff, d_ff_s multiples
 *     of 64, T*k < 2^31, T >= 0 (T = 0 is a valid no-op).  Pointers 16-byte
 *     aligned.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; on error nothing is enqueued and a negative moe_status is
 *     returned.  A failed launch returns MOE_ERR_HIP.  Device faults surface
 *     at the caller's next synchronisation.  Inputs must be finite: the
 *     result for NaN or Inf inputs is undefined.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    MOE_ERR_UNSUPPORTED = -3, /* outside the limits above (E > 256, k > 16, d % 64, dtype) */
    MOE_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required */
    MOE_ERR_HIP = -6          /* a HIP launch failed */
} moe_status;

typedef enum moe_score_fn {
    MOE_SCORE_SOFTMAX = 0,    /* softmax over all E experts */
    MOE_SCORE_SIGMOID = 1     /* independent sigmoid per expert */
} moe_score_fn;

typedef enum moe_dtype {
    MOE_F32 = 0,
    MOE_BF16 = 1
} moe_dtype;

typedef struct moe_config {
    int32_t num_tokens;   /* T */
    int32_t d_model;      /* d */
    int32_t num_experts;  /* E, routed experts */
    int32_t top_k;        /* k */
    int32_t d_ff;         /* width of each routed expert */
    int32_t num_shared;   /* 0 or 1 always-on shared expert(s), weight 1 */
    int32_t d_ff_shared;  /* width of the shared expert (ignored if num_shared == 0) */
    int32_t score_fn;     /* moe_score_fn */
    int32_t renormalize;  /* 1: gates renormalised over the k chosen; 0: raw scores */
    int32_t dtype;        /* moe_dtype of activations and weights */
} moe_config;

/* Bytes of device workspace moe_forward needs for `cfg` (also enough for
 * every other forward entry point; the backward has its own,
 * moe_backward_workspace_bytes).  0 for an invalid cfg.  Host only. */
size_t moe_workspace_bytes(const moe_config* cfg);

/* Human-readable name of a status code.  Host only; static storage. */
const char* moe_status_str(int status);

/*
 * Router + top-k + gates ("Mixture-of-Experts Internals" sec. 2.1; "from the
 * router to the all-to-all", The router).
 *   x [T,d], w_router [E,d]                 in
 *   topk_ids [T,k] int32                    out: chosen experts, by descending
 *                                                logit, ties to the lower index
 *   topk_weights [T,k] fp32                 out: gates
 *   topk_gap [T,2] fp32 (nullable)          out, per token:
 *       [t][0] = h_(k) - h_(k+1), the logit margin between the k-th and the
 *                (k+1)-th choice (with a selection bias, moe_options, the
 *                margin of the selection key);
 *       [t][1] = s_(k) - s_(k+1), the score margin of the same two experts
 *                (softmax over all E, or sigmoid; unbiased scores, so with
 *                a bias it can be negative), computed without cancellation.
 *       Both +inf when k == E.  A token whose margins are tiny (a near-tie:
 *       score margin below about 1e-6, logit margin below about 1e-4, the
 *       reach of fp32 accumulation) may be routed differently by an exact
 *       computation; the caller can tell which tokens those are.
 * Logits are accumulated in fp32 (products of bf16 inputs are exact in fp32).
 */
int moe_route(const moe_config* cfg, const void* x, const void* w_router, int32_t* topk_ids,
              float* topk_weights, float* topk_gap, void* stream);

/*
 * Group the T*k pairs by expert ("What Actually Happens...", Step 3: sort
 * tokens by assigned expert into contiguous blocks).  Stable: inside expert
 * e's block, pairs keep ascending p.
 *   topk_ids [T,k]                          in
 *   expert_counts [E] int32                 out: pairs per expert
 *   expert_offsets [E+1] int32              out: exclusive prefix sum; the
 *                                                block of expert e is rows
 *                                                [off[e], off[e+1])
 *   sorted_pairs [T*k] int32                out: pair p at each grouped row
 *   pair_pos [T*k] int32                    out: grouped row of each pair
 *   ws, ws_bytes                            scratch, >= moe_workspace_bytes
 * ids outside [0, E) are a precondition violation (undefined result).
 */
int moe_dispatch(const moe_config* cfg, const int32_t* topk_ids, int32_t* expert_counts,
                 int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos, void* ws,
                 size_t ws_bytes, void* stream);

/*
 * Expert SwiGLU FFNs as one grouped GEMM pair ("8.6 Mixture of Experts" sec.
 * 2; "What Actually Happens...", Step 4): for every grouped row r of expert
 * e with pair p = sorted_pairs[r] and token t = p / k,
 *   expert_out[r] = W_down,e (silu(W_gate,e x_t) * (W_up,e x_t)),
 * and, when cfg->num_shared == 1, for every token t
 *   shared_out[t] = W_sdown (silu(W_sgate x_t) * (W_sup x_t)).
 * The intermediate silu(.)*(.) is rounded to cfg->dtype.
 *   x [T,d], sorted_pairs [T*k], expert_offsets [E+1]   in
 *   w_gate, w_up, w_down                                in (routed experts)
 *   ws_gate, ws_up, ws_down                             in (nullable iff num_shared == 0)
 *   expert_out [T*k, d]                                 out
 *   shared_out [T, d]                                   out (nullable iff num_shared == 0)
 *   ws, ws_bytes                                        scratch
 */
int moe_expert_ffn(const moe_config* cfg, const void* x, const int32_t* sorted_pairs,
                   const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                   const void* w_down, const void* ws_gate, const void* ws_up,
                   const void* ws_down, void* expert_out, void* shared_out, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * Gate-weighted combine back into token order ("8.6 Mixture of Experts" sec.
 * 2 boxed equation and sec. 4.1):
 *   y[t] = sum_{j=0..k-1} topk_weights[t,j] * expert_out[pair_pos[t*k+j]]
 *          (+ shared_out[t])
 * summed in fp32 in slot order j = 0..k-1, then rounded to cfg->dtype.  No
 * atomics: every y row is written once.  A slot whose pair_pos is -1 (a pair
 * dropped for capacity, see moe_options) contributes nothing.
 *   shared_out nullable iff num_shared == 0.
 */
int moe_combine(const moe_config* cfg, const void* expert_out, const float* topk_weights,
                const int32_t* pair_pos, const void* shared_out, void* y, void* stream);

/*
 * The whole layer: route, dispatch, expert FFNs (and the shared expert) and
 * combine, enqueued back to back on `stream`.
 *   topk_ids_out [T,k], topk_weights_out [T,k], expert_counts_out [E]:
 *   optional copies of the routing (nullable; the workspace is used when
 *   NULL).
 *   topk_gap_out [T,2] (nullable): the margins of this call's own routing,
 *   as moe_route's topk_gap (the near-ties of the layer as it ran).
 * Same arithmetic as the entry points above, except that in bf16 the router
 * logits (below 8192 tokens) and the down projections may be summed over K
 * ranges (fixed order; deterministic), so results can differ from the
 * step-by-step calls in the last bits and routing at near-ties.
 * A bf16 shared expert as wide as the routed ones (d_ff_shared == d_ff)
 * runs inside the routed GEMMs' launches, as one more group of T rows with
 * its own weights, when those GEMMs take 256-row tiles without K splits and
 * no capacity is set; its products are the same as on its own launches.
 */
int moe_forward(const moe_config* cfg, const void* x, const void* w_router, const void* w_gate,
                const void* w_up, const void* w_down, const void* ws_gate, const void* ws_up,
                const void* ws_down, void* y, int32_t* topk_ids_out, float* topk_weights_out,
                int32_t* expert_counts_out, float* topk_gap_out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The caller passes inputs and outputs only (same meaning as moe_forward);
 * the workspace is the library's own: a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES in device memory, one per GPU, which each GPU the
 * library runs on holds from module load until the process ends.  Nothing
 * is allocated or freed: no hipMalloc, no allocating library routine.
 *   Limit: layers whose moe_workspace_bytes(cfg) exceed the array (decode-
 *   sized batches fit: Mixtral-8x7B widths up to about 256 tokens) return
 *   MOE_ERR_WORKSPACE before anything is enqueued.
 *   Sharing: every call on one GPU uses that GPU's array, which keeps the
 *   last call's contents (each call sets up what it needs, counters
 *   included).  Calls that overlap on one GPU, on different streams or from
 *   different threads, race on it: serialise them.
 * The first call on a device looks up the array's address on that device
 * (current device); a failure there returns MOE_ERR_HIP.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_config* cfg, const void* x, const void* w_router, const void* w_gate,
                        const void* w_up, const void* w_down, const void* ws_gate, const void* ws_up,
                        const void* ws_down, void* y, int32_t* topk_ids_out, float* topk_weights_out,
                        int32_t* expert_counts_out, float* topk_gap_out, void* stream);

/*
 * moe_forward with per-stage timing ("T2.6 -- What Mixture of Experts
 * Changes", In practice: watch per-expert counts and expert compute time;
 * profile each stage).  Same arguments and results as moe_forward, plus
 *   stage_events: MOE_NUM_STAGES hipEvent_t handles (passed as void*),
 *                 created by the caller, entries nullable; event i is
 *                 recorded on `stream` right after stage i is enqueued,
 *                 except events 1 and 2, which the routed gate/up kernel's
 *                 launch records at its start and at its end (so 1 -> 2 is
 *                 that kernel's own duration):
 *                 0 route, 1 dispatch, 2 routed gate/up GEMM (+SiLU*up),
 *                 3 routed down GEMM, 4 shared gate/up, 5 shared down,
 *                 6 combine.  Stages 4-5 are empty when num_shared == 0
 *                 and when the shared expert runs inside the routed GEMMs
 *                 (see moe_forward; its time then counts in stages 2-3);
 *                 stage 1 is empty when the batch is at most 32 bf16
 *                 tokens with a K-split router, whose last kernel then
 *                 also groups the pairs (its time counts in stage 0).
 *   start_event:  recorded before stage 0 (nullable).
 * The elapsed time between consecutive events is the stage's device time.
 */
#define MOE_NUM_STAGES 7
int moe_forward_staged(const moe_config* cfg, const void* x, const void* w_router,
                       const void* w_gate, const void* w_up, const void* w_down,
                       const void* ws_gate, const void* ws_up, const void* ws_down, void* y,
                       int32_t* topk_ids_out, float* topk_weights_out,
                       int32_t* expert_counts_out, float* topk_gap_out, void* ws, size_t ws_bytes,
                       void* start_event, void* const* stage_events, void* stream);

/*
 * Backward pass of the layer for the routing of a forward call ("8.6 Mixture
 * of Experts", sec. 2; the router learns only through the gates of the
 * chosen experts, "Mixture-of-Experts Internals", sec. 2.2).  With L the
 * loss and dy = dL/dy [T,d] (cfg->dtype):
 *   topk_ids, topk_weights [T,k]     in: the forward's routing (held fixed;
 *                                    the selection itself has no gradient)
 *   dx [T,d]                         out: dL/dx, through the experts, the
 *                                    gates and the shared expert
 *   dw_router [E,d]                  out: through the gates only
 *   dw_gate, dw_up [E,d_ff,d]; dw_down [E,d,d_ff]   out (0 for unused experts)
 *   dws_gate, dws_up [d_ff_s,d]; dws_down [d,d_ff_s] out, nullable iff
 *                                    num_shared == 0
 * All gradients are fp32 and overwritten (not accumulated).  The plain layer
 * (moe_backward_ex below adds an expert capacity).  The expert pre-activations are recomputed, nothing
 * is kept from the forward but its routing.  Sums run in a fixed order, no
 * atomics: the result is deterministic.  ws: at least
 * moe_backward_workspace_bytes(cfg) bytes; for bf16 layers whose d and d_ff
 * are multiples of 256 that includes transposed copies of the pairs'
 * activations (the weights are read as they are).
 */
size_t moe_backward_workspace_bytes(const moe_config* cfg);
int moe_backward(const moe_config* cfg, const void* x, const void* w_router, const void* w_gate,
                 const void* w_up, const void* w_down, const void* ws_gate, const void* ws_up,
                 const void* ws_down, const void* dy, const int32_t* topk_ids, const float* topk_weights,
                 float* dx, float* dw_router, float* dw_gate, float* dw_up, float* dw_down, float* dws_gate,
                 float* dws_up, float* dws_down, void* ws, size_t ws_bytes, void* stream);

/*
 * Optional routing features.  A NULL moe_options*, or one with every field
 * zero, is the plain layer above.
 *   expert_bias [E] fp32 (device, nullable): a per-expert bias used only to
 *       choose the experts; the gates stay the unbiased scores, renormalised
 *       over the chosen set when cfg->renormalize ("Mixture-of-Experts
 *       Internals", sec. 3.3, auxiliary-loss-free balancing; "from the router
 *       to the all-to-all", Load balancing).
 *   bias_on_scores: 0 = choose on logit + bias (the first page's form),
 *       1 = on score + bias (the second page's form; the score is the
 *       softmax probability or the sigmoid).  topk_gap is then the margin in
 *       that selection space.
 *   expert_capacity (> 0): each expert keeps at most this many pairs, the
 *       first ones in pair order; the others are dropped and contribute
 *       nothing ("8.6 Mixture of Experts", sec. 3.2; "from the router to the
 *       all-to-all", Capacity and token dropping: capacity = T k / E times
 *       the capacity factor, rounded as the caller chooses).  expert_counts
 *       and expert_offsets then count the kept pairs, pair_pos is -1 for a
 *       dropped pair, and sorted_pairs holds offsets[E] entries (the rest
 *       are unspecified).  <= 0: no limit.
 *   router_stats [2E + 3] fp32 (device, nullable): load statistics of the
 *       batch ("8.6 Mixture of Experts", sec. 3.1; "from the router to the
 *       all-to-all", Load balancing; "T2.6 -- What Mixture of Experts
 *       Changes", In practice: counts, maximum-to-mean load, overflow):
 *         [0, E)   f_e = (pairs routed to e, before any capacity drop) / T
 *         [E, 2E)  P_e = mean over tokens of e's router probability (softmax
 *                  score; sigmoid scores normalised over all experts)
 *         [2E]     L_aux = aux_alpha * E * sum_e f_e P_e  (sum_e f_e = k, so
 *                  uniform routing gives aux_alpha * k)
 *         [2E+1]   max_e n_e / mean_e n_e
 *         [2E+2]   capacity overflow: sum_e max(0, n_e - expert_capacity),
 *                  the pairs the capacity drops (0 without a capacity);
 *                  counts are exact below 2^24
 *       Needs the workspace.  Sums are taken in a fixed order.
 */
typedef struct moe_options {
    const float* expert_bias;
    int32_t bias_on_scores;
    int32_t expert_capacity;
    float* router_stats;
    float aux_alpha;
} moe_options;

/* moe_route with options.  ws: scratch of at least moe_workspace_bytes
 * bytes when router_stats is set, else unused (nullable). */
int moe_route_ex(const moe_config* cfg, const moe_options* opts, const void* x, const void* w_router,
                 int32_t* topk_ids, float* topk_weights, float* topk_gap, void* ws, size_t ws_bytes,
                 void* stream);

/* moe_dispatch with options (expert_capacity). */
int moe_dispatch_ex(const moe_config* cfg, const moe_options* opts, const int32_t* topk_ids,
                    int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_pairs,
                    int32_t* pair_pos, void* ws, size_t ws_bytes, void* stream);

/* moe_forward with options (bias, capacity, statistics). */
int moe_forward_ex(const moe_config* cfg, const moe_options* opts, const void* x, const void* w_router,
                   const void* w_gate, const void* w_up, const void* w_down, const void* ws_gate,
                   const void* ws_up, const void* ws_down, void* y, int32_t* topk_ids_out,
                   float* topk_weights_out, int32_t* expert_counts_out, float* topk_gap_out, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * Slots per expert for a capacity factor ("8.6 Mixture of Experts", sec. 3.2;
 * "Mixture-of-Experts, from the router to the all-to-all", Capacity and
 * token dropping: tokens per batch times k over the number of experts, times
 * the factor), for moe_options.expert_capacity:
 *   ceil(T * k / E * capacity_factor).
 * The pages leave the rounding open; the ceiling keeps every slot the formula
 * grants.  The factor is read as the decimal the caller wrote: a product
 * within 1e-12 (relative) of a whole number is that number, so 640 tokens,
 * k = 8, E = 8 and factor 1.1 give 704 slots although the product of the
 * doubles is 704.0000000000001.  The page's example (4,096 tokens, 64
 * experts, top-8, factor 1.0) gives 512.
 * Returns the capacity (>= 0), or a negative moe_status: an invalid cfg as
 * moe_workspace_bytes would reject it, MOE_ERR_SHAPE for a factor that is not
 * finite and positive, MOE_ERR_UNSUPPORTED for a result past INT32_MAX.
 * Host only. */
int moe_capacity(const moe_config* cfg, double capacity_factor);

/*
 * How moe_forward (no capacity) lays the layer out on kernels, for reading
 * its per-stage times and kernel traces ("T2.6 -- What Mixture of Experts
 * Changes", In practice: profile each stage).  plan_out [4] int32, host:
 *   [0] rows per tile of the routed expert GEMMs: 256; 288 when the experts
 *       hold 224 to 287 rows on average with the tile queue (fewer than 640
 *       rows per expert), so that experts of 257..288 rows are one tile; 32
 *       for few pairs (fp32 layers report 256 and use a plain tiled kernel);
 *       0 when each call chooses between 256 and 288 on the device from the
 *       expert counts (bf16, 640 or more rows per expert, d a multiple of
 *       256 and d_ff of 128): both kernels of each GEMM are launched and the
 *       one not chosen exits at once,
 *   [1] K splits of the routed down GEMM (1 = none; with [0] = 0, of its
 *       256-row kernel: the 288-row one does not split),
 *   [2] K splits of the shared down GEMM (0 when num_shared == 0),
 *   [3] 1 when the shared expert runs inside the routed GEMMs' launches
 *       (stages 4-5 of moe_forward_staged empty), else 0.
 * Returns MOE_OK, an invalid cfg's moe_status, or MOE_ERR_NULL.  Host only.
 */
int moe_forward_plan(const moe_config* cfg, int32_t* plan_out);

/* moe_backward with options, for training with an expert capacity ("8.6
 * Mixture of Experts", sec. 3.2; "Mixture-of-Experts, from the router to the
 * all-to-all", Capacity and token dropping): with expert_capacity > 0 the pairs past each
 * expert's first expert_capacity (in pair order, as moe_forward_ex dropped
 * them) added nothing to y, so they get no gradient: their gates' dL/dg is 0
 * and their experts get nothing from them; the router still gets the gates'
 * full Jacobian.  With aux_alpha != 0 the gradient of the load-balancing
 * loss L_aux = aux_alpha E sum_e f_e P_e (as moe_options' statistics define
 * it; "8.6 Mixture of Experts", sec. 3.1) is added to dx and dw_router: f_e
 * counts the hard assignment (before any capacity drop) and carries no
 * gradient, so the loss trains the router through P_e, the mean router
 * probability (softmax, or the sigmoids normalised over the experts).
 * expert_bias and bias_on_scores have no effect (the routing is an input);
 * router_stats must be NULL (MOE_ERR_UNSUPPORTED); a non-finite aux_alpha is
 * MOE_ERR_SHAPE.  Same arguments, workspace and errors as moe_backward; NULL
 * opts is moe_backward. */
int moe_backward_ex(const moe_config* cfg, const moe_options* opts, const void* x, const void* w_router,
                    const void* w_gate, const void* w_up, const void* w_down, const void* ws_gate,
                    const void* ws_up, const void* ws_down, const void* dy, const int32_t* topk_ids,
                    const float* topk_weights, float* dx, float* dw_router, float* dw_gate, float* dw_up,
                    float* dw_down, float* dws_gate, float* dws_up, float* dws_down, void* ws, size_t ws_bytes,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
