"""CPU oracle for the top-k MoE FFN layer forward pass (fp64, plain C).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline are the only callers.  The GPU library never imports, links or runs
anything from here, and this package imports nothing from it.

Each wrapper below states the definition it evaluates; the C source
(``moe_oracle.c``) cites the page and section of each step.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
in ``tests/test_oracle_pins.py``, ``tests/test_oracle_next.py`` and
``tests/test_oracle_backward.py`` (closed forms, special cases that reduce to
a dense softmax ensemble or a library routine, brute force over subsets, the
pages' printed counts, and central finite differences of the forward for the
backward).  None is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB_OVERRIDE loads another build of moe_oracle.c; the mutation tests
# use it to check that the pins fail on a copy with a planted mistake.
_LIB_PATH = os.environ.get("ORACLE_LIB_OVERRIDE") or os.path.join(_HERE, "liboracle.so")
_lib = None

SOFTMAX, SIGMOID = 0, 1
F32, BF16, F64 = 0, 1, 2


def build(verbose: bool = False) -> str:
    src = os.path.join(_HERE, "moe_oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC", src,
           "-o", out, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    return out


def _nthreads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        i32, i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        L.oracle_logits.argtypes = [i64, i64, i32, i32, vp, vp, i32, vp, i32]
        L.oracle_logits.restype = None
        L.oracle_route.argtypes = [i64, i32, i32, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp, vp, i32]
        L.oracle_route.restype = i32
        L.oracle_dispatch.argtypes = [i64, i32, i32, i64, vp, vp, vp, vp, vp]
        L.oracle_dispatch.restype = i32
        L.oracle_expert_rows.argtypes = [i32, i32, i32, vp, i32, vp, i64, vp, vp, vp, vp, vp, i32]
        L.oracle_expert_rows.restype = None
        L.oracle_forward_tokens.argtypes = ([i32] * 9 + [vp] * 8 + [vp, i32, vp, i64, vp, vp, vp, vp, vp, i32])
        L.oracle_forward_tokens.restype = i32
        L.oracle_forward_expert_loop.argtypes = ([i64] + [i32] * 7 + [vp] * 7 + [vp, vp, vp, i32])
        L.oracle_forward_expert_loop.restype = i32
        L.oracle_backward.argtypes = [i64] + [i32] * 9 + [vp] * 8 + [vp, vp] + [vp] * 8 + [vp]
        L.oracle_backward.restype = i32
        L.oracle_backward_weight_samples.argtypes = ([i64] + [i32] * 8 + [vp] * 8 + [vp, vp, i32] + [vp] * 5)
        L.oracle_backward_weight_samples.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs are fp32, bf16 bit patterns (uint16) or fp64, got {a.dtype}")


def _c(a):
    return None if a is None else np.ascontiguousarray(a)


def _f64(a: np.ndarray) -> np.ndarray:
    """The stored values widened exactly to fp64 (bf16 bit patterns, fp32 or fp64)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def logits(x: np.ndarray, w_router: np.ndarray, rows: slice | None = None,
           nthreads: int | None = None) -> np.ndarray:
    """h[t,e] = sum_i x[t,i] W_r[e,i] in fp64, for the tokens in ``rows``."""
    x, w_router = _c(x), _c(w_router)
    T, d = x.shape
    E = w_router.shape[0]
    t0, t1 = (0, T) if rows is None else (rows.start or 0, rows.stop if rows.stop is not None else T)
    out = np.empty((t1 - t0, E), dtype=np.float64)
    lib().oracle_logits(t1 - t0, t0, d, E, x.ctypes.data, w_router.ctypes.data, _dtype_of(x),
                        out.ctypes.data, nthreads or _nthreads())
    return out


def route(lg: np.ndarray, k: int, score_fn: int = SOFTMAX, renormalize: int = 1,
          bias: np.ndarray | None = None, forced_ids: np.ndarray | None = None,
          nthreads: int | None = None, bias_on_scores: int = 0) -> dict:
    """Scores, top-k ids (descending selection key, ties to the lower index),
    gates from the unbiased scores, and the k-th/(k+1)-th gaps in score space
    and in selection-key space (``gap_logit``: the key is the logit, or with a
    bias the logit + bias or the score + bias)."""
    lg = np.ascontiguousarray(lg, dtype=np.float64)
    n, E = lg.shape
    ids = np.empty((n, k), dtype=np.int32)
    gates = np.empty((n, k), dtype=np.float64)
    scores = np.empty((n, E), dtype=np.float64)
    gs = np.empty(n, dtype=np.float64)
    gl = np.empty(n, dtype=np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
    fi = None if forced_ids is None else np.ascontiguousarray(forced_ids, dtype=np.int32)
    rc = lib().oracle_route(n, E, k, score_fn, renormalize, lg.ctypes.data, _ptr(b), int(bias_on_scores),
                            _ptr(fi), ids.ctypes.data, gates.ctypes.data, scores.ctypes.data,
                            gs.ctypes.data, gl.ctypes.data, nthreads or _nthreads())
    if rc:
        raise ValueError(f"oracle_route failed ({rc})")
    return dict(ids=ids, gates=gates, scores=scores, gap_score=gs, gap_logit=gl)


def capacity(T: int, k: int, E: int, factor: float) -> int:
    """Slots per expert: ceil(T * k / E * factor) ("8.6 Mixture of Experts",
    sec. 3.2; "from the router to the all-to-all", Capacity and token
    dropping: tokens per batch over experts, times k, times the factor).  The
    pages leave the rounding open; the ceiling keeps every slot the formula
    grants.  Evaluated exactly in rational arithmetic, the factor taken as the
    decimal it prints as (1.1 is 11/10, not the nearest binary double)."""
    from fractions import Fraction
    q = Fraction(int(T) * int(k), int(E)) * Fraction(repr(float(factor)))
    return int(-((-q.numerator) // q.denominator))


def dispatch(ids: np.ndarray, E: int, cap: int | None = None) -> dict:
    """Pairs p = t*k + j grouped by expert (index order), ascending p inside;
    with ``cap`` each expert keeps its first ``cap`` pairs in that order and
    the rest are dropped (pair_pos -1, sorted_pairs -1 past the kept pairs)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sp = np.empty(T * k, dtype=np.int32)
    pp = np.empty(T * k, dtype=np.int32)
    rc = lib().oracle_dispatch(T, k, E, -1 if cap is None else int(cap), ids.ctypes.data,
                               counts.ctypes.data, offsets.ctypes.data, sp.ctypes.data,
                               pp.ctypes.data)
    if rc:
        raise ValueError(f"oracle_dispatch failed ({rc})")
    return dict(counts=counts, offsets=offsets, sorted_pairs=sp, pair_pos=pp)


def router_stats(scores: np.ndarray, ids: np.ndarray, score_fn: int = SOFTMAX,
                 alpha: float = 1.0, cap: int | None = None) -> dict:
    """Load-balancing statistics of one batch ("8.6 Mixture of Experts",
    sec. 3.1; "from the router to the all-to-all", Load balancing; "T2.6 --
    What Mixture of Experts Changes", In practice: per-expert counts,
    maximum-to-mean load and capacity overflow):
      f_e = n_e / T, with n_e the pairs routed to expert e (before any
            capacity drop); sum_e f_e = k;
      P_e = mean over tokens of the router probability of e: the softmax
            score, or the sigmoid score normalised over all experts;
      L_aux = alpha * E * sum_e f_e P_e (= alpha under uniform routing, k = 1);
      max_over_mean = max_e n_e / mean_e n_e;
      overflow = pairs an expert capacity ``cap`` drops, sum_e max(0, n_e - cap)
            (0 without a capacity)."""
    scores = np.asarray(scores, dtype=np.float64)
    T, E = scores.shape
    ids = np.asarray(ids)
    n = np.zeros(E, dtype=np.float64)
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            n[ids[t, j]] += 1.0
    prob = scores if score_fn == SOFTMAX else scores / scores.sum(1, keepdims=True)
    f = n / T
    P = prob.sum(0) / T
    l_aux = alpha * E * float(np.sum(f * P))
    overflow = 0.0
    if cap is not None:
        for e in range(E):
            if n[e] > cap:
                overflow += n[e] - cap
    return dict(f=f, P=P, l_aux=l_aux, max_over_mean=float(n.max() / n.mean()), counts=n,
                overflow=overflow)


def aux_loss_logit_grad(lg: np.ndarray, ids: np.ndarray, score_fn: int = SOFTMAX,
                        alpha: float = 1.0) -> np.ndarray:
    """dL_aux/dl [T,E] for the load-balancing loss of router_stats,
    L_aux = alpha E sum_e f_e P_e ("8.6 Mixture of Experts", sec. 3.1: f_e
    counts the hard assignment and carries no gradient, so the loss trains the
    router through P_e alone).  With p_t the router probabilities of token t
    (softmax over the logits, or the sigmoids normalised over the experts) and
    P_e = (1/T) sum_t p_te:
        dL_aux/dl_te' = (alpha E / T) sum_e f_e dp_te/dl_te',
    the Jacobian written out: softmax dp_e/dl_e' = p_e (delta_ee' - p_e');
    normalised sigmoid p_e = s_e / S, s = sigmoid(l), S = sum s, by the
    quotient rule dp_e/dl_e' = (delta_ee' s_e (1 - s_e) S - s_e s_e' (1 - s_e')) / S^2."""
    lg = np.asarray(lg, dtype=np.float64)
    T, E = lg.shape
    n = np.zeros(E)
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            n[ids[t, j]] += 1.0
    f = n / T
    out = np.empty((T, E))
    for t in range(T):
        if score_fn == SOFTMAX:
            p = np.exp(lg[t] - lg[t].max())
            p /= p.sum()
            J = np.diag(p) - np.outer(p, p)
        else:
            sg = 1.0 / (1.0 + np.exp(-lg[t]))
            S = sg.sum()
            ds = sg * (1.0 - sg)
            J = (np.diag(ds) * S - np.outer(sg, ds)) / (S * S)
        out[t] = alpha * E / T * (f @ J)
    return out


def expert_rows(e: int, x: np.ndarray, rows: np.ndarray, w_gate, w_up, w_down,
                want_h: bool = False, nthreads: int | None = None):
    """Expert e's SwiGLU on token rows ``rows``: (h [n,d_ff] or None, o [n,d])."""
    x, w_gate, w_up, w_down = _c(x), _c(w_gate), _c(w_up), _c(w_down)
    d = x.shape[1]
    f = w_gate.shape[-2]
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    n = rows.size
    h = np.empty((n, f), dtype=np.float64) if want_h else None
    o = np.empty((n, d), dtype=np.float64)
    lib().oracle_expert_rows(d, f, e, x.ctypes.data, _dtype_of(x), rows.ctypes.data, n,
                             w_gate.ctypes.data, w_up.ctypes.data, w_down.ctypes.data, _ptr(h),
                             o.ctypes.data, nthreads or _nthreads())
    return h, o


def forward_tokens(inp: dict, k: int, tokens, score_fn: int = SOFTMAX, renormalize: int = 1,
                   forced_ids: np.ndarray | None = None, bias: np.ndarray | None = None,
                   nthreads: int | None = None, bias_on_scores: int = 0,
                   keep: np.ndarray | None = None) -> dict:
    """y for the listed tokens, token by token: y = sum_j g_j f_{id_j}(x) (+ f_s(x)),
    skipping the pairs that ``keep`` [n,k] marks 0 (dropped for capacity)."""
    x = _c(inp["x"])
    wr, wg, wu, wd = (_c(inp[n]) for n in ("w_router", "w_gate", "w_up", "w_down"))
    sg, su, sd = (_c(inp.get(n)) for n in ("ws_gate", "ws_up", "ws_down"))
    T, d = x.shape
    E = wr.shape[0]
    f = wg.shape[-2]
    S = 0 if sg is None else 1
    f_s = 0 if sg is None else sg.shape[0]
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    n = tokens.size
    if n and (tokens.min() < 0 or tokens.max() >= T):
        raise ValueError("token index out of range")
    y = np.empty((n, d), dtype=np.float64)
    ids = np.empty((n, k), dtype=np.int32)
    gates = np.empty((n, k), dtype=np.float64)
    fi = None if forced_ids is None else np.ascontiguousarray(forced_ids, dtype=np.int32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
    kp = None if keep is None else np.ascontiguousarray(keep, dtype=np.int32)
    rc = lib().oracle_forward_tokens(d, E, k, f, S, f_s, score_fn, renormalize, _dtype_of(x),
                                     x.ctypes.data, wr.ctypes.data, wg.ctypes.data,
                                     wu.ctypes.data, wd.ctypes.data, _ptr(sg), _ptr(su), _ptr(sd),
                                     _ptr(b), int(bias_on_scores), tokens.ctypes.data, n, _ptr(fi),
                                     _ptr(kp), y.ctypes.data, ids.ctypes.data, gates.ctypes.data,
                                     nthreads or _nthreads())
    if rc:
        raise ValueError(f"oracle_forward_tokens failed ({rc})")
    return dict(y=y, ids=ids, gates=gates)


def forward_expert_loop(inp: dict, ids: np.ndarray, gates: np.ndarray,
                        nthreads: int | None = None) -> np.ndarray:
    """y [T,d] by looping over experts and the tokens that chose each."""
    x = _c(inp["x"])
    wg, wu, wd = (_c(inp[n]) for n in ("w_gate", "w_up", "w_down"))
    sg, su, sd = (_c(inp.get(n)) for n in ("ws_gate", "ws_up", "ws_down"))
    T, d = x.shape
    E, f = wg.shape[0], wg.shape[1]
    k = ids.shape[1]
    S = 0 if sg is None else 1
    f_s = 0 if sg is None else sg.shape[0]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    gates = np.ascontiguousarray(gates, dtype=np.float64)
    y = np.empty((T, d), dtype=np.float64)
    lib().oracle_forward_expert_loop(T, d, E, k, f, S, f_s, _dtype_of(x), x.ctypes.data,
                                     wg.ctypes.data, wu.ctypes.data, wd.ctypes.data, _ptr(sg),
                                     _ptr(su), _ptr(sd), ids.ctypes.data, gates.ctypes.data,
                                     y.ctypes.data, nthreads or _nthreads())
    return y


def forward(inp: dict, k: int, score_fn: int = SOFTMAX, renormalize: int = 1,
            bias: np.ndarray | None = None, nthreads: int | None = None) -> dict:
    """Whole layer for all tokens: routing, dispatch and y (expert-loop form)."""
    lg = logits(inp["x"], inp["w_router"], nthreads=nthreads)
    r = route(lg, k, score_fn, renormalize, bias=bias, nthreads=nthreads)
    E = inp["w_router"].shape[0]
    disp = dispatch(r["ids"], E)
    y = forward_expert_loop(inp, r["ids"], r["gates"], nthreads=nthreads)
    return dict(logits=lg, y=y, **r, **disp)


def backward(inp: dict, ids: np.ndarray, dy: np.ndarray, score_fn: int = SOFTMAX,
             renormalize: int = 1, weights: bool = True, keep=None, aux_alpha: float = 0.0) -> dict:
    """Gradients of L = sum(dy * y) for the routing ``ids`` [T,k] (held fixed):
    dx, dw_router, dw_gate, dw_up, dw_down (and ds_gate, ds_up, ds_down with a
    shared expert), fp64, by the chain rule written out per token.  With
    weights=False only dx (each token's row depends on that token alone).
    keep [T,k] (bool, optional): False marks pairs an expert capacity dropped
    (as in forward_tokens), which add nothing to y.  aux_alpha != 0 adds the
    gradient of the load-balancing loss L_aux (router_stats, same alpha) to dx
    and dw_router: dl_aux = aux_loss_logit_grad, dx += dl_aux W_r,
    dw_router += dl_aux^T x."""
    x = _c(inp["x"])
    wr, wg, wu, wd = (_c(inp[n]) for n in ("w_router", "w_gate", "w_up", "w_down"))
    sg, su, sd = (_c(inp.get(n)) for n in ("ws_gate", "ws_up", "ws_down"))
    T, d = x.shape
    E, f = wg.shape[0], wg.shape[1]
    k = ids.shape[1]
    S = 0 if sg is None else 1
    f_s = 0 if sg is None else sg.shape[0]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    out = dict(dx=np.empty((T, d)))
    if weights:
        out.update(dw_router=np.empty((E, d)), dw_gate=np.empty((E, f, d)), dw_up=np.empty((E, f, d)),
                   dw_down=np.empty((E, d, f)))
    if S and weights:
        out.update(ds_gate=np.empty((f_s, d)), ds_up=np.empty((f_s, d)), ds_down=np.empty((d, f_s)))
    wp = (lambda n: out[n].ctypes.data) if weights else (lambda n: None)
    kp = None if keep is None else np.ascontiguousarray(np.asarray(keep).reshape(T, k), dtype=np.int32)
    rc = lib().oracle_backward(T, d, E, k, f, S, f_s, score_fn, renormalize, _dtype_of(x), x.ctypes.data,
                               wr.ctypes.data, wg.ctypes.data, wu.ctypes.data, wd.ctypes.data, _ptr(sg),
                               _ptr(su), _ptr(sd), ids.ctypes.data, dy.ctypes.data,
                               out["dx"].ctypes.data, *(wp(n) for n in ("dw_router", "dw_gate", "dw_up", "dw_down")),
                               *((wp(n) for n in ("ds_gate", "ds_up", "ds_down")) if S else (None,) * 3),
                               None if kp is None else kp.ctypes.data)
    if rc:
        raise ValueError(f"oracle_backward failed ({rc})")
    if aux_alpha:
        dl = aux_loss_logit_grad(logits(x, wr), ids, score_fn, aux_alpha)
        out["dx"] += dl @ _f64(wr)
        if weights:
            out["dw_router"] += dl.T @ _f64(x)
    return out


WEIGHT_SAMPLE_KINDS = ("dw_gate", "dw_up", "dw_down", "ds_gate", "ds_up", "ds_down")


def backward_weight_samples(inp: dict, ids: np.ndarray, dy: np.ndarray, samples, score_fn: int = SOFTMAX,
                            renormalize: int = 1) -> np.ndarray:
    """Single elements of the weight gradients of ``backward``, each summed over
    its expert's pairs (all tokens for the shared expert), for checking
    full-size layers on a sample.  samples: (name, e, i, j) with name in
    WEIGHT_SAMPLE_KINDS, the element being grad[name][e][i][j] (routed) or
    grad[name][i][j] (shared; e ignored)."""
    x = _c(inp["x"])
    wr, wg, wu, wd = (_c(inp[n]) for n in ("w_router", "w_gate", "w_up", "w_down"))
    sg, su, sd = (_c(inp.get(n)) for n in ("ws_gate", "ws_up", "ws_down"))
    T, d = x.shape
    E, f = wg.shape[0], wg.shape[1]
    k = ids.shape[1]
    f_s = 0 if sg is None else sg.shape[0]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    kind, eidx, ridx, cidx = [], [], [], []
    for name, e, i, j in samples:
        kd = WEIGHT_SAMPLE_KINDS.index(name)
        if kd >= 3 and sg is None:
            raise ValueError(f"{name}: the layer has no shared expert")
        # the oracle takes (row r of the inner width, column c of the model width)
        down = name in ("dw_down", "ds_down")
        r, c = (j, i) if down else (i, j)
        kind.append(kd); eidx.append(e); ridx.append(r); cidx.append(c)
    arr = [np.ascontiguousarray(v, dtype=np.int32) for v in (kind, eidx, ridx, cidx)]
    out = np.empty(len(kind))
    rc = lib().oracle_backward_weight_samples(T, d, E, k, f, f_s, score_fn, renormalize, _dtype_of(x),
                                              x.ctypes.data, wr.ctypes.data, wg.ctypes.data, wu.ctypes.data,
                                              wd.ctypes.data, _ptr(sg), _ptr(su), _ptr(sd), ids.ctypes.data,
                                              dy.ctypes.data, len(kind), *(a.ctypes.data for a in arr),
                                              out.ctypes.data)
    if rc:
        raise ValueError(f"oracle_backward_weight_samples failed ({rc})")
    return out
