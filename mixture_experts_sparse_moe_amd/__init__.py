"""Top-k Mixture-of-Experts FFN layer forward on MI355X (gfx950).

Thin Python binding of ``libmoe.so`` (C ABI in ``include/moe.h``).  Every
step of the layer runs in the library's HIP kernels; this module only checks
tensor shapes, dtypes and devices on the host and passes device pointers.
PyTorch provides device memory and streams.  There is no fallback: if the
library is missing, importing works but every call raises.

Entry points (same names as the C ABI):
    moe_workspace_bytes, moe_route, moe_dispatch, moe_expert_ffn,
    moe_combine, moe_forward, moe_forward_staged, moe_status_str,
    moe_route_ex, moe_dispatch_ex, moe_forward_ex (with MoeOptions),
    moe_capacity, moe_forward_plan, moe_backward_workspace_bytes, moe_backward,
    moe_backward_ex, moe_forward_noalloc
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH loads another build of the same library (e.g. one compiled with
# different tile options) in place of the in-tree libmoe.so.
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED = -1, -2, -3
MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_HIP = -4, -5, -6
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_F32, MOE_BF16 = 0, 1

EXPORTS = ("moe_workspace_bytes", "moe_status_str", "moe_route", "moe_dispatch",
           "moe_expert_ffn", "moe_combine", "moe_forward", "moe_forward_staged",
           "moe_route_ex", "moe_dispatch_ex", "moe_forward_ex", "moe_capacity",
           "moe_backward_workspace_bytes", "moe_backward", "moe_backward_ex", "moe_forward_noalloc",
           "moe_forward_plan")
NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_NUM_STAGES = 7
STAGE_NAMES = ("route", "dispatch", "gate_up_gemm", "down_gemm", "shared_gate_up", "shared_down",
               "combine")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_status_str(status)} ({status})")


class MoeConfig(ctypes.Structure):
    """Mirror of ``moe_config``."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "d_model", "num_experts", "top_k", "d_ff", "num_shared", "d_ff_shared",
        "score_fn", "renormalize", "dtype")]

    def __repr__(self):
        return "MoeConfig(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"

    @classmethod
    def of(cls, T, d, E, k, d_ff, num_shared=0, d_ff_shared=0, score_fn=MOE_SCORE_SOFTMAX,
           renormalize=1, dtype=MOE_BF16):
        return cls(T, d, E, k, d_ff, num_shared, d_ff_shared, score_fn, renormalize, dtype)


class MoeOptions(ctypes.Structure):
    """Mirror of ``moe_options``: selection-only expert bias, per-expert
    capacity, router statistics.  Build with ``MoeOptions.of(...)``; the
    tensors it points to must stay alive while the call runs."""
    _fields_ = [("expert_bias", ctypes.c_void_p), ("bias_on_scores", ctypes.c_int32),
                ("expert_capacity", ctypes.c_int32), ("router_stats", ctypes.c_void_p),
                ("aux_alpha", ctypes.c_float)]

    @classmethod
    def of(cls, expert_bias=None, bias_on_scores=0, expert_capacity=0, router_stats=None, aux_alpha=0.0):
        o = cls(_ptr(expert_bias), int(bias_on_scores), int(expert_capacity), _ptr(router_stats),
                float(aux_alpha))
        o._keep = (expert_bias, router_stats)
        return o


def moe_capacity(cfg: "MoeConfig", capacity_factor: float) -> int:
    """Slots per expert for a capacity factor, from the library (moe_capacity)."""
    c = int(lib().moe_capacity(ctypes.byref(cfg), float(capacity_factor)))
    if c < 0:
        raise MoeError(c, "moe_capacity")
    return c


def moe_forward_plan(cfg: "MoeConfig") -> dict:
    """How moe_forward lays the layer out on kernels (moe_forward_plan):
    tile rows of the routed GEMMs, K splits of the routed and the shared down
    GEMMs, and whether the shared expert runs inside the routed launches."""
    out = (ctypes.c_int32 * 4)()
    st = int(lib().moe_forward_plan(ctypes.byref(cfg), out))
    if st != MOE_OK:
        raise MoeError(st, "moe_forward_plan")
    return dict(tile_rows=out[0], routed_splits=out[1], shared_splits=out[2], shared_merged=bool(out[3]))


def capacity(T: int, k: int, E: int, factor: float) -> int:
    """moe_capacity for a layer of T tokens, top-k of E experts."""
    return moe_capacity(MoeConfig.of(T, 64, E, k, 64), factor)


_lib = None


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m mixture_experts_sparse_moe_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        cfgp = ctypes.POINTER(MoeConfig)
        L.moe_workspace_bytes.argtypes = [cfgp]
        L.moe_workspace_bytes.restype = sz
        L.moe_status_str.argtypes = [i32]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_route.argtypes = [cfgp, vp, vp, vp, vp, vp, vp]
        L.moe_route.restype = i32
        L.moe_dispatch.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_dispatch.restype = i32
        L.moe_expert_ffn.argtypes = [cfgp] + [vp] * 11 + [vp, sz, vp]
        L.moe_expert_ffn.restype = i32
        L.moe_combine.argtypes = [cfgp, vp, vp, vp, vp, vp, vp]
        L.moe_combine.restype = i32
        L.moe_forward.argtypes = [cfgp] + [vp] * 13 + [vp, sz, vp]
        L.moe_forward.restype = i32
        L.moe_forward_staged.argtypes = [cfgp] + [vp] * 13 + [vp, sz, vp, vp, vp]
        L.moe_forward_staged.restype = i32
        optp = ctypes.POINTER(MoeOptions)
        L.moe_route_ex.argtypes = [cfgp, optp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_route_ex.restype = i32
        L.moe_dispatch_ex.argtypes = [cfgp, optp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_dispatch_ex.restype = i32
        L.moe_forward_ex.argtypes = [cfgp, optp] + [vp] * 13 + [vp, sz, vp]
        L.moe_forward_ex.restype = i32
        L.moe_capacity.argtypes = [cfgp, ctypes.c_double]
        L.moe_capacity.restype = i32
        L.moe_forward_plan.argtypes = [cfgp, vp]
        L.moe_forward_plan.restype = i32
        L.moe_forward_noalloc.argtypes = [cfgp] + [vp] * 13 + [vp]
        L.moe_forward_noalloc.restype = i32
        L.moe_backward_workspace_bytes.argtypes = [cfgp]
        L.moe_backward_workspace_bytes.restype = sz
        L.moe_backward.argtypes = [cfgp] + [vp] * 20 + [sz, vp]
        L.moe_backward.restype = i32
        L.moe_backward_ex.argtypes = [cfgp, optp] + [vp] * 20 + [sz, vp]
        L.moe_backward_ex.restype = i32
        _lib = L
    return _lib


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def moe_workspace_bytes(cfg: MoeConfig) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(cfg)))


# ----------------------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _act_dtype(cfg):
    torch = _torch()
    return torch.bfloat16 if cfg.dtype == MOE_BF16 else torch.float32


def _ptr(t):
    return None if t is None else (t.data_ptr() or None)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, name, shape, dtype, device=None, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on the GPU device of x ({device}), got {t.device}")


def _rc(status, where):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ws_bytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def moe_route(cfg, x, w_router, topk_ids, topk_weights, topk_gap=None, stream=None):
    torch = _torch()
    T, d, E, k = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k
    dt, dev = _act_dtype(cfg), x.device
    _check(x, "x", (T, d), dt, dev)
    _check(w_router, "w_router", (E, d), dt, dev)
    _check(topk_ids, "topk_ids", (T, k), torch.int32, dev)
    _check(topk_weights, "topk_weights", (T, k), torch.float32, dev)
    _check(topk_gap, "topk_gap", (T, 2), torch.float32, dev, optional=True)
    _rc(lib().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(topk_ids),
                        _ptr(topk_weights), _ptr(topk_gap), _stream(stream)), "moe_route")


def moe_dispatch(cfg, topk_ids, expert_counts, expert_offsets, sorted_pairs, pair_pos, ws,
                 stream=None):
    torch = _torch()
    T, E, k = cfg.num_tokens, cfg.num_experts, cfg.top_k
    dev = topk_ids.device
    _check(topk_ids, "topk_ids", (T, k), torch.int32, dev)
    _check(expert_counts, "expert_counts", (E,), torch.int32, dev)
    _check(expert_offsets, "expert_offsets", (E + 1,), torch.int32, dev)
    _check(sorted_pairs, "sorted_pairs", (T * k,), torch.int32, dev)
    _check(pair_pos, "pair_pos", (T * k,), torch.int32, dev)
    _rc(lib().moe_dispatch(ctypes.byref(cfg), _ptr(topk_ids), _ptr(expert_counts),
                           _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(pair_pos), _ptr(ws),
                           _ws_bytes(ws), _stream(stream)), "moe_dispatch")


def _check_experts(cfg, dev, w_gate, w_up, w_down, ws_gate, ws_up, ws_down):
    E, d, f, fs = cfg.num_experts, cfg.d_model, cfg.d_ff, cfg.d_ff_shared
    dt = _act_dtype(cfg)
    _check(w_gate, "w_gate", (E, f, d), dt, dev)
    _check(w_up, "w_up", (E, f, d), dt, dev)
    _check(w_down, "w_down", (E, d, f), dt, dev)
    if cfg.num_shared:
        _check(ws_gate, "ws_gate", (fs, d), dt, dev)
        _check(ws_up, "ws_up", (fs, d), dt, dev)
        _check(ws_down, "ws_down", (d, fs), dt, dev)


def moe_expert_ffn(cfg, x, sorted_pairs, expert_offsets, w_gate, w_up, w_down, ws_gate, ws_up,
                   ws_down, expert_out, shared_out, ws, stream=None):
    torch = _torch()
    T, d, E, k = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k
    dt, dev = _act_dtype(cfg), x.device
    _check(x, "x", (T, d), dt, dev)
    _check(sorted_pairs, "sorted_pairs", (T * k,), torch.int32, dev)
    _check(expert_offsets, "expert_offsets", (E + 1,), torch.int32, dev)
    _check_experts(cfg, dev, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    _check(expert_out, "expert_out", (T * k, d), dt, dev)
    _check(shared_out, "shared_out", (T, d), dt, dev, optional=not cfg.num_shared)
    _rc(lib().moe_expert_ffn(ctypes.byref(cfg), _ptr(x), _ptr(sorted_pairs), _ptr(expert_offsets),
                             _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up),
                             _ptr(ws_down), _ptr(expert_out), _ptr(shared_out), _ptr(ws),
                             _ws_bytes(ws), _stream(stream)), "moe_expert_ffn")


def moe_combine(cfg, expert_out, topk_weights, pair_pos, shared_out, y, stream=None):
    torch = _torch()
    T, d, k = cfg.num_tokens, cfg.d_model, cfg.top_k
    dt, dev = _act_dtype(cfg), y.device
    _check(expert_out, "expert_out", (T * k, d), dt, dev)
    _check(topk_weights, "topk_weights", (T, k), torch.float32, dev)
    _check(pair_pos, "pair_pos", (T * k,), torch.int32, dev)
    _check(shared_out, "shared_out", (T, d), dt, dev, optional=not cfg.num_shared)
    _check(y, "y", (T, d), dt, dev)
    _rc(lib().moe_combine(ctypes.byref(cfg), _ptr(expert_out), _ptr(topk_weights), _ptr(pair_pos),
                          _ptr(shared_out), _ptr(y), _stream(stream)), "moe_combine")


def moe_forward(cfg, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y,
                topk_ids=None, topk_weights=None, expert_counts=None, ws=None, stream=None,
                topk_gap=None):
    torch = _torch()
    T, d, E, k = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k
    dt, dev = _act_dtype(cfg), x.device
    _check(x, "x", (T, d), dt, dev)
    _check(w_router, "w_router", (E, d), dt, dev)
    _check_experts(cfg, dev, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    _check(y, "y", (T, d), dt, dev)
    _check(topk_ids, "topk_ids", (T, k), torch.int32, dev, optional=True)
    _check(topk_weights, "topk_weights", (T, k), torch.float32, dev, optional=True)
    _check(expert_counts, "expert_counts", (E,), torch.int32, dev, optional=True)
    _check(topk_gap, "topk_gap", (T, 2), torch.float32, dev, optional=True)
    _rc(lib().moe_forward(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up),
                          _ptr(w_down), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(y),
                          _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_counts), _ptr(topk_gap),
                          _ptr(ws), _ws_bytes(ws), _stream(stream)), "moe_forward")


def moe_forward_noalloc(cfg, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y,
                        topk_ids=None, topk_weights=None, expert_counts=None, topk_gap=None, stream=None):
    """moe_forward without a workspace argument: the library's own fixed
    device array (NOALLOC_SCRATCH_BYTES per GPU) serves as the workspace.
    Layers that need more raise MoeError(MOE_ERR_WORKSPACE); calls that
    overlap on one GPU race on the array."""
    torch = _torch()
    T, d, E, k = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k
    dt, dev = _act_dtype(cfg), x.device
    _check(x, "x", (T, d), dt, dev)
    _check(w_router, "w_router", (E, d), dt, dev)
    _check_experts(cfg, dev, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    _check(y, "y", (T, d), dt, dev)
    _check(topk_ids, "topk_ids", (T, k), torch.int32, dev, optional=True)
    _check(topk_weights, "topk_weights", (T, k), torch.float32, dev, optional=True)
    _check(expert_counts, "expert_counts", (E,), torch.int32, dev, optional=True)
    _check(topk_gap, "topk_gap", (T, 2), torch.float32, dev, optional=True)
    _rc(lib().moe_forward_noalloc(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up),
                                  _ptr(w_down), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(y),
                                  _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_counts), _ptr(topk_gap),
                                  _stream(stream)), "moe_forward_noalloc")


def moe_forward_staged(cfg, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y,
                       topk_ids=None, topk_weights=None, expert_counts=None, ws=None,
                       start_event=None, stage_events=None, stream=None, topk_gap=None):
    """moe_forward recording ``start_event`` and one event per stage (torch.cuda.Event
    objects created with enable_timing=True, or raw hipEvent_t handles) on the stream."""
    torch = _torch()
    T, d, E, k = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k
    dt, dev = _act_dtype(cfg), x.device
    _check(x, "x", (T, d), dt, dev)
    _check(w_router, "w_router", (E, d), dt, dev)
    _check_experts(cfg, dev, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    _check(y, "y", (T, d), dt, dev)
    _check(topk_ids, "topk_ids", (T, k), torch.int32, dev, optional=True)
    _check(topk_weights, "topk_weights", (T, k), torch.float32, dev, optional=True)
    _check(expert_counts, "expert_counts", (E,), torch.int32, dev, optional=True)
    _check(topk_gap, "topk_gap", (T, 2), torch.float32, dev, optional=True)
    if stage_events is not None and len(stage_events) != MOE_NUM_STAGES:
        raise ValueError(f"stage_events needs {MOE_NUM_STAGES} events")

    def ev_handle(e):
        if e is None or isinstance(e, int):     # a raw hipEvent_t handle
            return e
        if not e.cuda_event:        # torch creates its events on first record
            e.record()
        return e.cuda_event

    evs = None
    if stage_events is not None:
        evs = (ctypes.c_void_p * MOE_NUM_STAGES)(*[ev_handle(e) for e in stage_events])
    _rc(lib().moe_forward_staged(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(w_gate),
                                 _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up),
                                 _ptr(ws_down), _ptr(y), _ptr(topk_ids), _ptr(topk_weights),
                                 _ptr(expert_counts), _ptr(topk_gap), _ptr(ws), _ws_bytes(ws),
                                 ev_handle(start_event), evs, _stream(stream)),
        "moe_forward_staged")


def _opts(opts):
    return None if opts is None else ctypes.byref(opts)


def _check_opts(cfg, opts, dev):
    if opts is None:
        return
    torch = _torch()
    b, st = opts._keep if hasattr(opts, "_keep") else (None, None)
    _check(b, "expert_bias", (cfg.num_experts,), torch.float32, dev, optional=True)
    _check(st, "router_stats", (2 * cfg.num_experts + 3,), torch.float32, dev, optional=True)


def moe_route_ex(cfg, opts, x, w_router, topk_ids, topk_weights, topk_gap=None, ws=None, stream=None):
    torch = _torch()
    T, d, E, k = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k
    dt, dev = _act_dtype(cfg), x.device
    _check(x, "x", (T, d), dt, dev)
    _check(w_router, "w_router", (E, d), dt, dev)
    _check(topk_ids, "topk_ids", (T, k), torch.int32, dev)
    _check(topk_weights, "topk_weights", (T, k), torch.float32, dev)
    _check(topk_gap, "topk_gap", (T, 2), torch.float32, dev, optional=True)
    _check_opts(cfg, opts, dev)
    _rc(lib().moe_route_ex(ctypes.byref(cfg), _opts(opts), _ptr(x), _ptr(w_router), _ptr(topk_ids),
                           _ptr(topk_weights), _ptr(topk_gap), _ptr(ws), _ws_bytes(ws), _stream(stream)),
        "moe_route_ex")


def moe_dispatch_ex(cfg, opts, topk_ids, expert_counts, expert_offsets, sorted_pairs, pair_pos, ws,
                    stream=None):
    torch = _torch()
    T, E, k = cfg.num_tokens, cfg.num_experts, cfg.top_k
    dev = topk_ids.device
    _check(topk_ids, "topk_ids", (T, k), torch.int32, dev)
    _check(expert_counts, "expert_counts", (E,), torch.int32, dev)
    _check(expert_offsets, "expert_offsets", (E + 1,), torch.int32, dev)
    _check(sorted_pairs, "sorted_pairs", (T * k,), torch.int32, dev)
    _check(pair_pos, "pair_pos", (T * k,), torch.int32, dev)
    _check_opts(cfg, opts, dev)
    _rc(lib().moe_dispatch_ex(ctypes.byref(cfg), _opts(opts), _ptr(topk_ids), _ptr(expert_counts),
                              _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(pair_pos), _ptr(ws),
                              _ws_bytes(ws), _stream(stream)), "moe_dispatch_ex")


def moe_forward_ex(cfg, opts, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, y,
                   topk_ids=None, topk_weights=None, expert_counts=None, ws=None, stream=None,
                   topk_gap=None):
    torch = _torch()
    T, d, E, k = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k
    dt, dev = _act_dtype(cfg), x.device
    _check(x, "x", (T, d), dt, dev)
    _check(w_router, "w_router", (E, d), dt, dev)
    _check_experts(cfg, dev, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    _check(y, "y", (T, d), dt, dev)
    _check(topk_ids, "topk_ids", (T, k), torch.int32, dev, optional=True)
    _check(topk_weights, "topk_weights", (T, k), torch.float32, dev, optional=True)
    _check(expert_counts, "expert_counts", (E,), torch.int32, dev, optional=True)
    _check(topk_gap, "topk_gap", (T, 2), torch.float32, dev, optional=True)
    _check_opts(cfg, opts, dev)
    _rc(lib().moe_forward_ex(ctypes.byref(cfg), _opts(opts), _ptr(x), _ptr(w_router), _ptr(w_gate),
                             _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(y),
                             _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_counts), _ptr(topk_gap),
                             _ptr(ws), _ws_bytes(ws), _stream(stream)), "moe_forward_ex")


def moe_backward_workspace_bytes(cfg: MoeConfig) -> int:
    return int(lib().moe_backward_workspace_bytes(ctypes.byref(cfg)))


def _check_backward(cfg, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, dy, topk_ids,
                    topk_weights, dx, dw_router, dw_gate, dw_up, dw_down, dws_gate, dws_up, dws_down):
    torch = _torch()
    T, d, E, k, f, fs = cfg.num_tokens, cfg.d_model, cfg.num_experts, cfg.top_k, cfg.d_ff, cfg.d_ff_shared
    dt, dev = _act_dtype(cfg), x.device
    f32 = torch.float32
    _check(x, "x", (T, d), dt, dev)
    _check(w_router, "w_router", (E, d), dt, dev)
    _check_experts(cfg, dev, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    _check(dy, "dy", (T, d), dt, dev)
    _check(topk_ids, "topk_ids", (T, k), torch.int32, dev)
    _check(topk_weights, "topk_weights", (T, k), f32, dev)
    _check(dx, "dx", (T, d), f32, dev)
    _check(dw_router, "dw_router", (E, d), f32, dev)
    _check(dw_gate, "dw_gate", (E, f, d), f32, dev)
    _check(dw_up, "dw_up", (E, f, d), f32, dev)
    _check(dw_down, "dw_down", (E, d, f), f32, dev)
    if cfg.num_shared:
        _check(dws_gate, "dws_gate", (fs, d), f32, dev)
        _check(dws_up, "dws_up", (fs, d), f32, dev)
        _check(dws_down, "dws_down", (d, fs), f32, dev)
    return dev


def moe_backward(cfg, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, dy, topk_ids,
                 topk_weights, dx, dw_router, dw_gate, dw_up, dw_down, dws_gate=None, dws_up=None,
                 dws_down=None, ws=None, stream=None):
    """Gradients (fp32) of the layer for the forward's routing."""
    _check_backward(cfg, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, dy, topk_ids, topk_weights,
                    dx, dw_router, dw_gate, dw_up, dw_down, dws_gate, dws_up, dws_down)
    _rc(lib().moe_backward(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                           _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(dy), _ptr(topk_ids),
                           _ptr(topk_weights), _ptr(dx), _ptr(dw_router), _ptr(dw_gate), _ptr(dw_up),
                           _ptr(dw_down), _ptr(dws_gate), _ptr(dws_up), _ptr(dws_down), _ptr(ws),
                           _ws_bytes(ws), _stream(stream)), "moe_backward")


def moe_backward_ex(cfg, opts, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, dy, topk_ids,
                    topk_weights, dx, dw_router, dw_gate, dw_up, dw_down, dws_gate=None, dws_up=None,
                    dws_down=None, ws=None, stream=None):
    """moe_backward for a forward that ran with options: an expert capacity
    leaves the dropped pairs without gradient (opts.expert_capacity is the one
    field it reads; router_stats must be unset)."""
    dev = _check_backward(cfg, x, w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, dy, topk_ids,
                          topk_weights, dx, dw_router, dw_gate, dw_up, dw_down, dws_gate, dws_up, dws_down)
    _check_opts(cfg, opts, dev)
    _rc(lib().moe_backward_ex(ctypes.byref(cfg), _opts(opts), _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up),
                              _ptr(w_down), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(dy), _ptr(topk_ids),
                              _ptr(topk_weights), _ptr(dx), _ptr(dw_router), _ptr(dw_gate), _ptr(dw_up),
                              _ptr(dw_down), _ptr(dws_gate), _ptr(dws_up), _ptr(dws_down), _ptr(ws),
                              _ws_bytes(ws), _stream(stream)), "moe_backward_ex")


def alloc_backward_workspace(cfg, device="cuda"):
    """A device byte buffer of moe_backward_workspace_bytes(cfg) bytes."""
    n = moe_backward_workspace_bytes(cfg)
    if n == 0:
        raise ValueError(f"invalid config {cfg}")
    return _torch().empty(n, dtype=_torch().uint8, device=device)


def alloc_workspace(cfg, device="cuda"):
    """A device byte buffer of moe_workspace_bytes(cfg) bytes."""
    n = moe_workspace_bytes(cfg)
    if n == 0 and cfg.num_tokens != 0:
        raise ValueError(f"invalid config {cfg}")
    return _torch().empty(max(n, 256), dtype=_torch().uint8, device=device)
