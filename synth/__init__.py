"""Seeded synthetic inputs for the top-k MoE FFN layer.

This package is the only code shared by the CPU oracle's tests and the GPU
path's tests and benchmark.  It holds none of the layer's arithmetic: it draws
Gaussian tensors with a counter-based generator (``synth.c``), and describes
the five layer shapes the inputs are drawn for.

Layer shapes (the pages' workloads, drawn synthetically):

* ``tiny``            -- T=64, d=64, E=8, k=2, d_ff=128, fp32, softmax + renorm.
* ``mixtral_prefill`` -- Mixtral-8x7B-shaped: T=4096, d=4096, E=8, k=2,
  d_ff=14336, bf16, softmax + renorm, router weights scaled by 4.
* ``mixtral_decode``  -- the same layer at T=32 (weight-read bound).
* ``hunyuan_a13b``    -- T=8192, d=4096, E=64, k=8, d_ff=3072, bf16, softmax over
  64 then renorm over 8; expert popularity skewed Zipf(1.1) through a shift of
  the token vectors (``zipf_shift``).
* ``deepseek_v3``     -- T=8192, d=7168, E=256, k=8, d_ff=2048, sigmoid scores
  normalised over the 8 chosen, plus one always-on shared SwiGLU expert of
  width 2048, bf16.

Weights are N(0, 1/fan_in); token vectors are N(0, 1).  bf16 tensors are
handled as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# Tensor ids: each tensor draws from its own Philox key.
TID_X, TID_WR, TID_WGATE, TID_WUP, TID_WDOWN = 0, 1, 2, 3, 4
TID_SGATE, TID_SUP, TID_SDOWN, TID_ZIPF_PERM = 5, 6, 7, 8

SOFTMAX, SIGMOID = 0, 1
F32, BF16 = 0, 1


def build(verbose: bool = False) -> str:
    """Compile ``libsynth.so`` with gcc (OpenMP)."""
    src = os.path.join(_HERE, "synth.c")
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC", src,
           "-o", _LIB_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, u32, i32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p
        L.synth_normal.argtypes = [u64, u32, u64, u64, ctypes.c_double, vp, i32, vp, i32]
        L.synth_normal.restype = None
        L.synth_normal_rows.argtypes = [u64, u32, u64, u64, u64, u64, ctypes.c_double, vp, i32, vp, i32]
        L.synth_normal_rows.restype = None
        L.synth_u32.argtypes = [u64, u32, u64, u64, vp]
        L.synth_u32.restype = None
        L.synth_philox_block.argtypes = [u32, u32, vp, vp]
        L.synth_philox_block.restype = None
        _lib = L
    return _lib


def nthreads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def philox_block(k0: int, k1: int, ctr) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().synth_philox_block(k0, k1, c.ctypes.data, out.ctypes.data)
    return out


def normal(seed: int, tid: int, n: int, sigma: float, dtype: int, first: int = 0,
           add: np.ndarray | None = None, out: np.ndarray | None = None) -> np.ndarray:
    """Elements [first, first+n) of tensor ``tid``: sigma*z (+add), rounded."""
    npdt = np.float32 if dtype == F32 else np.uint16
    if out is None:
        out = np.empty(n, dtype=npdt)
    assert out.dtype == npdt and out.size == n and out.flags.c_contiguous
    addp = None
    if add is not None:
        add = np.ascontiguousarray(add, dtype=np.float64)
        assert add.size == n
        addp = add.ctypes.data
    lib().synth_normal(seed, tid, first, n, float(sigma), addp, dtype, out.ctypes.data, nthreads())
    return out


def normal_rows(seed: int, tid: int, first: int, nrows: int, row_len: int, row_stride: int,
                sigma: float, dtype: int, add_row: np.ndarray | None = None,
                out: np.ndarray | None = None) -> np.ndarray:
    """Rows r=0..nrows-1 of length row_len starting at first + r*row_stride."""
    npdt = np.float32 if dtype == F32 else np.uint16
    if out is None:
        out = np.empty((nrows, row_len), dtype=npdt)
    assert out.dtype == npdt and out.size == nrows * row_len and out.flags.c_contiguous
    addp = None
    if add_row is not None:
        add_row = np.ascontiguousarray(add_row, dtype=np.float64)
        assert add_row.size == row_len
        addp = add_row.ctypes.data
    lib().synth_normal_rows(seed, tid, first, nrows, row_len, row_stride, float(sigma), addp,
                            dtype, out.ctypes.data, nthreads())
    return out


def u32(seed: int, tid: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    lib().synth_u32(seed, tid, first, n, out.ctypes.data)
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One MoE layer workload: shapes, scoring and the input distributions."""
    name: str
    T: int
    d: int
    E: int
    k: int
    d_ff: int
    num_shared: int = 0
    d_ff_shared: int = 0
    score_fn: int = SOFTMAX
    renormalize: int = 1
    dtype: int = BF16
    router_scale: float = 1.0     # router weights ~ N(0, (router_scale^2)/d)
    zipf_s: float = 0.0           # > 0: skew popularity Zipf(zipf_s) via a token shift
    zipf_tau: float = 0.6

    def replace(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def npdtype(self):
        return np.float32 if self.dtype == F32 else np.uint16

    # sigmas: weights ~ N(0, 1/fan_in)
    @property
    def sigma_router(self) -> float:
        return self.router_scale / np.sqrt(self.d)

    @property
    def sigma_in(self) -> float:
        return 1.0 / np.sqrt(self.d)

    @property
    def sigma_down(self) -> float:
        return 1.0 / np.sqrt(self.d_ff)

    @property
    def sigma_sdown(self) -> float:
        return 1.0 / np.sqrt(self.d_ff_shared) if self.d_ff_shared else 0.0

    def flops(self) -> float:
        """Algorithmic FLOPs: router 2TdE, 6 d d_ff per routed pair, 6 d d_ff_s per token."""
        return (2.0 * self.T * self.d * self.E + 6.0 * self.d * self.d_ff * self.T * self.k
                + 6.0 * self.d * self.d_ff_shared * self.T * self.num_shared)


SHAPES = {
    "tiny": LayerShape("tiny", T=64, d=64, E=8, k=2, d_ff=128, dtype=F32),
    "mixtral_prefill": LayerShape("mixtral_prefill", T=4096, d=4096, E=8, k=2, d_ff=14336,
                                  router_scale=4.0),
    "mixtral_decode": LayerShape("mixtral_decode", T=32, d=4096, E=8, k=2, d_ff=14336,
                                 router_scale=4.0),
    "hunyuan_a13b": LayerShape("hunyuan_a13b", T=8192, d=4096, E=64, k=8, d_ff=3072,
                               zipf_s=1.1),
    "deepseek_v3": LayerShape("deepseek_v3", T=8192, d=7168, E=256, k=8, d_ff=2048,
                              num_shared=1, d_ff_shared=2048, score_fn=SIGMOID),
}


def zipf_perm_ranks(shape: LayerShape, seed: int) -> np.ndarray:
    """Popularity rank (1 = most popular) of each expert: a seeded permutation."""
    keys = u32(seed, TID_ZIPF_PERM, shape.E)
    order = np.argsort(keys, kind="stable")
    ranks = np.empty(shape.E, dtype=np.int64)
    ranks[order] = np.arange(1, shape.E + 1)
    return ranks


def zipf_shift(shape: LayerShape, w_router_bits: np.ndarray, seed: int) -> np.ndarray:
    """Token-vector shift m (fp64, length d) with W_r m = b, b_e = tau ln p_rank(e).

    p_r = r^-s / H_{E,s}.  Adding m to every token vector adds b to every
    router logit, so popular experts win more often while the router GEMM still
    does all the selecting.  m is the minimum-norm solution, computed in fp64
    from the already-rounded router weights.
    """
    E = shape.E
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-shape.zipf_s)
    p /= p.sum()
    ranks = zipf_perm_ranks(shape, seed)
    b = shape.zipf_tau * np.log(p[ranks - 1])
    W = (bf16_to_f64(w_router_bits) if shape.dtype == BF16
         else w_router_bits.astype(np.float64)).reshape(E, shape.d)
    G = W @ W.T
    return W.T @ np.linalg.solve(G, b)


class Inputs(dict):
    """Host tensors of one layer: x, w_router, w_gate, w_up, w_down (+ ws_*)."""


def make_router_and_x(shape: LayerShape, seed: int = 0):
    """x [T,d] and w_router [E,d] (host)."""
    dt = shape.dtype
    w_r = normal(seed, TID_WR, shape.E * shape.d, shape.sigma_router, dt).reshape(shape.E, shape.d)
    add = zipf_shift(shape, w_r, seed) if shape.zipf_s > 0 else None
    x = normal_rows(seed, TID_X, 0, shape.T, shape.d, shape.d, 1.0, dt, add_row=add)
    return x, w_r


def make_expert_weights(shape: LayerShape, seed: int = 0, experts=None):
    """w_gate, w_up [E?,d_ff,d] and w_down [E?,d,d_ff] for all or some experts."""
    dt = shape.dtype
    E, d, f = shape.E, shape.d, shape.d_ff
    ex = list(range(E)) if experts is None else list(experts)
    npdt = shape.npdtype
    wg = np.empty((len(ex), f, d), dtype=npdt)
    wu = np.empty((len(ex), f, d), dtype=npdt)
    wd = np.empty((len(ex), d, f), dtype=npdt)
    for i, e in enumerate(ex):
        normal(seed, TID_WGATE, f * d, shape.sigma_in, dt, first=e * f * d, out=wg[i].reshape(-1))
        normal(seed, TID_WUP, f * d, shape.sigma_in, dt, first=e * f * d, out=wu[i].reshape(-1))
        normal(seed, TID_WDOWN, d * f, shape.sigma_down, dt, first=e * d * f, out=wd[i].reshape(-1))
    return wg, wu, wd


def make_shared_weights(shape: LayerShape, seed: int = 0):
    if not shape.num_shared:
        return None, None, None
    dt = shape.dtype
    d, f = shape.d, shape.d_ff_shared
    sg = normal(seed, TID_SGATE, f * d, shape.sigma_in, dt).reshape(f, d)
    su = normal(seed, TID_SUP, f * d, shape.sigma_in, dt).reshape(f, d)
    sd = normal(seed, TID_SDOWN, d * f, shape.sigma_sdown, dt).reshape(d, f)
    return sg, su, sd


def make_inputs(shape: LayerShape, seed: int = 0) -> Inputs:
    x, w_r = make_router_and_x(shape, seed)
    wg, wu, wd = make_expert_weights(shape, seed)
    sg, su, sd = make_shared_weights(shape, seed)
    return Inputs(x=x, w_router=w_r, w_gate=wg, w_up=wu, w_down=wd,
                  ws_gate=sg, ws_up=su, ws_down=sd)
