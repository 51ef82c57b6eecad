"""Benchmark of the top-k MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--only]

One step = one whole forward of the layer (route, dispatch, routed SwiGLU
grouped GEMMs, shared expert, combine) over one batch of seeded synthetic
inputs already resident in HBM.  The headline workload is the DeepSeek-V3-
shaped layer (T=8192, d=7168, E=256, k=8, sigmoid gates renormalised over the
8 chosen, d_ff=2048, one shared expert of 2048, bf16), the largest of the five
layer shapes; the other four (the tiny fp32 layer, Mixtral-8x7B prefill and
decode, Hunyuan-A13B) are measured the same way in the same run and reported
as sub-records under "configs" (--only skips them).

Prints one JSON line: throughput (tokens/s), the roofline of the dominant
kernel (the routed gate/up GEMM) measured live with HIP events on the launch
stream, bound by the larger of its HBM and MFMA floors with the other
fraction reported beside it, and the CPU oracle timed on a bounded sample of
the same workload on the host cores; the oracle's outputs on that sample also
give the parity of the timed output.  The timed region records two timing
events per step, the gate/up kernel's own launch events (created without the
system-scope fence, so recording them costs the next kernel nothing
measurable); the per-stage breakdown comes from a separate pass with an
event after every stage.

Other modes: --copy-calibration and --traffic-from (HBM bytes of the gate/up
kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE runs), --counters-from (MFMA
busy fraction and clock per kernel from a rocprofv3 --pmc run).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
HEADLINE = "deepseek_v3"
OTHERS = ("mixtral_prefill", "mixtral_decode", "hunyuan_a13b", "tiny")
TAU = {"bf16": 2e-2, "f32": 1e-4}     # max|err| <= tau * max|y|


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--only", action="store_true", help="measure the --workload alone (no sub-records)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="target wall time of the CPU oracle sample of each workload")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the practical ceilings (device copy, torch.matmul yardstick)")
    p.add_argument("--no-options", action="store_true",
                   help="skip timing the layer with its optional routing features")
    p.add_argument("--no-backward", action="store_true",
                   help="skip timing the backward pass (moe_backward)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device copy of 1 GiB (the reference for HBM counters)")
    p.add_argument("--traffic-from", nargs=4, metavar=("READ_DIR", "WRITE_DIR", "COPY_READ_DIR", "COPY_WRITE_DIR"),
                   help="rocprofv3 --pmc output dirs: TCC_EA0_RDREQ_32B/64B/128B_sum and WRITE_SIZE runs "
                        "of the bench, the same two of --copy-calibration; writes profiles/traffic.json "
                        "for --workload")
    p.add_argument("--trace-summary", metavar="TRACE_DIR",
                   help="markdown table of a rocprofv3 --kernel-trace --stats run (its kernel_stats.csv)")
    p.add_argument("--counters-from", metavar="PMC_DIR",
                   help="summarise a rocprofv3 --pmc run of SQ_VALU_MFMA_BUSY_CYCLES, "
                        "SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE per kernel")
    return p.parse_args()


class TimingEvents:
    """HIP events for timing only, created with hipEventDisableSystemFence:
    recording one skips the system-scope cache write-back and invalidation
    that a default event performs, which would otherwise slow the next
    kernel.  Uses the HIP runtime already loaded in this process."""
    FLAG = 0x20000000   # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        path = next(ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln)
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.made = []

    def make(self, n, stream):
        out = []
        for _ in range(n):
            ev = self.ct.c_void_p()
            if self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.FLAG) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            # record once outside any timed region
            self.hip.hipEventRecord(ev, self.ct.c_void_p(stream.cuda_stream))
            out.append(ev.value)
        self.made += out
        return out

    def ms(self, a, b) -> float:
        t = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(t), self.ct.c_void_p(a), self.ct.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(self.ct.c_void_p(e))
        self.made = []


# The sources of the gate/up GEMM kernel and of its launch (tile path, K split).
GATE_UP_SOURCES = ("grouped_gemm.hip", "skinny.h", "device_util.h", "moe_internal.h", "moe_api.cpp")


def kernel_source_hash() -> str:
    """Hash of the gate/up kernel's sources: the traffic counters stay valid
    while it is unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_sparse_moe_amd", "csrc")
    for n in GATE_UP_SOURCES:
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(n.encode() + f.read())
    return h.hexdigest()[:16]


def upload(a: np.ndarray, torch, dev):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def device_tile_rows(counts, d_ff: int, slots: int = 256) -> int:
    """Tile height moe_forward takes on the device for a layer of 640 or
    more rows per expert: 288 when the gate/up GEMM's 288-row tiles take fewer
    rounds of the persistent grid than 256-row ones, a 288-row round weighing
    9/8 (the rule moe_forward_plan documents)."""
    tn = 2 * d_ff // 256
    r = {bm: -(-sum(-(-int(n) // bm) for n in counts) * tn // slots) for bm in (256, 288)}
    return 288 if 9 * r[288] < 8 * r[256] else 256


def algorithmic(sh, counts: np.ndarray, shared_merged: bool = False) -> dict:
    """Algorithmic work of the layer and of its two expert GEMM kernels.

    FLOPs: router 2TdE, routed experts 6 d d_ff per pair (4 in gate/up, 2 in
    down), shared expert 6 d d_ff_s per token.  Bytes: weights of the experts
    actually touched (union read), the router weights, x read once, y written
    once, 8 bytes of routing per pair; per kernel, its weights plus its
    activation input and output.  shared_merged: the two kernels also run the
    shared expert (its weights, T more rows of H and of the down product; x
    is still read once)."""
    w = sh.elem_bytes
    T, d, E, k, f, fs = sh.T, sh.d, sh.E, sh.k, sh.d_ff, sh.d_ff_shared
    touched = int((counts > 0).sum())
    P = T * k
    layer_flops = sh.flops()
    layer_bytes = (E * d * w + touched * 3 * d * f * w + sh.num_shared * 3 * d * fs * w
                   + 2 * T * d * w + P * 8)
    gate_up = dict(flops=4.0 * P * d * f, bytes=touched * 2 * d * f * w + T * d * w + P * f * w)
    down = dict(flops=2.0 * P * d * f, bytes=touched * d * f * w + P * f * w + P * d * w)
    if shared_merged:
        gate_up = dict(flops=gate_up["flops"] + 4.0 * T * d * fs,
                       bytes=gate_up["bytes"] + 2 * d * fs * w + T * fs * w)
        down = dict(flops=down["flops"] + 2.0 * T * d * fs,
                    bytes=down["bytes"] + d * fs * w + T * fs * w + T * d * w)
    return dict(layer_flops=layer_flops, layer_bytes=layer_bytes, gate_up=gate_up, down=down,
                touched=touched, shared_merged=shared_merged)


def options_cost(torch, moe, cfg, d, y, ws, stream, sh, steps: int) -> dict:
    """ms per layer (moe_forward_ex, no per-stage events) with each optional
    routing feature on: a selection-only bias on the scores (N(0, 0.01)),
    capacity factor 1.25, router statistics, and all three; next to the plain
    layer through the same entry point."""
    g = torch.Generator().manual_seed(0)
    bias = (torch.randn(sh.E, generator=g, dtype=torch.float32) * 0.01).to(d["x"].device)
    stats = torch.empty(2 * sh.E + 3, dtype=torch.float32, device=d["x"].device)
    cap = moe.capacity(sh.T, sh.k, sh.E, 1.25)
    variants = {
        "plain": moe.MoeOptions.of(),
        "bias_on_scores": moe.MoeOptions.of(expert_bias=bias, bias_on_scores=1),
        "capacity_1.25": moe.MoeOptions.of(expert_capacity=cap),
        "router_stats": moe.MoeOptions.of(router_stats=stats, aux_alpha=0.01),
        "all": moe.MoeOptions.of(expert_bias=bias, bias_on_scores=1, expert_capacity=cap,
                                 router_stats=stats, aux_alpha=0.01),
    }
    out = {}
    for name, o in variants.items():
        run = lambda: moe.moe_forward_ex(cfg, o, d["x"], d["w_router"], d["w_gate"], d["w_up"],
                                         d["w_down"], d["ws_gate"], d["ws_up"], d["ws_down"], y,
                                         ws=ws, stream=stream)
        for _ in range(2):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        out[name] = round((time.perf_counter() - t0) / steps * 1e3, 4)
    out["capacity"] = cap
    st = stats.cpu().numpy()
    out["l_aux_alpha_0.01"] = float(st[2 * sh.E])
    out["max_over_mean_load"] = float(st[2 * sh.E + 1])
    return out


def backward_cost(torch, moe, cfg, d, sh, stream, steps: int) -> dict:
    """ms per moe_backward for the layer's routing (dy seeded normal), and its
    algorithmic FLOPs: 12 d d_ff per routed pair (data and weight gradients of
    the three expert matrices), 4 d E per token for the router, 12 d d_ff_s per
    token for the shared expert.  The recomputation of the expert
    pre-activations (4 d d_ff per pair) is an implementation cost, not
    counted.  bf16 layers run its GEMMs on bf16 MFMA (roofline: the dense
    bf16 peak), fp32 layers on fp32 FMA (the fp32 vector peak)."""
    import synth
    dev = d["x"].device
    T, E, k, dm, f, fs = sh.T, sh.E, sh.k, sh.d, sh.d_ff, sh.d_ff_shared
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    moe.moe_route(cfg, d["x"], d["w_router"], ids, wts, stream=stream)
    dy = upload(synth.normal(7, 99, T * dm, 1.0, sh.dtype).reshape(T, dm), torch, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dx=torch.empty(T, dm, **f32), dw_router=torch.empty(E, dm, **f32),
             dw_gate=torch.empty(E, f, dm, **f32), dw_up=torch.empty(E, f, dm, **f32),
             dw_down=torch.empty(E, dm, f, **f32))
    if sh.num_shared:
        g.update(dws_gate=torch.empty(fs, dm, **f32), dws_up=torch.empty(fs, dm, **f32),
                 dws_down=torch.empty(dm, fs, **f32))
    ws = moe.alloc_backward_workspace(cfg, dev)
    run = lambda: moe.moe_backward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                                   d["ws_gate"], d["ws_up"], d["ws_down"], dy, ids, wts, g["dx"],
                                   g["dw_router"], g["dw_gate"], g["dw_up"], g["dw_down"], g.get("dws_gate"),
                                   g.get("dws_up"), g.get("dws_down"), ws=ws, stream=stream)
    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    flops = 12.0 * T * k * dm * f + 4.0 * T * dm * E + 12.0 * sh.num_shared * T * dm * fs
    bf16 = sh.dtype == synth.BF16
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    out = {"ms": round(ms, 3), "steps": steps, "alg_flops": flops, "tflops": flops / (ms * 1e-3) / 1e12,
           "bound": "mfma" if bf16 else "alu", "peak_tflops": peak}
    out["frac"] = out["tflops"] / peak
    del g, ws
    return out


def practical_ceilings(torch, dev, sh=None) -> dict:
    """Measured ceilings on the same GPU, next to the nominal peaks: a 1 GiB
    device copy (read + write bytes / time), a 4 GiB streaming read (torch row
    sums of an fp32 [2^18, 4096] tensor: read bytes / time, the writes are
    0.02 %), and one bf16 4096 x 14336 x 4096 torch.matmul (a library
    yardstick only; nothing of the layer uses any of them)."""
    out = {}
    big = torch.empty(READ_BYTES // 4, dtype=torch.float32, device=dev).uniform_().view(-1, 4096)
    for _ in range(3):
        r = big.sum(dim=1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        r = big.sum(dim=1)
    e1.record()
    e1.synchronize()
    out["read_gbs"] = READ_BYTES * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del big, r
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    out["copy_gbs"] = 2 * COPY_BYTES * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    a = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
    b = torch.randn(4096, 14336, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        c = a @ b
    e1.record()
    e1.synchronize()
    out["torch_matmul_bf16_tflops"] = 2.0 * 4096 * 14336 * 4096 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    out["torch_matmul_shape"] = "4096x14336x4096"
    del a, b, c
    if sh is not None and sh.dtype == synth_bf16():
        out["torch_bmm_bf16"] = grouped_yardstick(torch, dev, sh)
    return out


def synth_bf16():
    import synth
    return synth.BF16


def grouped_yardstick(torch, dev, sh) -> dict:
    """The layer's two routed expert products as torch.bmm (hipBLASLt
    batched GEMMs), one batch per routed expert, every expert holding the
    average T k / E rows: [E, M, d] x [E, d, 2 d_ff] (gate and up as one
    product) and [E, M, d_ff] x [E, d_ff, d], both operands contiguous.  The
    routed experts' weight bytes and FLOPs, without the routing's raggedness,
    the gathered rows, SiLU or the shared expert; a library yardstick only."""
    G = sh.E
    M = max(1, sh.T * sh.k // sh.E)
    res = {"groups": G, "rows": M}
    for tag, K, N in (("gate_up", sh.d, 2 * sh.d_ff), ("down", sh.d_ff, sh.d)):
        a = torch.empty(G, M, K, device=dev, dtype=torch.bfloat16).normal_()
        b = torch.empty(G, K, N, device=dev, dtype=torch.bfloat16).normal_(0.0, K ** -0.5)
        for _ in range(2):
            c = torch.bmm(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            c = torch.bmm(a, b)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / 5
        flops = 2.0 * G * M * K * N
        nbytes = 2.0 * G * (M * K + K * N + M * N)
        res[tag] = {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12, "gbs": nbytes / (ms * 1e-3) / 1e9}
        del a, b, c
    return res


def cpu_baseline(sh, inp, target_s: float) -> dict:
    """The oracle as it stands, on a bounded sample of tokens of the same
    layer: the first and the last token and seeded random ones, growing
    until about target_s / 4 to target_s of work.  Returns the rate and, for
    the parity of the timed output, the sampled tokens with the oracle's y
    and ids (its own routing)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    n = max(cores, 2)
    rng = np.random.default_rng(123)
    while True:
        rnd = rng.choice(sh.T, size=min(n, sh.T), replace=False)
        toks = np.unique(np.concatenate([[0, sh.T - 1], rnd]))[:max(n, 2)]
        t0 = time.perf_counter()
        r = oracle.forward_tokens(inp, sh.k, toks, sh.score_fn, sh.renormalize, nthreads=cores)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or toks.size >= sh.T:
            break
        n = int(min(sh.T, max(n * 2, n * (target_s / max(dt, 1e-3)) * 0.8)))
    sample = (f"{toks.size} of {sh.T} tokens (first, last, seeded random), full routing and {sh.k} "
              f"experts" + (" + shared expert" if sh.num_shared else "") + " per token, fp64")
    out = {"value": toks.size / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": sample, "seconds": round(dt, 3)}
    if toks.size >= sh.T:
        # a whole small layer: also on one thread, the per-core rate
        t0 = time.perf_counter()
        oracle.forward_tokens(inp, sh.k, toks, sh.score_fn, sh.renormalize, nthreads=1)
        out["single_thread_value"] = toks.size / (time.perf_counter() - t0)
    return out, (toks, r["y"], r["ids"])


def parity_of(y_gpu: np.ndarray, ids_gpu: np.ndarray, ref, dtype: str) -> dict:
    """max|y_gpu - y_oracle| / max|y_oracle| over the oracle's sampled tokens
    whose GPU routing equals the oracle's (a token routed differently at a
    near-tie is counted, not compared: the tests check those under the
    GPU's ids)."""
    toks, y_ref, ids_ref = ref
    same = (ids_gpu[toks] == ids_ref).all(1)
    yg = y_gpu[toks][same]
    yr = y_ref[same]
    rel = float(np.abs(yg - yr).max() / max(np.abs(yr).max(), 1e-30)) if same.any() else float("nan")
    return {"tokens": int(toks.size), "routing_differs": int((~same).sum()), "max_err_over_max_y": rel,
            "tau": TAU[dtype], "ok": bool(rel <= TAU[dtype])}


COPY_BYTES = 1 << 30
READ_BYTES = 4 << 30        # streaming-read ceiling


def copy_calibration():
    """A plain 1 GiB device-to-device copy: the HBM counters must read 1 GiB
    fetched and 1 GiB written for it (a check of the byte formulas)."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES}), flush=True)


# the routed GEMM kernels as rocprofv3 names them (prefix of the template
# argument list): the 256-row tile kernel, the 288-row one, or the 32-row one
# for decode-sized batches; dual = gate/up, single = down; the routed ones take
# the expert-aligned tile order (template argument 2), the shared expert's do
# not.  Where the tile height is chosen on the device both the 256- and the
# 288-row kernel are launched and one exits at once: the traffic is that of the
# kernel of the two that read the most
GATE_UP_KERNELS = ("gemm_bf16_persistent_kernel<true, true", "gemm_bf16_tall_kernel<true",
                   "gemm_bf16_skinny_kernel<true")
DOWN_KERNELS = ("gemm_bf16_persistent_kernel<false, true", "gemm_bf16_tall_kernel<false",
                "gemm_bf16_skinny_kernel<false")
READ_COUNTERS = ("TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")


def _pmc_rows(d):
    """Counter rows of a rocprofv3 --pmc output directory, from its CSV files
    or from its rocpd database: dicts with Kernel_Name, Counter_Name,
    Counter_Value, Dispatch_Id and the dispatch's duration in ns."""
    import csv
    import glob
    import sqlite3
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            dur = float(r["End_Timestamp"]) - float(r["Start_Timestamp"]) if "End_Timestamp" in r else None
            rows.append(dict(r, Duration=dur))
    for f in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
        con = sqlite3.connect(f)
        q = "select kernel_name, counter_name, value, dispatch_id, duration from counters_collection"
        for kn, cn, v, di, dur in con.execute(q):
            rows.append({"Kernel_Name": kn, "Counter_Name": cn, "Counter_Value": v, "Dispatch_Id": di,
                         "Duration": dur})
        con.close()
    return rows


def _per_dispatch(rows, counter, names):
    vals = [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and any(n in r["Kernel_Name"] for n in names)]
    return sum(vals) / len(vals) if vals else None


def _read_bytes(rows, names):
    """Fabric read bytes per dispatch: the L2's 32-, 64- and 128-byte read
    requests to the fabric, 32 n32 + 64 n64 + 128 n128 (FETCH_SIZE's formula
    counts this chip's 128-byte requests as 64 bytes: it reads half a copy)."""
    n = [_per_dispatch(rows, c, names) for c in READ_COUNTERS]
    return None if None in n else 32 * n[0] + 64 * n[1] + 128 * n[2]


def _busiest_kernel(rows, names):
    """Of the kernels matching names, the full name of the one whose
    dispatches read the most (None if none matches)."""
    kns = {r["Kernel_Name"] for r in rows if any(n in r["Kernel_Name"] for n in names)}
    best = max(kns, key=lambda kn: _read_bytes(rows, (kn,)) or 0.0, default=None)
    return best


def traffic_from(args):
    """HBM bytes per launch of the routed GEMMs from rocprofv3 runs: fabric
    reads from the TCC_EA0_RDREQ_32B/64B/128B counts, writes from WRITE_SIZE
    (KiB); both checked on a 1 GiB copy (--copy-calibration), which must read
    1 GiB and write 1 GiB.  Writes profiles/traffic.json for --workload."""
    rd_dir, wr_dir, crd_dir, cwr_dir = args.traffic_from
    copy_names = ("copyBuffer", "elementwise_kernel")
    crd = max((_read_bytes([r for r in _pmc_rows(crd_dir) if n in r["Kernel_Name"]], (n,)) or 0.0)
              for n in copy_names)
    cwr = max((float(r["Counter_Value"]) * 1024 for r in _pmc_rows(cwr_dir) if r["Counter_Name"] == "WRITE_SIZE"),
              default=None)
    rows_rd, rows_wr = _pmc_rows(rd_dir), _pmc_rows(wr_dir)
    rec = {"method": "reads: 32 TCC_EA0_RDREQ_32B + 64 TCC_EA0_RDREQ_64B + 128 TCC_EA0_RDREQ_128B; "
                     "writes: WRITE_SIZE KiB * 1024; per dispatch, averaged",
           "copy_check": {"copy_bytes": COPY_BYTES, "read_bytes": crd, "write_bytes": cwr},
           "source_hash": kernel_source_hash()}
    for tag, names in (("gate_up", GATE_UP_KERNELS), ("down", DOWN_KERNELS)):
        kn = _busiest_kernel(rows_rd, names)
        rb = _read_bytes(rows_rd, (kn,)) if kn else None
        wk = _per_dispatch(rows_wr, "WRITE_SIZE", (kn,)) if kn else None
        if rb is None or wk is None:
            sys.exit(f"missing counters for {tag}: read {rb}, write {wk}")
        rec[tag] = {"kernel": kn, "read_bytes": rb, "write_bytes": wk * 1024, "bytes_per_launch": rb + wk * 1024}
    rec["bytes_per_launch"] = rec["gate_up"]["bytes_per_launch"]
    data = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    data[args.workload] = rec
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(data, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(rec))


def trace_summary(args):
    """The kernel_stats.csv of a rocprofv3 --kernel-trace --stats run as a
    markdown table (durations in us; calls include warm-up launches)."""
    import csv
    import glob
    f = glob.glob(os.path.join(args.trace_summary, "**", "*kernel_stats.csv"), recursive=True)
    if not f:
        sys.exit(f"no kernel_stats.csv under {args.trace_summary}")
    print("| kernel | calls | avg (us) | min (us) | max (us) | share |")
    print("|---|---|---|---|---|---|")
    for r in csv.DictReader(open(f[0])):
        name = r["Name"].replace("void ", "").replace("moe::(anonymous namespace)::", "")
        name = name.replace("(moe::GemmGroup, int)", "").replace("(moe::", "(")
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
              f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} % |")


def counters_from(args):
    """MFMA busy fraction and clock of each kernel from a rocprofv3 --pmc run
    of SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16 and
    GRBM_GUI_ACTIVE, averaged over its dispatches:
      clock    = GRBM_GUI_ACTIVE / 8 (one GRBM per XCD, summed) / duration;
      mfma busy = SQ_VALU_MFMA_BUSY_CYCLES (summed over the 1024 SIMDs)
                  / (1024 * GRBM_GUI_ACTIVE / 8), rocprofv3's MfmaUtil;
      MFMA FLOPs = 512 * SQ_INSTS_VALU_MFMA_MOPS_BF16 (executed, padding included).
    Prints a markdown table."""
    per = {}
    for r in _pmc_rows(args.counters_from):
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        e = per.setdefault(key, {"dur": r["Duration"]})
        e[r["Counter_Name"]] = float(r["Counter_Value"])
    agg = {}
    for (kn, _), e in per.items():
        if "GRBM_GUI_ACTIVE" not in e or not e.get("dur"):
            continue
        a = agg.setdefault(kn, [])
        a.append(e)
    print("| kernel | dispatches | avg duration (us) | clock (GHz) | MFMA busy | MFMA FLOPs per dispatch | "
          "TFLOP/s executed |")
    print("|---|---|---|---|---|---|---|")
    for kn, es in sorted(agg.items(), key=lambda kv: -sum(e["dur"] for e in kv[1])):
        dur = np.mean([e["dur"] for e in es]) * 1e-9
        gui = np.mean([e["GRBM_GUI_ACTIVE"] for e in es]) / 8.0
        busy = np.mean([e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for e in es])
        flops = 512.0 * np.mean([e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for e in es])
        name = kn if len(kn) < 110 else kn[:107] + "..."
        print(f"| `{name}` | {len(es)} | {dur * 1e6:.1f} | {gui / dur / 1e9:.3f} | "
              f"{busy / (1024.0 * gui) * 100:.1f} % | {flops:.4g} | {flops / dur / 1e12:.1f} |")


def measure(name: str, args, torch, moe, dev, extras: bool) -> dict:
    """One workload: inputs resident in HBM, warmup, K timed steps of the
    whole layer (moe_forward_staged, gate/up kernel timed by its own launch
    events), a separate staged pass for the per-stage times, the roofline of
    the gate/up kernel, the CPU oracle on a sample (and the parity of the
    timed output on it); with extras the optional features, the backward and
    the practical ceilings."""
    import synth
    sh = synth.SHAPES[name]
    dt_name = "bf16" if sh.dtype == synth.BF16 else "f32"
    t_gen = time.perf_counter()
    inp = synth.make_inputs(sh, args.seed)
    d = {n: (None if a is None else upload(a, torch, dev)) for n, a in inp.items()}
    print(f"[bench] {sh.name}: inputs generated and resident in HBM in "
          f"{time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    cfg = moe.MoeConfig.of(sh.T, sh.d, sh.E, sh.k, sh.d_ff, sh.num_shared, sh.d_ff_shared,
                           sh.score_fn, sh.renormalize, sh.dtype)
    ws = moe.alloc_workspace(cfg, dev)
    y = torch.empty(sh.T, sh.d, dtype=torch.bfloat16 if sh.dtype else torch.float32, device=dev)
    counts = torch.empty(sh.E, dtype=torch.int32, device=dev)
    ids = torch.empty(sh.T, sh.k, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(start, evs):
        moe.moe_forward_staged(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                               d["ws_gate"], d["ws_up"], d["ws_down"], y, topk_ids=ids, expert_counts=counts,
                               ws=ws, start_event=start, stage_events=evs, stream=stream)

    tev = TimingEvents()
    for _ in range(args.warmup):
        step(None, None)
    torch.cuda.synchronize()
    # Timed region: the whole layer, with two timing events per step around
    # the dominant kernel (the routed gate/up GEMM, stage 2) on the layer's stream.
    gu_ev = [tev.make(2, stream) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs = [None] * moe.MOE_NUM_STAGES
        evs[1], evs[2] = gu_ev[i]
        step(None, evs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    gu_each = np.array([tev.ms(a, b) for a, b in gu_ev])
    gu_ms = float(gu_each.mean())
    y_host = y.float().cpu().numpy().astype(np.float64)
    ids_host = ids.cpu().numpy()

    # Stage breakdown: a separate pass with an event after every stage.
    starts = tev.make(args.steps, stream)
    stages = [tev.make(moe.MOE_NUM_STAGES, stream) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(starts[i], stages[i])
    torch.cuda.synchronize()
    stage_ms = np.zeros((args.steps, moe.MOE_NUM_STAGES))
    for i in range(args.steps):
        prev = starts[i]
        for j, e in enumerate(stages[i]):
            stage_ms[i, j] = tev.ms(prev, e)
            prev = e
    stage_avg = stage_ms.mean(0)
    tev.close()
    cnt = counts.cpu().numpy()
    plan = moe.moe_forward_plan(cfg)
    if plan["tile_rows"] == 0:
        # chosen on the device per call: the library's documented rule on these counts
        plan["tile_rows_chosen"] = device_tile_rows(cnt, sh.d_ff)
    alg = algorithmic(sh, cnt, plan["shared_merged"])
    bf16 = sh.dtype == synth.BF16
    peak_c = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    gu = alg["gate_up"]
    t_hbm = gu["bytes"] / (PEAK_HBM_GBS * 1e9)          # floors of the gate/up kernel, s
    t_mfma = gu["flops"] / (peak_c * 1e12)
    hbm_roof = {"bound": "hbm", "achieved": gu["bytes"] / (gu_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    cmp_roof = {"bound": "mfma" if bf16 else "alu", "achieved": gu["flops"] / (gu_ms * 1e-3) / 1e12,
                "peak": peak_c, "unit": "TFLOP/s"}
    for r_ in (hbm_roof, cmp_roof):
        r_["frac"] = r_["achieved"] / r_["peak"]
    roof, other = (hbm_roof, cmp_roof) if t_hbm >= t_mfma else (cmp_roof, hbm_roof)
    roof = dict(roof)
    roof["kernel"] = "gate_up_gemm (grouped gate/up GEMM + SiLU*up" + (
        ", the shared expert as one more group)" if plan["shared_merged"] else ")")
    roof["per_launch"] = {"flops": gu["flops"], "bytes": gu["bytes"], "avg_ms": gu_ms,
                          "floor_ms_hbm": t_hbm * 1e3, "floor_ms_compute": t_mfma * 1e3}
    roof["other_bound"] = other
    roof["traffic"] = None
    src_hash = kernel_source_hash()
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE)).get(sh.name, {})
        if rec.get("source_hash") == src_hash:
            roof["traffic"] = rec.get("bytes_per_launch")
    layer_s = ms_per_step * 1e-3
    floor_layer = max(alg["layer_bytes"] / (PEAK_HBM_GBS * 1e9), alg["layer_flops"] / (peak_c * 1e12))
    gg_ms = gu_ms + float(stage_avg[3])
    out = {
        "metric": "MoE-layer tokens/s",
        "value": sh.T / layer_s,
        "unit": "tokens/s",
        "ms_per_step": ms_per_step,
        "dtype": dt_name,
        "config": {"workload": sh.name, "T": sh.T, "d": sh.d, "E": sh.E, "k": sh.k,
                   "d_ff": sh.d_ff, "num_shared": sh.num_shared, "d_ff_shared": sh.d_ff_shared,
                   "score": "sigmoid" if sh.score_fn else "softmax",
                   "renormalize": sh.renormalize, "parallelism": "single GPU"},
        "layer_tflops": alg["layer_flops"] / layer_s / 1e12,
        "layer_pct_bf16_peak": alg["layer_flops"] / layer_s / 1e12 / PEAK_BF16_TFLOPS,
        "layer_gbs": alg["layer_bytes"] / layer_s / 1e9,
        "layer_pct_hbm": alg["layer_bytes"] / layer_s / 1e9 / PEAK_HBM_GBS,
        "layer_floor_ms": floor_layer * 1e3,
        "layer_frac_of_floor": floor_layer / layer_s,
        "stages_ms": {n: round(float(v), 4) for n, v in zip(moe.STAGE_NAMES, stage_avg)},
        "staged_ms_per_step": round(float(stage_ms.sum(1).mean()), 4),
        # spread over the steps: the whole layer per step (start event to the
        # last stage's, staged pass) and the gate/up kernel per launch (timed pass)
        "step_ms_stats": {"median": round(float(np.median(stage_ms.sum(1))), 4),
                          "min": round(float(stage_ms.sum(1).min()), 4),
                          "p90": round(float(np.percentile(stage_ms.sum(1), 90)), 4)},
        "gate_up_ms_stats": {"median": round(float(np.median(gu_each)), 4), "min": round(float(gu_each.min()), 4),
                             "p90": round(float(np.percentile(gu_each, 90)), 4)},
        "expert_load": {"max_over_mean": float(cnt.max() / max(cnt.mean(), 1e-9)),
                        "touched": alg["touched"], "min": int(cnt.min()), "max": int(cnt.max())},
        "plan": plan,
        "roofline": roof,
        # the routed grouped GEMM: gate/up (timed region) and down (stage pass) kernels
        "grouped_gemm": {"ms": gg_ms,
                         "tflops": (gu["flops"] + alg["down"]["flops"]) / (gg_ms * 1e-3) / 1e12,
                         "gbs": (gu["bytes"] + alg["down"]["bytes"]) / (gg_ms * 1e-3) / 1e9},
        "kernel_source_hash": src_hash,
    }
    gg = out["grouped_gemm"]
    gg["frac_bf16_peak"] = gg["tflops"] / PEAK_BF16_TFLOPS
    gg["frac_hbm"] = gg["gbs"] / PEAK_HBM_GBS
    if extras and not args.no_options:
        out["options_ms_per_step"] = options_cost(torch, moe, cfg, d, y, ws, stream, sh,
                                                  max(3, min(args.steps, 20)))
    if extras and not args.no_backward:
        out["backward"] = backward_cost(torch, moe, cfg, d, sh, stream, 3)
    if extras and not args.no_ceilings:
        out["practical_ceilings"] = practical_ceilings(torch, dev, sh)
    del d, ws, y, counts, ids
    torch.cuda.empty_cache()
    if args.no_cpu_baseline:
        out["cpu_baseline"] = None
        out["parity"] = None
    else:
        out["cpu_baseline"], ref = cpu_baseline(sh, inp, args.cpu_seconds)
        out["parity"] = parity_of(y_host, ids_host, ref, dt_name)
    del inp
    return out


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(args)
        return
    if args.counters_from:
        counters_from(args)
        return
    if args.trace_summary:
        trace_summary(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the layer is measured at N=1", file=sys.stderr)
        sys.exit(2)
    import torch

    import mixture_experts_sparse_moe_amd as moe

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    moe.lib()
    dev = torch.device("cuda:0")
    head = measure(args.workload, args, torch, moe, dev, extras=True)
    line = {
        "metric": head.pop("metric"), "value": head.pop("value"), "unit": head.pop("unit"), "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": head.pop("dtype"),
        "data": "synthetic (seeded Philox normals; weights N(0,1/fan_in))", "config": head.pop("config"),
    }
    line.update(head)
    if not args.only:
        subs = {}
        for name in OTHERS:
            if name == args.workload:
                continue
            try:
                subs[name] = measure(name, args, torch, moe, dev, extras=False)
            except Exception as exc:            # a failed sub-record is reported, not hidden
                subs[name] = {"error": f"{type(exc).__name__}: {exc}"}
            print(f"[bench] {name}: done", file=sys.stderr, flush=True)
        line["configs"] = subs
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
