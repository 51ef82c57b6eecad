"""Benchmark of the top-k MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one whole forward of the layer (route, dispatch, routed SwiGLU
grouped GEMMs, shared expert, combine) over one batch of seeded synthetic
inputs already resident in HBM.  The default workload is the Mixtral-8x7B-
shaped prefill layer (T=4096, d=4096, E=8, k=2, d_ff=14336, bf16).

Prints one JSON line with the throughput (tokens/s), the roofline of the
dominant kernel measured live with HIP events on the launch stream, and the
CPU oracle timed on a bounded sample of the same workload on the host cores.
The timed region records two timing events per step, around the dominant
kernel (created without the system-scope fence, so recording them costs the
next kernel nothing measurable); the per-stage breakdown comes from a
separate pass with an event after every stage.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mixtral_prefill")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target wall time of the CPU oracle sample")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the practical ceilings (device copy, torch.matmul yardstick)")
    p.add_argument("--no-options", action="store_true",
                   help="skip timing the layer with its optional routing features")
    p.add_argument("--no-backward", action="store_true",
                   help="skip timing the backward pass (moe_backward)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device copy of 1 GiB (the reference for HBM counters)")
    p.add_argument("--traffic-from", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_DIR"),
                   help="rocprofv3 --pmc output dirs (FETCH_SIZE run of the bench, WRITE_SIZE run "
                        "of the bench, FETCH_SIZE+WRITE_SIZE runs of --copy-calibration); writes "
                        "profiles/traffic.json for --workload")
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


def algorithmic(sh, counts: np.ndarray) -> dict:
    """Algorithmic work of the layer and of its two expert GEMM kernels.

    FLOPs: router 2TdE, routed experts 6 d d_ff per pair (4 in gate/up, 2 in
    down), shared expert 6 d d_ff_s per token.  Bytes: weights of the experts
    actually touched (union read), the router weights, x read once, y written
    once, 8 bytes of routing per pair; per kernel, its weights plus its
    activation input and output."""
    w = sh.elem_bytes
    T, d, E, k, f = sh.T, sh.d, sh.E, sh.k, sh.d_ff
    touched = int((counts > 0).sum())
    P = T * k
    layer_flops = sh.flops()
    layer_bytes = (E * d * w + touched * 3 * d * f * w + sh.num_shared * 3 * d * sh.d_ff_shared * w
                   + 2 * T * d * w + P * 8)
    gate_up = dict(flops=4.0 * P * d * f, bytes=touched * 2 * d * f * w + T * d * w + P * f * w)
    down = dict(flops=2.0 * P * d * f, bytes=touched * d * f * w + P * f * w + P * d * w)
    return dict(layer_flops=layer_flops, layer_bytes=layer_bytes, gate_up=gate_up, down=down,
                touched=touched)


def options_cost(torch, moe, cfg, d, y, ws, stream, sh, steps: int) -> dict:
    """ms per layer (moe_forward_ex, no per-stage events) with each optional
    routing feature on: a selection-only bias on the scores (N(0, 0.01)),
    capacity factor 1.25, router statistics, and all three; next to the plain
    layer through the same entry point."""
    g = torch.Generator().manual_seed(0)
    bias = (torch.randn(sh.E, generator=g, dtype=torch.float32) * 0.01).to(d["x"].device)
    stats = torch.empty(2 * sh.E + 2, dtype=torch.float32, device=d["x"].device)
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


def practical_ceilings(torch, dev) -> dict:
    """Measured ceilings on the same GPU, next to the nominal peaks: a 1 GiB
    device copy (read + write bytes / time) and one bf16 4096 x 14336 x 4096
    torch.matmul (a library yardstick only; nothing of the layer uses it)."""
    out = {}
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
    return out


def cpu_baseline(sh, inp, target_s: float) -> dict:
    """The oracle as it stands, on a bounded sample of tokens of the same layer."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    n = max(cores, 1)
    tokens_done, t_used, sample_desc = 0, 0.0, ""
    rng = np.random.default_rng(123)
    while True:
        toks = np.sort(rng.choice(sh.T, size=min(n, sh.T), replace=False))
        t0 = time.perf_counter()
        oracle.forward_tokens(inp, sh.k, toks, sh.score_fn, sh.renormalize, nthreads=cores)
        dt = time.perf_counter() - t0
        tokens_done, t_used = toks.size, dt
        sample_desc = (f"{toks.size} of {sh.T} tokens (seeded random), full routing and "
                       f"{sh.k} experts" + (" + shared expert" if sh.num_shared else "") +
                       " per token, fp64")
        if dt >= target_s / 4 or toks.size >= sh.T:
            break
        n = int(min(sh.T, max(n * 2, n * (target_s / max(dt, 1e-3)) * 0.8)))
    return {"value": tokens_done / t_used, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": sample_desc, "seconds": round(t_used, 3)}


COPY_BYTES = 1 << 30


def copy_calibration():
    """A plain 1 GiB device-to-device copy: its FETCH_SIZE / WRITE_SIZE readings
    give the scale between those counters and bytes moved."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES}), flush=True)


# the gate/up GEMM kernel as rocprofv3 names it (bf16, dual mode; prefix of
# the template argument list)
# the routed gate/up GEMM: the 256-row tile kernel, or the 32-row one for
# decode-sized batches (one of them runs per workload)
GATE_UP_KERNELS = ("gemm_bf16_persistent_kernel<true", "gemm_bf16_skinny_kernel<true")


def _pmc_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def _per_dispatch(rows, counter, names):
    vals = [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and any(n in r["Kernel_Name"] for n in names)]
    return sum(vals) / len(vals) if vals else None


def traffic_from(args):
    """HBM bytes per launch of the gate/up GEMM from rocprofv3 FETCH_SIZE and
    WRITE_SIZE runs, each scaled by the same counter's reading for the 1 GiB copy."""
    fetch_dir, write_dir, copy_dir = args.traffic_from
    copy_rows = _pmc_rows(copy_dir)
    # the copy kernel is the largest dispatch of the calibration run
    cf = max((float(r["Counter_Value"]) for r in copy_rows if r["Counter_Name"] == "FETCH_SIZE"),
             default=None)
    cw = max((float(r["Counter_Value"]) for r in copy_rows if r["Counter_Name"] == "WRITE_SIZE"),
             default=None)
    f_kib = _per_dispatch(_pmc_rows(fetch_dir), "FETCH_SIZE", GATE_UP_KERNELS)
    w_kib = _per_dispatch(_pmc_rows(write_dir), "WRITE_SIZE", GATE_UP_KERNELS)
    if None in (cf, cw, f_kib, w_kib):
        sys.exit(f"missing counters: copy {cf} {cw}, kernel {f_kib} {w_kib}")
    f_scale, w_scale = COPY_BYTES / cf, COPY_BYTES / cw
    rec = {"kernel": "grouped gate/up GEMM (" + " or ".join(GATE_UP_KERNELS) + ", ...>)",
           "fetch_kib": f_kib, "write_kib": w_kib,
           "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale_bytes_per_kib": f_scale, "write_scale_bytes_per_kib": w_scale,
           "bytes_per_launch": f_kib * f_scale + w_kib * w_scale,
           "source_hash": kernel_source_hash()}
    data = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    data[args.workload] = rec
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(data, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(rec))


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(args)
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
    import synth

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    moe.lib()
    sh = synth.SHAPES[args.workload]
    dev = torch.device("cuda:0")
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
    stream = torch.cuda.current_stream(dev)

    def step(start, evs):
        moe.moe_forward_staged(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                               d["ws_gate"], d["ws_up"], d["ws_down"], y, expert_counts=counts,
                               ws=ws, start_event=start, stage_events=evs, stream=stream)

    tev = TimingEvents()

    for _ in range(args.warmup):
        step(None, None)
    torch.cuda.synchronize()
    # Timed region: the whole layer, with two timing events per step around
    # the dominant kernel (the routed gate/up GEMM, stage 2) on the layer's
    # stream.
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
    gu_ms = float(np.mean([tev.ms(a, b) for a, b in gu_ev]))

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
    alg = algorithmic(sh, cnt)
    decode = sh.T * sh.k < 64 * sh.E          # under 64 rows per expert: weight-read bound
    if decode:
        achieved = alg["gate_up"]["bytes"] / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        peak = PEAK_BF16_TFLOPS if sh.dtype == synth.BF16 else PEAK_F32_TFLOPS
        achieved = alg["gate_up"]["flops"] / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = "gate_up_gemm (grouped gate/up GEMM + SiLU*up)"
    roof["per_launch"] = {"flops": alg["gate_up"]["flops"], "bytes": alg["gate_up"]["bytes"],
                          "avg_ms": gu_ms}
    roof["traffic"] = None
    src_hash = kernel_source_hash()
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE)).get(sh.name, {})
        if rec.get("source_hash") == src_hash:
            roof["traffic"] = rec.get("bytes_per_launch")
    layer_s = ms_per_step * 1e-3
    out = {
        "metric": "MoE-layer tokens/s",
        "value": sh.T / layer_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sh.dtype == synth.BF16 else "f32",
        "data": "synthetic (seeded Philox normals; weights N(0,1/fan_in))",
        "config": {"workload": sh.name, "T": sh.T, "d": sh.d, "E": sh.E, "k": sh.k,
                   "d_ff": sh.d_ff, "num_shared": sh.num_shared, "d_ff_shared": sh.d_ff_shared,
                   "score": "sigmoid" if sh.score_fn else "softmax",
                   "renormalize": sh.renormalize, "parallelism": "single GPU"},
        "layer_tflops": alg["layer_flops"] / layer_s / 1e12,
        "layer_pct_bf16_peak": alg["layer_flops"] / layer_s / 1e12 / PEAK_BF16_TFLOPS,
        "layer_gbs": alg["layer_bytes"] / layer_s / 1e9,
        "layer_pct_hbm": alg["layer_bytes"] / layer_s / 1e9 / PEAK_HBM_GBS,
        # separate pass with an event after every stage
        "stages_ms": {n: round(float(v), 4) for n, v in zip(moe.STAGE_NAMES, stage_avg)},
        "staged_ms_per_step": round(float(stage_ms.sum(1).mean()), 4),
        "expert_load": {"max_over_mean": float(cnt.max() / max(cnt.mean(), 1e-9)),
                        "touched": alg["touched"], "min": int(cnt.min()), "max": int(cnt.max())},
        "roofline": roof,
        # the routed grouped GEMM: gate/up (timed region) and down (stage pass) kernels
        "grouped_gemm": {"ms": gu_ms + float(stage_avg[3]),
                         "tflops": (alg["gate_up"]["flops"] + alg["down"]["flops"]) /
                                   ((gu_ms + float(stage_avg[3])) * 1e-3) / 1e12,
                         "gbs": (alg["gate_up"]["bytes"] + alg["down"]["bytes"]) /
                                ((gu_ms + float(stage_avg[3])) * 1e-3) / 1e9},
        "kernel_source_hash": src_hash,
    }
    gg = out["grouped_gemm"]
    gg["frac_bf16_peak"] = gg["tflops"] / PEAK_BF16_TFLOPS
    gg["frac_hbm"] = gg["gbs"] / PEAK_HBM_GBS
    if not args.no_options:
        out["options_ms_per_step"] = options_cost(torch, moe, cfg, d, y, ws, stream, sh,
                                                  max(3, min(args.steps, 20)))
    if not args.no_backward:
        out["backward"] = backward_cost(torch, moe, cfg, d, sh, stream, 3)
    if not args.no_ceilings:
        out["practical_ceilings"] = practical_ceilings(torch, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(sh, inp, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
