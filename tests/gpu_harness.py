"""Helpers for the GPU parity tests: device copies of seeded inputs, calls
through the C ABI, and the comparison rules against the CPU oracle."""
from __future__ import annotations

import numpy as np

import mixture_experts_sparse_moe_amd as moe
import oracle
import synth

# Output tolerance, max |y_gpu - y_ref| <= TAU * max |y_ref|: 2e-2 for bf16
# layers, 1e-4 for fp32 layers.
TAU = {synth.BF16: 2e-2, synth.F32: 1e-4}
# Routing near-tie rule: a GPU/oracle difference in the chosen ids is allowed
# only where the oracle's adjacent score gap at that position is below this.
NEAR_TIE = 1e-6
LOGIT_TIE = 1e-4


def torch():
    import torch as _t
    return _t


def to_dev(a: np.ndarray, device="cuda"):
    t = torch()
    if a.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(t.bfloat16)
    return t.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(x) -> np.ndarray:
    t = torch()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def widen(a: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def cfg_of(sh: synth.LayerShape, T: int | None = None) -> moe.MoeConfig:
    return moe.MoeConfig.of(sh.T if T is None else T, sh.d, sh.E, sh.k, sh.d_ff, sh.num_shared,
                            sh.d_ff_shared, sh.score_fn, sh.renormalize, sh.dtype)


class DeviceLayer:
    """Device copies of one layer's inputs and the calls of the C ABI."""

    def __init__(self, sh: synth.LayerShape, inp: dict, device="cuda"):
        self.sh, self.inp, self.device = sh, inp, device
        self.d = {n: (None if a is None else to_dev(a, device)) for n, a in inp.items()}
        self.cfg = cfg_of(sh)
        self.ws = moe.alloc_workspace(self.cfg, device)

    def empty_act(self, *shape):
        t = torch()
        dt = t.bfloat16 if self.sh.dtype == synth.BF16 else t.float32
        return t.empty(*shape, dtype=dt, device=self.device)

    def forward(self, stream=None) -> dict:
        t = torch()
        sh, dv = self.sh, self.d
        y = self.empty_act(sh.T, sh.d)
        ids = t.empty(sh.T, sh.k, dtype=t.int32, device=self.device)
        wts = t.empty(sh.T, sh.k, dtype=t.float32, device=self.device)
        counts = t.empty(sh.E, dtype=t.int32, device=self.device)
        gap = t.empty(sh.T, 2, dtype=t.float32, device=self.device)
        moe.moe_forward(self.cfg, dv["x"], dv["w_router"], dv["w_gate"], dv["w_up"], dv["w_down"],
                        dv["ws_gate"], dv["ws_up"], dv["ws_down"], y, ids, wts, counts, self.ws,
                        stream=stream, topk_gap=gap)
        return dict(y=y, ids=ids, weights=wts, counts=counts, gap=gap)

    def steps(self) -> dict:
        """The layer through the four step entry points, keeping every output."""
        t = torch()
        sh, dv, dev = self.sh, self.d, self.device
        P = sh.T * sh.k
        ids = t.empty(sh.T, sh.k, dtype=t.int32, device=dev)
        wts = t.empty(sh.T, sh.k, dtype=t.float32, device=dev)
        gap = t.empty(sh.T, 2, dtype=t.float32, device=dev)
        moe.moe_route(self.cfg, dv["x"], dv["w_router"], ids, wts, gap)
        counts = t.empty(sh.E, dtype=t.int32, device=dev)
        offsets = t.empty(sh.E + 1, dtype=t.int32, device=dev)
        sp = t.empty(P, dtype=t.int32, device=dev)
        pp = t.empty(P, dtype=t.int32, device=dev)
        moe.moe_dispatch(self.cfg, ids, counts, offsets, sp, pp, self.ws)
        out = self.empty_act(P, sh.d)
        so = self.empty_act(sh.T, sh.d) if sh.num_shared else None
        moe.moe_expert_ffn(self.cfg, dv["x"], sp, offsets, dv["w_gate"], dv["w_up"], dv["w_down"],
                           dv["ws_gate"], dv["ws_up"], dv["ws_down"], out, so, self.ws)
        y = self.empty_act(sh.T, sh.d)
        moe.moe_combine(self.cfg, out, wts, pp, so, y)
        return dict(ids=ids, weights=wts, gap=gap, counts=counts, offsets=offsets,
                    sorted_pairs=sp, pair_pos=pp, expert_out=out, shared_out=so, y=y)


def check_ids(gpu_ids: np.ndarray, oracle_ids: np.ndarray, key: np.ndarray, key_score: np.ndarray,
              key_tol: float, score_tol: float = NEAR_TIE) -> np.ndarray:
    """GPU ids against the oracle's, slot by slot, with near-ties exempted.

    key [T,E]: the oracle's selection key (fp64: the logit, or the logit or
    score plus a selection bias); key_score [T,E]: the same key in score
    space (the scores themselves for a logit key, the key itself when it is
    already a score).  A token's list may differ from the oracle's only at
    slots j where the GPU's expert is tied with the oracle's expert of that
    slot: |key gap| < key_tol (fp32 accumulation reach; a larger gap is a
    bug) and |score gap| < score_tol (1e-6, the near-tie rule).  So every
    reorder and every set change sits at a near-tie, and the list stays a
    valid top-k in descending order up to that band.  The k ids must be
    distinct experts.  Returns the exempted token indices."""
    T, k = oracle_ids.shape
    E = key.shape[1]
    exempt = []
    for t in np.nonzero((gpu_ids != oracle_ids).any(1))[0]:
        g, o = gpu_ids[t], oracle_ids[t]
        ok = len(set(g.tolist())) == k and bool(np.all((g >= 0) & (g < E)))
        bad = []
        for j in np.nonzero(g != o)[0]:
            if not ok:
                break
            dk = abs(key[t, g[j]] - key[t, o[j]])
            ds = abs(key_score[t, g[j]] - key_score[t, o[j]])
            if not (dk < key_tol and ds < score_tol):
                bad.append((int(j), int(g[j]), int(o[j]), float(dk), float(ds)))
        assert ok and not bad, (f"token {t}: gpu ids {g.tolist()} != oracle {o.tolist()}; "
                                f"(slot, gpu, oracle, key gap, score gap) outside the near-tie band: {bad}")
        exempt.append(int(t))
    return np.array(exempt, dtype=np.int64)


def check_routing(gpu_ids: np.ndarray, ref: dict, k: int) -> np.ndarray:
    """Plain routing (key = logit): check_ids with the oracle's logits and
    scores, logit band LOGIT_TIE, score band NEAR_TIE."""
    return check_ids(gpu_ids, ref["ids"], ref["logits"], ref["scores"], LOGIT_TIE, NEAR_TIE)


def oracle_routing(inp: dict, sh: synth.LayerShape) -> dict:
    lg = oracle.logits(inp["x"], inp["w_router"])
    r = oracle.route(lg, sh.k, sh.score_fn, sh.renormalize)
    r["logits"] = lg
    return r


def check_gaps(gap: np.ndarray, ref: dict, k: int, E: int, skip=()) -> None:
    """GPU margins [T,2] against the oracle's: the key (logit) margin within
    1e-3 absolute + 1e-4 relative (fp32 logits), the score margin within
    2e-6 absolute + 1e-3 relative (fp32 scores); +inf for both when k == E.
    Tokens in ``skip`` (routed differently at a near-tie) are left out."""
    if k == E:
        assert np.all(np.isinf(gap))
        return
    ok = np.setdiff1d(np.arange(gap.shape[0]), np.asarray(skip, dtype=np.int64))
    np.testing.assert_allclose(gap[ok, 0], ref["gap_logit"][ok], atol=1e-3, rtol=1e-4, err_msg="key margin")
    np.testing.assert_allclose(gap[ok, 1], ref["gap_score"][ok], atol=2e-6, rtol=1e-3, err_msg="score margin")


def assert_close(got: np.ndarray, want: np.ndarray, tau: float, what: str):
    scale = float(np.abs(want).max())
    err = float(np.abs(got - want).max())
    assert err <= tau * max(scale, 1e-30), f"{what}: max|err| {err:.3e} > {tau} * max|ref| {scale:.3e}"
    return err / max(scale, 1e-30)
