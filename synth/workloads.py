"""Seeded synthetic workloads for the liveness-sparse routed-expert MoE layer.

This module only draws inputs: weights, router biases, hidden states and the
per-iteration decoded / forced masks.  It holds none of the layer's arithmetic
(no routing, no top-k, no fresh-set logic, no expert math), so both the HIP
path and the CPU oracle can take their inputs from it.

Why the inputs look the way they do (the pages have no public weights or
traces for this layer; Epoch: Compiling Diffusion Blocks for Sparse MoE
Serving, and the pinghaoyang.com.cn teardown of it):

* block-diffusion refinement: a block of positions starts fully masked and
  positions commit over the iterations (teardown, "why diffusion LMs stall
  serving systems"); commit schedules below stand in for a threshold decoder.
* hidden states drift less for decoded positions than for live ones
  (teardown, "refresh period" section: decoded routed outputs are more stable
  across iterations than masked ones); an AR(1) drift with a larger
  correlation for decoded positions keeps N(0,1) marginals.
* the active expert set is stable inside a block and routing mass is
  concentrated (teardown, Expert Atlas section, Figure 3); Zipf-shaped router
  biases give a concentrated load.

Every array is a pure function of (workload, layer, tensor, expert) seeds, so a
single expert's weights can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import json
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

# tensor codes used in the seed sequence
_T_ROUTER_W, _T_ROUTER_PERM, _T_W1, _T_W3, _T_W2 = 0, 1, 2, 3, 4
_T_SW1, _T_SW3, _T_SW2 = 5, 6, 7
_T_HIDDEN, _T_LIVE, _T_FORCE = 10, 11, 12


@dataclass(frozen=True)
class Workload:
    """Shape and statistics of one synthetic MoE-layer workload."""

    name: str
    seed: int
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    n_shared: int
    shared_inter: int
    batch: int
    block: int
    iters: int
    staleness_R: int
    n_layers: int
    gate: str            # "softmax" | "sigmoid"
    norm_topk: bool
    act: str             # "f32" | "bf16"
    sigma: float         # std of every weight tensor
    zipf: Optional[float]  # target Zipf exponent of the expert load, or None
    liveness: str        # "per_iter" | "uniform" | "forced"
    commits_per_iter: int = 0
    forced_fraction: Optional[float] = None
    redraw_every: int = 0  # hidden state piecewise constant over windows of this many iterations
    rho_live: float = 0.9
    rho_decoded: float = 0.99
    # Expert Atlas plan parameters (the pages give no values; see the design notes)
    atlas_m: int = -1     # -1: m = top_k
    atlas_B: int = -1     # -1: ceil(E / 2)
    atlas_c: int = -1     # -1: c = top_k
    alpha: tuple = (9, 10)
    q: tuple = (95, 100)
    beta: tuple = (1, 1)
    # routing over all experts ("exact") or inside the layer's Atlas support ("restricted");
    # atlas_period > 0 rebuilds a restricted support after that many iterations
    routing: str = "exact"
    atlas_period: int = 0
    # group-limited top-k: experts in n_group contiguous groups, each position selecting among
    # the experts of its topk_group best groups (n_group <= 1: no grouping)
    n_group: int = 0
    topk_group: int = 0

    @property
    def M(self) -> int:
        return self.batch * self.block

    @property
    def m_ext(self) -> int:
        return self.top_k if self.atlas_m < 0 else self.atlas_m

    @property
    def k_ext(self) -> int:
        return min(self.top_k + self.m_ext, self.n_experts)

    @property
    def B(self) -> int:
        return (self.n_experts + 1) // 2 if self.atlas_B < 0 else self.atlas_B

    @property
    def c(self) -> int:
        return self.top_k if self.atlas_c < 0 else self.atlas_c

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _cfg(i: int, **kw) -> Workload:
    return Workload(seed=20260909 + i, **kw)


# The five workloads: tiny fp32 layer, single bf16 layer, 20 stacked layers with a
# shared expert and Zipf(1.1) load, 4 large stacked layers, and the forced-fresh sweep
# on the 20-layer shape with Zipf(1.5) load.
WORKLOADS = {
    1: _cfg(1, name="tiny-fp32-h64-e8-k2", hidden=64, n_experts=8, top_k=2, inter=32,
            n_shared=0, shared_inter=0, batch=1, block=16, iters=4, staleness_R=2,
            n_layers=1, gate="softmax", norm_topk=False, act="f32", sigma=0.02, zipf=None,
            liveness="per_iter", commits_per_iter=4),
    2: _cfg(2, name="bf16-h2048-e64-k8-i1024-b8x32", hidden=2048, n_experts=64, top_k=8,
            inter=1024, n_shared=0, shared_inter=0, batch=8, block=32, iters=16,
            staleness_R=4, n_layers=1, gate="softmax", norm_topk=False, act="bf16",
            sigma=0.02, zipf=None, liveness="uniform"),
    3: _cfg(3, name="bf16-20L-h2048-e256-k8-i512-shared-b32x32-zipf1.1", hidden=2048,
            n_experts=256, top_k=8, inter=512, n_shared=1, shared_inter=512, batch=32,
            block=32, iters=32, staleness_R=4, n_layers=20, gate="sigmoid", norm_topk=True,
            act="bf16", sigma=0.02, zipf=1.1, liveness="uniform"),
    4: _cfg(4, name="bf16-4L-h4096-e256-k8-i1536-shared-b64x32", hidden=4096, n_experts=256,
            top_k=8, inter=1536, n_shared=1, shared_inter=1536, batch=64, block=32, iters=32,
            staleness_R=8, n_layers=4, gate="sigmoid", norm_topk=True, act="bf16",
            sigma=0.01, zipf=None, liveness="uniform"),
    5: _cfg(5, name="bf16-sweep-h2048-e256-k8-i512-shared-b128x64-zipf1.5", hidden=2048,
            n_experts=256, top_k=8, inter=512, n_shared=1, shared_inter=512, batch=128,
            block=64, iters=32, staleness_R=4, n_layers=1, gate="sigmoid", norm_topk=True,
            act="bf16", sigma=0.02, zipf=1.5, liveness="forced", forced_fraction=1.0,
            redraw_every=8),
}

SWEEP_FRACTIONS = (1.0, 0.5, 0.25, 0.10, 0.05)
SWEEP_R = (1, 4, 16)


def workload(i: int, **overrides) -> Workload:
    w = WORKLOADS[i]
    return w.replace(**overrides) if overrides else w


# --------------------------------------------------------------------------- helpers

def _rng(w: Workload, *codes: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([w.seed, *codes]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16, round-to-nearest-even, returned as uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_act(rng: np.random.Generator, shape, sigma: float, act: str) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return f32_to_bf16_bits(a) if act == "bf16" else a


def act_dtype(w: Workload):
    return np.uint16 if w.act == "bf16" else np.float32


# --------------------------------------------------------------------------- weights

def expert_weight(w: Workload, layer: int, which: str, e: int) -> np.ndarray:
    """One routed expert's weight, row-major [out x in]: w1/w3 are [I x H], w2 is [H x I]."""
    code = {"w1": _T_W1, "w3": _T_W3, "w2": _T_W2}[which]
    shape = (w.inter, w.hidden) if which != "w2" else (w.hidden, w.inter)
    return _normal_act(_rng(w, layer, code, e), shape, w.sigma, w.act)


def shared_weight(w: Workload, layer: int, which: str) -> np.ndarray:
    code = {"w1": _T_SW1, "w3": _T_SW3, "w2": _T_SW2}[which]
    shape = (w.shared_inter, w.hidden) if which != "w2" else (w.hidden, w.shared_inter)
    return _normal_act(_rng(w, layer, code), shape, w.sigma, w.act)


def router_weight(w: Workload, layer: int) -> np.ndarray:
    """Router weight [E x H], fp32, N(0, sigma)."""
    a = _rng(w, layer, _T_ROUTER_W).standard_normal((w.n_experts, w.hidden), dtype=np.float32)
    return a * np.float32(w.sigma)


def zipf_scale(w: Workload) -> float:
    """Bias scale s for the Zipf-shaped router bias b_e = -s * ln(rank_e).

    The table is written by oracle/calibrate_zipf.py, which fits s so that the
    expert load (top-k selections) of this workload follows the target exponent.
    """
    path = os.path.join(_HERE, "zipf_scale.json")
    with open(path) as f:
        table = json.load(f)
    key = f"{w.n_experts}:{w.top_k}:{w.hidden}:{w.sigma}:{w.gate}:{w.zipf}"
    if key not in table:
        raise KeyError(f"no Zipf calibration for {key}; run oracle/calibrate_zipf.py")
    return float(table[key])


def router_bias(w: Workload, layer: int, scale: Optional[float] = None) -> Optional[np.ndarray]:
    """Router bias [E] fp32, or None when the workload has no load skew."""
    if w.zipf is None:
        return None
    s = zipf_scale(w) if scale is None else scale
    rank = _rng(w, layer, _T_ROUTER_PERM).permutation(w.n_experts) + 1
    return (-s * np.log(rank.astype(np.float64))).astype(np.float32)


def layer_weights(w: Workload, layer: int, threads: int = 0) -> dict:
    """All weights of one layer as host arrays (bf16 as uint16 bit patterns)."""
    E = w.n_experts
    out = {"router_w": router_weight(w, layer), "router_b": router_bias(w, layer)}
    dt = act_dtype(w)
    for which, shape in (("w1", (E, w.inter, w.hidden)), ("w3", (E, w.inter, w.hidden)),
                         ("w2", (E, w.hidden, w.inter))):
        arr = np.empty(shape, dtype=dt)

        def fill(e, arr=arr, which=which):
            arr[e] = expert_weight(w, layer, which, e)

        nthreads = threads or min(16, os.cpu_count() or 1)
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, range(E)))
        out[which] = arr
    if w.n_shared:
        for which in ("w1", "w3", "w2"):
            out["s" + which] = shared_weight(w, layer, which)
    else:
        out["sw1"] = out["sw3"] = out["sw2"] = None
    return out


# --------------------------------------------------------------------------- liveness

def decoded_masks(w: Workload) -> np.ndarray:
    """D_i for every iteration, uint8 [iters x M]; D_0 is empty (a block starts fully masked)."""
    M, T = w.M, w.iters
    D = np.zeros((T, M), dtype=np.uint8)
    rng = _rng(w, 0, _T_LIVE)
    if w.liveness == "per_iter":
        order = rng.permutation(M)
        for i in range(1, T):
            n = min(M, i * w.commits_per_iter)
            D[i, order[:n]] = 1
    elif w.liveness == "uniform":
        commit_iter = rng.integers(0, T, size=M)  # position commits after forward c_t
        for i in range(T):
            D[i] = (commit_iter < i).astype(np.uint8)
    elif w.liveness == "forced":
        D[1:] = 1
    else:
        raise ValueError(w.liveness)
    return D


def force_masks(w: Workload) -> Optional[np.ndarray]:
    """Forced-fresh masks uint8 [iters x M] (a rotating window of ceil(f*M) positions), or None."""
    if w.liveness != "forced" or w.forced_fraction is None:
        return None
    M, T = w.M, w.iters
    n = int(math.ceil(w.forced_fraction * M))
    start = int(_rng(w, 0, _T_FORCE).integers(0, M))
    F = np.zeros((T, M), dtype=np.uint8)
    for i in range(T):
        idx = (start + i * n + np.arange(n)) % M
        F[i, idx] = 1
    return F


# --------------------------------------------------------------------------- hidden states

def hidden_states(w: Workload, layer: int, D: Optional[np.ndarray] = None,
                  iters: Optional[int] = None) -> np.ndarray:
    """x_i for every iteration, [iters x M x H] (uint16 bf16 bits or fp32).

    AR(1) drift x_i = rho x_{i-1} + sqrt(1 - rho^2) eps with rho = rho_decoded for
    positions in D_i and rho_live otherwise; with redraw_every > 0 the state is
    piecewise constant and redrawn from N(0,1) at every window start.
    """
    T = w.iters if iters is None else iters
    if D is None:
        D = decoded_masks(w)
    M, H = w.M, w.hidden
    rng = _rng(w, layer, _T_HIDDEN)
    out = np.empty((T, M, H), dtype=act_dtype(w))
    state = rng.standard_normal((M, H), dtype=np.float32)
    for i in range(T):
        if i > 0:
            if w.redraw_every:
                if i % w.redraw_every == 0:
                    state = rng.standard_normal((M, H), dtype=np.float32)
            else:
                rho = np.where(D[i].astype(bool), w.rho_decoded, w.rho_live).astype(np.float32)[:, None]
                eps = rng.standard_normal((M, H), dtype=np.float32)
                state = rho * state + np.sqrt(1.0 - rho * rho) * eps
        out[i] = f32_to_bf16_bits(state) if w.act == "bf16" else state
    return out


def describe_recipe() -> str:
    lines = []
    for i, w in WORKLOADS.items():
        lines.append(f"{i}: {w.name} M={w.M} iters={w.iters} R={w.staleness_R} layers={w.n_layers}")
    return "\n".join(lines)


def desc_fields(w: Workload, **overrides) -> dict:
    """The C-ABI descriptor fields (include/epoch.h, epoch_desc) of a workload."""
    f = dict(n_layers=w.n_layers, hidden=w.hidden, n_experts=w.n_experts, top_k=w.top_k,
             inter=w.inter, n_shared=w.n_shared, shared_inter=w.shared_inter if w.n_shared else 0,
             batch=w.batch, block=w.block, gate=1 if w.gate == "sigmoid" else 0,
             norm_topk=int(w.norm_topk), act_dtype=1 if w.act == "bf16" else 0,
             staleness_R=w.staleness_R, atlas_m=w.m_ext, atlas_B=w.B, atlas_c=w.c,
             alpha_num=w.alpha[0], alpha_den=w.alpha[1], q_num=w.q[0], q_den=w.q[1],
             beta_num=w.beta[0], beta_den=w.beta[1], flags=0,
             routing=1 if w.routing == "restricted" else 0, atlas_period=w.atlas_period,
             n_group=w.n_group, topk_group=w.topk_group)
    f.update(overrides)
    return f


def decode_inputs(seed: int, batch: int, block: int, hidden: int, vocab: int, steps: int = 1,
                  sigma: float = 0.02, lean_fraction: float = 0.4):
    """Seeded inputs of live-only output decoding: LM-head weights [V, H] (bf16 bits, N(0,
    sigma)), hidden states [steps, M, H] (bf16 bits) and the starting decoded mask [M] (u8,
    about a quarter of the positions).  A lean_fraction of the rows leans toward one token:
    h = c w_v / (sigma^2 H) + N(0, 1/4), which puts that token's logit about c above the
    others (c drawn from {6, 10, 14, 18, 22}); the rest are N(0, 1) rows.  With a vocabulary of
    thousands of tokens this spreads the top-token probability on both sides of 0.95."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7001]))
    M = batch * block
    W = (rng.standard_normal((vocab, hidden), dtype=np.float32) * np.float32(sigma))
    Wb = f32_to_bf16_bits(W)
    Wf = bf16_bits_to_f32(Wb)
    hs = np.empty((steps, M, hidden), dtype=np.uint16)
    for s in range(steps):
        h = rng.standard_normal((M, hidden), dtype=np.float32)
        lean = rng.random(M) < lean_fraction
        tok = rng.integers(0, vocab, size=M)
        c = rng.choice(np.array([6.0, 10.0, 14.0, 18.0, 22.0], np.float32), size=M)
        scale = (c / np.float32(sigma * sigma * hidden)).astype(np.float32)
        h[lean] = Wf[tok[lean]] * scale[lean, None] + 0.5 * h[lean]
        hs[s] = f32_to_bf16_bits(h)
    D = (rng.random(M) < 0.25).astype(np.uint8)
    return hs, Wb, D
