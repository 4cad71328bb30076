"""Lock-step GPU-vs-oracle replay of MoE-layer blocks, shared by the GPU tests and smoke().

The HIP path runs through the C ABI (block_diffusion_sparse_amd.binding via
EpochPlan); the oracle replays the same block on the CPU from the same seeded
host arrays.  Every stage is compared each iteration:
  bit-exact: top-k ids, planner weights q, support and slots, fresh set and list,
             worklist order, offsets, inverse map, path counters;
  <= 1 ulp:  fp32 router logits;
  rtol 1e-6: gate scores and routing weights (fp32 of the oracle's double);
  row-normwise max_t |a_t - b_t|_inf / |b_t|_inf <= 2e-2 (bf16) or 1e-5 (fp32): outputs.
Plus the GPU-internal invariant that a stable row's routed output is its cache row,
bitwise, unchanged since the row's last fresh iteration.

Near ties: a position whose GPU ranking differs from the oracle's only among experts whose
logits are closer than NEAR_TIE is reported (counted and logged), not failed; the oracle then
takes the GPU's order for that position (after checking that it is a tie order of its own
logits) and the block continues, every stage still compared.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
import synth
from block_diffusion_sparse_amd import binding as B
from block_diffusion_sparse_amd.plan import EpochPlan

TOL = {"bf16": 2e-2, "f32": 1e-5}
NEAR_TIE = 1e-6


# the library's rule for compute-bound routed tiles (block_diffusion_sparse_amd/csrc/
# epoch_internal.h, kBigRows): experts with at least this many fresh pairs, on shapes whose
# iterations can hold 32768 pairs or more
BIG_ROWS = 128


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, device="cuda"):
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload_weights(W: dict, device="cuda") -> dict:
    return {k: to_dev(v, device) for k, v in W.items()}


def act_to_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype in (np.int16, np.uint16):
        return synth.bf16_bits_to_f32(a.view(np.uint16)).astype(np.float64)
    return a.astype(np.float64)


def rownorm_err(a: np.ndarray, b: np.ndarray) -> float:
    if a.size == 0:
        return 0.0
    den = np.maximum(np.abs(b).max(axis=-1), 1e-30)
    return float((np.abs(a - b).max(axis=-1) / den).max())


@dataclass
class BlockReport:
    iters: int = 0
    logits_ulp1: int = 0
    near_ties: int = 0
    max_err_y: float = 0.0
    max_err_routed: float = 0.0
    fresh_counts: list = field(default_factory=list)
    paths: list = field(default_factory=list)
    stable_rows_checked: int = 0
    rows_checked: int = 0
    big_experts: int = 0  # experts the worklist sends to 256-row compute-bound tiles, summed
    big_pairs: int = 0    # and their fresh pairs


def make_plan(w: synth.Workload, Wdev: list, n_layers: int) -> EpochPlan:
    desc = B.make_desc(**synth.desc_fields(w, n_layers=n_layers))
    return EpochPlan(desc, Wdev)


def _near_tie_rows(G_orc, ids_gpu, ids_orc):
    bad = np.nonzero((ids_gpu != ids_orc).any(1))[0]
    ties, real = [], []
    for t in bad:
        diff = ids_gpu[t] != ids_orc[t]
        experts = set(ids_gpu[t][diff].tolist()) | set(ids_orc[t][diff].tolist())
        g = G_orc[t, sorted(experts)].astype(np.float64)
        (ties if g.max() - g.min() < NEAR_TIE else real).append(int(t))
    return ties, real


def compare_iteration(w, out, ins, y, y_routed, it, rows, rep: BlockReport, prev_cache=None,
                      prev_fresh_gpu=None):
    """Compare one forward's stage outputs (GPU inspect views) with the oracle's."""
    M, K, E = w.M, w.top_k, w.n_experts
    g = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in ins.items()}
    tag = f"iter {it}"
    # router logits: the fp32-rounded value of an (almost) exact sum on both sides
    ulps = np.abs(g["logits"].view(np.int32).astype(np.int64) -
                  out["G"].view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, f"{tag}: router logits differ by {ulps.max()} ulp"
    rep.logits_ulp1 += int((ulps == 1).sum())
    # the oracle took the GPU's order on near-tie rows (run_block), so the ids agree in full
    assert np.array_equal(g["ids"], out["ids"]), f"{tag}: top-k ids differ"
    np.testing.assert_allclose(g["scores"], out["s"], rtol=1e-6, atol=1e-12, err_msg=tag)
    np.testing.assert_allclose(g["weights"], out["w"], rtol=1e-6, atol=1e-12, err_msg=tag)
    assert np.array_equal(g["atlas_q"], out["q"]), f"{tag}: planner weights q differ"
    nS = int(g["support_size"][0])
    assert np.array_equal(g["support"][:nS], out["S_list"]), f"{tag}: support differs"
    assert np.array_equal(g["slot_of"], out["slot_of"]), f"{tag}: slots differ"
    assert np.array_equal(g["in_support"], out["inS"]), f"{tag}: support mask differs"
    if w.routing == "restricted":
        assert np.array_equal(g["atlas"], out["inA"]), f"{tag}: Atlas support differs"
    # the routing the worklist used (all-expert top-K, or top-K inside the support)
    assert np.array_equal(g["routed_ids"], out["routed_ids"]), f"{tag}: routed ids differ"
    np.testing.assert_allclose(g["routed_w"], out["routed_w"], rtol=1e-6, atol=1e-12,
                               err_msg=tag)
    fresh = out["fresh"].astype(bool)
    assert np.array_equal(g["fresh"].astype(bool), fresh), f"{tag}: fresh set differs"
    nf = int(fresh.sum())
    assert int(g["n_fresh"][0]) == nf
    assert np.array_equal(g["fresh_list"][:nf], np.nonzero(fresh)[0]), f"{tag}: fresh list"
    wl = out["worklist"]
    P = wl["P"]
    assert int(g["n_pairs"][0]) == P
    assert np.array_equal(g["wl_pos"][:P], wl["wl_pos"]), f"{tag}: worklist positions differ"
    assert np.array_equal(g["wl_k"][:P], wl["wl_k"]), f"{tag}: worklist k differ"
    np.testing.assert_allclose(g["wl_w"][:P], wl["wl_w"], rtol=1e-6, atol=1e-12, err_msg=tag)
    assert np.array_equal(g["offs"][:nS + 1], wl["offs"]), f"{tag}: offsets differ"
    # bf16 shapes whose iterations can hold >= 32768 pairs run experts with >= BIG_ROWS fresh
    # pairs on the compute-bound tiles
    if w.act == "bf16" and w.M * w.top_k >= 32768:
        per_slot = np.diff(wl["offs"])
        rep.big_experts += int((per_slot >= BIG_ROWS).sum())
        rep.big_pairs += int(per_slot[per_slot >= BIG_ROWS].sum())
    assert np.array_equal(g["inv"], wl["inv"]), f"{tag}: inverse map differs"
    # outputs on the oracle's evaluated rows
    tol = TOL[w.act]
    y_np = act_to_f64(y.cpu().numpy())[rows]
    yr_np = act_to_f64(y_routed.cpu().numpy())[rows]
    e_y = rownorm_err(y_np, out["Y"])
    e_r = rownorm_err(yr_np, out["R"])
    assert e_y <= tol, f"{tag}: output error {e_y:.3g} > {tol}"
    assert e_r <= tol, f"{tag}: routed output error {e_r:.3g} > {tol}"
    rep.max_err_y = max(rep.max_err_y, e_y)
    rep.max_err_routed = max(rep.max_err_routed, e_r)
    rep.rows_checked += len(rows)
    # stable rows: routed output == cache row, bitwise, and the cache row did not move
    yr_raw = y_routed.cpu().numpy()
    cache = g["cache"]
    stable = np.nonzero(~fresh)[0]
    if len(stable):
        assert np.array_equal(yr_raw[stable], cache[stable]), f"{tag}: stable rows != cache"
        if prev_cache is not None:
            assert np.array_equal(cache[stable], prev_cache[stable]), f"{tag}: stale cache moved"
        rep.stable_rows_checked += len(stable)
    return True


def pick_rows(fresh, known, n, seed):
    """Rows whose outputs the oracle evaluates in one forward: a seeded sample of n fresh
    positions (all of them when fewer) and up to n/2 stable positions whose oracle cache row
    holds a computed value.  `fresh` (the GPU's flags) only chooses the sample; the fresh set
    itself is compared exactly."""
    rng = np.random.default_rng(seed)
    f = np.nonzero(fresh)[0]
    st = np.nonzero(~fresh & known)[0]
    pick = set(rng.choice(f, size=min(n, len(f)), replace=False).tolist()) if len(f) else set()
    if len(st):
        pick |= set(rng.choice(st, size=min(n // 2, len(st)), replace=False).tolist())
    return np.array(sorted(pick), dtype=np.int32)


def run_block(w: synth.Workload, layers=(0,), iters=None, rows=None, weights=None, Wdev=None,
              bias_override=None, force_override=None, check=True, verbose=True,
              D_override=None, hook=None, fresh_sample=None) -> BlockReport:
    """Replay one block of `iters` iterations over `layers` on GPU and oracle, comparing.

    rows: positions whose outputs the oracle evaluates on every forward (None = all).
    fresh_sample: instead, a new sample per forward of this many fresh positions plus stable
    positions whose oracle cache row was computed (pick_rows).
    hook(it, plan, orcs) runs before each iteration (e.g. to rebuild the plan mid-block); it
    may return a replacement (plan, orcs) pair.
    """
    iters = w.iters if iters is None else iters
    D = synth.decoded_masks(w) if D_override is None else D_override
    F = synth.force_masks(w) if force_override is None else force_override
    rep = BlockReport()
    if weights is None:
        weights = [synth.layer_weights(w, l) for l in layers]
    if bias_override is not None:
        for W in weights:
            W["router_b"] = bias_override
    if Wdev is None:
        Wdev = [upload_weights(W) for W in weights]
    plan = make_plan(w, Wdev, len(layers))
    orcs = [oracle.OracleLayer(w, W, rows=rows) for W in weights]
    X = [synth.hidden_states(w, l, D, iters=iters) for l in layers]
    Xdev = [to_dev(x) for x in X]
    Ddev = to_dev(D)
    Fdev = None if F is None else to_dev(F)
    prev_cache = [None] * len(layers)
    known = [np.zeros(w.M, dtype=bool) for _ in layers]  # oracle cache rows with a computed value
    for it in range(iters):
        if hook is not None:
            repl = hook(it, plan, orcs)
            if repl is not None:
                plan, orcs = repl
                prev_cache = [None] * len(layers)
        for li, l in enumerate(layers):
            x = Xdev[li][it]
            y = torch.empty_like(x)
            yr = torch.empty_like(x)
            force = None if Fdev is None else Fdev[it]
            plan.forward(li, x, Ddev[it], force, y, yr)
            torch.cuda.synchronize()
            ins = plan.inspect(li)
            pick = None
            if fresh_sample:
                pick = pick_rows(ins["fresh"].cpu().numpy().astype(bool), known[li], fresh_sample,
                                 [w.seed, l, it, 99])
            # ranking first: rows where the GPU's order differs from the oracle's only among
            # logits closer than NEAR_TIE are ties (both orders correct); they are reported and
            # the oracle continues on the GPU's order, so every later stage stays comparable
            pre = orcs[li].route(X[li][it])
            ids_g = ins["ids"].cpu().numpy()
            tie_ids = None
            if not np.array_equal(ids_g, pre["ids"]):
                ties, real = _near_tie_rows(pre["G"], ids_g, pre["ids"])
                assert not real, f"iter {it}: top-k ids differ on rows {real[:8]} (not near-ties)"
                rep.near_ties += len(ties)
                log(f"  iter {it}: {len(ties)} near-tie rows (logit gap < {NEAR_TIE}) reported; "
                    "the oracle continues on the GPU's order")
                tie_ids = {t: ids_g[t].copy() for t in ties}
            routed_g = ins["routed_ids"].cpu().numpy()

            def tie_routed(rids, it=it):
                # the same for the ranking inside the support (restricted routing)
                if np.array_equal(routed_g, rids):
                    return None
                ties, real = _near_tie_rows(pre["G"], routed_g, rids)
                assert not real, f"iter {it}: routed ids differ on rows {real[:8]} (not near-ties)"
                rep.near_ties += len(ties)
                log(f"  iter {it}: {len(ties)} near-tie rows in the routing inside the support "
                    "reported; the oracle continues on the GPU's order")
                return {t: routed_g[t].copy() for t in ties}

            out = orcs[li].forward(X[li][it], D[it], None if F is None else F[it], rows=pick,
                                   pre=pre, tie_ids=tie_ids, tie_routed=tie_routed)
            ofresh = out["fresh"].astype(bool)
            evaluated = np.zeros(w.M, dtype=bool)
            evaluated[out["rows"]] = True
            known[li] = np.where(ofresh, evaluated, known[li])
            if check:
                compare_iteration(w, out, ins, y, yr, it, out["rows"], rep, prev_cache[li])
            prev_cache[li] = ins["cache"].cpu().numpy().copy()
            rep.fresh_counts.append(int(out["fresh"].sum()))
            rep.paths.append(out["path"])
            plan.commit(li)
            orcs[li].commit()
        rep.iters += 1
        if verbose:
            nfr = int(out["fresh"][out["rows"]].sum())
            log(f"  iter {it}: fresh {rep.fresh_counts[-1]}/{w.M} path {rep.paths[-1]} "
                f"rows compared {len(out['rows'])} ({nfr} fresh) err_y {rep.max_err_y:.2e}")
    torch.cuda.synchronize()
    for li, l in enumerate(layers):
        c = plan.counters(li)
        oc = orcs[li].counters
        assert c["cold"] == oc["cold"] and c["hot_update"] == oc["hot_update"]
        assert c["hot_skip"] == oc["hot_skip"] and c["anomaly"] == oc["anomalies"]
        assert c["fresh_rows"] == oc["fresh_rows"] and c["pairs"] == oc["pairs"]
        assert plan.inspect(li)["iteration"] == c["forwards"] == orcs[li].iter
        assert c["restricted"] == oc["restricted"]
        assert c["coverage_fallback"] == oc["coverage_fallback"]
        assert c["period_update"] == oc["period_update"]
    if check and len(layers) == 1:
        c = plan.counters(0)
        assert c["big_experts"] == rep.big_experts and c["big_pairs"] == rep.big_pairs, (
            c["big_experts"], rep.big_experts, c["big_pairs"], rep.big_pairs)
    rep.counters = [plan.counters(li) for li in range(len(layers))]
    plan.close()
    return rep
