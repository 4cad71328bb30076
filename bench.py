#!/usr/bin/env python3
"""Benchmark of the liveness-sparse routed-expert MoE layer forward on one MI355X.

One step = one pass of the whole hot path over one block of synthetic input:
block-plan build (cold path), then for every refinement iteration and layer the
forward (router + top-k, support check / rebuild, fresh set, worklist, grouped
SwiGLU experts, shared expert, combine / stale merge / dense restore) and the
cache commit.  Inputs (weights, every iteration's hidden states and masks) are
resident in HBM before the timed region starts.

Prints one JSON line: fresh token-expert pairs/s over the timed steps, the
per-layer-iteration time, the roofline of the dominant kernel (measured live with
HIP events on the stream the kernels run on), the rooflines of the combine, the
router and the compaction steps (from the untimed per-kernel breakdown), and the
CPU oracle timed on a bounded sample of the same workload as a baseline.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
TIMED_EVERY = 4            # the timed region times the dominant kernel on every 4th forward
MFMA_BF16_PEAK_TFS = 2500.0  # dense bf16 MFMA, TFLOP/s
MFMA_FP64_PEAK_TFS = 78.6    # dense fp64 MFMA, TFLOP/s (the router's contraction)
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4,
                    help="workload id 1..5 (default 4: the largest single-GPU configuration)")
    ap.add_argument("--layers", type=int, default=0, help="layers to run (0 = all of the workload)")
    ap.add_argument("--fraction", type=float, default=None, help="forced fresh fraction (workload 5)")
    ap.add_argument("--R", type=int, default=None, help="staleness bound override")
    ap.add_argument("--routing", choices=("exact", "restricted"), default="exact",
                    help="top-K over all experts, or inside the layer's Atlas support")
    ap.add_argument("--atlas-period", type=int, default=0,
                    help="restricted routing: rebuild the support after this many iterations")
    ap.add_argument("--decode", action="store_true",
                    help="measure live-only output decoding (LM head on live rows + threshold "
                         "commit) instead of the MoE layer")
    ap.add_argument("--vocab", type=int, default=32768, help="--decode: vocabulary size")
    ap.add_argument("--decode-batch", type=int, default=0,
                    help="--decode: sequences of the workload's block length (default: the "
                         "workload's batch)")
    ap.add_argument("--n-group", type=int, default=0,
                    help="group-limited top-k: number of contiguous expert groups (0: off)")
    ap.add_argument("--topk-group", type=int, default=0,
                    help="group-limited top-k: groups each position selects from")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle work of the all-core CPU-baseline leg (the one-core leg: 2/3)")
    ap.add_argument("--cpu-rows", type=int, default=128,
                    help="positions whose expert outputs the all-core CPU-baseline leg evaluates "
                         "(the one-core leg: 1/8 of them)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB elementwise copy (HBM counter calibration)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 29  # 2^29 bf16 = 1 GiB read + 1 GiB written
    a = torch.randn(n, device="cuda", dtype=torch.bfloat16)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 2 * n, "bytes_written": 2 * n, "launches": 3}))


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in ("expert_gemm.h", "experts.hip", "epoch_internal.h", "device_common.h"):
        with open(os.path.join(ROOT, "block_diffusion_sparse_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload_name: str, kernel: str):
    """HBM traffic per launch from the committed rocprofv3 PMC summary, if it matches the source."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_hash():
        return None
    return t.get("bytes_per_launch")


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every expert is resident on one MI355X; no collectives). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from block_diffusion_sparse_amd import binding as B
    B.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.decode:
        bench_decode(args)
        return
    over = {}
    if args.fraction is not None:
        over["forced_fraction"] = args.fraction
    if args.R is not None:
        over["staleness_R"] = args.R
    if args.routing != "exact":
        over["routing"] = args.routing
        over["atlas_period"] = args.atlas_period
    if args.n_group > 1:
        over["n_group"] = args.n_group
        over["topk_group"] = args.topk_group
    w = synth.workload(args.workload, **over)
    n_layers = w.n_layers if args.layers <= 0 else min(args.layers, w.n_layers)
    M, H, I, E, K = w.M, w.hidden, w.inter, w.n_experts, w.top_k
    iters = w.iters

    # ---------------------------------------------------------------- inputs resident in HBM
    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    D = synth.decoded_masks(w)
    F = synth.force_masks(w)
    host_weights = []
    Wdev, Xdev = [], []
    for l in range(n_layers):
        Wl = synth.layer_weights(w, l)
        if l == 0:
            host_weights.append(Wl)
        Wdev.append({k: dev(v) for k, v in Wl.items()})
        Xdev.append(dev(synth.hidden_states(w, l, D)))
        if l > 0:
            del Wl
    Ddev = dev(D)
    Fdev = dev(F) if F is not None else None
    Y = torch.empty((M, H), dtype=Xdev[0].dtype, device="cuda")

    desc = B.make_desc(**synth.desc_fields(w, n_layers=n_layers))
    nbytes = B.epoch_plan_workspace_bytes(desc)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    lw = [B.layer_weights(d["router_w"], d.get("router_b"), d["w1"], d["w3"], d["w2"],
                          d.get("sw1"), d.get("sw3"), d.get("sw2")) for d in Wdev]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def one_block(timing_groups: int, every: int = 1):
        # timing_groups on every `every`-th forward (a timed dispatch costs a few us of gap on
        # each side, so the timed region samples its launches instead of timing them all)
        plan = B.epoch_block_plan_build(desc, lw, ws, nbytes, sp)
        n_fwd = 0
        for it in range(iters):
            for l in range(n_layers):
                if timing_groups and (every == 1 or n_fwd % every in (0, 1)):
                    B.epoch_plan_set_timing(plan, timing_groups if n_fwd % every == 0 else 0)
                n_fwd += 1
                B.epoch_moe_fresh_forward(plan, l, Xdev[l][it], Ddev[it],
                                          None if Fdev is None else Fdev[it], Y, None, sp)
                B.epoch_cache_update(plan, l, sp)
        return plan

    def layer_counters(plan, l):
        ins = B.epoch_plan_inspect(plan, l)
        off = ins.counters - ws.data_ptr()
        return ws[off:off + 8 * B.EPOCH_NUM_COUNTERS].view(torch.int64).cpu().numpy()

    def block_counters(plan):
        tot = sum(layer_counters(plan, l) for l in range(n_layers))
        return dict(zip(B.COUNTERS, tot.tolist()))

    def reference_block():
        """An untimed block, read after every forward: the block's counters and each forward's
        touched experts and fresh pairs (blocks are deterministic, so they hold for every
        block)."""
        plan = B.epoch_block_plan_build(desc, lw, ws, nbytes, sp)
        prev = [layer_counters(plan, l) for l in range(n_layers)]
        idx = [B.COUNTERS.index(n)
               for n in ("touched", "pairs", "big_experts", "big_pairs", "fresh_rows")]
        fwd = []
        for it in range(iters):
            for l in range(n_layers):
                B.epoch_moe_fresh_forward(plan, l, Xdev[l][it], Ddev[it],
                                          None if Fdev is None else Fdev[it], Y, None, sp)
                B.epoch_cache_update(plan, l, sp)
                c = layer_counters(plan, l)
                fwd.append(tuple(int(c[i] - prev[l][i]) for i in idx))
                prev[l] = c
        counters = block_counters(plan)
        B.epoch_block_plan_destroy(plan)
        return counters, fwd

    def collect(plans):
        ms_ = {g: 0.0 for g in B.TIMING_GROUPS}
        n_ = {g: 0 for g in B.TIMING_GROUPS}
        for p in plans:
            for g, (ms, n) in B.epoch_plan_timing(p).items():
                ms_[g] += ms
                n_[g] += n
            B.epoch_block_plan_destroy(p)
        return ms_, n_

    # ---------------------------------------------------------------- warmup
    for _ in range(args.warmup):
        B.epoch_block_plan_destroy(one_block(0))
    torch.cuda.synchronize()
    per_block, per_fwd = reference_block()
    # per-kernel breakdown (every group timed; outside the timed region).  Its events go back
    # to the library's pool, so the timed region below creates none.
    brk_ms, brk_n = collect([one_block(-1) for _ in range(args.steps)])

    # ---------------------------------------------------------------- timed region
    # the dominant expert kernel group (by the breakdown) is the one timed live, two events a
    # forward: the weight-stream tiles, or (shapes with them) the 256-row compute-bound tiles
    routed = [g for g in ("routed_gateup", "routed_down", "routed_gateup_big", "routed_down_big")
              if brk_n[g]]
    dom = max(routed, key=lambda g: brk_ms[g] / max(brk_n[g], 1))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    plans = [one_block(1 << B.TIMING_GROUPS.index(dom), TIMED_EVERY) for _ in range(args.steps)]
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    last = block_counters(plans[-1])
    assert last["pairs"] == per_block["pairs"], "blocks are not deterministic"
    group_ms, group_n = collect(plans)

    pairs_per_block = per_block["pairs"]
    ms_per_step = 1e3 * elapsed / args.steps
    value = pairs_per_block * args.steps / elapsed
    layer_iters = iters * n_layers
    us_per_layer_iter = 1e3 * ms_per_step / layer_iters

    # ---------------------------------------------------------------- roofline of the dominant kernel
    # the forwards the timed region timed (every TIMED_EVERY-th of each block): their touched
    # experts and fresh pairs, and how many of each the big tiles took, from the reference block
    sampled = per_fwd[::TIMED_EVERY]
    touched = sum(f[0] for f in sampled)     # experts with fresh pairs, summed over forwards
    P = sum(f[1] for f in sampled)
    Eb = sum(f[2] for f in sampled)          # of which on big tiles, and their pairs
    Pb = sum(f[3] for f in sampled)
    El, Pl = touched - Eb, P - Pb            # on the weight-stream tiles
    act = 2 if w.act == "bf16" else 4
    # (bound, algorithmic bytes, flops) per group over the sampled forwards
    work = {
        # W1 + W3 of every expert of the group, gathered x rows, h written
        "routed_gateup": ("hbm", El * 2 * I * H * act + Pl * H * act + Pl * I * act, 4.0 * Pl * H * I),
        # W2 of every expert of the group, h read, y_pair written
        "routed_down": ("hbm", El * H * I * act + Pl * I * act + Pl * H * act, 2.0 * Pl * H * I),
        "routed_gateup_big": ("mfma", Eb * 2 * I * H * act + Pb * (H + I) * act, 4.0 * Pb * H * I),
        "routed_down_big": ("mfma", Eb * H * I * act + Pb * (I + H) * act, 2.0 * Pb * H * I),
    }
    bound, nbytes, nflop = work[dom]
    launches = max(group_n[dom], 1)
    assert launches == len(sampled) * args.steps, (launches, len(sampled), args.steps)
    avg_ms = group_ms[dom] / launches
    steps = args.steps
    bytes_per_launch = nbytes * steps / launches
    flop_per_launch = nflop * steps / launches
    gbs = bytes_per_launch / (avg_ms * 1e-3) / 1e9
    tfs = flop_per_launch / (avg_ms * 1e-3) / 1e12
    traffic = load_traffic(w.name, dom)
    common = {"traffic": traffic, "kernel": dom,
              "algorithmic_bytes_per_launch": int(bytes_per_launch),
              "algorithmic_flop_per_launch": int(flop_per_launch),
              "avg_launch_us": round(avg_ms * 1e3, 2), "timed_launches": launches,
              "timed_every": TIMED_EVERY}
    if bound == "hbm":
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), **common,
                    "mfma_tflops": round(tfs, 2),
                    "mfma_frac_of_bf16_peak": round(tfs / MFMA_BF16_PEAK_TFS, 4)}
    else:
        roofline = {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS,
                    "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4), **common,
                    "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    kernels_us = {g: round(1e3 * brk_ms[g] / max(brk_n[g], 1), 2) for g in B.TIMING_GROUPS
                  if brk_n[g]}

    # ------------------------------------------------- rooflines of the other kernel groups
    # per launch, averaged over every forward of a block, against the breakdown pass's event
    # times (every group timed, so each carries a few us of event gap):
    #   combine: y_pair rows of the fresh pairs and cached rows of the stable positions read,
    #            y and the committed copy written, the shared expert's output read -> HBM;
    #   logits + top-k: 2 M E H flop in fp64 -> the fp64 MFMA peak (the top-k kernel is
    #            latency-bound and inside the same group);
    #   compaction (plan step + placement): ids and scores of the K_ext candidates read,
    #            the worklist (12 bytes a pair) and the inverse map written: latency-bound.
    n_fwd = max(len(per_fwd), 1)
    Pavg = sum(f[1] for f in per_fwd) / n_fwd
    Favg = sum(f[4] for f in per_fwd) / n_fwd
    Kx = w.k_ext
    other = {}
    if brk_n["combine"]:
        t = brk_ms["combine"] / brk_n["combine"] * 1e-3
        nb = (Pavg + (M - Favg) + 2 * M + (M if w.n_shared else 0)) * H * act
        other["combine"] = {"bound": "hbm", "achieved": round(nb / t / 1e9, 1),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(nb / t / 1e9 / HBM_PEAK_GBS, 4),
                            "algorithmic_bytes_per_launch": int(nb),
                            "avg_launch_us": round(t * 1e6, 2)}
    if brk_n["router"]:
        t = brk_ms["router"] / brk_n["router"] * 1e-3
        fl = 2.0 * M * E * H
        other["router"] = {"bound": "mfma_fp64", "achieved": round(fl / t / 1e12, 2),
                           "peak": MFMA_FP64_PEAK_TFS, "unit": "TFLOP/s",
                           "frac": round(fl / t / 1e12 / MFMA_FP64_PEAK_TFS, 4),
                           "algorithmic_flop_per_launch": int(fl),
                           "algorithmic_bytes_per_launch": int(M * H * act + 4 * E * H),
                           "avg_launch_us": round(t * 1e6, 2),
                           "groups": "logits + top-k"}
    t = sum(brk_ms[g] for g in ("plan", "place")) / max(brk_n["plan"], 1) * 1e-3
    if brk_n["plan"]:
        nb = M * Kx * 12 + Pavg * 12 + M * K * 4
        other["compaction"] = {"bound": "latency", "achieved": round(nb / t / 1e9, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(nb / t / 1e9 / HBM_PEAK_GBS, 4),
                               "algorithmic_bytes_per_launch": int(nb),
                               "avg_launch_us": round(t * 1e6, 2),
                               "groups": "plan step + placement"}
    kernels_share = {g: round(brk_ms[g] / max(sum(brk_ms.values()), 1e-9), 4)
                     for g in B.TIMING_GROUPS if brk_n[g]}

    # ---------------------------------------------------------------- CPU baseline (the oracle)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, host_weights[0], D, F, args.cpu_seconds, args.cpu_rows)

    rec = {
        "metric": "fresh token-expert pairs/s & MoE-layer µs/iteration; MFMA % peak; HBM GB/s",
        "value": round(value, 1),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.act == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": n_layers, "iterations_per_block": iters,
                   "positions": M, "hidden": H, "experts": E, "top_k": K, "inter": I,
                   "shared_expert": bool(w.n_shared), "staleness_R": w.staleness_R,
                   "forced_fraction": w.forced_fraction, "routing": w.routing,
                   "atlas_period": w.atlas_period, "n_group": w.n_group,
                   "topk_group": w.topk_group, "step": "one block"},
        "us_per_layer_iteration": round(us_per_layer_iter, 2),
        "fresh_pairs_per_block": pairs_per_block,
        "fresh_fraction": round(per_block["fresh_rows"] / (M * layer_iters), 4),
        "support_paths": {"cold": per_block["cold"], "hot_update": per_block["hot_update"],
                          "hot_skip": per_block["hot_skip"],
                          "restricted": per_block["restricted"],
                          "coverage_fallback": per_block["coverage_fallback"],
                          "repair_rounds": per_block["repair_rounds"]},
        "touched_experts_per_forward": round(per_block["touched"] / layer_iters, 2),
        "kernel_us_per_launch": kernels_us,
        "kernel_time_share": kernels_share,
        "roofline": roofline,
        "other_rooflines": other,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, Wl, D, F, seconds, n_rows):
    """The oracle on layer 0 of the same block, on the host's cores: all of them, then one.

    Every forward runs the discrete stages (router, top-k, support, fresh set, worklist) over
    all positions; expert outputs are evaluated on a seeded sample of positions (all of them
    when the block has no more than `n_rows`).  The per-fresh-row expert cost measured on the
    sample prices the fresh rows outside it, so the rate is that of whole iterations:
        pairs/s = sum of fresh pairs / (stage seconds + expert seconds per sampled fresh row
                                        x fresh rows).
    Iterations run in block order until the leg's budget is spent."""
    import numpy as np

    import oracle
    import synth
    X0 = synth.hidden_states(w, 0, D)
    order = np.random.default_rng(w.seed + 7).permutation(w.M)
    all_cores = oracle.num_threads()

    def leg(threads, rows_n, budget):
        oracle.set_num_threads(threads)
        rows = np.sort(order[:min(rows_n, w.M)]).astype(np.int32)
        L = oracle.OracleLayer(w, Wl, rows=rows)
        t_stage = t_expert = 0.0
        fresh_all = fresh_sampled = done = 0
        while done < w.iters and t_stage + t_expert < budget:
            out = L.forward(X0[done], D[done], None if F is None else F[done])
            L.commit()
            t_stage += L.last_stage_s
            t_expert += L.last_expert_s
            fresh_all += int(out["fresh"].sum())
            fresh_sampled += int(out["fresh"][rows].sum())
            done += 1
        per_row = t_expert / max(fresh_sampled, 1)
        t_full = t_stage + per_row * fresh_all
        pairs = fresh_all * w.top_k
        return {"value": round(pairs / t_full, 1), "cores": threads,
                "iterations": done, "rows_sampled": int(len(rows)),
                "fresh_rows": fresh_all, "fresh_rows_sampled": fresh_sampled,
                "stage_s": round(t_stage, 2), "expert_s_sampled": round(t_expert, 2),
                "expert_s_per_fresh_row": round(per_row, 5), "seconds_priced": round(t_full, 2)}

    multi = leg(all_cores, n_rows, seconds)
    single = leg(1, max(n_rows // 8, 1), seconds * 2 / 3)
    oracle.set_num_threads(all_cores)
    return {"value": multi["value"], "unit": "pairs/s", "cores": all_cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"layer 0, iterations 0-{multi['iterations'] - 1} of the block in order; "
                       f"router, top-k, support, fresh set and worklist over all {w.M} positions "
                       f"each iteration; expert outputs (double precision) on a seeded sample of "
                       f"{multi['rows_sampled']} positions, whose cost per fresh row "
                       f"({multi['expert_s_per_fresh_row']} s) prices all "
                       f"{multi['fresh_rows']} fresh rows"),
            "all_cores": multi, "one_core": single}


def bench_decode(args):
    """Live-only output decoding of one refinement step on the workload's block batch: the
    LM head ([V x H] bf16) over the live positions, then the threshold commit."""
    import numpy as np
    import torch

    import synth
    from block_diffusion_sparse_amd import binding as B
    w = synth.workload(args.workload)
    batch = args.decode_batch or w.batch
    M, H, V = batch * w.block, w.hidden, args.vocab
    hs, Wb, D = synth.decode_inputs(w.seed, batch, w.block, H, V)

    def dev(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    h, Wv, Dd = dev(hs[0]), dev(Wb), dev(D)
    d = B.make_decode_desc(batch, w.block, H, V)
    n = B.epoch_decode_workspace_bytes(d)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    Dn = torch.empty(M, dtype=torch.uint8, device="cuda")
    tok = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    conf = torch.empty(M, dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        B.epoch_live_decode(d, h, Wv, Dd, Dn, tok, conf, ws, n)
    reps = 10 * args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        B.epoch_live_decode(d, h, Wv, Dd, Dn, tok, conf, ws, n)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    live = int((D == 0).sum())
    # algorithmic bytes: the vocabulary once, the live rows, the partials (one per live row
    # and 256-token block; 128-token blocks from the streamed LM head, which takes up to 128
    # live rows, when the vocabulary has fewer 256-token blocks than the chip has CUs)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blk = 128 if (live <= 128 and V // 256 < n_cu) else 256
    lm_bytes = V * H * 2 + live * H * 2 + live * (V // blk) * 12
    flops = 2.0 * live * V * H
    print(json.dumps({
        "metric": "live positions decoded per second (LM head + threshold commit)",
        "value": round(live / dt, 1), "unit": "live positions/s", "n_gpus": 1,
        "steps": reps, "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"live-decode {batch}x{w.block} h{H} v{V}", "live": live,
                   "tau": 0.95},
        "us_per_step": round(dt * 1e6, 2),
        "lm_head_gbs": round(lm_bytes / dt / 1e9, 1),
        "lm_head_tflops": round(flops / dt / 1e12, 2),
    }), flush=True)


if __name__ == "__main__":
    main()
