"""Fit the router-bias scale of the Zipf-skewed workloads; writes synth/zipf_scale.json.

The workloads with a Zipf load ask for gate biases under which the expert load
(number of top-k selections per expert) follows rank^-a.  The bias is
b_e = -s * ln(rank_e) for a seeded rank permutation; this script bisects s so
that the least-squares slope of log(load) against log(rank) over the 64 most
loaded experts equals -a.  Loads are measured with the oracle's router and
top-k on 1024 N(0,1) positions drawn from the workload's own seed.

Run: python oracle/calibrate_zipf.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402
import synth  # noqa: E402
from synth import workloads as wl  # noqa: E402

ROWS = 1024
TOP = 64


def slope_for(w, s, x, Wg):
    b = wl.router_bias(w, 0, scale=s)
    G = oracle.router_logits(x, Wg, b)
    ids, _, _, _ = oracle.route(G, w.top_k, w.top_k, w.gate == "sigmoid", w.norm_topk)
    load = np.bincount(ids.ravel(), minlength=w.n_experts).astype(np.float64)
    load = np.sort(load)[::-1][:TOP]
    load = np.maximum(load, 0.5)
    r = np.arange(1, TOP + 1, dtype=np.float64)
    return np.polyfit(np.log(r), np.log(load), 1)[0]


def calibrate(w):
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 999]))
    x = rng.standard_normal((ROWS, w.hidden), dtype=np.float32)
    x = synth.f32_to_bf16_bits(x) if w.act == "bf16" else x
    Wg = wl.router_weight(w, 0)
    lo, hi = 0.0, 4.0
    for _ in range(24):
        mid = 0.5 * (lo + hi)
        if slope_for(w, mid, x, Wg) > -w.zipf:
            lo = mid
        else:
            hi = mid
    s = 0.5 * (lo + hi)
    return s, slope_for(w, s, x, Wg)


def main():
    out = {}
    for i, w in synth.WORKLOADS.items():
        if w.zipf is None:
            continue
        key = f"{w.n_experts}:{w.top_k}:{w.hidden}:{w.sigma}:{w.gate}:{w.zipf}"
        s, slope = calibrate(w)
        print(f"workload {i} ({w.name}): s = {s:.6f}, fitted slope {slope:.4f}", flush=True)
        out[key] = round(s, 6)
    path = os.path.join(os.path.dirname(wl.__file__), "zipf_scale.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
