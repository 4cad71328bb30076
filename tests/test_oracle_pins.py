"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Each pin compares the oracle with something other than itself: a library
routine that computes the same definition (numpy matmul, stable argsort,
scipy softmax / expit, Python's sorted), a closed form, a special case, a
hand-worked example, or an invariant the pages state.  `test_planted_mistakes`
rebuilds the oracle with one mistake planted at a time and checks that some
pin fails for each.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- independent helpers

def f64(a):
    return synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def np_router(x, Wg, b):
    G = f64(x) @ Wg.astype(np.float64).T
    if b is not None:
        G = G + b.astype(np.float64)
    return G.astype(np.float32)


def np_swiglu(xrow, W1, W3, W2):
    g = f64(W1) @ xrow
    u = f64(W3) @ xrow
    return f64(W2) @ (g * expit(g) * u)


def np_dense(x, W, K, sigmoid, norm):
    xf = f64(x)
    G = np_router(x, W["router_w"], W["router_b"])
    order = np.argsort(-G, axis=1, kind="stable")[:, :K]
    s = expit(G.astype(np.float64)) if sigmoid else softmax(G.astype(np.float64), axis=1)
    M, H = xf.shape
    R = np.zeros((M, H))
    Y = np.zeros((M, H))
    for t in range(M):
        wt = s[t, order[t]]
        if norm:
            wt = wt / wt.sum()
        for e, we in zip(order[t], wt):
            R[t] += we * np_swiglu(xf[t], W["w1"][e], W["w3"][e], W["w2"][e])
        Y[t] = R[t]
        if W.get("sw1") is not None:
            Y[t] += np_swiglu(xf[t], W["sw1"], W["sw3"], W["sw2"])
    return R, Y


def rownorm_err(a, b):
    den = np.maximum(np.abs(b).max(axis=-1), 1e-300)
    return float((np.abs(a - b).max(axis=-1) / den).max())


def small_workload(**kw):
    base = dict(name="small", hidden=64, n_experts=16, top_k=4, inter=24, n_shared=1,
                shared_inter=20, batch=2, block=8, iters=6, staleness_R=3, n_layers=1,
                zipf=None, sigma=0.1)
    base.update(kw)
    return synth.workload(3, **base)


def rand_x(rng, M, H, bf16):
    x = rng.standard_normal((M, H), dtype=np.float32)
    return synth.f32_to_bf16_bits(x) if bf16 else x


# ----------------------------------------------------------------- pins (each takes the library)

def pin_router(orc, lib):
    rng = np.random.default_rng(5)
    for bf16 in (True, False):
        M, H, E = 37, 96, 13
        x = rand_x(rng, M, H, bf16)
        Wg = rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.05)
        b = rng.standard_normal(E).astype(np.float32)
        G = orc.router_logits(x, Wg, b, lib=lib)
        ref = np_router(x, Wg, b)
        ulps = np.abs(G.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
        assert ulps.max() <= 1, "router logits differ from fp32(x W^T + b) by more than 1 ulp"
        assert (ulps == 0).mean() > 0.99
    # one-hot rows select a column of W exactly: G[t, e] = fp32(W[e, t] + b[e])
    H = E = 8
    x = np.eye(H, dtype=np.float32)
    Wg = rng.standard_normal((E, H), dtype=np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    G = orc.router_logits(x, Wg, b, lib=lib)
    assert np.array_equal(G, (Wg.T.astype(np.float64) + b.astype(np.float64)).astype(np.float32))


def pin_topk(orc, lib):
    rng = np.random.default_rng(6)
    M, E, K, Kext = 50, 24, 4, 9
    G = rng.standard_normal((M, E)).astype(np.float32)
    G[:, 7] = G[:, 3]               # exact ties between experts 3 and 7 ...
    G[::2, 3] = G[::2, 7] = 9.0     # ... that sit at the top on even rows
    ids, s, w, q = orc.route(G, K, Kext, True, True, lib=lib)
    ref = np.argsort(-G, axis=1, kind="stable")[:, :Kext]
    assert np.array_equal(ids, ref), "top-k must equal a stable sort on (-G) (ties -> lower id)"
    assert (ids[::2, 0] == 3).all() and (ids[::2, 1] == 7).all()


def pin_weights(orc, lib):
    rng = np.random.default_rng(7)
    M, E, K, Kext = 40, 16, 4, 8
    G = rng.standard_normal((M, E)).astype(np.float32)
    for sigmoid in (True, False):
        for norm in (True, False):
            ids, s, w, q = orc.route(G, K, Kext, sigmoid, norm, lib=lib)
            full = expit(G.astype(np.float64)) if sigmoid else softmax(G.astype(np.float64), axis=1)
            s_ref = np.take_along_axis(full, ids, axis=1)
            np.testing.assert_allclose(s, s_ref, rtol=1e-13, atol=0)
            w_ref = s_ref[:, :K] / s_ref[:, :K].sum(1, keepdims=True) if norm else s_ref[:, :K]
            np.testing.assert_allclose(w, w_ref, rtol=1e-13, atol=0)
            assert np.array_equal(q, np.floor(s * 65536.0 + 0.5).astype(np.int64))
            if norm:
                np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-13)
            elif not sigmoid:
                assert (w.sum(1) <= 1.0 + 1e-12).all()
    ids, s, w, q = orc.route(G, E, E, False, False, lib=lib)   # K = E softmax: all mass
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-13)


def pin_score_given(orc, lib):
    """Scoring a selection the top-k itself produced reproduces its scores bit for bit, and
    swapping two experts whose logits tie exactly is a valid order with swapped scores."""
    rng = np.random.default_rng(21)
    M, E, K, Kext = 30, 16, 4, 8
    G = rng.standard_normal((M, E)).astype(np.float32)
    G[:, 9] = G[:, 2]
    for sigmoid in (True, False):
        for norm in (True, False):
            ids, s, w, q = orc.route(G, K, Kext, sigmoid, norm, lib=lib)
            s2, w2, q2 = orc.score_given(G, ids, K, sigmoid, norm, lib=lib)
            assert np.array_equal(s, s2) and np.array_equal(w, w2) and np.array_equal(q, q2)
            t = int(np.nonzero((ids == 2).any(1) & (ids == 9).any(1))[0][0])
            alt = ids[t].copy()
            i2, i9 = int(np.nonzero(alt == 2)[0][0]), int(np.nonzero(alt == 9)[0][0])
            alt[i2], alt[i9] = 9, 2
            assert orc.tie_order_ok(G[t], ids[t], alt, 1e-6)
            assert not orc.tie_order_ok(G[t], ids[t], np.roll(ids[t], 1), 1e-6)
            s3, _, q3 = orc.score_given(G[t:t + 1], alt[None], K, sigmoid, norm, lib=lib)
            assert np.array_equal(s3[0][[i2, i9]], s[t][[i9, i2]]) and np.array_equal(q3[0][[i2, i9]], q[t][[i9, i2]])


def pin_atlas_hand(orc, lib):
    with open(os.path.join(GOLDEN, "atlas_hand_worked.json")) as f:
        g = json.load(f)
    inst = g["instance"]
    ids = np.array(inst["ids"], dtype=np.int32)
    q = np.array(inst["q"], dtype=np.int64)
    for case in g["cases"]:
        inS, slot_of, S, stats = orc.support_build(ids, q, inst["E"], inst["K"], inst["B"],
                                                   case["c"], case["alpha"], case["q"],
                                                   case["beta"], lib=lib)
        assert list(S) == case["support"], case["name"]
        assert int(stats[1]) == case["rounds"], case["name"]
        assert int(stats[0]) == case["final_U"], case["name"]
        assert int(stats[2]) == case["unmet"], case["name"]
        assert int(stats[4]) == len(case["support_before_closure"]), case["name"]


def pin_atlas_special(orc, lib):
    rng = np.random.default_rng(8)
    M, E, K, Kext = 64, 32, 4, 8
    G = (rng.standard_normal((M, E)) + np.linspace(2, -2, E)).astype(np.float32)
    ids, s, w, q = orc.route(G, K, Kext, True, True, lib=lib)
    p = np.bincount(ids.ravel(), weights=q.ravel(), minlength=E).astype(np.int64)
    closure = set(ids[:, :K].ravel().tolist())
    # alpha = 0: nothing is under-covered; S = top-B by popularity (p desc, id asc) plus closure
    for B in (0, 3, 10):
        inS, slot_of, S, stats = orc.support_build(ids, q, E, K, B, 4, (0, 1), (95, 100), (1, 1), lib=lib)
        order = sorted([e for e in range(E) if p[e] > 0], key=lambda e: (-p[e], e))[:B]
        assert set(S.tolist()) == set(order) | closure
        assert stats[1] == 0 and stats[0] == 0
    # B at least the number of experts with popularity: S = every candidate expert
    inS, slot_of, S, stats = orc.support_build(ids, q, E, K, E, 4, (9, 10), (95, 100), (1, 1), lib=lib)
    assert set(S.tolist()) == set(np.nonzero(p > 0)[0].tolist())
    # invariants on the real goal: closure inside S, goal met or flagged, slots are ranks
    for B, c in ((2, 1), (4, 2), (8, 4)):
        inS, slot_of, S, stats = orc.support_build(ids, q, E, K, B, c, (9, 10), (95, 100), (1, 1), lib=lib)
        assert closure <= set(S.tolist())
        assert stats[2] == 1 or 100 * stats[0] <= 5 * M
        assert list(S) == sorted(S)
        assert all(slot_of[e] == i for i, e in enumerate(S))
        assert (slot_of[[e for e in range(E) if e not in set(S.tolist())]] == -1).all()


def pin_fresh(orc, lib):
    # tiny fp32 workload: 4 commits per iteration, R = 2 -> fresh counts 16, 16, 12, 12
    w = synth.workload(1)
    D = synth.decoded_masks(w)
    M = w.M
    valid = np.zeros(M, np.uint8)
    last = np.full(M, -(1 << 30), np.int32)
    prev = np.zeros(M, np.uint8)
    counts = []
    for i in range(w.iters):
        fresh, an = orc.fresh_set(w.staleness_R, i, valid, last, prev, D[i], lib=lib)
        counts.append(int(fresh.sum()))
        lib.orc_commit(M, i, fresh.ctypes.data_as(np.ctypeslib.ctypes.c_void_p),
                       D[i].ctypes.data_as(np.ctypeslib.ctypes.c_void_p),
                       valid.ctypes.data_as(np.ctypeslib.ctypes.c_void_p),
                       last.ctypes.data_as(np.ctypeslib.ctypes.c_void_p),
                       prev.ctypes.data_as(np.ctypeslib.ctypes.c_void_p))
    assert counts == [16, 16, 12, 12], counts


def pin_worklist(orc, lib):
    rng = np.random.default_rng(9)
    M, E, K, Kext = 45, 20, 3, 5
    G = rng.standard_normal((M, E)).astype(np.float32)
    ids, s, w, q = orc.route(G, K, Kext, False, False, lib=lib)
    fresh = (rng.random(M) < 0.6).astype(np.uint8)
    used = sorted(set(ids[:, :K].ravel().tolist()) | {0, 19})
    slot_of = np.full(E, -1, np.int32)
    slot_of[used] = np.arange(len(used))
    wl = orc.worklist(ids, w, K, fresh, slot_of, len(used), lib=lib)
    pairs = sorted((int(ids[t, k]), t, k) for t in range(M) if fresh[t] for k in range(K))
    assert wl["P"] == len(pairs)
    assert [(int(ids[t, k]), int(t), int(k)) for t, k in zip(wl["wl_pos"], wl["wl_k"])] == pairs
    cnt = np.bincount([slot_of[e] for e, _, _ in pairs], minlength=len(used))
    assert np.array_equal(wl["offs"], np.concatenate([[0], np.cumsum(cnt)]))
    for p, (t, k) in enumerate(zip(wl["wl_pos"], wl["wl_k"])):
        assert wl["inv"][t, k] == p and wl["wl_w"][p] == w[t, k]
    assert (wl["inv"][fresh == 0] == -1).all()


def pin_expert(orc, lib):
    rng = np.random.default_rng(10)
    for bf16 in (True, False):
        H, I = 40, 28
        x = rand_x(rng, 1, H, bf16)[0]
        W1, W3 = rand_x(rng, I, H, bf16), rand_x(rng, I, H, bf16)
        W2 = rand_x(rng, H, I, bf16)
        y = orc.expert(x, W1, W3, W2, lib=lib)
        np.testing.assert_allclose(y, np_swiglu(f64(x), W1, W3, W2), rtol=1e-12, atol=1e-14)


def pin_dense(orc, lib):
    w = small_workload()
    W = synth.layer_weights(w, 0)
    W["router_b"] = np.random.default_rng(11).standard_normal(w.n_experts).astype(np.float32)
    x = synth.hidden_states(w, 0)[0]
    for sig, norm in ((True, True), (False, False)):
        R, Y = orc.dense_moe(x, W["router_w"], W["router_b"], W["w1"], W["w3"], W["w2"],
                             W["sw1"], W["sw3"], W["sw2"], w.top_k, sig, norm, lib=lib)
        Rr, Yr = np_dense(x, W, w.top_k, sig, norm)
        assert rownorm_err(R, Rr) < 1e-12 and rownorm_err(Y, Yr) < 1e-12


def pin_all_fresh_equals_dense(orc, lib):
    # staleness bound R = 1: every iteration is exact and equals the dense layer
    w = small_workload(staleness_R=1)
    W = synth.layer_weights(w, 0)
    D = synth.decoded_masks(w)
    X = synth.hidden_states(w, 0, D)
    L = orc.OracleLayer(w, W, lib=lib)
    for i in range(w.iters):
        out = L.forward(X[i], D[i])
        assert out["fresh"].all()
        Rr, Yr = np_dense(X[i], W, w.top_k, True, True)
        assert rownorm_err(out["R"], Rr) < 1e-12 and rownorm_err(out["Y"], Yr) < 1e-12
        L.commit()


def pin_staleness(orc, lib):
    # stable rows reuse the routed output of their last fresh iteration, bitwise, and
    # that output is the dense routed output of that iteration; age <= R - 1
    w = small_workload(staleness_R=3, iters=9)
    W = synth.layer_weights(w, 0)
    D = synth.decoded_masks(w)
    X = synth.hidden_states(w, 0, D)
    L = orc.OracleLayer(w, W, lib=lib)
    dense_R = []
    n_stable = 0
    for i in range(w.iters):
        dense_R.append(np_dense(X[i], W, w.top_k, True, True)[0])
        last = L.last_fresh.copy()
        cache = L.cache.copy()
        out = L.forward(X[i], D[i])
        fresh = out["fresh"].astype(bool)
        newly = D[i].astype(bool) & ~L.prev_D.astype(bool)
        assert fresh[~D[i].astype(bool)].all() and fresh[newly].all()
        for t in np.nonzero(~fresh)[0]:
            n_stable += 1
            assert 0 <= i - last[t] <= w.staleness_R - 1
            assert np.array_equal(out["R"][t], cache[t])
            assert rownorm_err(out["R"][t:t + 1], dense_R[last[t]][t:t + 1]) < 1e-12
        assert rownorm_err(out["R"][fresh], dense_R[i][fresh]) < 1e-12
        L.commit()
    assert n_stable > 0


def pin_restricted_topk(orc, lib):
    """Top-K inside a support mask against a masked stable sort (brute force), with the
    scores defined over all experts; the all-experts mask reduces to the plain top-K."""
    rng = np.random.default_rng(11)
    M, E, K = 45, 20, 4
    G = rng.standard_normal((M, E)).astype(np.float32)
    G[:, 9] = G[:, 4]                       # exact ties inside the support
    inA = np.zeros(E, np.uint8)
    inA[[0, 2, 4, 5, 9, 11, 12, 17, 19]] = 1
    for sigmoid in (True, False):
        for norm in (True, False):
            rids, rw = orc.route_restricted(G, K, inA, sigmoid, norm, lib=lib)
            masked = np.where(inA.astype(bool)[None, :], -G.astype(np.float64), np.inf)
            ref = np.argsort(masked, axis=1, kind="stable")[:, :K]
            assert np.array_equal(rids, ref), "restricted top-K must be the masked stable sort"
            assert inA[rids].all()
            full = expit(G.astype(np.float64)) if sigmoid else softmax(G.astype(np.float64), axis=1)
            sk = np.take_along_axis(full, ref, axis=1)
            np.testing.assert_allclose(rw, sk / sk.sum(1, keepdims=True) if norm else sk,
                                       rtol=1e-13, atol=0)
    ids, s, w, q = orc.route(G, K, 2 * K, False, True, lib=lib)
    rids, rw = orc.route_restricted(G, K, np.ones(E, np.uint8), False, True, lib=lib)
    assert np.array_equal(rids, ids[:, :K]) and np.array_equal(rw, w)


def pin_atlas_without_closure(orc, lib):
    """The restricted-routing support is the hand-worked support before its closure step,
    and the exact-mode support is exactly that set plus every routed expert."""
    with open(os.path.join(GOLDEN, "atlas_hand_worked.json")) as f:
        g = json.load(f)
    inst = g["instance"]
    ids = np.array(inst["ids"], dtype=np.int32)
    q = np.array(inst["q"], dtype=np.int64)
    for case in g["cases"]:
        args = (ids, q, inst["E"], inst["K"], inst["B"], case["c"], case["alpha"], case["q"],
                case["beta"])
        inA, _, A, stats = orc.atlas_build(*args, lib=lib)
        assert list(A) == case["support_before_closure"], case["name"]
        inS, _, S, _ = orc.support_build(*args, lib=lib)
        assert set(S.tolist()) == set(A.tolist()) | set(ids[:, :inst["K"]].ravel().tolist())
    rng = np.random.default_rng(12)
    M, E, K, Kext = 64, 32, 4, 8
    G = (rng.standard_normal((M, E)) + np.linspace(2, -2, E)).astype(np.float32)
    ids, s, w, q = orc.route(G, K, Kext, True, True, lib=lib)
    for B, c in ((2, 1), (4, 2), (8, 4)):
        inA, _, A, st = orc.atlas_build(ids, q, E, K, B, c, (9, 10), (95, 100), (1, 1), lib=lib)
        inS, _, S, _ = orc.support_build(ids, q, E, K, B, c, (9, 10), (95, 100), (1, 1), lib=lib)
        assert set(S.tolist()) == set(A.tolist()) | set(ids[:, :K].ravel().tolist())
        assert int(st[4]) == len(A)


def pin_support_lifecycle(orc, lib):
    """Teardown, "cold / hot-update / hot-skip": a forward keeps the block's support
    (hot-skip) while every routed expert has a slot in it, and rebuilds it (hot-update)
    once one does not.  Only the K routed experts decide this: the planner's extra
    candidates (ranks K..K_ext-1) are not routed and need no slot.

    Hand-built block: one-hot hidden rows make the logits the router's columns, so every
    position routes to experts {0, 1} and ranks experts 2..9 as its extra candidates.
    With B = 0 and alpha = 0 the support is the closure {0, 1} alone, so the extra
    candidates lie outside it on every iteration."""
    w = small_workload(n_experts=16, top_k=2, atlas_m=2, atlas_B=0, alpha=(0, 1), iters=5,
                       n_shared=0, shared_inter=0, liveness="uniform")
    M, H, E, K, Kext = w.M, w.hidden, w.n_experts, w.top_k, w.k_ext
    assert Kext == 4 and M <= H
    G = np.full((M, E), -5.0, np.float32)
    for t in range(M):
        G[t, 0], G[t, 1] = 5.0, 4.0
        G[t, 2 + t % 4], G[t, 6 + t % 4] = 3.0, 2.0
    Wl = dict(synth.layer_weights(w, 0))
    Wl["router_w"] = np.zeros((E, H), np.float32)
    Wl["router_w"][:, :M] = G.T
    Wl["router_b"] = None
    x = synth.f32_to_bf16_bits(np.eye(M, H, dtype=np.float32))
    D = np.zeros(M, np.uint8)
    L = orc.OracleLayer(w, Wl, lib=lib)
    paths = []
    for it in range(w.iters):
        out = L.forward(x, D)
        assert set(out["ids"][:, K:].ravel().tolist()) == set(range(2, 10))
        assert out["S_list"].tolist() == [0, 1]
        paths.append(out["path"])
        L.commit()
    assert paths == [1] + [0] * (w.iters - 1)
    assert (L.counters["cold"], L.counters["hot_update"], L.counters["hot_skip"]) == (1, 0, w.iters - 1)
    # a routed expert outside the support: hot-update; no support yet: cold
    ids = np.ascontiguousarray(out["ids"]).copy()
    inS = out["inS"]
    assert orc.support_status(ids, K, inS, True, lib=lib) == 0
    ids[3, 1] = 12
    assert orc.support_status(ids, K, inS, True, lib=lib) == 2
    assert orc.support_status(ids, K, inS, False, lib=lib) == 1


def pin_under_covered(orc, lib):
    """Teardown, Expert Atlas, the U_l equation: a position is under-covered when the
    support's share of its candidate weight is strictly below alpha times its top-K weight.
    Hand-worked rows with alpha = 3/4 and S = {0, 2} (C = covered weight, R = top-K weight):
      row 0  C 150, R 200: 4*150 = 600 = 3*200, on the boundary -> covered
      row 1  C 120, R 200: 480 < 600                       -> under-covered
      row 2  C 180, R 180: 720 >= 540                      -> covered
      row 3  C  60, R 120: 240 < 360                       -> under-covered
      row 4  C  30, R 120: 120 < 360                       -> under-covered
      row 5  C  90, R 120: 360 = 360, on the boundary      -> covered"""
    ids = np.array([[0, 1, 2, 3], [1, 0, 3, 2], [2, 0, 1, 4],
                    [4, 5, 0, 2], [1, 3, 0, 2], [0, 4, 2, 5]], np.int32)
    q = np.array([[100, 100, 50, 50], [120, 80, 40, 40], [90, 90, 10, 10],
                  [60, 60, 30, 30], [80, 40, 20, 10], [60, 60, 30, 30]], np.int64)
    inS = np.zeros(6, np.uint8)
    inS[[0, 2]] = 1
    assert orc.under_covered(ids, q, 2, inS, (3, 4), lib=lib) == 3
    assert orc.under_covered(ids, q, 2, inS, (0, 1), lib=lib) == 0        # alpha = 0: none
    assert orc.under_covered(ids, q, 2, np.ones(6, np.uint8), (1, 1), lib=lib) == 0  # C >= R
    assert orc.under_covered(ids, q, 2, np.zeros(6, np.uint8), (1, 1), lib=lib) == 6


def pin_restricted_lifecycle(orc, lib):
    """Support-restricted routing over small blocks:
    - the first forward (cold) and every rebuild route over all experts;
    - hot-skip forwards route inside the support (masked stable sort of the logits);
    - with the support holding every routed expert, restricted routing reproduces the
      exact mode bit for bit (ids, weights, outputs, cache);
    - an update period rebuilds on schedule; a support built on one hidden state and
      confronted with an unrelated one fails the coverage goal and falls back."""
    w = small_workload(routing="restricted", n_experts=16, top_k=3, iters=6,
                       liveness="uniform", n_shared=0, shared_inter=0)
    Wl = synth.layer_weights(w, 0)
    D = synth.decoded_masks(w)
    X = synth.hidden_states(w, 0, D)
    L = orc.OracleLayer(w, Wl, lib=lib)
    for it in range(w.iters):
        out = L.forward(X[it], D[it])
        K = w.top_k
        if out["path"]:
            assert np.array_equal(out["routed_ids"], out["ids"][:, :K])
            assert np.array_equal(out["routed_w"], out["w"])
        else:
            masked = np.where(out["inA"].astype(bool)[None, :], -out["G"].astype(np.float64), np.inf)
            assert np.array_equal(out["routed_ids"], np.argsort(masked, axis=1, kind="stable")[:, :K])
        assert set(out["routed_ids"].ravel().tolist()) <= set(out["S_list"].tolist())
        L.commit()
    assert L.counters["cold"] == 1 and L.counters["restricted"] == L.counters["hot_skip"]
    # B = E: the support holds every candidate expert, so no routed expert is ever outside it
    wx = w.replace(routing="exact", atlas_B=w.n_experts)
    wr = w.replace(routing="restricted", atlas_B=w.n_experts)
    Lx = orc.OracleLayer(wx, Wl, lib=lib)
    Lr = orc.OracleLayer(wr, Wl, lib=lib)
    for it in range(w.iters):
        ox = Lx.forward(X[it], D[it])
        orr = Lr.forward(X[it], D[it])
        if set(ox["ids"][:, :w.top_k].ravel().tolist()) <= set(np.flatnonzero(orr["inA"]).tolist()):
            assert np.array_equal(ox["ids"][:, :w.top_k], orr["routed_ids"])
            assert np.array_equal(ox["Y"], orr["Y"]) and np.array_equal(Lx.cache, Lr.cache)
        Lx.commit()
        Lr.commit()
    assert Lr.counters["restricted"] >= 1
    # update period 2: no forward reuses a support built two or more iterations earlier
    Lp = orc.OracleLayer(w.replace(atlas_period=2), Wl, lib=lib)
    last = None
    for it in range(w.iters):
        path = Lp.forward(X[it], D[it])["path"]
        Lp.commit()
        assert (path == 1) == (it == 0)
        if path:
            last = it
        else:
            assert it - last < 2
    assert Lp.counters["period_update"] >= 1
    # a narrow support (B = c = 1) built on one hidden state, then unrelated hidden states
    wn = w.replace(atlas_B=1, atlas_c=1, redraw_every=1, rho_live=0.0, rho_decoded=0.0)
    Xn = synth.hidden_states(wn, 0, D)
    Ln = orc.OracleLayer(wn, Wl, lib=lib)
    for it in range(w.iters):
        out = Ln.forward(Xn[it], D[it])
        Ln.commit()
    assert Ln.counters["coverage_fallback"] >= 1


def _groups_by_first_appearance(G, n_group, topk_group, base=None):
    """Brute force of the group-limited selectable set by a second formulation: walk the
    experts in key order (stable sort on -G, so ties -> lower id) and keep the groups in the
    order their first (allowed) expert appears; a group's first appearance is its best expert."""
    M, E = G.shape
    gs = E // n_group
    order = np.argsort(-G.astype(np.float64), axis=1, kind="stable")
    out = np.zeros((M, E), np.uint8)
    for t in range(M):
        kept = []
        for e in order[t]:
            if base is not None and not base[e]:
                continue
            if e // gs not in kept:
                kept.append(e // gs)
            if len(kept) == topk_group:
                break
        for gr in kept:
            lo = gr * gs
            out[t, lo:lo + gs] = 1 if base is None else base[lo:lo + gs]
    return out


def pin_group_limited(orc, lib):
    """Group-limited top-k: the kept groups against the first-appearance walk (with and
    without a support mask); the candidates lie in at most topk_group groups and start with
    the overall best expert; topk_group = n_group and single-expert groups reduce to the
    plain top-K."""
    rng = np.random.default_rng(13)
    M, E, K, Kext, ng, tg = 60, 24, 3, 6, 6, 2
    G = rng.standard_normal((M, E)).astype(np.float32)
    G[:, 13] = G[:, 2]                              # exact ties across groups
    for base in (None, (rng.random(E) < 0.6).astype(np.uint8)):
        al = orc.group_allowed(G, ng, tg, base=base, lib=lib)
        assert np.array_equal(al, _groups_by_first_appearance(G, ng, tg, base)), \
            "kept groups must be the first topk_group groups met in key order"
    al = orc.group_allowed(G, ng, tg, lib=lib)
    ids, s, w, q = orc.route(G, K, Kext, True, True, allowed=al, lib=lib)
    plain = np.argsort(-G.astype(np.float64), axis=1, kind="stable")
    assert (ids[:, 0] == plain[:, 0]).all()
    assert all(len(set((ids[t] // (E // ng)).tolist())) <= tg for t in range(M))
    masked = np.where(al.astype(bool), -G.astype(np.float64), np.inf)
    assert np.array_equal(ids, np.argsort(masked, axis=1, kind="stable")[:, :Kext])
    full = expit(G.astype(np.float64))
    np.testing.assert_allclose(s, np.take_along_axis(full, ids, axis=1), rtol=1e-13, atol=0)
    ids0, s0, w0, q0 = orc.route(G, K, Kext, True, True, lib=lib)
    for ng2, tg2 in ((ng, ng), (E, Kext)):
        al2 = orc.group_allowed(G, ng2, tg2, lib=lib)
        ids2, s2, w2, q2 = orc.route(G, K, Kext, True, True, allowed=al2, lib=lib)
        assert np.array_equal(ids2, ids0) and np.array_equal(w2, w0)


def pin_group_limited_restricted(orc, lib):
    """Group-limited routing inside the support over a small block: candidates and routed
    experts stay within topk_group groups; hot-skip forwards route to the masked stable sort
    over the experts of the groups met first among the support's experts."""
    w = small_workload(routing="restricted", n_experts=16, top_k=3, iters=6,
                       liveness="uniform", n_shared=0, shared_inter=0, n_group=4, topk_group=2)
    Wl = synth.layer_weights(w, 0)
    D = synth.decoded_masks(w)
    X = synth.hidden_states(w, 0, D)
    L = orc.OracleLayer(w, Wl, lib=lib)
    gs = w.n_experts // w.n_group
    for it in range(w.iters):
        out = L.forward(X[it], D[it])
        for t in range(w.M):
            assert len(set((out["ids"][t] // gs).tolist())) <= w.topk_group
            assert len(set((out["routed_ids"][t] // gs).tolist())) <= w.topk_group
        if not out["path"]:
            al = _groups_by_first_appearance(out["G"], w.n_group, w.topk_group, out["inA"])
            masked = np.where(al.astype(bool), -out["G"].astype(np.float64), np.inf)
            assert np.array_equal(out["routed_ids"],
                                  np.argsort(masked, axis=1, kind="stable")[:, :w.top_k])
        L.commit()
    assert L.counters["restricted"] >= 1


def pin_live_decode(orc, lib):
    """Live-only threshold decoding against numpy / scipy: logits as a float64 matmul of the
    live rows, the top token as numpy argmax (first maximum, i.e. lower id on exact ties),
    the confidence as the largest softmax probability; commits by the threshold rule, with
    the most confident live position of an otherwise uncommitted sequence; decoded positions
    untouched; one-token vocabularies commit every live position."""
    rng = np.random.default_rng(14)
    block, nb, H, V = 8, 3, 32, 50
    M = block * nb
    W = (rng.standard_normal((V, H)) * 0.3).astype(np.float32)
    W[17] = W[5]                                   # exact tie between tokens 5 and 17
    h = rng.standard_normal((M, H)).astype(np.float32) * 0.2
    h[block + 2] = W[5] * 40.0                     # a row split between the tied tokens
    # confident rows of sequence 1 ...
    h[block + 6] = W[30] * 40.0
    h[2 * block:3 * block] = W[9] * 40.0           # ... every row of sequence 2
    D = np.zeros(M, np.uint8)
    D[[0, 3, block + 1, 2 * block + 4]] = 1        # decoded positions
    hb, Wb = synth.f32_to_bf16_bits(h), synth.f32_to_bf16_bits(W)
    out = orc.live_decode(hb, Wb, D, block, 0.95, lib=lib)
    z = synth.bf16_bits_to_f32(hb).astype(np.float64) @ synth.bf16_bits_to_f32(Wb).astype(np.float64).T
    live = ~D.astype(bool)
    top = np.argmax(z, axis=1)
    conf = softmax(z, axis=1).max(axis=1)
    assert np.array_equal(out["top"][live], top[live])
    assert (out["top"][block + 2] == 5)                   # the tie goes to the lower id
    np.testing.assert_allclose(out["conf"][live], conf[live], rtol=1e-12)
    srt = np.sort(z, axis=1)
    np.testing.assert_allclose(out["gap"][live], (srt[:, -1] - srt[:, -2])[live], rtol=1e-9, atol=1e-12)
    expect = D.copy()
    for b in range(nb):
        rows = [t for t in range(b * block, (b + 1) * block) if live[t]]
        hit = [t for t in rows if conf[t] >= 0.95]
        for t in hit or [max(rows, key=lambda t: (conf[t], -t))]:
            expect[t] = 1
    assert np.array_equal(out["D_next"], expect)
    assert not expect[block + 2]                   # the tied row holds at most half the mass
    assert expect[block + 6] and expect[2 * block:3 * block].all()
    assert expect[:block].sum() == D[:block].sum() + 1          # sequence 0: one fallback commit
    new = (expect == 1) & (D == 0)
    assert np.array_equal(out["token"][new], top[new]) and (out["token"][~new] == -1).all()
    assert out["commits"] == int(new.sum())
    one = orc.live_decode(hb, Wb[:1], D, block, 0.95, lib=lib)
    assert one["D_next"].all() and np.allclose(one["conf"][live], 1.0)


PINS = [pin_router, pin_topk, pin_weights, pin_score_given, pin_atlas_hand, pin_atlas_special, pin_fresh,
        pin_worklist, pin_expert, pin_dense, pin_all_fresh_equals_dense, pin_staleness,
        pin_restricted_topk, pin_atlas_without_closure, pin_restricted_lifecycle,
        pin_group_limited, pin_group_limited_restricted, pin_live_decode, pin_support_lifecycle,
        pin_under_covered]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc, orc.load())


def test_anomaly_and_special_fresh_cases(orc):
    M = 10
    valid = np.ones(M, np.uint8)
    last = np.full(M, 5, np.int32)
    prev = np.ones(M, np.uint8)
    D = np.ones(M, np.uint8)
    fresh, an = orc.fresh_set(4, 6, valid, last, prev, D)
    assert an == 0 and fresh.sum() == 0          # all stable, age 1 < R
    fresh, an = orc.fresh_set(1, 6, valid, last, prev, D)
    assert fresh.all()                             # R = 1: never stale
    D2 = D.copy()
    D2[3] = 0                                      # decoded -> live: anomaly, full fresh pass
    fresh, an = orc.fresh_set(4, 6, valid, last, prev, D2)
    assert an == 1 and fresh.all()
    fresh, an = orc.fresh_set(4, 6, np.zeros(M, np.uint8), last, prev, D)
    assert fresh.all()                             # cache miss
    force = np.zeros(M, np.uint8)
    force[[1, 7]] = 1
    fresh, an = orc.fresh_set(4, 6, valid, last, prev, D, force)
    assert fresh.nonzero()[0].tolist() == [1, 7]


MUTATIONS = {1: "router bias dropped", 2: "down-projection operand indexed wrongly",
             3: "SiLU sign flipped", 4: "ties broken toward the higher id",
             5: "refresh-due test dropped", 6: "worklist in position order",
             7: "H_e uses a strict inequality", 8: "restricted top-K ignores the support",
             9: "groups ranked by their first expert, not their best",
             10: "decoded token ties broken toward the higher id",
             11: "support rebuilt when an extra (not routed) candidate lies outside it",
             12: "boundary rows counted as under-covered (<= instead of <)"}


@pytest.mark.parametrize("m", sorted(MUTATIONS), ids=[MUTATIONS[m] for m in sorted(MUTATIONS)])
def test_planted_mistakes(orc, m, tmp_path):
    path = str(tmp_path / f"liboracle_m{m}.so")
    orc.build_oracle(path, mutate=m, quiet=True)
    lib = orc.load(path)
    caught = []
    for pin in PINS:
        try:
            pin(orc, lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake: {MUTATIONS[m]}"


def test_tie_order_continuation(orc):
    """The GPU harness's near-tie rule: where two experts' logits tie exactly, the oracle accepts
    the other order for a position, scores it from its own logits and routes through it.
    Experts 3 and 11 get identical router rows (exact ties everywhere); on positions where the
    tie straddles the top-K boundary, swapping them changes which expert runs."""
    w = small_workload(n_experts=16, top_k=3, iters=2, n_shared=0, shared_inter=0)
    Wl = dict(synth.layer_weights(w, 0))
    Wl["router_w"] = Wl["router_w"].copy()
    Wl["router_w"][11] = Wl["router_w"][3]
    Wl["router_w"][3] += 0.3 * np.abs(Wl["router_w"][3])   # rank 3 and 11 high on most rows
    Wl["router_w"][11] = Wl["router_w"][3]
    Wl["router_b"] = None
    D = synth.decoded_masks(w)
    X = synth.hidden_states(w, 0, D)
    K = w.top_k
    La = orc.OracleLayer(w, Wl)
    Lb = orc.OracleLayer(w, Wl)
    pre = La.route(X[0])
    ids = pre["ids"]
    straddle = [t for t in range(w.M)
                if 3 in ids[t, :K].tolist() and ids[t, K] == 11]
    assert straddle, "no position with the tie on the top-K boundary"
    ties = {}
    for t in straddle:
        alt = ids[t].copy()
        alt[K - 1 if ids[t, K - 1] == 3 else list(alt).index(3)] = 11
        alt[K] = 3
        ties[t] = alt
    oa = La.forward(X[0], D[0], pre=pre)
    ob = Lb.forward(X[0], D[0], pre=pre, tie_ids=ties)
    for t in straddle:
        assert 11 in ob["routed_ids"][t].tolist() and 3 not in ob["routed_ids"][t].tolist()
        assert np.allclose(ob["w"][t], oa["w"][t])            # tied logits: same weights
    assert np.array_equal(np.delete(ob["Y"], straddle, 0), np.delete(oa["Y"], straddle, 0))
    assert ob["worklist"]["P"] == oa["worklist"]["P"]
