"""CPU oracle of the liveness-sparse routed-expert MoE layer forward.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and
the CPU-baseline leg of bench.py may import this package.  The product path
(block_diffusion_sparse_amd and its HIP library) never imports it.

This module is argument marshalling around oracle.c (plain C, double sums);
the per-step citations of the pages live there.  `OracleLayer` replays the
per-layer state machine of one block (plan build, then forward + commit per
refinement iteration) by calling those steps in the pages' order.
"""
from __future__ import annotations

import ctypes
import os
import time
from typing import Optional

import numpy as np

from .build import LIB, build as build_oracle

_c_int = ctypes.c_int
_ptr = ctypes.c_void_p
_libs: dict = {}


def load(path: str = LIB) -> ctypes.CDLL:
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        build_oracle(path, quiet=True)
    lib = ctypes.CDLL(path)
    lib.orc_num_threads.restype = _c_int
    lib.orc_support_status.restype = _c_int
    lib.orc_support_build.restype = _c_int
    lib.orc_under_covered.restype = ctypes.c_int64
    lib.orc_fresh_set.restype = _c_int
    lib.orc_worklist.restype = _c_int
    lib.orc_atlas_build.restype = _c_int
    lib.orc_route_restricted.restype = _c_int
    lib.orc_group_allowed.restype = None
    lib.orc_live_decode.restype = _c_int
    for name in ("orc_router_logits", "orc_route", "orc_score_given", "orc_expert",
                 "orc_moe_rows", "orc_commit", "orc_dense_moe"):
        getattr(lib, name).restype = None
    _libs[path] = lib
    return lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _is_bf16(a: np.ndarray) -> int:
    return 1 if a.dtype == np.uint16 else 0


def num_threads(lib=None) -> int:
    return (lib or load()).orc_num_threads()


def set_num_threads(n: int, lib=None) -> None:
    (lib or load()).orc_set_num_threads(_c_int(int(n)))


def router_logits(x, Wg, bias=None, lib=None) -> np.ndarray:
    lib = lib or load()
    x = np.ascontiguousarray(x)
    Wg = np.ascontiguousarray(Wg, dtype=np.float32)
    M, H = x.shape
    E = Wg.shape[0]
    G = np.empty((M, E), dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    lib.orc_router_logits(_c_int(M), _c_int(H), _c_int(E), _c_int(_is_bf16(x)), _p(x), _p(Wg),
                          _p(b), _p(G))
    return G


def route(G, K, Kext, gate_sigmoid, norm_topk, allowed=None, lib=None):
    """Top-K_ext candidates (key: logit desc, id asc) over all experts, or over the
    selectable ones of each row when allowed [M, E] is given."""
    lib = lib or load()
    G = np.ascontiguousarray(G, dtype=np.float32)
    M, E = G.shape
    ids = np.empty((M, Kext), dtype=np.int32)
    s = np.empty((M, Kext), dtype=np.float64)
    w = np.empty((M, K), dtype=np.float64)
    q = np.empty((M, Kext), dtype=np.int64)
    al = None if allowed is None else np.ascontiguousarray(allowed, dtype=np.uint8)
    if al is not None and (al.sum(axis=1) < Kext).any():
        raise ValueError("fewer selectable experts than K_ext candidates in some row")
    lib.orc_route(_c_int(M), _c_int(E), _c_int(K), _c_int(Kext), _c_int(int(gate_sigmoid)),
                  _c_int(int(norm_topk)), _p(G), _p(al), _p(ids), _p(s), _p(w), _p(q))
    return ids, s, w, q


def score_given(G, ids, K, gate_sigmoid, norm_topk, lib=None):
    """Scores s, routing weights w and planner weights q of a given ranked selection ids
    [M x Kext] (the scoring half of route)."""
    lib = lib or load()
    G = np.ascontiguousarray(G, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    M, E = G.shape
    Kext = ids.shape[1]
    s = np.empty((M, Kext), dtype=np.float64)
    w = np.empty((M, K), dtype=np.float64)
    q = np.empty((M, Kext), dtype=np.int64)
    lib.orc_score_given(_c_int(M), _c_int(E), _c_int(K), _c_int(Kext), _c_int(int(gate_sigmoid)),
                        _c_int(int(norm_topk)), _p(G), _p(ids), _p(s), _p(w), _p(q))
    return s, w, q


def tie_order_ok(g_row, ids_row, alt_row, tie):
    """True if alt_row ranks the same candidates as ids_row up to ties: distinct experts whose
    logit at every rank is within `tie` of the logit the key order puts there (an order that
    differs only among logits closer than `tie`)."""
    g = np.asarray(g_row, dtype=np.float64)
    alt = np.asarray(alt_row)
    if len(set(alt.tolist())) != len(alt):
        return False
    return bool(np.all(np.abs(g[alt] - g[np.asarray(ids_row)]) < tie))


def group_allowed(G, n_group, topk_group, base=None, lib=None):
    """[M, E] mask of the experts of each row's topk_group best groups (groups ranked by
    their best expert among base, the [E] support mask, or all experts)."""
    lib = lib or load()
    G = np.ascontiguousarray(G, dtype=np.float32)
    M, E = G.shape
    out = np.empty((M, E), dtype=np.uint8)
    b = None if base is None else np.ascontiguousarray(base, dtype=np.uint8)
    lib.orc_group_allowed(_c_int(M), _c_int(E), _c_int(n_group), _c_int(topk_group), _p(G),
                          _p(b), _p(out))
    return out


def support_status(ids, K, inS, support_valid, lib=None) -> int:
    lib = lib or load()
    M, Kext = ids.shape
    return lib.orc_support_status(_c_int(M), _c_int(K), _c_int(Kext), _p(ids), _p(inS),
                                  _c_int(int(support_valid)))


def support_build(ids, q, E, K, B, c, alpha, qfrac, beta, lib=None):
    lib = lib or load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    q = np.ascontiguousarray(q, dtype=np.int64)
    M, Kext = ids.shape
    inS = np.zeros(E, dtype=np.uint8)
    slot_of = np.empty(E, dtype=np.int32)
    S_list = np.empty(E, dtype=np.int32)
    stats = np.zeros(5, dtype=np.int64)
    n = lib.orc_support_build(_c_int(M), _c_int(E), _c_int(K), _c_int(Kext), _p(ids), _p(q),
                              _c_int(B), _c_int(c), _c_int(alpha[0]), _c_int(alpha[1]),
                              _c_int(qfrac[0]), _c_int(qfrac[1]), _c_int(beta[0]),
                              _c_int(beta[1]), _p(inS), _p(slot_of), _p(S_list), _p(stats))
    return inS, slot_of, S_list[:n].copy(), stats


def atlas_build(ids, q, E, K, B, c, alpha, qfrac, beta, lib=None):
    """The Atlas support without the closure over routed experts (restricted routing)."""
    lib = lib or load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    q = np.ascontiguousarray(q, dtype=np.int64)
    M, Kext = ids.shape
    inA = np.zeros(E, dtype=np.uint8)
    slot_of = np.empty(E, dtype=np.int32)
    S_list = np.empty(E, dtype=np.int32)
    stats = np.zeros(5, dtype=np.int64)
    n = lib.orc_atlas_build(_c_int(M), _c_int(E), _c_int(K), _c_int(Kext), _p(ids), _p(q),
                            _c_int(B), _c_int(c), _c_int(alpha[0]), _c_int(alpha[1]),
                            _c_int(qfrac[0]), _c_int(qfrac[1]), _c_int(beta[0]),
                            _c_int(beta[1]), _p(inA), _p(slot_of), _p(S_list), _p(stats))
    return inA, slot_of, S_list[:n].copy(), stats


def route_restricted(G, K, inA, gate_sigmoid, norm_topk, lib=None):
    """Top-K inside the support: inA is the [E] support mask or an [M, E] per-row mask of
    selectable experts.  Returns ids [M, K] int32 and weights [M, K] double, or None when
    some row has fewer than K selectable experts."""
    lib = lib or load()
    G = np.ascontiguousarray(G, dtype=np.float32)
    M, E = G.shape
    al = np.ascontiguousarray(np.broadcast_to(np.asarray(inA, dtype=np.uint8), (M, E)))
    rids = np.empty((M, K), dtype=np.int32)
    rw = np.empty((M, K), dtype=np.float64)
    n_short = lib.orc_route_restricted(_c_int(M), _c_int(E), _c_int(K),
                                       _c_int(int(gate_sigmoid)), _c_int(int(norm_topk)), _p(G),
                                       _p(al), _p(rids), _p(rw))
    return None if n_short else (rids, rw)


def slots_of(mask):
    """Slots in expert-id order of the experts with mask = 1: (slot_of, S_list)."""
    S_list = np.flatnonzero(np.asarray(mask)).astype(np.int32)
    slot_of = np.full(len(mask), -1, dtype=np.int32)
    slot_of[S_list] = np.arange(len(S_list), dtype=np.int32)
    return slot_of, S_list


def under_covered(ids, q, K, inS, alpha, lib=None) -> int:
    lib = lib or load()
    M, Kext = ids.shape
    return int(lib.orc_under_covered(_c_int(M), _c_int(K), _c_int(Kext), _p(ids), _p(q),
                                     _p(inS), _c_int(alpha[0]), _c_int(alpha[1])))


def fresh_set(R, it, valid, last_fresh, prev_D, D, force=None, lib=None):
    lib = lib or load()
    M = D.shape[0]
    fresh = np.empty(M, dtype=np.uint8)
    D = np.ascontiguousarray(D, dtype=np.uint8)
    f = None if force is None else np.ascontiguousarray(force, dtype=np.uint8)
    anomaly = lib.orc_fresh_set(_c_int(M), _c_int(R), _c_int(it), _p(valid), _p(last_fresh),
                                _p(prev_D), _p(D), _p(f), _p(fresh))
    return fresh, int(anomaly)


def worklist(ids, w, K, fresh, slot_of, nS, lib=None) -> dict:
    lib = lib or load()
    M, Kext = ids.shape
    P_max = M * K
    wl_pos = np.empty(max(P_max, 1), dtype=np.int32)
    wl_k = np.empty(max(P_max, 1), dtype=np.int32)
    wl_w = np.empty(max(P_max, 1), dtype=np.float64)
    offs = np.empty(nS + 1, dtype=np.int32)
    inv = np.empty(M * K, dtype=np.int32)
    P = lib.orc_worklist(_c_int(M), _c_int(K), _c_int(Kext), _p(ids), _p(w), _p(fresh),
                         _p(slot_of), _c_int(nS), _p(wl_pos), _p(wl_k), _p(wl_w), _p(offs),
                         _p(inv))
    assert P >= 0, "a routed expert of a fresh position has no slot in the support"
    return dict(P=P, wl_pos=wl_pos[:P].copy(), wl_k=wl_k[:P].copy(), wl_w=wl_w[:P].copy(),
                offs=offs, inv=inv.reshape(M, K))


def expert(x_row, W1e, W3e, W2e, lib=None) -> np.ndarray:
    lib = lib or load()
    x_row = np.ascontiguousarray(x_row)
    I, H = W1e.shape
    y = np.empty(H, dtype=np.float64)
    lib.orc_expert(_c_int(H), _c_int(I), _c_int(_is_bf16(x_row)), _p(x_row),
                   _p(np.ascontiguousarray(W1e)), _p(np.ascontiguousarray(W3e)),
                   _p(np.ascontiguousarray(W2e)), _p(y))
    return y


def dense_moe(x, Wg, bias, W1, W3, W2, SW1, SW3, SW2, K, gate_sigmoid, norm_topk, lib=None):
    lib = lib or load()
    x = np.ascontiguousarray(x)
    M, H = x.shape
    E, I, _ = W1.shape
    Is = SW1.shape[0] if SW1 is not None else 0
    R = np.empty((M, H), dtype=np.float64)
    Y = np.empty((M, H), dtype=np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    lib.orc_dense_moe(_c_int(M), _c_int(H), _c_int(I), _c_int(Is), _c_int(E), _c_int(K),
                      _c_int(int(gate_sigmoid)), _c_int(int(norm_topk)), _c_int(_is_bf16(x)),
                      _p(x), _p(np.ascontiguousarray(Wg, dtype=np.float32)), _p(b), _p(W1),
                      _p(W3), _p(W2), _p(SW1), _p(SW3), _p(SW2), _p(R), _p(Y))
    return R, Y


def live_decode(h, Wv, D, block, tau=0.95, token=None, lib=None) -> dict:
    """Live-only threshold decoding of one refinement step (see orc_live_decode)."""
    lib = lib or load()
    h = np.ascontiguousarray(h)
    Wv = np.ascontiguousarray(Wv)
    M, H = h.shape
    V = Wv.shape[0]
    D = np.ascontiguousarray(D, dtype=np.uint8)
    D_next = np.empty(M, np.uint8)
    tok = np.full(M, -1, np.int32) if token is None else np.ascontiguousarray(token, np.int32).copy()
    conf = np.empty(M, np.float64)
    gap = np.empty(M, np.float64)
    top = np.empty(M, np.int32)
    n = lib.orc_live_decode(_c_int(M), _c_int(H), _c_int(V), _c_int(block), _c_int(_is_bf16(h)),
                            _p(h), _p(Wv), _p(D), ctypes.c_double(tau), _p(D_next), _p(tok),
                            _p(conf), _p(gap), _p(top))
    return dict(D_next=D_next, token=tok, conf=conf, gap=gap, top=top, commits=int(n))


class OracleLayer:
    """Replays one MoE layer over one block: plan build, then forward/commit per iteration.

    weights: dict with router_w [E,H] f32, router_b [E] f32 or None, w1/w3 [E,I,H],
    w2 [E,H,I], sw1/sw3 [Is,H], sw2 [H,Is] or None (uint16 bf16 bits or f32).
    rows: positions whose expert outputs are evaluated (None = all); the discrete
    stages (router, top-k, support, fresh set, worklist) always cover every position.
    """

    NEG_INF_ITER = -(1 << 30)
    TIE = 1e-6  # logits closer than this are a tie: either order is a correct ranking

    def __init__(self, w, weights: dict, lib=None, rows=None):
        self.lib = lib or load()
        self.w = w
        self.W = {k: (None if v is None else np.ascontiguousarray(v)) for k, v in weights.items()}
        M, E, H = w.M, w.n_experts, w.hidden
        self.rows = np.arange(M, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
        # plan build / cold path: caches cleared, support invalid, iteration 0
        self.valid = np.zeros(M, dtype=np.uint8)
        self.last_fresh = np.full(M, self.NEG_INF_ITER, dtype=np.int32)
        self.prev_D = np.zeros(M, dtype=np.uint8)
        self.cache = np.zeros((M, H), dtype=np.float64)
        self.inS = np.zeros(E, dtype=np.uint8)
        self.slot_of = np.full(E, -1, dtype=np.int32)
        self.S_list = np.zeros(0, dtype=np.int32)
        self.support_valid = False
        self.iter = 0
        self.counters = dict(cold=0, hot_update=0, hot_skip=0, anomalies=0, fresh_rows=0,
                             pairs=0, coverage_unmet=0, restricted=0, coverage_fallback=0,
                             period_update=0)
        self._pending = None
        # restricted routing: the Atlas support (no closure) and the iteration it was built at
        self.inA = np.zeros(E, dtype=np.uint8)
        self.built_iter = 0

    def route(self, x) -> dict:
        """Router logits and the ranked candidates of every position (no state is touched)."""
        w, lib, W = self.w, self.lib, self.W
        G = router_logits(x, W["router_w"], W["router_b"], lib=lib)
        # group-limited rule: each row selects among the experts of its best groups
        allowed = (group_allowed(G, w.n_group, w.topk_group, lib=lib) if w.n_group > 1
                   else None)
        ids, s, wts, q = route(G, w.top_k, w.k_ext, w.gate == "sigmoid", w.norm_topk,
                               allowed=allowed, lib=lib)
        return dict(G=G, ids=ids, s=s, w=wts, q=q)

    def forward(self, x, D, force=None, rows=None, pre=None, tie_ids=None,
                tie_routed=None) -> dict:
        """One forward of the layer.  rows: positions whose outputs this forward evaluates
        (default: the rows given at construction).  A stable row's output is the oracle's
        cache row, which holds the row's value only if the row was evaluated at its last fresh
        iteration.  Wall-clock seconds of the two parts are kept in `last_stage_s` (router,
        top-k, support, fresh set, worklist over every position) and `last_expert_s` (expert
        outputs of the evaluated rows, merge of the stable ones)."""
        t_start = time.perf_counter()
        w, lib = self.w, self.lib
        K, Kext, E = w.top_k, w.k_ext, w.n_experts
        W = self.W
        r = self.route(x) if pre is None else pre
        G, ids, s, wts, q = r["G"], r["ids"], r["s"], r["w"], r["q"]
        if tie_ids:
            # positions whose ranking is a tie of their logits take the given (equally correct)
            # order, checked against this forward's own logits; their scores follow from it
            ids, s, wts, q = ids.copy(), s.copy(), wts.copy(), q.copy()
            for t, alt in tie_ids.items():
                assert tie_order_ok(G[t], ids[t], alt, self.TIE), f"row {t}: not a tie order"
                ids[t] = alt
            tr = np.array(sorted(tie_ids), dtype=np.int64)
            s[tr], wts[tr], q[tr] = score_given(G[tr], ids[tr], K, w.gate == "sigmoid",
                                                w.norm_topk, lib=lib)
        stats = None
        if w.routing == "restricted":
            path, stats, rids, rw = self._restricted_step(G, ids, q, wts, tie_routed)
        else:
            path = support_status(ids, K, self.inS, self.support_valid, lib=lib)
            if path:
                self.inS, self.slot_of, self.S_list, stats = support_build(
                    ids, q, E, K, w.B, w.c, w.alpha, w.q, w.beta, lib=lib)
                self.support_valid = True
                self.counters["cold" if path == 1 else "hot_update"] += 1
                if stats[2]:
                    self.counters["coverage_unmet"] += 1
            else:
                self.counters["hot_skip"] += 1
            rids, rw = np.ascontiguousarray(ids[:, :K]), wts
        fresh, anomaly = fresh_set(w.staleness_R, self.iter, self.valid, self.last_fresh,
                                   self.prev_D, D, force, lib=lib)
        wl = worklist(rids, rw, K, fresh, self.slot_of, len(self.S_list), lib=lib)
        H, I = w.hidden, w.inter
        Is = w.shared_inter if W.get("sw1") is not None else 0
        rows = self.rows if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
        R = np.empty((len(rows), H), dtype=np.float64)
        Y = np.empty((len(rows), H), dtype=np.float64)
        x = np.ascontiguousarray(x)
        t_rows = time.perf_counter()
        lib.orc_moe_rows(_c_int(w.M), _c_int(H), _c_int(I), _c_int(Is), _c_int(E), _c_int(K),
                         _c_int(K), _c_int(_is_bf16(x)), _p(x), _p(rids), _p(rw), _p(fresh),
                         _p(W["w1"]), _p(W["w3"]), _p(W["w2"]), _p(W.get("sw1")),
                         _p(W.get("sw3")), _p(W.get("sw2")), _c_int(len(rows)), _p(rows),
                         _p(self.cache), _p(R), _p(Y))
        t_end = time.perf_counter()
        self.last_stage_s, self.last_expert_s = t_rows - t_start, t_end - t_rows
        self._pending = (fresh, np.ascontiguousarray(D, dtype=np.uint8).copy(), anomaly)
        return dict(G=G, ids=ids, s=s, w=wts, q=q, path=path, support_stats=stats,
                    routed_ids=rids, routed_w=rw, inA=self.inA.copy(),
                    inS=self.inS.copy(), slot_of=self.slot_of.copy(), S_list=self.S_list.copy(),
                    fresh=fresh, anomaly=anomaly, worklist=wl, rows=rows, R=R, Y=Y,
                    iter=self.iter)

    def _restricted_step(self, G, ids, q, wts, tie_routed=None):
        """Support lifecycle and routing of one forward under support-restricted routing.

        Teardown, Expert Atlas (third step) and the block-plan lifecycle: the hot path keeps
        the support mask and picks each position's top-K inside it (hot-skip); the support is
        rebuilt from the current candidates (all-expert top-K_ext, recomputed every
        iteration) at the block's first forward (cold), when its update period has run out,
        or when the current candidates show that it no longer meets the coverage goal
        |U| <= (1 - q) M (or holds fewer than K experts) -- hot-update.  A forward that
        (re)builds the support routes over all experts (the full path) and gives every
        routed expert a slot for that forward only; the stored support has no closure.
        """
        w, lib = self.w, self.lib
        K, E = w.top_k, w.n_experts
        stats = None
        restricted = None
        if self.support_valid:
            # the model's rule with the selectable experts limited to the support; None when
            # some row is left with fewer than K selectable experts
            allowed = (group_allowed(G, w.n_group, w.topk_group, base=self.inA, lib=lib)
                       if w.n_group > 1 else self.inA)
            restricted = route_restricted(G, K, allowed, w.gate == "sigmoid", w.norm_topk,
                                          lib=lib)
        if not self.support_valid:
            path = 1
        elif w.atlas_period > 0 and self.iter - self.built_iter >= w.atlas_period:
            path = 2
            self.counters["period_update"] += 1
        else:
            nU = under_covered(ids, q, K, self.inA, w.alpha, lib=lib)
            short = restricted is None
            if short or w.q[1] * nU > (w.q[1] - w.q[0]) * w.M:
                path = 2
                self.counters["coverage_fallback"] += 1
            else:
                path = 0
        if path:
            self.inA, _, _, stats = atlas_build(ids, q, E, K, w.B, w.c, w.alpha, w.q, w.beta,
                                                lib=lib)
            self.support_valid = True
            self.built_iter = self.iter
            self.counters["cold" if path == 1 else "hot_update"] += 1
            if stats[2]:
                self.counters["coverage_unmet"] += 1
            rids, rw = np.ascontiguousarray(ids[:, :K]), wts
            mask = self.inA.copy()
            mask[rids.ravel()] = 1
        else:
            self.counters["hot_skip"] += 1
            self.counters["restricted"] += 1
            rids, rw = restricted
            if tie_routed is not None:
                # rows whose in-support ranking is a tie of their logits take the given order
                ov = tie_routed(rids)
                if ov:
                    rids, rw = rids.copy(), rw.copy()
                    for t, alt in ov.items():
                        assert tie_order_ok(G[t], rids[t], alt, self.TIE), f"row {t}: not a tie"
                        al = allowed[t] if np.ndim(allowed) == 2 else allowed
                        assert np.asarray(al)[np.asarray(alt)].all(), f"row {t}: outside the support"
                        rids[t] = alt
                    tr = np.array(sorted(ov), dtype=np.int64)
                    _, rw[tr], _ = score_given(G[tr], rids[tr], K, w.gate == "sigmoid",
                                               w.norm_topk, lib=lib)
            mask = self.inA
        self.inS = np.ascontiguousarray(mask, dtype=np.uint8).copy()
        self.slot_of, self.S_list = slots_of(self.inS)
        return path, stats, rids, rw

    def commit(self):
        assert self._pending is not None, "commit without a forward"
        fresh, D, anomaly = self._pending
        self.lib.orc_commit(_c_int(self.w.M), _c_int(self.iter), _p(fresh), _p(D),
                            _p(self.valid), _p(self.last_fresh), _p(self.prev_D))
        self.counters["anomalies"] += anomaly
        self.counters["fresh_rows"] += int(fresh.sum())
        self.counters["pairs"] += int(fresh.sum()) * self.w.top_k
        self.iter += 1
        self._pending = None
