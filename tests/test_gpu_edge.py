"""Edge cases and degenerate cases of the layer on the GPU, through the C ABI, against the oracle."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_sparse_amd import binding
    binding.load()


def H():
    import gpu_harness
    return gpu_harness


def small(**kw):
    base = dict(hidden=128, n_experts=24, top_k=4, inter=64, shared_inter=64, batch=3, block=11,
                iters=6, staleness_R=3, n_layers=1, zipf=None)
    base.update(kw)
    return synth.workload(3, **base)


def test_liveness_anomaly_falls_back_to_full_fresh():
    """A position decoded in the previous forward that is live again makes the whole
    layer-iteration fresh and counts an anomaly (teardown, cold / hot paths: conservative
    fallback on an abnormal liveness transition)."""
    h = H()
    w = small()
    D = synth.decoded_masks(w)
    t = int(np.nonzero(D[3])[0][0])
    D[4:, t] = 0                                   # decoded at 3, live again from 4
    rep = h.run_block(w, D_override=D, verbose=False)
    assert rep.fresh_counts[4] == w.M and rep.counters[0]["anomaly"] == 1


def test_empty_fresh_set_restores_from_cache():
    """Every position decoded from the start and a long staleness bound: after the cold
    iteration no position is fresh, the worklist is empty and y comes from the cache."""
    h = H()
    w = small(staleness_R=50, iters=4)
    D = np.ones((w.iters, w.M), dtype=np.uint8)
    rep = h.run_block(w, D_override=D, verbose=False)
    assert rep.fresh_counts == [w.M, 0, 0, 0]   # from iteration 1 every position is stable
    assert rep.stable_rows_checked == 3 * w.M


def test_force_all_equals_dense_layer():
    """force_fresh = all on every iteration gives the dense MoE layer (teardown, FreshLane:
    for a valid fresh pair the expert computation is the dense path's)."""
    import oracle
    h = H()
    w = small(staleness_R=3)
    F = np.ones((w.iters, w.M), dtype=np.uint8)
    W = synth.layer_weights(w, 0)
    D = synth.decoded_masks(w)
    X = synth.hidden_states(w, 0, D)
    plan = h.make_plan(w, [h.upload_weights(W)], 1)
    for it in range(w.iters):
        x = h.to_dev(X[it])
        y = torch.empty_like(x)
        plan.forward(0, x, h.to_dev(D[it]), h.to_dev(F[it]), y)
        plan.commit(0)
        R, Y = oracle.dense_moe(X[it], W["router_w"], W["router_b"], W["w1"], W["w3"], W["w2"],
                                W["sw1"], W["sw3"], W["sw2"], w.top_k, True, True)
        assert h.rownorm_err(h.act_to_f64(y.cpu().numpy()), Y) <= h.TOL["bf16"]
    plan.close()


def test_repeat_forward_is_idempotent_and_commit_state():
    from block_diffusion_sparse_amd import binding as B
    h = H()
    w = small()
    W = synth.layer_weights(w, 0)
    D = synth.decoded_masks(w)
    X = synth.hidden_states(w, 0, D)
    plan = h.make_plan(w, [h.upload_weights(W)], 1)
    with pytest.raises(B.EpochError) as ei:
        plan.commit(0)                             # no forward yet
    assert ei.value.status == -6
    with pytest.raises(B.EpochError) as ei:
        plan.forward(1, h.to_dev(X[0]), h.to_dev(D[0]))
    assert ei.value.status == -5                   # layer out of range
    for it in range(3):
        x, d = h.to_dev(X[it]), h.to_dev(D[it])
        y1 = plan.forward(0, x, d)
        y2 = plan.forward(0, x, d)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), f"repeat forward differs at iteration {it}"
        plan.commit(0)
        with pytest.raises(B.EpochError):
            plan.commit(0)                         # one commit per forward
    plan.close()


def test_plan_rebuild_mid_block_invalidates_caches():
    """A new plan on the same workspace clears every cache entry: the next iteration runs
    all positions fresh, like a new block (teardown: plans are not reused across blocks)."""
    import oracle
    h = H()
    w = small(iters=6)

    def hook(it, plan, orcs):
        if it != 3:
            return None
        from block_diffusion_sparse_amd import binding as B
        plan.close()
        plan.handle = B.epoch_block_plan_build(plan.desc, [B.layer_weights(
            d["router_w"], d.get("router_b"), d["w1"], d["w3"], d["w2"], d.get("sw1"),
            d.get("sw3"), d.get("sw2")) for d in plan._weights], plan.ws, plan.nbytes)
        o = orcs[0]
        fresh_orc = oracle.OracleLayer(o.w, o.W, rows=o.rows)
        fresh_orc.iter = 0
        return plan, [fresh_orc]

    rep = h.run_block(w, hook=hook, verbose=False)
    assert rep.fresh_counts[3] == w.M


@pytest.mark.parametrize("case", ["max-experts-k16", "k-equals-e", "one-expert", "one-position"])
def test_extreme_shapes(case):
    h = H()
    if case == "max-experts-k16":   # E = 1024, K = 16, K_ext = 32: the kernels' upper limits
        w = small(n_experts=1024, top_k=16, inter=64, hidden=64, batch=2, block=40, iters=3)
    elif case == "k-equals-e":      # every expert routed: the support is everything
        w = small(n_experts=6, top_k=6, iters=4)
    elif case == "one-expert":
        w = small(n_experts=1, top_k=1, iters=4)
    else:                           # a single position
        w = small(batch=1, block=1, iters=4)
    rep = h.run_block(w, verbose=False)
    assert rep.iters == w.iters
