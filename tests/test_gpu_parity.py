"""GPU parity: the HIP path through the C ABI against the CPU oracle (needs an MI355X).

Small shapes span several tiles and ragged tails in every dimension the kernels tile
(positions, experts, pairs per expert); the five workload shapes run at full size with
every discrete stage compared in full and the outputs compared on sampled rows.
"""
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
    binding.load()  # fails loudly when the library is missing


def H():
    import gpu_harness
    return gpu_harness


def sample_rows(M, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(n, M), replace=False).tolist()) | {0, M - 1}
    return np.array(sorted(rows), dtype=np.int32)


def test_tiny_fp32_full_block():
    h = H()
    w = synth.workload(1)
    h.log(f"[tiny fp32] {w.name}")
    rep = h.run_block(w)
    assert rep.fresh_counts == [16, 16, 12, 12]
    assert rep.max_err_y <= 1e-5


@pytest.mark.parametrize("variant", ["softmax-unnorm", "sigmoid-norm-shared", "softmax-bias-ksplit"])
def test_small_bf16_ragged(variant):
    """Ragged in positions (M = 63 / 65), experts (E = 20 / 40 / 48: partial router tiles),
    pairs per expert (partial GEMM tiles), with several k tiles.  softmax-bias-ksplit: the
    router's contraction split over 4 workgroups (fp64 partials added by the top-k, the bias
    carried by the first) with a router bias."""
    h = H()
    if variant == "softmax-unnorm":
        w = synth.workload(2, hidden=256, n_experts=20, top_k=4, inter=128, batch=3, block=21,
                           iters=8, staleness_R=3)
        bias = None
    elif variant == "softmax-bias-ksplit":
        w = synth.workload(2, hidden=512, n_experts=48, top_k=4, inter=128, batch=3, block=21,
                           iters=6, staleness_R=2)
        bias = (np.random.default_rng(78).standard_normal(w.n_experts) * 0.3).astype(np.float32)
    else:
        w = synth.workload(3, hidden=192, n_experts=40, top_k=6, inter=192, shared_inter=128,
                           batch=5, block=13, iters=8, staleness_R=2, n_layers=1, zipf=None)
        bias = (np.random.default_rng(77).standard_normal(w.n_experts) * 0.3).astype(np.float32)
    h.log(f"[small {variant}] M={w.M} E={w.n_experts}")
    rep = h.run_block(w, bias_override=bias)
    assert rep.iters == w.iters and rep.stable_rows_checked > 0


def test_workload2_full_size():
    h = H()
    w = synth.workload(2)
    h.log(f"[full] {w.name}")
    rep = h.run_block(w, fresh_sample=128)
    assert rep.iters == w.iters and rep.stable_rows_checked > 0


def test_many_positions_one_expert_per_lane():
    """4096 positions of the single-layer expert shape: the top-k's 16-wave workgroups with one
    expert per lane (per-chunk counts summed in LDS over 16 positions), one k part."""
    h = H()
    w = synth.workload(2, batch=128, block=32, iters=4)
    h.log(f"[many positions] M={w.M} E={w.n_experts}")
    rep = h.run_block(w, rows=sample_rows(w.M, 24, 5))
    assert rep.iters == w.iters and rep.stable_rows_checked > 0


def test_workload3_full_shape_two_layers():
    """Layers 0 and 19 of the 20-layer shape in one plan over the whole block of 32
    iterations (R = 4: refresh-due rows from iteration 4 on)."""
    h = H()
    w = synth.workload(3)
    h.log(f"[full] {w.name}: layers 0 and 19 of 20, 32 iterations, 128 fresh rows a forward")
    rep = h.run_block(w, layers=(0, 19), fresh_sample=128)
    assert rep.iters == w.iters
    assert all(c["due_rows"] > 0 for c in rep.counters)


@pytest.mark.parametrize("layer", [0, 3])
def test_workload4_full_shape(layer):
    """One layer of the 4-layer H 4096 shape at a time (host memory) over the whole block of 32
    iterations; R = 8, so refresh-due rows appear from iteration 8 on."""
    h = H()
    w = synth.workload(4)
    h.log(f"[full] {w.name}: layer {layer} of 4, 32 iterations, 128 fresh rows a forward")
    rep = h.run_block(w, layers=(layer,), fresh_sample=128)
    assert rep.iters == w.iters
    assert rep.counters[0]["due_rows"] > 0


@pytest.mark.parametrize("frac,R,iters", [(0.25, 4, 10), (1.0, 1, 10), (0.5, 4, 32),
                                          (0.1, 16, 32), (0.05, 16, 32), (0.05, 4, 10)])
def test_workload5_sweep_points(frac, R, iters):
    """Forced-fraction sweep points of the 8192-position shape (hidden state redrawn every 8
    iterations, so the support is rebuilt mid-block)."""
    h = H()
    w = synth.workload(5, forced_fraction=frac, staleness_R=R)
    h.log(f"[full] {w.name}: f={frac} R={R}, {iters} iterations, 128 fresh rows a forward")
    rep = h.run_block(w, iters=iters, fresh_sample=128)
    assert rep.iters == iters
    if R == 1:
        assert all(c == w.M for c in rep.fresh_counts)
    # the rotating forced window refreshes each position every ~1/f iterations, so rows reach
    # the age bound R only when that period exceeds it
    if 1.0 / frac > R + 1 and iters > R + 1:
        assert rep.counters[0]["due_rows"] > 0


@pytest.mark.parametrize("frac,R", [(1.0, 1), (0.5, 4)])
def test_big_tiles_every_row(frac, R):
    """Shapes whose iterations can hold >= 32768 pairs route experts with >= BIG_ROWS fresh
    rows to 256-row compute-bound tiles and run the shared expert (M >= 2048) on them too.
    Small hidden/inter sizes keep the oracle quick, so every row is compared; H = 192 leaves a
    partial 128-column block in the down projection, and the skewed bias gives a mix of
    big-tile experts (ragged last tiles) and weight-stream experts in the same iteration."""
    h = H()
    w = synth.workload(5, hidden=192, n_experts=48, top_k=2, inter=128, shared_inter=192,
                       batch=400, block=41, iters=3, staleness_R=R, forced_fraction=frac,
                       zipf=None, redraw_every=0)
    assert w.M * w.top_k >= 32768
    bias = (-0.2 * np.log(np.arange(1, w.n_experts + 1))).astype(np.float32)
    # the routed load of the first iteration must put experts on both sides of BIG_ROWS pairs
    W0 = synth.layer_weights(w, 0)
    x0 = synth.bf16_bits_to_f32(synth.hidden_states(w, 0, synth.decoded_masks(w), iters=1)[0])
    G = x0.astype(np.float64) @ W0["router_w"].astype(np.float64).T + bias
    top = np.argsort(-G, axis=1, kind="stable")[:, : w.top_k]
    load = np.bincount(top.ravel(), minlength=w.n_experts)
    big = h.BIG_ROWS
    assert load.max() >= big and (load[load > 0] < big).any(), load
    h.log(f"[big tiles] M={w.M} f={frac} R={R} load={load.tolist()}")
    rep = h.run_block(w, weights=[W0], bias_override=bias)
    assert rep.iters == w.iters


def test_wide_shared_expert_tiles_every_row():
    """Shared-expert layers whose 256 x 256 tiles are at least as many as the device's CUs run
    both projections on the one-wave-per-SIMD tiles: M = 32800 positions (129 row tiles, the
    last one of 32 rows), I_s = 192 and H = 320 (each projection's second column block only
    partly inside the matrix).  The routed experts take the big tiles too (M K >= 32768).
    Small hidden/inter sizes keep the oracle quick, so every row is compared."""
    h = H()
    w = synth.workload(5, hidden=320, n_experts=16, top_k=1, inter=64, shared_inter=192,
                       batch=800, block=41, iters=2, staleness_R=1, forced_fraction=1.0,
                       zipf=None, redraw_every=0)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    t256 = -(-w.M // 256)
    assert t256 * -(-w.shared_inter // 128) >= n_cu and t256 * -(-w.hidden // 256) >= n_cu
    assert w.M * w.top_k >= 32768
    h.log(f"[wide shared tiles] M={w.M} H={w.hidden} Is={w.shared_inter} n_cu={n_cu}")
    rep = h.run_block(w)
    assert rep.iters == w.iters


def test_kernel_timing_on_both_streams():
    """Kernel timing with every group on, at a shape with big tiles and a shared expert: the
    shared expert and the big tiles run on the device's side stream and are timed there, and
    every group reads back one duration per forward."""
    h = H()
    w = synth.workload(5, hidden=192, n_experts=48, top_k=2, inter=128, shared_inter=192,
                       batch=400, block=41, iters=3, staleness_R=1, forced_fraction=1.0,
                       zipf=None, redraw_every=0)
    W0 = synth.layer_weights(w, 0)
    W0["router_b"] = (-0.2 * np.log(np.arange(1, w.n_experts + 1))).astype(np.float32)
    plan = h.make_plan(w, [h.upload_weights(W0)], 1)
    D = synth.decoded_masks(w)
    X = h.to_dev(synth.hidden_states(w, 0, D, iters=w.iters))
    Dd = h.to_dev(D)
    plan.set_timing(-1)
    for it in range(w.iters):
        y = torch.empty_like(X[it])
        plan.forward(0, X[it], Dd[it], None, y, None)
        plan.commit(0)
    torch.cuda.synchronize()
    t = plan.timing()
    c = plan.counters(0)
    plan.close()
    from block_diffusion_sparse_amd import binding as B
    assert list(t) == B.TIMING_GROUPS
    for g, (ms, n) in t.items():
        assert n == w.iters and ms > 0.0, (g, ms, n)
    assert c["big_experts"] > 0 and c["big_pairs"] >= h.BIG_ROWS * c["big_experts"]


@pytest.mark.parametrize("frac,R", [(1.0, 1), (0.5, 3)])
def test_tall_tiles_every_row(frac, R):
    """bf16 shapes without big tiles take 128-row routed tiles when that needs fewer tiles than
    64-row ones (an expert with more than 64 fresh pairs): the skewed bias gives experts with
    several tall tiles (ragged last tile), experts with one short tile, and iterations where
    the fresh fraction leaves every expert at 64 pairs or fewer (short tiles again); H = 192
    leaves waves without columns in the down projection.  Every row is compared."""
    h = H()
    w = synth.workload(5, hidden=192, n_experts=12, top_k=2, inter=128, shared_inter=128,
                       batch=20, block=33, iters=4, staleness_R=R, forced_fraction=frac,
                       zipf=None, redraw_every=0)
    assert w.M * w.top_k < 32768
    bias = (-0.3 * np.log(np.arange(1, w.n_experts + 1))).astype(np.float32)
    W0 = synth.layer_weights(w, 0)
    x0 = synth.bf16_bits_to_f32(synth.hidden_states(w, 0, synth.decoded_masks(w), iters=1)[0])
    G = x0.astype(np.float64) @ W0["router_w"].astype(np.float64).T + bias
    top = np.argsort(-G, axis=1, kind="stable")[:, : w.top_k]
    load = np.bincount(top.ravel(), minlength=w.n_experts)
    tiles64 = int(np.sum((load + 63) // 64))
    tiles128 = int(np.sum((load + 127) // 128))
    assert load.max() > 128 and tiles128 < tiles64, load
    h.log(f"[tall tiles] M={w.M} f={frac} R={R} load={load.tolist()}")
    rep = h.run_block(w, weights=[W0], bias_override=bias)
    assert rep.iters == w.iters
