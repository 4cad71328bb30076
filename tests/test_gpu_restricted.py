"""GPU parity of support-restricted routing (the Atlas hot path: top-K inside the support).

Every iteration compares, besides every stage the exact-mode tests compare, the Atlas support
(no closure), the routing the worklist used (all-expert top-K on cold / rebuild forwards,
top-K inside the support on hot-skip forwards) and its weights, and at the end of the block
the restricted / coverage-fallback / period-update counters.
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


def test_tiny_fp32_restricted():
    h = H()
    w = synth.workload(1, routing="restricted", iters=6)
    h.log(f"[restricted tiny fp32] {w.name}")
    rep = h.run_block(w)
    assert rep.max_err_y <= 1e-5
    assert rep.counters[0]["restricted"] >= 1


@pytest.mark.parametrize("variant", ["softmax-unnorm", "sigmoid-norm-shared-period3"])
def test_small_bf16_restricted_every_row(variant):
    """Ragged positions and experts; every output row compared."""
    h = H()
    if variant == "softmax-unnorm":
        w = synth.workload(2, hidden=256, n_experts=20, top_k=4, inter=128, batch=3, block=21,
                           iters=8, staleness_R=3, routing="restricted")
        bias = None
    else:
        w = synth.workload(3, hidden=192, n_experts=40, top_k=6, inter=192, shared_inter=128,
                           batch=5, block=13, iters=8, staleness_R=2, n_layers=1, zipf=None,
                           routing="restricted", atlas_period=3)
        bias = (np.random.default_rng(77).standard_normal(w.n_experts) * 0.3).astype(np.float32)
    h.log(f"[restricted small {variant}] M={w.M} E={w.n_experts}")
    rep = h.run_block(w, bias_override=bias)
    c = rep.counters[0]
    assert c["restricted"] >= 1
    if w.atlas_period:
        assert c["period_update"] >= 1


def test_coverage_fallback():
    """A narrow support (B = c = 1) facing a new, unrelated hidden state every iteration
    misses the coverage goal: those forwards rebuild it and route over all experts."""
    h = H()
    w = synth.workload(2, hidden=128, n_experts=16, top_k=3, inter=64, batch=2, block=24,
                       iters=6, staleness_R=2, routing="restricted", atlas_B=1, atlas_c=1,
                       redraw_every=1, rho_live=0.0, rho_decoded=0.0)
    h.log(f"[restricted coverage fallback] M={w.M}")
    rep = h.run_block(w)
    assert rep.counters[0]["coverage_fallback"] >= 1


def test_workload2_restricted_full_size():
    h = H()
    w = synth.workload(2, routing="restricted")
    h.log(f"[restricted full] {w.name}")
    rep = h.run_block(w, rows=sample_rows(w.M, 24, 12))
    assert rep.iters == w.iters and rep.counters[0]["restricted"] >= 1


def test_workload5_restricted_full_shape():
    h = H()
    w = synth.workload(5, forced_fraction=0.25, staleness_R=4, routing="restricted")
    h.log(f"[restricted full] {w.name}: f=0.25 R=4, 10 iterations (hidden state redrawn at 8)")
    rep = h.run_block(w, iters=10, rows=sample_rows(w.M, 8, 15))
    assert rep.iters == 10 and rep.counters[0]["restricted"] >= 1
