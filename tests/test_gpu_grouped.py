"""GPU parity of the group-limited top-k (experts in contiguous groups; each position selects
among the experts of its best groups), over all experts and inside the support."""
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


def groups_of(ids, gsz):
    return max(len(set((row // gsz).tolist())) for row in ids)


@pytest.mark.parametrize("routing", ["exact", "restricted"])
@pytest.mark.parametrize("variant", ["softmax-e20-g4", "sigmoid-e40-g8-shared"])
def test_small_grouped_every_row(variant, routing):
    """Ragged positions; groups of 5 experts; every output row compared."""
    h = H()
    if variant == "softmax-e20-g4":
        w = synth.workload(2, hidden=256, n_experts=20, top_k=4, inter=128, batch=3, block=21,
                           iters=8, staleness_R=3, n_group=4, topk_group=2, routing=routing)
    else:
        w = synth.workload(3, hidden=192, n_experts=40, top_k=6, inter=192, shared_inter=128,
                           batch=5, block=13, iters=8, staleness_R=2, n_layers=1, zipf=None,
                           n_group=8, topk_group=3, routing=routing)
    h.log(f"[grouped {routing} {variant}] M={w.M} E={w.n_experts}")
    seen = []
    def hook(it, plan, orcs):
        if it:
            seen.append(plan.inspect(0)["routed_ids"].cpu().numpy())
    rep = h.run_block(w, hook=hook)
    gsz = w.n_experts // w.n_group
    assert all(groups_of(r, gsz) <= w.topk_group for r in seen)
    if routing == "restricted":
        assert rep.counters[0]["restricted"] >= 1


def test_grouped_restricted_short_rows_fall_back():
    """A support too narrow for some position's chosen groups to hold K of its experts sends
    those forwards down the full path (counted as coverage fallbacks)."""
    h = H()
    w = synth.workload(2, hidden=128, n_experts=16, top_k=3, inter=64, batch=2, block=24,
                       iters=6, staleness_R=2, routing="restricted", atlas_B=2, atlas_c=1,
                       n_group=4, topk_group=2, alpha=(0, 1))
    h.log(f"[grouped restricted short rows] M={w.M}")
    rep = h.run_block(w)
    assert rep.counters[0]["coverage_fallback"] >= 1


def test_workload2_grouped_full_size():
    h = H()
    w = synth.workload(2, n_group=8, topk_group=4)
    h.log(f"[grouped full] {w.name} n_group 8 topk_group 4")
    rep = h.run_block(w, rows=sample_rows(w.M, 24, 21))
    assert rep.iters == w.iters


def test_workload5_grouped_restricted_full_shape():
    h = H()
    w = synth.workload(5, forced_fraction=0.25, staleness_R=4, routing="restricted",
                       n_group=8, topk_group=4)
    h.log(f"[grouped restricted full] {w.name}: f=0.25 R=4, 10 iterations")
    rep = h.run_block(w, iters=10, rows=sample_rows(w.M, 8, 22))
    assert rep.iters == 10
