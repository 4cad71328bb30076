"""The seeded generators are deterministic and per-expert regenerable (CPU only)."""
import numpy as np

import synth


def test_expert_regenerable_and_deterministic():
    w = synth.workload(2, hidden=64, inter=32, n_experts=6)
    W = synth.layer_weights(w, 0, threads=3)
    for e in (0, 5):
        assert np.array_equal(W["w1"][e], synth.expert_weight(w, 0, "w1", e))
        assert np.array_equal(W["w2"][e], synth.expert_weight(w, 0, "w2", e))
    W2 = synth.layer_weights(w, 0, threads=1)
    assert all(np.array_equal(W[k], W2[k]) for k in ("router_w", "w1", "w3", "w2"))
    assert not np.array_equal(W["w1"], synth.layer_weights(w, 1)["w1"])


def test_bf16_rounding_is_nearest_even():
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], dtype=np.float32)
    b = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a))
    assert b[0] == 1.0 and b[1] == 1.0 and b[2] == 1.0 + 2 ** -6 and b[3] == -2.5
    assert abs(b[4] - 3.0e-3) <= 2 ** -8 * 3.0e-3  # unit roundoff of an 8-bit significand


def test_liveness_schedules():
    w = synth.workload(2)
    D = synth.decoded_masks(w)
    assert D.shape == (w.iters, w.M) and D[0].sum() == 0
    assert (np.diff(D.astype(int), axis=0) >= 0).all()           # decoded stays decoded
    w5 = synth.workload(5, forced_fraction=0.25)
    F = synth.force_masks(w5)
    assert (F.sum(1) == int(np.ceil(0.25 * w5.M))).all()
    D5 = synth.decoded_masks(w5)
    assert D5[0].sum() == 0 and D5[1:].all()


def test_hidden_state_marginals():
    w = synth.workload(2, hidden=256, batch=4, iters=6)
    X = synth.hidden_states(w, 0)
    x = synth.bf16_bits_to_f32(X)
    assert abs(x.std() - 1.0) < 0.05 and abs(x.mean()) < 0.05
    w5 = synth.workload(5, hidden=64, batch=2, iters=10)
    X5 = synth.hidden_states(w5, 0)
    assert np.array_equal(X5[0], X5[7]) and not np.array_equal(X5[7], X5[8])
