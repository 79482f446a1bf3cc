"""Seeded input generator: determinism and bf16 rounding."""
import numpy as np
import pytest

import gdn_synth as gs


def test_bf16_round_to_nearest_even_matches_torch():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 3,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8,
                                  0.0, -0.0, 1e-30, 65504.0], dtype=np.float32)])
    ours = gs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = gs.bf16_bits_to_f64(ours)
    np.testing.assert_array_equal(
        back, torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())


def test_window_inputs_deterministic_and_keyed():
    s = gs.WindowShape(2, 3, 4, 2, 16, 8, 5)
    a = gs.window_inputs(s, (7, 1), ragged=True)
    b = gs.window_inputs(s, (7, 1), ragged=True)
    c = gs.window_inputs(s, (7, 2), ragged=True)
    for x, y in zip((a.q, a.k, a.v, a.beta, a.g), (b.q, b.k, b.v, b.beta, b.g)):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a.q, c.q)
    assert a.q.shape == (2, 3, 5, 2, 16) and a.v.shape == (2, 3, 5, 4, 8)
    assert np.all((a.t_lane >= 1) & (a.t_lane <= 5))
    assert np.all((a.beta > 0) & (a.beta < 1)) and np.all(a.g < 0)
    m = gs.accepted_uniform(a.t_lane, (7, 1))
    assert np.all((m >= 0) & (m <= a.t_lane))
    mb = gs.accepted_binomial(a.t_lane, 0.7, (7, 1))
    assert np.all((mb >= 0) & (mb <= a.t_lane))


def test_prefill_gate_distribution_is_slow_decay():
    p = gs.prefill_inputs(4096, 2, 2, 8, 8, (4,))
    alpha = np.exp(p.g.astype(np.float64))
    # g = -softplus(N(-2, 1)): alpha is close to 1 on average
    assert alpha.mean() > 0.8
