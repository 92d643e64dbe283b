"""CPU tests of the seeded workload generator (not of the method): realized activation
frequencies against the closed form the biases are calibrated to, and union growth with
batch against its closed form. numpy does the matrix products here."""
import math

import numpy as np
import pytest
import torch
from scipy.stats import norm

from synth import get_config, make_layer, make_tokens, zipf_targets


def test_zipf_targets_mean_and_shape():
    for n, s, a in [(3072, 1.1, 0.10), (16384, 1.1, 0.05), (11008, 1.0, 0.10), (49152, 1.2, 0.05)]:
        f = zipf_targets(n, s, a)
        assert abs(f.mean() - a) < 1e-9
        assert np.all(np.diff(f) <= 0) and f.max() <= 0.99 and f.min() >= 1e-4


def test_hot_share():
    # the top 20% of neurons carry most activations (power-law locality)
    f = zipf_targets(3072, 1.1, 0.10)
    assert f[: int(0.2 * 3072)].sum() / f.sum() > 0.6


def _emp(cfg, layer, N, **kw):
    L = make_layer(cfg, layer, "cpu", **kw)
    d = L.w_a.shape[1]
    X = make_tokens(cfg, N, 100, "cpu", d=d).double().numpy()
    A = X @ L.w_a.double().numpy().T + L.b_a.double().numpy()
    S = (X @ L.p1.double().numpy().T) @ L.p2.double().numpy().T + L.c.double().numpy()
    return L, A, S


def test_frequencies_gaussian_tokens():
    """Gaussian tokens: W x is exactly Gaussian, so each neuron's realized activation
    frequency must sit within 5 binomial sigmas of its target, and the mean near the target."""
    cfg = get_config("C1")
    N = 4096
    L, A, S = _emp(cfg, 0, N)
    f = L.freq
    for M in (A, S):   # true pre-activations and predictor scores are both calibrated
        emp = (M > 0).mean(axis=0)
        sig = np.sqrt(f * (1 - f) / N)
        assert np.all(np.abs(emp - f) <= 5 * sig + 1e-3), np.max(np.abs(emp - f) / sig)
        assert abs(emp.mean() - 0.10) < 0.005


def test_frequencies_relu_rmsnorm_tokens():
    """relu(rmsnorm(z)) tokens (the gated stack's input): about half the coordinates are zero,
    and the calibrated mean activity holds to the central-limit approximation."""
    cfg = get_config("C3")
    L, A, S = _emp(cfg, 0, 2048, d=1024, n=2048, rank=64)
    X = make_tokens(cfg, 512, 100, "cpu", d=1024).numpy()
    assert abs((X == 0).mean() - 0.5) < 0.02
    assert abs((A > 0).mean() - 0.10) < 0.01
    assert abs((S > 0).mean() - 0.10) < 0.01


def test_union_closed_form():
    """E[n_union(B)] = sum_i 1 - (1 - p_i)^B for independent tokens, p_i the per-neuron
    frequency of the predicted mask."""
    cfg = get_config("C1")
    N = 4096
    _, _, S = _emp(cfg, 0, N)
    Mk = S > 0
    p = Mk.mean(axis=0)
    for B in (4, 16, 32):
        groups = Mk[: (N // B) * B].reshape(N // B, B, -1).any(axis=1).sum(axis=1)
        expect = np.sum(1 - (1 - p) ** B)
        sem = groups.std(ddof=1) / math.sqrt(len(groups))
        assert abs(groups.mean() - expect) < 3 * sem + 1.0, (B, groups.mean(), expect)


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C5"])
def test_configs_shapes(name):
    cfg = get_config(name)
    assert cfg.d % 8 == 0 and cfg.rank % 8 == 0
    assert len(cfg.activity) == cfg.layers


def test_generator_is_seeded():
    cfg = get_config("C1")
    a = make_layer(cfg, 0, "cpu", d=64, n=128, rank=8)
    b = make_layer(cfg, 0, "cpu", d=64, n=128, rank=8)
    c = make_layer(cfg, 1, "cpu", d=64, n=128, rank=8)
    assert torch.equal(a.w_a, b.w_a) and torch.equal(a.c, b.c) and torch.equal(a.p1, b.p1)
    assert not torch.equal(a.w_a, c.w_a)
    assert np.allclose(norm.cdf(0.0), 0.5)
