"""The offline STS temperature fit (host code) against facts it does not
compute itself: recovery of known temperatures from logs drawn from the
model, agreement with a general-purpose optimiser on the same likelihood, and
the degenerate cases."""
import numpy as np
import pytest
from scipy.optimize import minimize_scalar

from confidence_scheduled_ragged_amd.calibrate import (fit_sts_temperatures,
                                                       head_logits_from_scores,
                                                       position_log_likelihood)


def _logs(rng, N, T_true, mu=1.5, sd=2.0):
    g = T_true.size
    z = rng.normal(mu, sd, (N, g))
    acc = np.full(N, g)
    alive = np.ones(N, bool)
    for i in range(g):
        p = 1.0 / (1.0 + np.exp(-z[:, i] / T_true[i]))
        rejected = alive & (rng.random(N) >= p)
        acc[rejected] = i
        alive &= ~rejected
    return z, acc


def test_recovers_known_temperatures():
    rng = np.random.default_rng(0)
    T_true = 1.0 + 0.15 * np.arange(6)
    z, acc = _logs(rng, 200_000, T_true)
    T = fit_sts_temperatures(z, acc)
    # the reached sample shrinks along the block; 6 % relative covers the
    # sampling error at the last position with a wide margin
    assert np.all(np.abs(T / T_true - 1.0) < 0.06), T


def test_matches_a_general_optimiser():
    rng = np.random.default_rng(1)
    T_true = np.array([0.8, 1.3, 2.0])
    z, acc = _logs(rng, 20_000, T_true, mu=0.5)
    T = fit_sts_temperatures(z, acc)
    for i in range(3):
        reached = acc >= i
        y = (acc[reached] > i).astype(float)
        res = minimize_scalar(lambda b: -position_log_likelihood(b, z[reached, i], y),
                              bounds=(1e-3, 50.0), method="bounded",
                              options={"xatol": 1e-10})
        assert abs(1.0 / T[i] - res.x) < 1e-6


def test_degenerate_positions_keep_the_default():
    z = np.zeros((100, 3)) + 1.0
    acc = np.full(100, 3)                  # every draft accepted: no rejection to fit
    assert np.all(fit_sts_temperatures(z, acc, default=1.7) == 1.7)
    acc = np.zeros(100, int)               # only position 0 is ever reached
    T = fit_sts_temperatures(z, acc, min_samples=10, default=2.0)
    assert np.all(T[1:] == 2.0)
    with pytest.raises(ValueError):
        fit_sts_temperatures(z, np.full(100, 4))


def test_head_logits_round_trip():
    rng = np.random.default_rng(2)
    z = rng.normal(0, 2, (50, 4))
    temps = np.array([1.0, 1.1, 1.2, 1.3])
    conf = 1.0 / (1.0 + np.exp(-z / temps))
    assert np.allclose(head_logits_from_scores(conf, temps), z, atol=1e-9)
