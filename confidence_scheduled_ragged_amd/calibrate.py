"""Offline fit of the Sequential Temperature Scaling (STS) temperatures from
cap-accept audit logs (host code, numpy only).

[P1] "DFlash to DSpark in SGLang", section "DSpark: a sequential head and a
verify budget": the head estimates, per drafted token, the probability that
the target keeps it; multiplied along the block these give the survival
probability, and STS tunes one temperature per position so the estimates
match measured acceptance; section "The confidence scheduler and verify
modes": the cap-accept arm logs, beside what it commits, the acceptance of the
whole block. Those records are the labels this fit needs.

Model (the same one the kernels apply): position i of a drafted block survives,
given that every earlier draft survived, with probability sigma(z_i / T_i),
where z_i = w.h_i + bias is the untempered head logit. A logged request with
full-verify acceptance a_full reached positions 0..min(a_full, gamma-1);
position i was accepted when a_full > i and rejected when a_full == i. For
each position the temperature is the maximum-likelihood one over the requests
that reached it; each position's likelihood involves only its own T_i, so the
positions are fitted one after another, in block order.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

__all__ = ["head_logits_from_scores", "fit_sts_temperatures", "position_log_likelihood"]


def head_logits_from_scores(conf: np.ndarray, temps: np.ndarray) -> np.ndarray:
    """Untempered head logits z = T_i * logit(conf) from logged scores (as
    written by dspark_confidence) and the temperatures they were taken with.
    Scores are clipped away from 0 and 1 first."""
    c = np.clip(np.asarray(conf, np.float64), 1e-12, 1.0 - 1e-12)
    return np.asarray(temps, np.float64)[None, :] * np.log(c / (1.0 - c))


def position_log_likelihood(beta: float, z: np.ndarray, y: np.ndarray) -> float:
    """Log-likelihood of outcomes y (1 accepted, 0 rejected) at logits z under
    acceptance sigma(beta * z), beta = 1 / T."""
    x = beta * np.asarray(z, np.float64)
    # log sigma(x) = -log(1 + e^-x); log(1 - sigma(x)) = -log(1 + e^x)
    return float(-np.sum(y * np.logaddexp(0.0, -x) + (1 - y) * np.logaddexp(0.0, x)))


def _fit_beta(z: np.ndarray, y: np.ndarray, iters: int, tol: float) -> Optional[float]:
    """Newton's method on beta for one position; None when the data cannot pin
    a finite positive optimum (no mixed outcomes, or a non-positive slope)."""
    if z.size == 0 or y.min() == y.max():
        return None
    beta = 1.0
    for _ in range(iters):
        p = 1.0 / (1.0 + np.exp(-beta * z))
        grad = float(np.sum((y - p) * z))
        hess = -float(np.sum(p * (1.0 - p) * z * z))
        if hess >= 0.0:
            return None
        step = grad / hess
        new = beta - step
        # stay on the side of positive slopes; halve the step when it overshoots
        while new <= 0.0:
            step *= 0.5
            new = beta - step
        if abs(new - beta) <= tol * max(1.0, abs(beta)):
            beta = new
            break
        beta = new
    return beta if beta > 0.0 and np.isfinite(beta) else None


def fit_sts_temperatures(z: np.ndarray, accepted_full: np.ndarray, min_samples: int = 32,
                         default: float = 1.0, iters: int = 100,
                         tol: float = 1e-12) -> np.ndarray:
    """Temperatures T[gamma] that fit sigma(z_i / T_i) to the logged outcomes.

    z: [N, gamma] untempered head logits of N logged drafted blocks;
    accepted_full: [N] full-verify acceptance counts (cap-accept's record),
    in [0, gamma]. A position with fewer than `min_samples` requests reaching
    it, or with outcomes that do not pin a finite temperature, gets `default`.
    """
    z = np.asarray(z, np.float64)
    a = np.asarray(accepted_full, np.int64)
    if z.ndim != 2 or a.shape != (z.shape[0],):
        raise ValueError("z must be [N, gamma] and accepted_full [N]")
    gamma = z.shape[1]
    if np.any(a < 0) or np.any(a > gamma):
        raise ValueError("accepted_full must lie in [0, gamma]")
    temps = np.full(gamma, float(default))
    for i in range(gamma):
        reached = a >= i
        if int(reached.sum()) < min_samples:
            continue
        y = (a[reached] > i).astype(np.float64)
        beta = _fit_beta(z[reached, i], y, iters, tol)
        if beta is not None:
            temps[i] = 1.0 / beta
    return temps
