"""Predicted-KL reduction q(D) and the step controller (TEST INFRASTRUCTURE ONLY).

[LoGRA] PKL: before an update is applied, the method estimates how much it
would change next-token probabilities.  It takes a small sample of responses
from the current batch and compares, at one common temperature, the model's
current vocabulary distribution with the distribution after the proposed
update.  The predicted change is quadratic in the step: the mean predicted KL
scales as alpha^2 q(D), so halving alpha divides it by four.  For a KL budget
delta the controller sets alpha = min(alpha_max, sqrt(delta / q(D))); with
q(D) = 4 delta the proposal is at most halved, and alpha_max stops tiny
predicted KLs from blowing the step up.  The budget may be constant or
annealed downward.

Readings where the pages leave a step open:
  * q(D) is the mean over the sampled token positions (rows) of the forward
    KL(p_cur || p_prop), p = softmax(z / tau), with p_prop the alpha = 1
    proposal; every row has equal weight.
  * controller edges: q = 0 or q < 0 (rounding) gives alpha_max; a NaN q
    gives a NaN alpha; an infinite q gives alpha = 0.
  * masked vocabulary entries: a logit of -inf is a token of probability
    zero.  Such a token of the current distribution contributes nothing to
    KL(p || p') (the convention 0 log 0 = 0); a token with p > 0 and p' = 0
    makes the KL +inf.  A row whose every logit is -inf has no distribution:
    its KL is NaN.  Other non-finite logits (NaN, +inf) give NaN.
All arithmetic is fp64.
"""
import numpy as np


def log_softmax(a):
    """Row-wise log softmax of a 2-D fp64 array."""
    a = np.asarray(a, np.float64)
    m = a.max(axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):      # rows with no finite logit give NaN
        return a - m - np.log(np.exp(a - m).sum(axis=1, keepdims=True))


def kl_rows(z_cur, z_prop, tau):
    """Per-row forward KL(softmax(z_cur/tau) || softmax(z_prop/tau)), the sum
    of p (log p - log p') over the tokens with p > 0 (masked tokens, z_cur =
    -inf, contribute nothing; p > 0 with p' = 0 contributes +inf)."""
    lp = log_softmax(np.asarray(z_cur, np.float64) / tau)
    lq = log_softmax(np.asarray(z_prop, np.float64) / tau)
    with np.errstate(invalid="ignore"):
        terms = np.where(lp == -np.inf, 0.0,                    # p = 0
                         np.where(lq == -np.inf, np.inf,        # p > 0, p' = 0
                                  np.exp(lp) * (lp - lq)))
    # (a row with no finite current logit gives NaN from log_softmax, which
    # propagates, as do NaN and +inf logits)
    return terms.sum(axis=1)


def predicted_kl(z_cur, z_prop, tau):
    """q(D): the mean per-row KL."""
    return float(kl_rows(z_cur, z_prop, tau).mean())


def step_size(q, kl_budget, alpha_max):
    """alpha = min(alpha_max, sqrt(delta / q)) with the edge readings above."""
    q = float(q)
    if np.isnan(q):
        return float("nan")
    if q <= 0.0:
        return float(alpha_max)
    return float(min(float(alpha_max), np.sqrt(float(kl_budget) / q)))


# --------------------------------------------------------------------------
# Direction-form sweep (the KL at several step multipliers in one call).
#
# [LoGRA] PKL: the proposal is the current model moved along the update
# direction; the predicted KL is quadratic in the step multiplier alpha.
# Here the proposed logits are z + alpha * delta, formed exactly (fp64, no
# rounding to bf16), so the alpha^2 law holds on the inputs as given.
# Readings: the weighted mean uses non-negative per-row weights (None means
# equal weights); a token mask or per-response averaging is a choice of
# weights, and a row of weight zero is left out whatever its KL.  A zero
# weight sum gives NaN.

def kl_sweep_rows(z, delta, alphas, tau):
    """(n_alpha, n_tok) array: row t, multiplier a -> KL(p(z_t) || p(z_t + a delta_t)).
    A masked token (z = -inf) stays masked in every proposal, whatever its
    direction entry."""
    z = np.asarray(z, np.float64)
    delta = np.asarray(delta, np.float64)
    masked = z == -np.inf
    with np.errstate(invalid="ignore"):
        props = [np.where(masked, -np.inf, z + float(a) * delta) for a in alphas]
    return np.stack([kl_rows(z, zp, tau) for zp in props])


def predicted_kl_sweep(z, delta, alphas, tau, weights=None):
    """Weighted mean over rows of kl_sweep_rows, one value per multiplier.  A
    row of weight zero is left out whatever its KL (a masked position, e.g.
    padding past a response's end, may have no distribution at all)."""
    rows = kl_sweep_rows(z, delta, alphas, tau)
    if weights is None:
        return rows.mean(axis=1)
    w = np.asarray(weights, np.float64)
    tot = w.sum()
    if tot == 0.0:
        return np.full(rows.shape[0], np.nan)
    with np.errstate(invalid="ignore"):
        terms = np.where(w[None, :] != 0.0, rows * w[None, :], 0.0)
    return terms.sum(axis=1) / tot
