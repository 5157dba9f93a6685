"""Oracle: the step-time model fitted from recorded step times.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix
------------------
DSpark-in-SGLang page, §A2 "cost-table profiling and modelling" (and the
additive model of §速读): the step time is profiled over batch size and verify
tokens and modelled as ``T(bs, K) = bias + alpha(bs) + theta(M)`` with
``M = bs + K``; the scheduler reads that table.

Readings taken where the pages are silent
-----------------------------------------
The pages give neither the form of ``alpha`` and ``theta`` nor how the table is
fitted.  The plainest reading that the additive model supports: both terms are
linear, ``alpha(bs) = a * bs`` and ``theta(M) = th * M``, and ``(bias, a, th)``
is the ordinary least-squares fit of ``T`` over the recorded samples
``(bs, M, T)``.  The scheduler's tables are ``alpha[b] = a * b`` and
``theta[m] = th * m``.
"""

import numpy as np


def fit_cost_model(bs, M, t):
    """Least-squares ``(bias, a, th)`` of ``t ~ bias + a*bs + th*M``.

    Raises ValueError when the samples do not determine the three
    coefficients (fewer than three samples, or samples on one line)."""
    bs = np.asarray(bs, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    if bs.ndim != 1 or not (len(bs) == len(M) == len(t)) or len(bs) < 3:
        raise ValueError("need at least three samples (bs, M, t)")
    A = np.stack([np.ones_like(bs), bs, M], axis=1)
    coef, _, rank, _ = np.linalg.lstsq(A, t, rcond=None)
    if rank < 3:
        raise ValueError("samples do not determine bias, alpha and theta")
    return coef


def cost_tables(coef, alpha_len, theta_len):
    """The scheduler's tables from fitted coefficients: ``bias``,
    ``alpha[b] = a*b`` for ``b < alpha_len``, ``theta[m] = th*m`` for
    ``m < theta_len``."""
    bias, a, th = (float(x) for x in coef)
    return bias, a * np.arange(alpha_len, dtype=np.float64), th * np.arange(theta_len, dtype=np.float64)
