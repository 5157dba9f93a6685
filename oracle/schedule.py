"""Oracle stage 1: confidence scheduler (per-request verify windows).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix
------------------
* DSpark-in-SGLang page, §A2 "DSpark core components": the confidence head
  scores each draft token's chance of passing verification, and the product of
  the scores over the block is the block's survival probability.
* Same page, §速读 and §A2 "cost-table profiling and modelling": the scheduler
  estimates the step time with the additive model
  ``T(bs, K) = bias + alpha(bs) + theta(M)``, ``M = bs + K``, where ``K`` is the
  batch's extra verify tokens; ``alpha`` is not trimmable and ``theta`` is the
  only term trimming recovers.  The scheduler's argmax weighs expected accepted
  tokens against that real marginal cost.
* Same page, §A3: compact mode is a per-step "SPS-argmax" budget; static
  verifies the whole block, cap-accept verifies the whole block but commits up
  to the scheduled window, no-trim is compact without a cost table (full
  windows).

Readings taken where the pages are silent
-----------------------------------------
* Block layout: ``gamma`` rows per request, row 0 is the anchor (last committed
  token), rows ``1..gamma-1`` carry drafts ``d_1..d_{gamma-1}`` whose
  confidences are ``conf[i, 0..gamma-2]``.  A window ``w`` in ``[1, gamma]``
  counts packed rows, so ``K = sum(w_i - 1)`` and ``M = sum(w_i)``.
* Survival of draft ``k`` (all of ``d_1..d_k`` accepted) is
  ``S[i,k] = c[i,1] * ... * c[i,k]``, formed left to right in fp64.
* Objective: expected committed tokens per unit step time,
  ``E(K) / T(bs, K)``, where ``E`` counts one bonus token per request plus the
  survival of every verified draft.  Because ``c <= 1`` every request's
  survival is non-increasing in ``k``, so the best window vector for a given
  ``K`` takes the ``K`` largest survivals, and the optimum is found by scanning
  ``K``.
* Determinism contract (so an integer output can be compared bit for bit):
  survivals are summed as int64 fixed point ``floor(S * 2**40)``; ``T`` is
  ``(bias + alpha[bs]) + theta[bs + K]`` with two fp64 adds in that order; the
  ratio is one IEEE fp64 divide of the exactly converted fixed-point sum;
  ``K*`` is the first (smallest) ``K`` reaching the maximum; candidates are
  ranked by ``(S desc, request asc, position asc)``.
"""

import math

import numpy as np

STATIC, COMPACT, CAP_ACCEPT, NO_TRIM = 0, 1, 2, 3
MODE_NAMES = {STATIC: "static", COMPACT: "compact", CAP_ACCEPT: "cap_accept",
              NO_TRIM: "no_trim"}

FIXED_SHIFT = 40  # survival fixed point: Q = floor(S * 2**40)


def survival(conf):
    """Block survival probabilities ``S[i, k]``, ``k = 0..gamma-1``.

    ``conf`` holds ``c[i, 1..gamma-1]`` in its columns ``0..gamma-2``.
    ``S[i, 0] = 1`` (the anchor row is always verified); ``S[i, k]`` is the
    running product of the first ``k`` confidences, one fp64 rounding per step.
    DSpark-in-SGLang page, §A2 (product of confidence scores = survival).
    """
    conf = np.asarray(conf, dtype=np.float64)
    B, g1 = conf.shape
    if np.any(~(conf >= 0.0)) or np.any(~(conf <= 1.0)):
        raise ValueError("confidence outside [0, 1] (or NaN)")
    S = np.empty((B, g1 + 1), dtype=np.float64)
    S[:, 0] = 1.0
    for k in range(1, g1 + 1):
        S[:, k] = S[:, k - 1] * conf[:, k - 1]
    return S


def step_time(bias, alpha, theta, bs, K):
    """Additive step-time model ``T(bs, K) = bias + alpha(bs) + theta(bs + K)``.

    DSpark-in-SGLang page, §速读 (equation for T) and §A2 (M = bs + K).
    ``alpha`` and ``theta`` are tables indexed by ``bs`` and ``M``.
    """
    return (float(bias) + float(alpha[bs])) + float(theta[bs + K])


def _fixed(s):
    # s * 2**40 is exact in fp64 (power-of-two scale, s <= 1); floor is exact.
    return int(math.floor(s * float(1 << FIXED_SHIFT)))


def schedule(conf, gamma, mode, bias, alpha, theta):
    """Pick per-request windows.

    Returns ``(w_commit, w_verify, k_star, e_star)``:

    * ``w_commit[i]`` -- rows whose verdicts may be committed,
    * ``w_verify[i]`` -- rows packed and verified,
    * ``k_star`` -- extra verify tokens of the chosen budget,
    * ``e_star`` -- expected committed tokens at ``k_star`` (fixed point / 2**40).

    static and no-trim verify and commit full blocks; compact verifies and
    commits the scheduled windows; cap-accept verifies full blocks and commits
    the scheduled windows (DSpark-in-SGLang page, §A2 "verify modes").
    """
    conf = np.asarray(conf, dtype=np.float64)
    B = conf.shape[0]
    if conf.shape[1] != gamma - 1:
        raise ValueError("conf must have gamma-1 columns")
    S = survival(conf)
    Q = [[_fixed(S[i, k]) for k in range(gamma)] for i in range(B)]
    base = B << FIXED_SHIFT  # one bonus token per request

    if mode in (STATIC, NO_TRIM):
        n = base + sum(Q[i][k] for i in range(B) for k in range(1, gamma))
        w = np.full(B, gamma, dtype=np.int64)
        return w.copy(), w.copy(), B * (gamma - 1), n / float(1 << FIXED_SHIFT)
    if mode not in (COMPACT, CAP_ACCEPT):
        raise ValueError("unknown mode")

    cands = [(i, k) for i in range(B) for k in range(1, gamma)]
    order = sorted(cands, key=lambda ik: (-S[ik[0], ik[1]], ik[0], ik[1]))

    best_r, k_star, n_star = None, 0, base
    n = base
    for K in range(len(order) + 1):
        if K > 0:
            i, k = order[K - 1]
            n += Q[i][k]
        T = step_time(bias, alpha, theta, B, K)
        if not (T > 0.0):
            raise ValueError("step-time model must be positive")
        r = float(n) / T
        if best_r is None or r > best_r:
            best_r, k_star, n_star = r, K, n

    w = np.ones(B, dtype=np.int64)
    for i, _k in order[:k_star]:
        w[i] += 1
    e_star = n_star / float(1 << FIXED_SHIFT)
    if mode == COMPACT:
        return w.copy(), w.copy(), k_star, e_star
    return w.copy(), np.full(B, gamma, dtype=np.int64), k_star, e_star
