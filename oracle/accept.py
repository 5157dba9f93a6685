"""Oracle stage 4b: acceptance (greedy and ``min(1, p/q)``) with the
cap-accept ceiling.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix
------------------
* Greedy: drafts are accepted while they agree with the target and everything
  from the first disagreement on is dropped (explainer page, §1.2).
* Rejection sampling: draft token ``x`` is kept with probability
  ``min(1, p(x) / q(x))`` (explainer page, §2.3 and §3.3), ``p`` the target and
  ``q`` the draft distribution.
* cap-accept verifies the full block but commits only up to the scheduled
  window: its commits equal compact's and it exposes how many tokens the full
  block would have accepted (DSpark-in-SGLang page, §A2 "verify modes" and
  "observability").

Readings taken where the pages are silent
-----------------------------------------
* Row ``j - 1`` of a request (``j = 1..w-1``) predicts the token at draft
  position ``j``; ``ceiling`` counts the leading accepted drafts over all
  verified rows, ``accept = min(ceiling, w_commit - 1)``.
* Greedy bonus token: the target's prediction at row ``accept``.
* ``min(1, p/q)`` is evaluated as ``u * q(x) < p(x)`` with a uniform ``u`` per
  draft position (no epsilon); ``p = softmax(z)`` at temperature 1.
* Bonus token under rejection sampling (the standard rule the explainer page
  attributes to the speculative-decoding paper): after a rejection at draft
  ``j`` it is drawn from ``norm(max(0, p_{j-1} - q_j))``; if every committed
  draft was accepted it is drawn from ``p`` at row ``w_commit - 1``.  The draw
  is an inverse CDF in vocabulary order with one uniform ``u'`` per request:
  the smallest ``v`` whose running mass exceeds ``u' * total``.
* By causality, a cap-accept request whose ceiling reaches its commit window
  resolves its bonus at row ``w_commit - 1`` exactly as compact does.
"""

import numpy as np

GREEDY, REJECTION = 0, 1


def accept_greedy(pred, cu, w_commit, w_verify, drafts):
    """Returns ``(accept, bonus, ceiling)`` per request."""
    B = len(w_commit)
    accept = np.zeros(B, dtype=np.int64)
    bonus = np.zeros(B, dtype=np.int64)
    ceiling = np.zeros(B, dtype=np.int64)
    for i in range(B):
        base = int(cu[i])
        c = 0
        while c < int(w_verify[i]) - 1 and int(drafts[i][c]) == int(pred[base + c]):
            c += 1
        a = min(c, int(w_commit[i]) - 1)
        ceiling[i] = c
        accept[i] = a
        bonus[i] = int(pred[base + a])
    return accept, bonus, ceiling


def softmax(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def residual_sample(r, u):
    """Inverse CDF of the non-negative weights ``r`` in index order.

    Returns ``(index, margin, neighbour)``: the smallest ``v`` with
    ``cumsum(r)[v] > u * sum(r)``; the distance of ``u * sum(r)`` to the
    nearest cumulative boundary relative to ``sum(r)``; and the token on the
    other side of that nearest boundary (the largest earlier ``v`` of non-zero
    weight when the lower boundary is nearer, else the smallest later one; the
    index itself when there is none).  Tests use the last two to tell a
    well-posed draw from one that rounding may move to the neighbouring token.
    """
    r = np.asarray(r, dtype=np.float64)
    cdf = np.cumsum(r)
    total = cdf[-1]
    target = u * total
    idx = int(np.searchsorted(cdf, target, side="right"))
    if idx >= len(r):  # rounding pushed the target past the last step
        idx = int(np.nonzero(r > 0)[0][-1])
    lo = cdf[idx - 1] if idx > 0 else 0.0
    d_lo, d_hi = abs(target - lo), abs(cdf[idx] - target)
    margin = min(d_lo, d_hi) / total
    nz = np.nonzero(r > 0)[0]
    if d_lo <= d_hi:
        before = nz[nz < idx]
        neighbour = int(before[-1]) if len(before) else idx
    else:
        after = nz[nz > idx]
        neighbour = int(after[0]) if len(after) else idx
    return idx, margin, neighbour


def accept_rejection(z_rows, cu, w_commit, w_verify, drafts, q_rows, u,
                     u_bonus, diag=None):
    """Rejection-sampling acceptance.

    ``z_rows`` [>=M, V] logits of the packed rows; ``q_rows`` [B, gamma-1, V]
    draft distributions; ``u`` [B, gamma-1]; ``u_bonus`` [B].  Returns
    ``(accept, bonus, ceiling)``.  If ``diag`` is a dict it receives, per
    request, the relative margins of every accept decision and of the bonus
    draw, and the token across the bonus draw's nearest CDF step.
    """
    B = len(w_commit)
    accept = np.zeros(B, dtype=np.int64)
    bonus = np.zeros(B, dtype=np.int64)
    ceiling = np.zeros(B, dtype=np.int64)
    for i in range(B):
        base = int(cu[i])
        wv, wc = int(w_verify[i]), int(w_commit[i])
        dec_margins = []
        c = 0
        for j in range(1, wv):
            d = int(drafts[i][j - 1])
            p = softmax(z_rows[base + j - 1])
            lhs = float(u[i][j - 1]) * float(q_rows[i][j - 1][d])
            dec_margins.append(abs(lhs - p[d]) / max(p[d], 1e-300))
            if lhs < p[d]:
                c += 1
            else:
                break
        a = min(c, wc - 1)
        if c < wc - 1:
            p = softmax(z_rows[base + c])
            r = np.maximum(0.0, p - np.asarray(q_rows[i][c], dtype=np.float64))
        else:
            r = softmax(z_rows[base + wc - 1])
        b, margin, neighbour = residual_sample(r, float(u_bonus[i]))
        ceiling[i], accept[i], bonus[i] = c, a, b
        if diag is not None:
            diag.setdefault("decision_margin", []).append(dec_margins)
            diag.setdefault("bonus_margin", []).append(margin)
            diag.setdefault("bonus_neighbour", []).append(neighbour)
    return accept, bonus, ceiling
