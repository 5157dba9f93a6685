"""Oracle: the block-accept estimator (the ceiling that truncation hides).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix
------------------
DSpark-in-SGLang page, §A2 "observability and ceiling recovery" and "the
ceiling estimator under truncation": compact mode verifies only the
scheduled window, so how many tokens the full block would have accepted is
not observed; cap-accept exposes it by verifying the whole block.  For runs
without that companion mode, a block-accept estimator recovers the hidden
ceiling from a compact run itself: it uses the target's token usage and
log-probabilities in later steps and assumes the anchor behaves alike in the
truncated and the untruncated trajectory, giving an interval estimate of the
counterfactual tail.

Readings taken where the pages are silent
-----------------------------------------
* A request of a step is *censored* when its window was truncated
  (``w_verify < gamma``) and every verified draft was accepted
  (``accept == w_verify - 1``): the full block might have accepted more.
  Otherwise its ceiling is observed (a rejection inside the window, or a
  full block).
* The counterfactual tail of a censored request is its drafts
  ``d_w .. d_{gamma-1}``, proposals for positions ``ctx + w .. ctx + gamma - 1``.
  Later steps commit those positions; the row of a later step whose prediction
  is committed at position ``P`` (rows ``0..accept`` of that step predict
  positions ``ctx' + 1 .. ctx' + accept + 1``) is the target at ``P`` on the
  realised prefix, which the similarity assumption takes for the
  counterfactual one.  Its verdict on the tail draft at ``P`` is an
  acceptance probability ``alpha``: greedy, 1 if the draft equals the row's
  prediction and 0 otherwise; rejection sampling, ``min(1, p(d) / q(d))``
  with ``p`` the row's softmax and ``q`` the draft distribution of the
  censored step.
* With ``S_m`` the product of the first ``m`` resolved ``alpha`` (survival),
  the expected counterfactual tail over ``R`` resolved positions is
  ``E = S_1 + ... + S_R``.  The ceiling interval is
  ``[base + E, base + E + S_R * (unresolved positions)]`` with
  ``base = w - 1``; it closes when every tail position is resolved or a
  resolved ``alpha`` is 0 (the tail is cut there).  Under greedy every
  ``alpha`` is 0 or 1, so a closed interval is one integer: the ceiling the
  full block would have reached.
* One probe per request at a time: a censored step opens a probe only when
  the request has none open (after this step's resolutions).  The step that
  opens a probe resolves its first tail position at once (its row
  ``w - 1`` predicts the bonus position ``ctx + w``).
* A probe whose next position is at or before a step's anchor position was
  passed without being resolved (steps were skipped); it is dropped
  uncounted.
"""

import math

import numpy as np

GREEDY, REJECTION = 0, 1


def new_state(B, gamma):
    """Per-request probe state, no probe open."""
    return {
        "pos": np.zeros(B, dtype=np.int64),      # position of the next unresolved tail draft
        "left": np.zeros(B, dtype=np.int64),     # unresolved tail drafts (0: no open probe)
        "done": np.zeros(B, dtype=np.int64),     # resolved tail drafts
        "base": np.zeros(B, dtype=np.int64),     # w - 1 of the censored step
        "tok": np.zeros((B, gamma - 1), dtype=np.int64),    # tail drafts
        "lq": np.zeros((B, gamma - 1), dtype=np.float64),   # their log q (rejection)
        "S": np.zeros(B, dtype=np.float64),      # survival through the resolved tail
        "E": np.zeros(B, dtype=np.float64),      # expected resolved tail
        "count": np.zeros(B, dtype=np.int64),    # closed probes
        "last": np.zeros(B, dtype=np.float64),   # ceiling estimate of the last closed probe (0: none yet)
        "sum": np.zeros(B, dtype=np.float64),    # sum of closed probes' estimates
    }


def _log_softmax_at(z, tok):
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z)
    return float(z[tok] - m - math.log(np.sum(np.exp(z - m))))


def _alpha(rule, row, tok, lq, pred, logits):
    if rule == GREEDY:
        return 1.0 if int(pred[row]) == int(tok) else 0.0
    return min(1.0, math.exp(_log_softmax_at(logits[row], tok) - lq))


def estimate_update(state, cu, w_verify, accept, drafts, ctx, rule, pred=None,
                    logits=None, q_rows=None, closed=None):
    """One step of the estimator, after the step's acceptance and before its
    scatter (``ctx`` is the anchor position of the step).  Updates ``state``
    in place and returns it.  ``pred`` [rows] (greedy) or ``logits``
    [rows, V] and ``q_rows`` [B, gamma-1, V] (rejection).  If ``closed`` is a
    list, each probe closed in this step appends ``(request, first tail
    position, estimate)`` to it."""
    B, g1 = np.asarray(drafts).shape
    gamma = g1 + 1
    st = state

    def resolve(i, row, P):
        if st["left"][i] == 0 or P != st["pos"][i]:
            return
        a = _alpha(rule, row, st["tok"][i][st["done"][i]], st["lq"][i][st["done"][i]], pred, logits)
        st["S"][i] *= a
        st["E"][i] += st["S"][i]
        st["done"][i] += 1
        st["left"][i] -= 1
        st["pos"][i] += 1
        if st["S"][i] == 0.0:          # the tail is cut at this draft
            st["left"][i] = 0
        if st["left"][i] == 0:
            est = float(st["base"][i]) + st["E"][i]
            st["count"][i] += 1
            st["last"][i] = est
            st["sum"][i] += est
            if closed is not None:
                closed.append((i, int(st["pos"][i] - st["done"][i]), est))

    for i in range(B):
        base, a, wv, c = int(cu[i]), int(accept[i]), int(w_verify[i]), int(ctx[i])
        if st["left"][i] > 0 and st["pos"][i] <= c:
            st["left"][i] = 0                 # passed unresolved: dropped
        # rows 0..a predict positions c+1..c+a+1, all committed this step
        for k in range(a + 1):
            resolve(i, base + k, c + k + 1)
        if st["left"][i] == 0 and wv < gamma and a == wv - 1:
            n = gamma - wv
            st["pos"][i] = c + wv
            st["left"][i] = n
            st["done"][i] = 0
            st["base"][i] = wv - 1
            st["S"][i] = 1.0
            st["E"][i] = 0.0
            st["tok"][i][:] = 0
            st["lq"][i][:] = 0.0
            for j in range(n):
                d = int(drafts[i][wv - 1 + j])
                st["tok"][i][j] = d
                if rule == REJECTION:
                    st["lq"][i][j] = math.log(float(q_rows[i][wv - 1 + j][d]))
            resolve(i, base + a, c + a + 1)
    return st


def open_interval(state, i):
    """The ceiling interval of request ``i``'s open probe, or None."""
    if state["left"][i] == 0:
        return None
    lo = float(state["base"][i]) + state["E"][i]
    return lo, lo + state["S"][i] * float(state["left"][i])
