"""Oracle stage 4a: target LM head over the packed rows.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The verify forward ends in the target model's vocabulary projection of every
packed row; the target's prediction for a row is the arg-max logit (explainer
page, §1.2: the target computes logits for every draft position in one pass and
drafts are checked against them; §3.3 takes ``softmax`` / ``argmax`` of those
logits).

Readings: ``z[r, v] = sum_h W[v, h] * x[r, h]`` in fp64 on the exact input
values; the prediction is the lowest vocabulary index among the maximal logits.
"""

import numpy as np


def lm_head_logits(hidden, W, chunk=8192):
    """``hidden`` [R, H] and ``W`` [V, H] -> fp64 logits [R, V].

    The vocabulary is processed in slices only to bound host memory; every
    logit is one independent dot product.
    """
    x = np.asarray(hidden, dtype=np.float64)
    V = W.shape[0]
    z = np.empty((x.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, chunk):
        Wc = np.asarray(W[v0:v0 + chunk], dtype=np.float64)
        z[:, v0:v0 + chunk] = x @ Wc.T
    return z


def lm_head_pred(z):
    """Lowest index of the maximal logit of each row (``np.argmax`` returns
    the first occurrence)."""
    return np.argmax(np.asarray(z), axis=1).astype(np.int64)
