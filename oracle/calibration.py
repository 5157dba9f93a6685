"""Oracle: per-request confidence statistics and the calibration error (ECE)
of the draft confidences against the target's verdicts.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix
------------------
DSpark-in-SGLang page, §A2 "observability and ceiling recovery": the system
reports per-request confidence and calibration metrics such as ECE for
post-hoc analysis; compact verifies only the scheduled window, so only those
positions carry a verdict, while cap-accept verifies the whole block.

Readings taken where the pages are silent
-----------------------------------------
* A verified draft is draft ``j`` (``1 <= j <= w_verify[i] - 1``) of request
  ``i``; its confidence is ``conf[i, j-1]`` and its label is whether it equals
  the target's prediction at row ``cu[i] + j - 1`` (the greedy per-token
  verdict, independent of earlier drafts).
* ECE with ``n_bins`` equal-width bins over [0, 1]: draft to bin
  ``min(floor(c * n_bins), n_bins - 1)`` (``c * n_bins`` one fp64 product of
  the fp32 confidence), ``ECE = sum_b (n_b / N) |acc_b - conf_b|``, which is
  ``sum_b |matches_b - sum_conf_b| / N``; 0 when nothing was verified.
* Determinism contract (so the GPU's sums compare bit for bit): each bin's
  confidence sum is kept in int64 fixed point, ``sum floor(c * 2**48)``; the
  ECE is ``(sum_b |matches_b * 2**48 - conf_fx_b|) / 2**48 / N`` with the
  numerator an exact integer and two fp64 divides in that order.
"""

import math

FIX_SHIFT = 48


def calibration(conf, drafts, pred, cu, w_verify, n_bins):
    """Returns (bin_count, bin_match, bin_conf_fx, ece, req_verified,
    req_matched) as Python ints / float, looping over every verified draft."""
    B = len(w_verify)
    count = [0] * n_bins
    match = [0] * n_bins
    conf_fx = [0] * n_bins
    req_verified = [0] * B
    req_matched = [0] * B
    for i in range(B):
        for j in range(1, int(w_verify[i])):
            c = float(conf[i][j - 1])
            label = int(drafts[i][j - 1]) == int(pred[int(cu[i]) + j - 1])
            b = min(int(math.floor(c * n_bins)), n_bins - 1)
            count[b] += 1
            match[b] += int(label)
            conf_fx[b] += int(math.floor(c * 2.0 ** FIX_SHIFT))
            req_verified[i] += 1
            req_matched[i] += int(label)
    N = sum(count)
    num = sum(abs(match[b] * 2 ** FIX_SHIFT - conf_fx[b]) for b in range(n_bins))
    ece = (float(num) / 2.0 ** FIX_SHIFT) / N if N else 0.0
    return count, match, conf_fx, ece, req_verified, req_matched
