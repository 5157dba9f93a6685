"""Oracle stage 2: ragged front-packing and capture-tier rounding.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

DSpark-in-SGLang page, §A2 "ragged verify over a full CUDA graph" and Fig. 2:
variable-length requests are front-packed into one compact buffer with a
cu_seqlens-style variable-length layout, no per-request padding; only the total
is rounded up to the nearest captured tier, and a smaller total replays a
smaller tier.

Readings: row ``k`` of request ``i`` sits at sequence position ``ctx[i] + k``
(``ctx`` = committed tokens before the anchor); its token is the anchor for
``k == 0`` and draft ``d_k`` otherwise; its KV slot is
``page_table[i][pos // P] * P + pos % P``.  Rows between the real total ``M``
and the tier ``M_pad`` are padding and carry ``-1`` in every field.  Without
tiers ``M_pad = M``; a total above the largest tier is an error.
"""

import numpy as np


def select_tier(M, tiers):
    """Smallest tier ``>= M``; ``M`` itself when no tiers are given."""
    if not tiers:
        return int(M)
    for t in sorted(tiers):
        if t >= M:
            return int(t)
    raise OverflowError("packed total exceeds the largest capture tier")


def pack(w_verify, anchor, drafts, ctx, page_table, page_size, tiers):
    """Return ``(cu, M, M_pad, row_req, row_pos, tok, slot)``."""
    w = [int(x) for x in w_verify]
    B = len(w)
    cu = np.zeros(B + 1, dtype=np.int64)
    for i in range(B):
        cu[i + 1] = cu[i] + w[i]
    M = int(cu[B])
    M_pad = select_tier(M, tiers)
    row_req = np.full(M_pad, -1, dtype=np.int64)
    row_pos = np.full(M_pad, -1, dtype=np.int64)
    tok = np.full(M_pad, -1, dtype=np.int64)
    slot = np.full(M_pad, -1, dtype=np.int64)
    P = int(page_size)
    for i in range(B):
        for k in range(w[i]):
            r = int(cu[i]) + k
            pos = int(ctx[i]) + k
            row_req[r] = i
            row_pos[r] = pos
            tok[r] = int(anchor[i]) if k == 0 else int(drafts[i][k - 1])
            slot[r] = int(page_table[i][pos // P]) * P + pos % P
    return cu, M, M_pad, row_req, row_pos, tok, slot
