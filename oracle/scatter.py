"""Oracle stage 5: compact scatter of committed tokens and KV slots.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

DSpark-in-SGLang page, §A2 "performance and zero-overhead scheduling": a fused
compact-scatter kernel writes the step's accepted results back, and the page
table lives on the device so no per-step host sync is needed.

Readings taken where the pages are silent
-----------------------------------------
* A request that accepts ``a`` drafts commits ``a + 1`` tokens: the drafts
  ``d_1..d_a`` and the bonus token.
* The KV written for rows ``0..a`` (anchor and accepted drafts) becomes
  committed: ``req_to_token[i][ctx + k] = slot(row k)``, ``ctx += a + 1``, and
  the bonus token becomes the new anchor (its KV is written next step).
* The KV slots of rows ``a+1..w_verify-1`` are released, listed compactly.
* Committed tokens are appended to a per-request history when one is given.
"""

import numpy as np


def compact_scatter(cu, w_verify, accept, bonus, drafts, slot, ctx, anchor,
                    req_to_token, hist=None, hist_len=None):
    """Returns a dict with ``commit_cu``, ``commit_tok``, ``commit_slot``,
    ``free_slots`` and the updated copies of ``ctx``, ``anchor``,
    ``req_to_token``, ``hist``, ``hist_len`` (inputs are not modified)."""
    B = len(w_verify)
    ctx = np.array(ctx, dtype=np.int64, copy=True)
    anchor = np.array(anchor, dtype=np.int64, copy=True)
    req_to_token = np.array(req_to_token, dtype=np.int64, copy=True)
    if hist is not None:
        hist = np.array(hist, dtype=np.int64, copy=True)
        hist_len = np.array(hist_len, dtype=np.int64, copy=True)
    commit_cu = np.zeros(B + 1, dtype=np.int64)
    for i in range(B):
        commit_cu[i + 1] = commit_cu[i] + int(accept[i]) + 1
    commit_tok = np.zeros(int(commit_cu[B]), dtype=np.int64)
    commit_slot = np.zeros(int(commit_cu[B]), dtype=np.int64)
    free_slots = []
    for i in range(B):
        a = int(accept[i])
        base = int(cu[i])
        toks = [int(drafts[i][j]) for j in range(a)] + [int(bonus[i])]
        for j in range(a + 1):
            commit_tok[commit_cu[i] + j] = toks[j]
            commit_slot[commit_cu[i] + j] = int(slot[base + j])
            req_to_token[i][int(ctx[i]) + j] = int(slot[base + j])
        for j in range(a + 1, int(w_verify[i])):
            free_slots.append(int(slot[base + j]))
        if hist is not None:
            for j in range(a + 1):
                hist[i][int(hist_len[i]) + j] = toks[j]
            hist_len[i] += a + 1
        ctx[i] += a + 1
        anchor[i] = int(bonus[i])
    return {
        "commit_cu": commit_cu, "commit_tok": commit_tok,
        "commit_slot": commit_slot,
        "free_slots": np.array(free_slots, dtype=np.int64),
        "ctx": ctx, "anchor": anchor, "req_to_token": req_to_token,
        "hist": hist, "hist_len": hist_len,
    }
