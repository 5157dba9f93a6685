"""Oracle: the fixed-shape padded verify that static mode must equal.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

DSpark-in-SGLang page, §A2 and Fig. 2: a fixed-shape decode graph pads every
request to the full block width; the ragged path front-packs the scheduled
tokens instead and yields the same accepted tokens while computing far fewer
padded cells.  This routine is the padded side of that comparison, written as
a masked batch computation (no packing, no page-table walk per row): every
request contributes ``gamma`` query rows, keys are padded to the batch's
longest sequence and hidden behind a mask.
"""

import numpy as np


def dense_padded_verify(q_block, k_cache, v_cache, page_table, page_size, ctx,
                        sm_scale, hidden_block, W, drafts, Dv=None):
    """Returns ``(o [B, gamma, Hq, Dv], pred [B, gamma], accept [B],
    bonus [B])`` for full-block greedy verification.

    ``q_block`` [B, gamma, Hq, Dqk]; ``hidden_block`` [B, gamma, H].
    """
    q_block = np.asarray(q_block, dtype=np.float64)
    B, gamma, Hq, Dqk = q_block.shape
    Hkv = k_cache.shape[2]
    if Dv is None:
        Dv = v_cache.shape[-1] if v_cache is not None else Dqk
    P = int(page_size)
    L = int(np.max(ctx)) + gamma
    keys = np.zeros((B, L, Hkv, Dqk))
    vals = np.zeros((B, L, Hkv, Dv))
    mask = np.zeros((B, gamma, L), dtype=bool)
    for i in range(B):
        n = int(ctx[i]) + gamma
        pos = np.arange(n)
        pages = np.asarray(page_table[i])[pos // P]
        keys[i, :n] = k_cache[pages, pos % P]
        vals[i, :n] = (k_cache[pages, pos % P][..., :Dv] if v_cache is None
                       else v_cache[pages, pos % P])
        for k in range(gamma):
            mask[i, k, :int(ctx[i]) + k + 1] = True
    group = Hq // Hkv
    kv_of_head = np.arange(Hq) // group
    # scores[b, k, h, j] = sm_scale * q[b,k,h,:] . keys[b,j,g(h),:]
    kh = keys[:, :, kv_of_head, :]                 # [B, L, Hq, Dqk]
    vh = vals[:, :, kv_of_head, :]                 # [B, L, Hq, Dv]
    scores = sm_scale * np.einsum("bkhd,bjhd->bkhj", q_block, kh)
    scores = np.where(mask[:, :, None, :], scores, -np.inf)
    m = np.max(scores, axis=-1, keepdims=True)
    e = np.exp(scores - m)
    o = np.einsum("bkhj,bjhd->bkhd", e, vh) / np.sum(e, axis=-1)[..., None]

    x = np.asarray(hidden_block, dtype=np.float64).reshape(B * gamma, -1)
    z = x @ np.asarray(W, dtype=np.float64).T
    pred = np.argmax(z, axis=1).reshape(B, gamma)
    accept = np.zeros(B, dtype=np.int64)
    bonus = np.zeros(B, dtype=np.int64)
    for i in range(B):
        a = 0
        while a < gamma - 1 and int(drafts[i][a]) == int(pred[i, a]):
            a += 1
        accept[i] = a
        bonus[i] = int(pred[i, a])
    return o, pred, accept, bonus
