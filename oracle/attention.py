"""Oracle stage 3: varlen causal verify attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

DSpark-in-SGLang page, §A2 "ragged verify over a full CUDA graph": the packed
buffer uses a cu_seqlens-style variable-length layout, so compact verify reuses
the backend's existing variable-length attention (on DeepSeek-V4 the native
sparse-MLA path); each backend only rebuilds its variable-length metadata for
the packed layout.  The method therefore computes ordinary causal attention for
each packed row against the request's cached keys.

Readings taken where the pages are silent:

* A row at sequence position ``p`` attends to keys ``0..p`` of its own request
  (bottom-right causal); the KV of every verified block position is already in
  the cache when attention runs.
* Grouped-query attention maps query head ``h`` to KV head
  ``h // (Hq // Hkv)``.
* Latent (MLA-style) attention has one KV head whose row serves as the key;
  the value is the first ``Dv`` entries of that same row (``v_cache is None``).
* ``sm_scale`` multiplies the raw dot products (callers pass ``1/sqrt(Dqk)``).
* Padding rows (``row_req < 0``) produce zeros; their ``lse`` is ``-inf``.
* Sliding-window layers (the pages name SWA page indexing among the fused
  kernels but do not define it): with a window of ``W`` keys the row at
  position ``p`` attends to keys ``max(0, p-W+1)..p``; ``W = 0`` is full
  causal attention.
* Sparse latent attention (the pages name DeepSeek-V4's native sparse-MLA
  path, not its selector): a row given a key list attends to the listed
  positions in list order, entries outside ``0..p`` (``-1`` pads) skipped; a
  repeated position counts once per entry; a row with no listed position
  gets ``o = 0`` and ``lse = -inf``.

Arithmetic: fp64 throughout; ``lse`` is the natural log of the softmax
normaliser of the scaled scores.
"""

import numpy as np


def attention_row(q_row, keys, values, sm_scale):
    """Softmax attention of one row's heads against ``L`` keys.

    ``q_row`` [Hq, Dqk]; ``keys`` [L, Hkv, Dqk]; ``values`` [L, Hkv, Dv].
    Returns ``(o [Hq, Dv], lse [Hq])``; textbook definition
    ``o_h = sum_j softmax_j(sm_scale * q_h . k_j) v_j``.
    """
    q_row = np.asarray(q_row, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    Hq = q_row.shape[0]
    Hkv = keys.shape[1]
    group = Hq // Hkv
    o = np.zeros((Hq, values.shape[2]), dtype=np.float64)
    lse = np.zeros(Hq, dtype=np.float64)
    for g in range(Hkv):
        heads = slice(g * group, (g + 1) * group)   # query heads sharing KV head g
        s = sm_scale * (q_row[heads] @ keys[:, g, :].T)        # [group, L]
        m = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - m)
        denom = np.sum(e, axis=1)
        o[heads] = (e @ values[:, g, :]) / denom[:, None]
        lse[heads] = m[:, 0] + np.log(denom)
    return o, lse


def gather_kv(k_cache, v_cache, page_table_row, page_size, length, Dv, start=0, positions=None):
    """Keys/values of positions ``start..length-1`` (or of the listed
    ``positions``) read through the page table.

    ``k_cache`` [num_pages, P, Hkv, Dqk]; ``v_cache`` same with ``Dv`` or None
    (latent layout: value = first ``Dv`` entries of the key row).
    """
    P = int(page_size)
    pos = np.arange(start, length) if positions is None else np.asarray(positions, dtype=np.int64)
    pages = np.asarray(page_table_row)[pos // P]
    if np.any(pages < 0) or np.any(pages >= k_cache.shape[0]):
        raise IndexError("page index out of range")
    keys = np.asarray(k_cache[pages, pos % P], dtype=np.float64)
    if v_cache is None:
        values = keys[:, :, :Dv]
    else:
        values = np.asarray(v_cache[pages, pos % P], dtype=np.float64)
    return keys, values


def verify_attention(q, k_cache, v_cache, page_table, page_size, row_req,
                     row_pos, M_pad, sm_scale, Dv=None, rows=None, window=0, topk_idx=None):
    """Attention for packed rows (``window`` > 0: sliding window of that many
    keys; ``topk_idx`` [>=M_pad, K]: each row's sparse key list).

    ``q`` [>=M_pad, Hq, Dqk] (packed order).  Returns ``(o, lse)`` shaped
    ``[M_pad, Hq, Dv]`` and ``[M_pad, Hq]``; if ``rows`` is given only those
    rows are computed (the others stay zero / -inf).
    """
    q = np.asarray(q)
    Hq = q.shape[1]
    if Dv is None:
        Dv = v_cache.shape[-1] if v_cache is not None else q.shape[2]
    o = np.zeros((M_pad, Hq, Dv), dtype=np.float64)
    lse = np.full((M_pad, Hq), -np.inf, dtype=np.float64)
    todo = range(M_pad) if rows is None else rows
    for r in todo:
        i = int(row_req[r])
        if i < 0:
            continue
        p = int(row_pos[r])
        start = max(0, p - int(window) + 1) if window else 0
        positions = None
        if topk_idx is not None:
            positions = [int(j) for j in topk_idx[r] if 0 <= int(j) <= p]
            if not positions:   # nothing listed: o = 0, lse = -inf, as for padding
                continue
        keys, values = gather_kv(k_cache, v_cache, page_table[i], page_size,
                                 p + 1, Dv, start=start, positions=positions)
        o[r], lse[r] = attention_row(q[r], keys, values, sm_scale)
    return o, lse
