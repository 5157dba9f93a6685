"""Pins for the oracle's packing (stage 2) and compact scatter (stage 5)."""

import os

import numpy as np
import pytest

import oracle
from oracle.pack import pack, select_tier
from oracle.scatter import compact_scatter

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, *vals = line.split()
                out[key] = [int(v) for v in vals]
    return out


def _contiguous_inputs(w, gamma, P=64, seed=0):
    rng = np.random.default_rng(seed)
    B = len(w)
    ctx = rng.integers(0, P - gamma, size=B)
    anchor = rng.integers(0, 1000, size=B)
    drafts = rng.integers(0, 1000, size=(B, gamma - 1))
    page_table = np.arange(B).reshape(B, 1)
    return ctx, anchor, drafts, page_table


def test_fig2_example_golden():
    g = _read_golden("ragged_pack_fig2.txt")
    w, gamma = g["windows"], g["gamma"][0]
    ctx, anchor, drafts, pt = _contiguous_inputs(w, gamma)
    cu, M, M_pad, row_req, row_pos, tok, slot = pack(w, anchor, drafts, ctx, pt, 64, g["tiers"])
    assert list(cu) == g["cu"]
    assert M == g["packed"][0]
    assert len(w) * gamma == g["padded_cells"][0]
    assert M_pad == g["tier"][0]


def test_tier_selection():
    assert select_tier(5, ()) == 5
    assert select_tier(64, (64, 128, 256)) == 64
    assert select_tier(65, (64, 128, 256)) == 128
    assert select_tier(1, (256, 64, 128)) == 64
    with pytest.raises(OverflowError):
        select_tier(257, (64, 128, 256))


def test_pack_contents_contiguous_cache():
    """With one page per request (identity table) the slot of position p is
    i*P + p, independent of the page arithmetic."""
    w = [3, 1, 4, 2]
    gamma, P = 4, 64
    ctx, anchor, drafts, pt = _contiguous_inputs(w, gamma, P, seed=2)
    cu, M, M_pad, row_req, row_pos, tok, slot = pack(w, anchor, drafts, ctx, pt, P, (16,))
    assert M == 10 and M_pad == 16
    r = 0
    for i, wi in enumerate(w):
        for k in range(wi):
            assert row_req[r] == i and row_pos[r] == ctx[i] + k
            assert tok[r] == (anchor[i] if k == 0 else drafts[i][k - 1])
            assert slot[r] == i * P + ctx[i] + k
            r += 1
    assert np.all(row_req[M:] == -1) and np.all(slot[M:] == -1)


def test_pack_paged_slots_are_distinct_and_static_offsets():
    rng = np.random.default_rng(4)
    B, gamma, P = 7, 8, 16
    ctx = rng.integers(20, 100, size=B)
    pages = (ctx + gamma + P - 1) // P
    perm = rng.permutation(int(pages.sum()))
    pt = np.full((B, int(pages.max())), -1)
    o = 0
    for i in range(B):
        pt[i, :pages[i]] = perm[o:o + pages[i]]
        o += pages[i]
    w = [gamma] * B
    cu, M, M_pad, row_req, row_pos, tok, slot = pack(
        w, rng.integers(0, 9, B), rng.integers(0, 9, (B, gamma - 1)), ctx, pt, P, ())
    assert list(cu) == [i * gamma for i in range(B + 1)]
    assert M == M_pad == B * gamma
    assert len(set(slot.tolist())) == M
    for r in range(M):
        page, off = divmod(int(slot[r]), P)
        assert off == row_pos[r] % P
        assert pt[row_req[r]][row_pos[r] // P] == page


def _scatter_case(seed):
    rng = np.random.default_rng(seed)
    B, gamma, P = 6, 5, 64
    w = rng.integers(1, gamma + 1, size=B)
    ctx, anchor, drafts, pt = _contiguous_inputs(list(w), gamma, P, seed)
    cu, M, M_pad, row_req, row_pos, tok, slot = pack(w, anchor, drafts, ctx, pt, P, ())
    accept = np.array([rng.integers(0, wi) for wi in w])
    bonus = rng.integers(0, 1000, size=B)
    r2t = np.full((B, P), -7)
    hist = np.full((B, 32), -1)
    hist_len = rng.integers(0, 8, size=B)
    out = compact_scatter(cu, w, accept, bonus, drafts, slot, ctx, anchor, r2t, hist, hist_len)
    return locals()


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_scatter_invariants(seed):
    c = _scatter_case(seed)
    out, w, accept, ctx = c["out"], c["w"], c["accept"], c["ctx"]
    B = len(w)
    n_commit = int(np.sum(accept + 1))
    assert out["commit_cu"][-1] == n_commit
    assert np.array_equal(np.diff(out["commit_cu"]), accept + 1)
    # committed + released slots are exactly the verified slots
    all_slots = sorted(c["slot"][:c["M"]].tolist())
    got = sorted(out["commit_slot"].tolist() + out["free_slots"].tolist())
    assert got == all_slots
    for i in range(B):
        a = int(accept[i])
        base = int(out["commit_cu"][i])
        toks = out["commit_tok"][base:base + a + 1]
        assert list(toks[:a]) == list(c["drafts"][i][:a])
        assert toks[a] == c["bonus"][i]
        # req_to_token gets the committed slots at positions ctx..ctx+a
        row = out["req_to_token"][i]
        assert np.all(row[ctx[i]:ctx[i] + a + 1] == c["slot"][c["cu"][i]:c["cu"][i] + a + 1])
        assert np.sum(row != -7) == a + 1
        assert out["ctx"][i] == ctx[i] + a + 1
        assert out["anchor"][i] == c["bonus"][i]
        h0 = int(c["hist_len"][i])
        assert list(out["hist"][i][h0:h0 + a + 1]) == list(toks)
        assert out["hist_len"][i] == h0 + a + 1
