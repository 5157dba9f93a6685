"""Pins for the oracle's acceptance rules (stage 4b) and the mode
equivalences (compact and cap-accept commit the same tokens)."""

import numpy as np
import pytest
import torch
from scipy import stats

import oracle
from oracle.accept import accept_greedy, accept_rejection, residual_sample, softmax
from ragged_verification_amd import synth


def test_greedy_matches_planted_drafts():
    """The generator knows which drafts equal the planted target, so the
    accept length is known without the oracle's arithmetic."""
    wl = synth.workload("gqa_bf16", V=400, H=64)
    d = synth.make_inputs(wl, B=24)
    B, gamma = d["B"], d["gamma"]
    x = d["hidden_block"].to(torch.float64).numpy().reshape(B * gamma, -1)
    pred = oracle.lm_head_pred(oracle.lm_head_logits(x, d["W"].to(torch.float64).numpy()))
    assert np.array_equal(pred, d["targets"].reshape(-1).numpy())
    correct = d["correct"].numpy()
    rng = np.random.default_rng(1)
    for mode in ("static", "compact"):
        w = np.full(B, gamma) if mode == "static" else rng.integers(1, gamma + 1, size=B)
        cu = np.concatenate([[0], np.cumsum(w)])
        # rows of a ragged pack: request i keeps its first w_i block rows
        rows = np.concatenate([np.arange(w[i]) + i * gamma for i in range(B)])
        acc, bonus, ceil = accept_greedy(pred[rows], cu, w, w, d["drafts"].numpy())
        for i in range(B):
            lead = 0
            while lead < gamma - 1 and correct[i, lead]:
                lead += 1
            assert acc[i] == min(lead, w[i] - 1)
            assert bonus[i] == d["targets"][i, acc[i]]


def _rejection_inputs(p, q, n, seed):
    """n independent one-draft requests with target p and draft q."""
    rng = np.random.default_rng(seed)
    V = len(p)
    drafts = rng.choice(V, size=(n, 1), p=q)
    z = np.tile(np.log(np.maximum(p, 1e-300)), (n, 1))
    q_rows = np.tile(q, (n, 1, 1))
    u = rng.uniform(size=(n, 1))
    ub = rng.uniform(size=n)
    cu = np.arange(0, 2 * n + 1, 2)
    zz = np.repeat(z, 2, axis=0)   # two rows per request, identical target
    return zz, cu, drafts, q_rows, u, ub


def test_rejection_equal_distributions_always_accept():
    V = 11
    p = softmax(np.random.default_rng(0).standard_normal(V))
    zz, cu, drafts, q_rows, u, ub = _rejection_inputs(p, p, 300, 1)
    w = np.full(300, 2)
    acc, bonus, ceil = accept_rejection(zz, cu, w, w, drafts, q_rows, u, ub)
    assert np.all(acc == 1) and np.all(ceil == 1)


def test_rejection_draft_where_target_is_tiny_rejects():
    V = 6
    p = np.array([0.5, 0.5 - 1e-9, 1e-9, 0, 0, 0])
    p = p / p.sum()
    q = np.array([0, 0, 1.0, 0, 0, 0])
    zz, cu, drafts, q_rows, u, ub = _rejection_inputs(p, q, 50, 2)
    u[:] = np.maximum(u, 1e-3)
    w = np.full(50, 2)
    acc, bonus, ceil = accept_rejection(zz, cu, w, w, drafts, q_rows, u, ub)
    assert np.all(acc == 0)
    # residual max(0, p - q) is supported on tokens 0 and 1 only
    assert set(bonus.tolist()) <= {0, 1}


def test_rejection_sampling_is_unbiased():
    """Speculative sampling theorem: the first committed token is distributed
    as p, and a draft is accepted with probability sum_v min(p_v, q_v)."""
    V, n = 16, 40000
    rng = np.random.default_rng(3)
    p = softmax(rng.standard_normal(V))
    q = softmax(rng.standard_normal(V) * 1.5)
    zz, cu, drafts, q_rows, u, ub = _rejection_inputs(p, q, n, 4)
    w = np.full(n, 2)
    acc, bonus, ceil = accept_rejection(zz, cu, w, w, drafts, q_rows, u, ub)
    rate = acc.mean()
    expect = np.minimum(p, q).sum()
    assert abs(rate - expect) < 4 * np.sqrt(expect * (1 - expect) / n)
    first = np.where(acc == 1, drafts[:, 0], bonus)
    counts = np.bincount(first, minlength=V)
    chi2, pval = stats.chisquare(counts, n * p)
    assert pval > 1e-3


def test_residual_sample_inverse_cdf():
    r = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert residual_sample(r, 0.0)[0] == 1
    assert residual_sample(r, 0.2)[0] == 1
    assert residual_sample(r, 0.26)[0] == 3
    assert residual_sample(r, 0.74)[0] == 3
    assert residual_sample(r, 0.76)[0] == 4
    assert residual_sample(r, 0.999999)[0] == 4


def test_residual_sample_neighbour_across_nearest_boundary():
    """The token on the far side of the nearest CDF step, skipping tokens of
    zero weight (the interval of token 3 is [0.25, 0.75))."""
    r = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    idx, margin, nb = residual_sample(r, 0.26)
    assert (idx, nb) == (3, 1) and abs(margin - 0.01) < 1e-12
    idx, margin, nb = residual_sample(r, 0.70)
    assert (idx, nb) == (3, 4) and abs(margin - 0.05) < 1e-12
    assert residual_sample(r, 0.01)[2] == 1        # nothing of weight below token 1
    assert residual_sample(r, 0.99)[2] == 4        # nothing above token 4


def test_cap_accept_commits_equal_compact_greedy():
    rng = np.random.default_rng(5)
    B, gamma, V = 40, 6, 7
    pred_full = rng.integers(0, V, size=(B, gamma))
    drafts = np.where(rng.uniform(size=(B, gamma - 1)) < 0.7, pred_full[:, :-1],
                      rng.integers(0, V, size=(B, gamma - 1)))
    w = rng.integers(1, gamma + 1, size=B)
    cu_c = np.concatenate([[0], np.cumsum(w)])
    rows_c = np.concatenate([np.arange(w[i]) + i * gamma for i in range(B)])
    a_c, b_c, c_c = accept_greedy(pred_full.reshape(-1)[rows_c], cu_c, w, w, drafts)
    cu_f = np.arange(0, B * gamma + 1, gamma)
    a_f, b_f, c_f = accept_greedy(pred_full.reshape(-1), cu_f, w, np.full(B, gamma), drafts)
    assert np.array_equal(a_c, a_f) and np.array_equal(b_c, b_f)
    assert np.all(c_f >= a_f) and np.all(c_c == a_c)
    assert np.any(c_f > a_f)  # the ceiling is visible only under cap-accept


def test_cap_accept_commits_equal_compact_rejection():
    wl = synth.workload("rejection_bf16", V=64, H=32, ctx=("lognormal", 30, 1.0, 60))
    d = synth.make_inputs(wl, B=30)
    B, gamma = d["B"], d["gamma"]
    x = d["hidden_block"].to(torch.float64).numpy().reshape(B * gamma, -1)
    z = oracle.lm_head_logits(x, d["W"].to(torch.float64).numpy())
    w = np.random.default_rng(6).integers(1, gamma + 1, size=B)
    cu_c = np.concatenate([[0], np.cumsum(w)])
    rows_c = np.concatenate([np.arange(w[i]) + i * gamma for i in range(B)])
    args = (d["drafts"].numpy(), d["q_rows"].numpy(), d["u"].numpy(), d["u_bonus"].numpy())
    a_c, b_c, c_c = accept_rejection(z[rows_c], cu_c, w, w, *args)
    cu_f = np.arange(0, B * gamma + 1, gamma)
    a_f, b_f, c_f = accept_rejection(z, cu_f, w, np.full(B, gamma), *args)
    assert np.array_equal(a_c, a_f) and np.array_equal(b_c, b_f)
    assert np.all(c_f >= a_f)


def test_rejection_bonus_uses_the_right_row():
    """Hand-worked two-draft request whose rows have different targets.
    Row 0 target p0 = (1/2, 1/2, 0, 0), row 1 target p1 = (0, 0, 1, 0),
    row 2 target p2 = (0, 0, 0, 1)."""
    neg = -1e4  # exp(-1e4) underflows to exactly 0 in fp64
    z = np.array([[0.0, 0.0, neg, neg], [neg, neg, 0.0, neg], [neg, neg, neg, 0.0]])
    cu = np.array([0, 3])
    w = np.array([3])
    q = np.zeros((1, 2, 4))
    q[0, 0] = [0.0, 1.0, 0.0, 0.0]   # draft 1 = token 1: p0(1)/q(1) = 1/2
    q[0, 1] = [0.0, 0.0, 1.0, 0.0]   # draft 2 = token 2: p1(2)/q(2) = 1
    drafts = np.array([[1, 2]])
    # u = 0.75 >= 1/2: reject draft 1; residual max(0, p0 - q1) = (1/2, 0, 0, 0)
    a, b, c = accept_rejection(z, cu, w, w, drafts, q, np.array([[0.75, 0.1]]), np.array([0.9]))
    assert (a[0], b[0], c[0]) == (0, 0, 0)
    # u = 0.25 < 1/2: accept draft 1, then draft 2 (ratio 1); bonus from p2
    a, b, c = accept_rejection(z, cu, w, w, drafts, q, np.array([[0.25, 0.9]]), np.array([0.3]))
    assert (a[0], b[0], c[0]) == (2, 3, 2)
    # commit window 2 (cap-accept): draft 2 is verified but not committed;
    # the bonus comes from p1, as compact with window 2 would draw it
    a, b, c = accept_rejection(z, cu, np.array([2]), w, drafts, q, np.array([[0.25, 0.9]]),
                               np.array([0.3]))
    assert (a[0], b[0], c[0]) == (1, 2, 2)


def test_attention_large_scores_do_not_overflow():
    from oracle.attention import attention_row
    rng = np.random.default_rng(8)
    q = np.ones((1, 4))
    keys = np.zeros((3, 1, 4))
    keys[0, 0] = 300.0   # scores 1200 and 0: exp of an unshifted score overflows
    vals = rng.standard_normal((3, 1, 2))
    o, lse = attention_row(q, keys, vals, 1.0)
    np.testing.assert_allclose(o[0], vals[0, 0], atol=1e-12)
    assert lse[0] == pytest.approx(1200.0, rel=1e-12)
