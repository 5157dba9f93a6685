"""Pins for the oracle's confidence scheduler (CPU only).

The scheduler's contract is an exact optimum: the window vector that
maximises expected committed tokens per unit of modelled step time.  These
tests check it by exhaustive enumeration in exact rational arithmetic, by the
closed form of the cost model, and by special cases whose answer is known
without running the scheduler.
"""

import itertools
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.schedule import survival, step_time, schedule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def linear_costs(B, gamma, bias=1.0, a=0.01, th=0.004):
    alpha = np.arange(B + 1, dtype=np.float64) * a
    theta = np.arange(B * gamma + 1, dtype=np.float64) * th
    return bias, alpha, theta


def test_cost_model_closed_form_golden():
    rows = []
    with open(os.path.join(GOLDEN, "cost_model.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                bs, K, T = line.split()
                rows.append((int(bs), int(K), float(T)))
    assert len(rows) == 6
    bias, alpha, theta = linear_costs(256, 8)
    for bs, K, T in rows:
        assert step_time(bias, alpha, theta, bs, K) == pytest.approx(T, abs=1e-12)


def test_survival_equal_confidences_is_a_power():
    c = np.full((3, 7), np.float32(0.75), dtype=np.float32)
    S = survival(c)
    for k in range(8):
        assert S[0, k] == 0.75 ** k  # 0.75**k is exact in fp64 for k <= 7


def test_survival_rejects_out_of_range():
    with pytest.raises(ValueError):
        survival(np.array([[0.5, 1.5]], dtype=np.float32))
    with pytest.raises(ValueError):
        survival(np.array([[np.nan, 0.5]], dtype=np.float32))


def _exact_best(conf, gamma, bias, alpha, theta):
    """Brute force over every window vector, exact rationals."""
    B = conf.shape[0]
    S = []
    for i in range(B):
        row, acc = [Fraction(1)], Fraction(1)
        for k in range(gamma - 1):
            acc *= Fraction(float(conf[i, k]))
            row.append(acc)
        S.append(row)
    base = Fraction(float(bias)) + Fraction(float(alpha[B]))
    best, best_ws = None, []
    for ws in itertools.product(range(1, gamma + 1), repeat=B):
        E = B + sum(sum(S[i][1:ws[i]], Fraction(0)) for i in range(B))
        K = sum(ws) - B
        T = base + Fraction(float(theta[B + K]))
        R = E / T
        if best is None or R > best:
            best, best_ws = R, [ws]
        elif R == best:
            best_ws.append(ws)
    return best, best_ws, S, base


def _exact_ratio(w, S, base, theta, B):
    E = B + sum(sum(S[i][1:int(w[i])], Fraction(0)) for i in range(B))
    K = int(sum(w)) - B
    return E / (base + Fraction(float(theta[B + K])))


def _check_against_brute(conf, gamma, bias, alpha, theta):
    B = conf.shape[0]
    wc, wv, k_star, e_star = schedule(conf, gamma, oracle.COMPACT, bias, alpha, theta)
    assert np.array_equal(wc, wv)
    assert k_star == int(wc.sum()) - B
    best, best_ws, S, base = _exact_best(conf, gamma, bias, alpha, theta)
    mine = _exact_ratio(wc, S, base, theta, B)
    # fixed point (2^-40) and fp64 rounding are the only departures from exact
    assert float(mine) >= float(best) * (1 - 1e-9)
    E = B + sum(sum(S[i][1:int(wc[i])], Fraction(0)) for i in range(B))
    assert abs(e_star - float(E)) <= B * gamma * 2.0 ** -40 + 1e-12
    return wc, best_ws


def test_brute_force_tiny_workload_shape():
    """B=4, gamma=4 (the tiny workload): all 256 window vectors."""
    rng = np.random.default_rng(7)
    for trial in range(12):
        conf = rng.uniform(0.3, 0.99, size=(4, 3)).astype(np.float32)
        th = [0.004, 0.05, 0.2, 0.6][trial % 4]
        bias, alpha, theta = linear_costs(4, 4, bias=0.2, a=0.01, th=th)
        _check_against_brute(conf, 4, bias, alpha, theta)


def test_brute_force_random_small():
    rng = np.random.default_rng(11)
    pyr = random.Random(11)
    for trial in range(25):
        B = pyr.randint(1, 5)
        gamma = pyr.randint(2, 5)
        if gamma ** B > 4000:
            gamma = 3
        conf = rng.beta(pyr.choice([0.5, 2, 4, 9]), pyr.choice([1, 2, 3]),
                        size=(B, gamma - 1)).astype(np.float32)
        bias = pyr.uniform(0.05, 1.0)
        alpha = np.cumsum(rng.uniform(0, 0.05, size=B + 1))
        # non-linear increasing theta exercises the table lookup
        theta = np.cumsum(rng.uniform(0, pyr.choice([0.01, 0.1, 0.5]), size=B * gamma + 1))
        _check_against_brute(conf, gamma, bias, alpha, theta)


def test_trimming_happens_and_is_optimal():
    """A case where the optimum is strictly between 'all ones' and 'full'."""
    conf = np.array([[0.99, 0.98, 0.97], [0.2, 0.9, 0.9], [0.6, 0.5, 0.1]], dtype=np.float32)
    bias, alpha, theta = linear_costs(3, 4, bias=0.1, a=0.0, th=0.05)
    wc, best_ws = _check_against_brute(conf, 4, bias, alpha, theta)
    assert 3 < wc.sum() < 12
    assert tuple(int(x) for x in wc) in best_ws


def test_zero_theta_keeps_every_positive_survival():
    rng = np.random.default_rng(3)
    conf = rng.uniform(0.0, 1.0, size=(9, 6)).astype(np.float32)
    conf[2, 3] = 0.0  # survival is zero from position 4 on
    bias, alpha, _ = linear_costs(9, 7)
    theta = np.zeros(9 * 7 + 1)
    wc, wv, _, _ = schedule(conf, 7, oracle.COMPACT, bias, alpha, theta)
    expect = np.full(9, 7)
    expect[2] = 4
    assert np.array_equal(wc, expect)


def test_negative_zero_confidence_is_zero():
    """-0.0 is a valid confidence equal to 0.0: the windows, K* and E* equal
    those of the same batch with +0.0, under a cost table where zeros tie
    with each other (theta flat past the positives) and under a linear one."""
    rng = np.random.default_rng(11)
    conf = rng.uniform(0.2, 1.0, size=(7, 5)).astype(np.float32)
    conf[1, 0] = 0.0
    conf[4, 2] = 0.0
    neg = conf.copy()
    neg[1, 0] = -0.0
    neg[4, 2] = -0.0
    assert np.signbit(neg[1, 0]) and not np.signbit(conf[1, 0])
    bias, alpha, theta = linear_costs(7, 6)
    for th in (theta, np.zeros_like(theta)):
        for mode in (oracle.COMPACT, oracle.CAP_ACCEPT):
            a = schedule(conf, 6, mode, bias, alpha, th)
            b = schedule(neg, 6, mode, bias, alpha, th)
            assert all(np.array_equal(x, y) for x, y in zip(a[:2], b[:2])) and a[2:] == b[2:]


def test_huge_theta_verifies_anchor_only():
    rng = np.random.default_rng(4)
    conf = rng.uniform(0.5, 1.0, size=(5, 7)).astype(np.float32)
    bias, alpha, _ = linear_costs(5, 8)
    theta = np.arange(5 * 8 + 1, dtype=np.float64) * 1e6
    wc, wv, k_star, e_star = schedule(conf, 8, oracle.COMPACT, bias, alpha, theta)
    assert np.all(wc == 1) and k_star == 0 and e_star == 5.0


def test_modes():
    rng = np.random.default_rng(5)
    conf = rng.beta(3, 2, size=(16, 7)).astype(np.float32)
    bias, alpha, theta = linear_costs(16, 8, th=0.1)
    c_w, c_v, c_k, c_e = schedule(conf, 8, oracle.COMPACT, bias, alpha, theta)
    a_w, a_v, a_k, a_e = schedule(conf, 8, oracle.CAP_ACCEPT, bias, alpha, theta)
    assert np.array_equal(c_w, a_w) and np.all(a_v == 8) and c_k == a_k and c_e == a_e
    for mode in (oracle.STATIC, oracle.NO_TRIM):
        w, v, k, e = schedule(conf, 8, mode, bias, alpha, theta)
        assert np.all(w == 8) and np.all(v == 8) and k == 16 * 7
        S = survival(conf)
        assert e == pytest.approx(16 + S[:, 1:].sum(), rel=1e-12)
    assert c_w.min() >= 1 and c_w.max() <= 8


def test_ratio_unimodal_for_linear_theta():
    """With linear theta, E(K)/T(K) rises then falls along the ranked
    candidates (each step is a mediant of the current ratio and s/theta)."""
    rng = np.random.default_rng(6)
    for _ in range(20):
        B = int(rng.integers(1, 40))
        conf = rng.beta(2, 2, size=(B, 7)).astype(np.float32)
        bias, alpha, theta = linear_costs(B, 8, th=float(rng.choice([0.004, 0.05, 0.3])))
        S = survival(conf)
        s = np.sort(S[:, 1:].ravel())[::-1]
        E = B + np.concatenate([[0.0], np.cumsum(s)])
        T = np.array([step_time(bias, alpha, theta, B, K) for K in range(len(s) + 1)])
        R = E / T
        k = int(np.argmax(R))
        assert np.all(np.diff(R[:k + 1]) >= -1e-12)
        assert np.all(np.diff(R[k:]) <= 1e-12)
        wc, _, k_star, _ = schedule(conf, 8, oracle.COMPACT, bias, alpha, theta)
        assert abs(R[k_star] - R[k]) <= 1e-12 * R[k]


def test_windows_shrink_with_difficulty():
    """Mixed traffic: requests of a harder confidence class get smaller
    windows (the DSpark-in-SGLang page reports this ordering in section A3;
    its numbers come from trained models and are not pinned)."""
    rng = np.random.default_rng(9)
    B = 240
    classes = [(9, 1), (3, 2), (2, 3)]
    conf = np.empty((B, 7), dtype=np.float32)
    for j, (a, b) in enumerate(classes):
        conf[j::3] = rng.beta(a, b, size=(B // 3, 7))
    bias, alpha, theta = linear_costs(B, 8)
    w, _, _, _ = schedule(conf, 8, oracle.COMPACT, bias, alpha, theta)
    means = [w[j::3].mean() for j in range(3)]
    assert means[0] > means[1] > means[2]
