"""Calibration oracle (ECE and per-request verdict counts) pinned to closed
forms, a textbook identity and the law of large numbers."""

import numpy as np
import pytest

import oracle


def _flat(conf, labels):
    """Arrange per-draft (conf, label) pairs as one request per draft (window
    2: one verified draft each), with pred chosen to produce the labels."""
    n = len(conf)
    conf2 = np.asarray(conf, dtype=np.float32).reshape(n, 1)
    drafts = np.arange(n).reshape(n, 1)
    pred = np.where(np.asarray(labels, dtype=bool), np.arange(n), -1)
    pred = np.stack([pred, np.full(n, 7)], axis=1).reshape(-1)   # rows 2i (checked), 2i+1 (bonus row)
    cu = np.arange(n + 1) * 2
    w = np.full(n, 2)
    return conf2, drafts, pred, cu, w


def test_constant_overconfidence():
    """Every draft at confidence 0.875, 60 of 100 right: ECE = 0.875 - 0.6."""
    conf = [0.875] * 100
    labels = [1] * 60 + [0] * 40
    cnt, match, cfx, ece, rv_, rm = oracle.calibration(*_flat(conf, labels), 10)
    assert cnt[8] == 100 and sum(cnt) == 100 and match[8] == 60
    assert ece == pytest.approx(0.275, abs=1e-15)
    assert sum(rv_) == 100 and sum(rm) == 60


def test_one_bin_is_calibration_in_the_large():
    """With one bin, ECE = |mean label - mean confidence|."""
    rng = np.random.default_rng(3)
    conf = rng.random(500).astype(np.float32)
    labels = rng.random(500) < 0.4
    ece = oracle.calibration(*_flat(conf, labels), 1)[3]
    assert ece == pytest.approx(abs(labels.mean() - conf.astype(np.float64).mean()), abs=1e-12)


def test_bins_that_match_exactly_give_zero():
    conf = [0.25] * 4 + [0.75] * 4
    labels = [1, 0, 0, 0, 1, 1, 1, 0]
    cnt, match, cfx, ece, _, _ = oracle.calibration(*_flat(conf, labels), 4)
    assert cnt == [0, 4, 0, 4] and match == [0, 1, 0, 3]
    assert ece == 0.0


def test_bin_edges():
    conf = [0.0, 0.5, 1.0, 0.099999994]   # the last is the fp32 just below 0.1
    cnt = oracle.calibration(*_flat(conf, [1, 1, 1, 1]), 10)[0]
    assert cnt[0] == 2 and cnt[5] == 1 and cnt[9] == 1


def test_law_of_large_numbers():
    """Labels drawn with probability conf: ECE near 0.  Drawn with
    probability conf^2 (overconfident): ECE near the mean of c - c^2 over
    uniform c, 1/6."""
    rng = np.random.default_rng(11)
    n = 200_000
    conf = rng.random(n).astype(np.float32)
    c64 = conf.astype(np.float64)
    good = rng.random(n) < c64
    bad = rng.random(n) < c64 ** 2
    e_good = oracle.calibration(*_flat(conf, good), 10)[3]
    e_bad = oracle.calibration(*_flat(conf, bad), 10)[3]
    assert e_good < 0.01
    assert abs(e_bad - 1 / 6) < 0.01


def test_only_verified_drafts_count():
    """Drafts past the verify window carry no verdict."""
    conf = np.array([[0.9, 0.8, 0.7], [0.6, 0.5, 0.4]], dtype=np.float32)
    drafts = np.array([[1, 2, 3], [4, 5, 6]])
    pred = np.array([1, 9, 3, 9, 4, 5, 6, 9])        # request 0 rows 0..1, request 1 rows 2..5
    cu = np.array([0, 2, 6])
    w = np.array([2, 4])
    cnt, match, cfx, ece, rver, rmat = oracle.calibration(conf, drafts, pred, cu, w, 10)
    assert rver == [1, 3]
    # request 0: draft 1 (1) against row 0 (1) matches; request 1: drafts 4, 5, 6
    # against rows 2, 3, 4 (3, 9, 4): none matches
    assert rmat == [1, 0]
    assert sum(cnt) == 4 and sum(match) == 1
