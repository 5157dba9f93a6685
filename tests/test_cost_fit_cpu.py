"""Cost-table fit: the oracle pinned to the pages' closed form and to the
least-squares optimality conditions, and the library's host routine
(rv_fit_cost_model, C ABI) against the oracle.  No GPU needed."""

import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cost_model.txt")


def _golden():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    bs = np.array([float(r[0]) for r in rows])
    K = np.array([float(r[1]) for r in rows])
    T = np.array([float(r[2]) for r in rows])
    return bs, bs + K, T


def _noisy(seed, n=40):
    rng = np.random.default_rng(seed)
    bs = rng.integers(1, 257, n).astype(float)
    M = bs + rng.integers(0, 8, n) * bs
    t = 0.15 + 0.0007 * bs + 0.00021 * M + rng.normal(0, 0.01, n)
    return bs, M, t


def test_oracle_recovers_the_pages_closed_form():
    """Samples of T(bs, K) = 1.0 + 0.01 bs + 0.004 (bs + K) ms, worked by hand
    from the mixed-confidence sweep's coefficients, give those coefficients."""
    bs, M, T = _golden()
    coef = oracle.fit_cost_model(bs, M, T)
    np.testing.assert_allclose(coef, [1.0, 0.01, 0.004], rtol=0, atol=1e-12)
    bias, alpha, theta = oracle.cost_tables(coef, 257, 2049)
    assert bias == pytest.approx(1.0, abs=1e-12)
    assert alpha[32] == pytest.approx(0.32, abs=1e-12) and theta[256] == pytest.approx(1.024, abs=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_oracle_meets_the_least_squares_conditions(seed):
    """With noise: the residual is orthogonal to each column (1, bs, M), and
    moving any coefficient either way raises the sum of squares."""
    bs, M, t = _noisy(seed)
    b0, a, th = oracle.fit_cost_model(bs, M, t)
    r = [t[i] - (b0 + a * bs[i] + th * M[i]) for i in range(len(t))]
    for col in (np.ones_like(bs), bs, M):
        s = sum(c * ri for c, ri in zip(col, r))
        assert abs(s) <= 1e-9 * max(1.0, float(np.abs(col).sum()))
    sse = sum(x * x for x in r)
    for k, h in ((0, 1e-3), (1, 1e-5), (2, 1e-6)):
        for sgn in (1, -1):
            c = [b0, a, th]
            c[k] += sgn * h
            sse2 = sum((t[i] - (c[0] + c[1] * bs[i] + c[2] * M[i])) ** 2 for i in range(len(t)))
            assert sse2 > sse


def test_oracle_order_and_degenerate_samples():
    bs, M, t = _noisy(5)
    p = np.random.default_rng(9).permutation(len(bs))
    np.testing.assert_allclose(oracle.fit_cost_model(bs[p], M[p], t[p]), oracle.fit_cost_model(bs, M, t),
                               rtol=1e-10, atol=1e-13)
    with pytest.raises(ValueError):
        oracle.fit_cost_model([4, 4, 4, 4], [8, 9, 10, 11], [1, 2, 3, 4])      # one batch size
    with pytest.raises(ValueError):
        oracle.fit_cost_model([1, 2, 3, 4], [2, 4, 6, 8], [1, 2, 3, 4])        # M = 2 bs
    with pytest.raises(ValueError):
        oracle.fit_cost_model([1, 2], [1, 3], [1, 2])                          # two samples


@pytest.fixture(scope="module")
def rv():
    from ragged_verification_amd import rv as _rv
    if not os.path.exists(_rv.LIB_PATH):
        pytest.fail("librv.so is not built (run __graft_entry__.build())")
    _rv.load()
    return _rv


@pytest.mark.parametrize("seed", [0, 3, 7])
def test_library_fit_matches_oracle(rv, seed):
    bs, M, t = _noisy(seed, n=25 + seed)
    coef, alpha, theta = rv.rv_fit_cost_model(bs, M, t, alpha_len=257, theta_len=2049)
    want = oracle.fit_cost_model(bs, M, t)
    np.testing.assert_allclose(coef, want, rtol=1e-9, atol=1e-12)
    b, wa, wt = oracle.cost_tables(want, 257, 2049)
    np.testing.assert_allclose(alpha, wa, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(theta, wt, rtol=1e-9, atol=1e-12)


def test_library_fit_golden_and_errors(rv):
    bs, M, T = _golden()
    coef, _, _ = rv.rv_fit_cost_model(bs, M, T)
    np.testing.assert_allclose(coef, [1.0, 0.01, 0.004], rtol=0, atol=1e-12)
    for args in (([4, 4, 4, 4], [8, 9, 10, 11], [1, 2, 3, 4]), ([1, 2, 3, 4], [2, 4, 6, 8], [1, 2, 3, 4]),
                 ([1, 2], [1, 3], [1, 2]), ([1, 2, 3], [1, 5, 2], [1, float("nan"), 2])):
        with pytest.raises(rv.RVError):
            rv.rv_fit_cost_model(*args)
