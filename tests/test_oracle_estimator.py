"""Pins of the oracle's block-accept estimator (oracle/estimator.py).

* Greedy, exact: on trajectories where the target's continuation is a fixed
  token sequence per request (so the truncated and the untruncated
  trajectory see the same target at every position, the pages' similarity
  assumption holding exactly), every closed probe equals the ceiling that
  cap-accept exposes for the probe's step, computed by the oracle's own
  acceptance on the full block.
* Rejection, statistical: with the target and draft distributions fixed per
  position, the estimate of a fully resolved probe is the expected tail the
  full block would accept; it matches the mean of cap-accept ceilings over
  many draws of the acceptance uniforms.
* Special cases: uncensored steps open no probe; a mismatch at the first
  tail draft closes the probe at w - 1; block width 2; skipped steps drop a
  probe.
"""

import numpy as np

import oracle
from oracle.estimator import GREEDY, REJECTION


def _costs(B, gamma, th):
    return 1.0, np.arange(B + 1) * 0.01, np.arange(B * gamma + 1) * th


def _greedy_trajectory(B, gamma, steps, seed, th=0.02, p_match=0.85):
    """Compact steps over per-request target sequences T.  Returns the
    estimator state and, per closed probe, (estimate, the ceiling cap-accept
    exposes for the probe's step); a probe is identified by its first tail
    position, ctx + w of the censored step."""
    rng = np.random.default_rng(seed)
    V = 50
    L = 8 + steps * gamma + gamma
    T = rng.integers(0, V, size=(B, L))
    ctx = rng.integers(0, 4, size=B)
    st = oracle.estimator_state(B, gamma)
    cap_at = {}
    pairs = []
    bias, alpha, theta = _costs(B, gamma, th)
    for s in range(steps):
        conf = rng.uniform(0.3, 1.0, size=(B, gamma - 1)).astype(np.float32)
        drafts = np.empty((B, gamma - 1), dtype=np.int64)
        for i in range(B):
            for j in range(1, gamma):
                t = T[i, ctx[i] + j]
                drafts[i, j - 1] = t if rng.uniform() < p_match else (t + 1 + rng.integers(0, V - 1)) % V
        wc, wv, _, _ = oracle.schedule(conf, gamma, oracle.COMPACT, bias, alpha, theta)
        cu = np.concatenate([[0], np.cumsum(wv)])
        # row k of request i predicts the target's token at ctx + k + 1
        pred = np.concatenate([[T[i, ctx[i] + k + 1] for k in range(wv[i])] for i in range(B)])
        acc, bonus, _ = oracle.accept_greedy(pred, cu, wc, wv, drafts)
        # cap-accept on the same step: the whole block verified
        cu_f = np.arange(B + 1) * gamma
        pred_f = np.concatenate([[T[i, ctx[i] + k + 1] for k in range(gamma)] for i in range(B)])
        _, _, cap = oracle.accept_greedy(pred_f, cu_f, wc, np.full(B, gamma), drafts)
        for i in range(B):
            cap_at[(i, int(ctx[i] + wv[i]))] = int(cap[i])
        closed = []
        oracle.estimate_update(st, cu, wv, acc, drafts, ctx, GREEDY, pred=pred, closed=closed)
        for i, first, est in closed:
            pairs.append((est, cap_at[(i, first)]))
        ctx = ctx + acc + 1
        # committed tokens are the target's: the bonus is T at the new anchor
        assert all(bonus[i] == T[i, ctx[i]] for i in range(B))
    return st, pairs


def test_greedy_closed_probes_equal_cap_accept_ceiling():
    total = 0
    for seed in range(6):
        st, pairs = _greedy_trajectory(B=12, gamma=8, steps=40, seed=seed)
        for est, cap in pairs:
            assert est == float(cap), (seed, est, cap)
            total += 1
    assert total > 100


def test_greedy_block_width_two():
    st, pairs = _greedy_trajectory(B=6, gamma=2, steps=30, seed=9, th=0.5)
    assert len(pairs) > 10
    for est, cap in pairs:
        assert est == float(cap)


def test_uncensored_steps_open_no_probe():
    B, gamma = 3, 5
    st = oracle.estimator_state(B, gamma)
    drafts = np.array([[1, 2, 3, 4], [5, 6, 7, 8], [9, 9, 9, 9]])
    cu = np.array([0, 5, 7, 10])
    wv = np.array([5, 2, 3])
    acc = np.array([4, 0, 1])          # full block; rejection inside window; rejection inside window
    ctx = np.array([10, 20, 30])
    pred = np.zeros(10, dtype=np.int64)
    oracle.estimate_update(st, cu, wv, acc, drafts, ctx, GREEDY, pred=pred)
    assert np.all(st["left"] == 0) and np.all(st["count"] == 0)


def test_first_tail_mismatch_closes_at_window():
    # gamma 4, window 2, the one verified draft accepted: tail d_2, d_3 at
    # positions ctx+2, ctx+3; the bonus row predicts 7 != d_2 = 6
    st = oracle.estimator_state(1, 4)
    oracle.estimate_update(st, np.array([0, 2]), np.array([2]), np.array([1]), np.array([[5, 6, 8]]),
                           np.array([100]), GREEDY, pred=np.array([5, 7]))
    assert st["count"][0] == 1 and st["last"][0] == 1.0 and st["left"][0] == 0


def test_open_interval_and_resolution_across_steps():
    # gamma 4, window 1 (anchor only), accept 0: tail d_1..d_3 at 51..53;
    # the bonus row resolves d_1 (match); the next step commits 52 and 53
    st = oracle.estimator_state(1, 4)
    oracle.estimate_update(st, np.array([0, 1]), np.array([1]), np.array([0]), np.array([[4, 5, 6]]),
                           np.array([50]), GREEDY, pred=np.array([4]))
    assert oracle.open_interval(st, 0) == (1.0, 3.0)
    # next step: anchor at 51, accepts 1 draft; rows 0, 1 predict 52 (=5), 53 (=9 != 6)
    oracle.estimate_update(st, np.array([0, 3]), np.array([3]), np.array([1]), np.array([[5, 1, 1]]),
                           np.array([51]), GREEDY, pred=np.array([5, 9, 0]))
    assert st["count"][0] == 1 and st["last"][0] == 2.0 and oracle.open_interval(st, 0) is None


def test_skipped_steps_drop_the_probe():
    st = oracle.estimator_state(1, 4)
    oracle.estimate_update(st, np.array([0, 1]), np.array([1]), np.array([0]), np.array([[4, 5, 6]]),
                           np.array([50]), GREEDY, pred=np.array([4]))
    assert st["left"][0] == 2
    # a later step whose anchor already lies past the probe's next position
    oracle.estimate_update(st, np.array([0, 4]), np.array([4]), np.array([3]), np.array([[1, 1, 1]]),
                           np.array([60]), GREEDY, pred=np.array([1, 1, 1, 0]))
    assert st["left"][0] == 0 and st["count"][0] == 0


def test_rejection_estimate_is_expected_cap_accept_tail():
    """Fixed per-position target p and draft q over a small vocabulary; a
    censored step (window 2 of 6, its draft accepted) and a later step that
    commits the rest of the tail.  The estimate equals the mean of the
    ceilings cap-accept reaches on the same drafts over many uniforms."""
    rng = np.random.default_rng(12)
    V, gamma, c = 6, 6, 40
    npos = gamma + 2
    p = rng.dirichlet(np.ones(V) * 0.7, size=npos)      # target at positions c+1 ..
    q = rng.dirichlet(np.ones(V) * 0.7, size=npos)      # draft at positions c+1 ..
    z = np.log(p)                                       # logits whose softmax is p
    drafts = np.array([[rng.choice(V, p=q[j]) for j in range(gamma - 1)]])
    q_rows = q[None, :gamma - 1]
    st = oracle.estimator_state(1, gamma)
    # step 1: window 2 (anchor + d_1), d_1 accepted: tail d_2..d_5 at c+2..c+5
    oracle.estimate_update(st, np.array([0, 2]), np.array([2]), np.array([1]), drafts, np.array([c]), REJECTION,
                           logits=z[0:2], q_rows=q_rows)
    assert st["left"][0] == 3 or st["count"][0] == 1
    # step 2: anchor at c+2, four rows committed (positions c+3..c+6)
    oracle.estimate_update(st, np.array([0, 5]), np.array([5]), np.array([3]), np.zeros((1, gamma - 1), dtype=int),
                           np.array([c + 2]), REJECTION, logits=z[2:7], q_rows=q_rows)
    assert st["count"][0] == 1
    est = st["last"][0]
    # Monte Carlo: cap-accept verifying the whole block of step 1
    n = 20000
    u = rng.uniform(size=(n, gamma - 1))
    acc_p = np.array([p[j][drafts[0, j]] for j in range(gamma - 1)])
    acc_q = np.array([q[j][drafts[0, j]] for j in range(gamma - 1)])
    ok = u * acc_q < acc_p                  # the oracle's accept test per draft
    lead = np.argmin(np.concatenate([ok, np.zeros((n, 1), bool)], axis=1), axis=1)
    sel = lead >= 1                          # draws where d_1 was accepted (the censored case)
    mc = lead[sel].mean()
    se = lead[sel].std() / np.sqrt(sel.sum())
    assert abs(mc - est) < 5 * se + 1e-3, (mc, est, se)
    # and the same through the oracle's acceptance routine on a few draws
    for k in range(5):
        zf = z[:gamma]
        a, _, ceil = oracle.accept_rejection(zf, np.array([0, gamma]), np.array([gamma]), np.array([gamma]), drafts,
                                             q_rows, u[k:k + 1], np.array([0.5]))
        assert ceil[0] == lead[k]
