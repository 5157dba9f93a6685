"""GPU parity of the block-accept estimator (rv_block_accept_estimate)
against the oracle's (oracle/estimator.py).

* Greedy, end to end: a 24-step compact trajectory through the five stages
  on per-request target continuations; after every step the estimator state
  on the GPU equals the oracle's, which runs its own schedule, pack and
  acceptance on the planted predictions (integers and the survival sums,
  which are integers under greedy, bit for bit).
* Rejection sampling, the kernel alone: an oracle-built multi-step
  trajectory over a small vocabulary with target logits and draft
  distributions fixed per position; both sides consume the same step inputs;
  integers exact, survival sums within 1e-4 relative.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import parity_util as pu
from oracle.estimator import GREEDY, REJECTION
from ragged_verification_amd import rv, synth
from ragged_verification_amd.pipeline import VerifyStep

pytestmark = pytest.mark.gpu


def _gpu_state(state, B, gamma):
    v = rv.estimator_state_views(state, B, gamma)
    return {k: t.cpu().numpy() for k, t in v.items()}


def _check_state(g, o, exact_float=True):
    for k in ("pos", "left", "done", "base", "count"):
        assert np.array_equal(g[k].astype(np.int64), o[k]), k
    for k in ("S", "E", "last", "sum"):
        if exact_float:
            assert np.array_equal(g[k].astype(np.float64), o[k]), (k, g[k], o[k])
        else:
            np.testing.assert_allclose(g[k], o[k], rtol=1e-4, atol=1e-5, err_msg=k)
    for i in range(len(o["left"])):      # tail drafts of open probes
        n = int(o["done"][i] + o["left"][i])
        if o["left"][i] > 0:
            assert np.array_equal(g["tok"][i][:n].astype(np.int64), o["tok"][i][:n]), i


def test_estimator_greedy_trajectory_end_to_end():
    B, gamma, steps = 16, 8, 24
    inp = pu.make_inputs("gqa_bf16", B=B, V=1000, H=256, tiers=(), ctx=("uniform", 20, 200),
                         spare_tokens=(steps + 2) * gamma)
    wl = inp["workload"]
    inp["cost_theta"] = inp["cost_theta"] * 4.0          # more truncated windows
    seq = synth.target_sequences(wl, B, int(inp["ctx"].max()) + (steps + 2) * gamma + 2, seed=77)
    step = VerifyStep(inp, mode="compact", hist_cap=(steps + 1) * gamma, r2t_extra=(steps + 2) * gamma)
    state = torch.zeros(rv.rv_estimator_state_bytes(B, gamma), dtype=torch.uint8, device="cuda")
    ost = oracle.estimator_state(B, gamma)
    ctx = pu.npi(inp["ctx"])
    alpha, theta = inp["cost_alpha"].cpu().numpy(), inp["cost_theta"].cpu().numpy()
    opened = 0
    for s in range(steps):
        tr = synth.trajectory_step(wl, inp["W"], step.ctx, seq, seed=5000 + s, device="cuda")
        for k in ("conf", "drafts", "hidden_block"):
            inp[k].copy_(tr[k])
        step.schedule()
        step.pack()
        step.stage_payload()
        step.attn()
        step.lm()
        step.block_accept_estimate(state)
        step.scatter()
        torch.cuda.synchronize()
        assert step.status() == 0
        # the oracle's own step on the planted predictions
        conf, drafts = tr["conf"].cpu().numpy(), pu.npi(tr["drafts"])
        wc, wv, _, _ = oracle.schedule(conf, gamma, oracle.COMPACT, inp["cost_bias"], alpha, theta)
        cu = np.concatenate([[0], np.cumsum(wv)])
        pred = np.concatenate([[int(seq[i, ctx[i] + k + 1]) for k in range(wv[i])] for i in range(B)])
        acc, bonus, _ = oracle.accept_greedy(pred, cu, wc, wv, drafts)
        assert np.array_equal(pu.npi(step.w_verify), wv)
        assert np.array_equal(pu.npi(step.pred)[:cu[-1]], pred)
        assert np.array_equal(pu.npi(step.accept), acc) and np.array_equal(pu.npi(step.bonus), bonus)
        before = int(ost["count"].sum())
        oracle.estimate_update(ost, cu, wv, acc, drafts, ctx, GREEDY, pred=pred)
        _check_state(_gpu_state(state, B, gamma), ost)
        opened += int((ost["left"] > 0).sum()) + int(ost["count"].sum()) - before
        ctx = ctx + acc + 1
        assert np.array_equal(pu.npi(step.ctx), ctx)
    pu.log(f"greedy trajectory: {int(ost['count'].sum())} probes closed, "
           f"{int((ost['left'] > 0).sum())} open at the end")
    assert int(ost["count"].sum()) >= 20


def test_estimator_rejection_kernel_alone():
    rng = np.random.default_rng(31)
    B, gamma, V, steps = 7, 6, 3000, 8
    g1 = gamma - 1
    ctx = rng.integers(5, 40, size=B)
    npos = int(ctx.max()) + (steps + 2) * gamma + 2
    Z = (rng.normal(size=(B, npos, V)) * 1.5).astype(np.float32)          # target logits at each position
    Q = rng.dirichlet(np.ones(V) * 0.3, size=(B, npos)).astype(np.float32)  # draft distribution at each position
    state = torch.zeros(rv.rv_estimator_state_bytes(B, gamma), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    ost = oracle.estimator_state(B, gamma)
    dev = lambda a, dt: torch.tensor(a, dtype=dt, device="cuda").contiguous()
    closed = 0
    for s in range(steps):
        wv = rng.integers(1, gamma + 1, size=B)
        cu = np.concatenate([[0], np.cumsum(wv)])
        drafts = np.array([[rng.choice(V, p=Q[i, ctx[i] + j] / Q[i, ctx[i] + j].sum()) for j in range(1, gamma)]
                           for i in range(B)])
        q_rows = np.stack([Q[i, ctx[i] + 1:ctx[i] + gamma] for i in range(B)])     # [B, g1, V]
        logits = np.concatenate([Z[i, ctx[i] + 1:ctx[i] + 1 + wv[i]] for i in range(B)])
        # accept: some requests take their whole window (censored when w < gamma)
        acc = np.array([wv[i] - 1 if rng.uniform() < 0.6 else rng.integers(0, wv[i]) for i in range(B)])
        rows_cap = B * gamma
        logits_pad = np.zeros((rows_cap, V), dtype=np.float32)
        logits_pad[:cu[-1]] = logits
        rv.rv_block_accept_estimate(dev(cu, torch.int32), dev(wv, torch.int32), dev(acc, torch.int32),
                                    dev(drafts, torch.int32), dev(ctx, torch.int32), rv.RV_REJECTION, state, ws,
                                    logits=dev(logits_pad, torch.float32), q_rows=dev(q_rows, torch.float32))
        torch.cuda.synchronize()
        assert rv.rv_device_status(ws) == 0
        before = int(ost["count"].sum())
        oracle.estimate_update(ost, cu, wv, acc, drafts, ctx, REJECTION, logits=logits_pad.astype(np.float64),
                               q_rows=q_rows)
        closed += int(ost["count"].sum()) - before
        _check_state(_gpu_state(state, B, gamma), ost, exact_float=False)
        ctx = ctx + acc + 1
    assert closed >= 3, closed
