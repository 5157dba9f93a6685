"""The cost-table loop on the GPU (DSpark-in-SGLang page, §A2 "cost-table
profiling and modelling"): five-stage step times recorded on this GPU over
batch sizes and modes go through the library's fit (rv_fit_cost_model), and
the fitted tables drive rv_schedule; the oracle fits the same samples
(oracle.fit_cost_model) and schedules with its own tables.

The fits agree to 1e-9 relative.  Windows, K* and E* must then be equal bit
for bit when the integer decision is well posed (the oracle's best ratio
E/T beats every other K by more than the table difference could move it,
1e-7 relative); when measured step times happen to make a near tie, the
GPU's K* must be one of the near-best K and its E* that K's exact E."""

import numpy as np
import pytest
import torch

import oracle
import parity_util as pu
from ragged_verification_amd import rv, synth
from ragged_verification_amd.pipeline import VerifyStep

pytestmark = pytest.mark.gpu


def _step_ms(step, n=5):
    for _ in range(2):
        step.restore()
        step.run()
    torch.cuda.synchronize()
    ev = []
    for _ in range(n):
        step.restore()
        step.schedule()
        step.pack()
        step.stage_payload()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        step.attn()
        step.lm()
        step.scatter()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    return float(np.median([x.elapsed_time(y) for x, y in ev]))


def _ratios(conf, gamma, bias, alpha, theta):
    """The oracle's ratio E(K)/T(K) for every K, and E(K) in fixed point."""
    B = conf.shape[0]
    S = oracle.survival(conf)
    vals = sorted((S[i, k] for i in range(B) for k in range(1, gamma)), reverse=True)
    q = [int(np.floor(v * 2.0 ** 40)) for v in vals]
    n = B << 40
    r, e = [], []
    for K in range(len(q) + 1):
        if K:
            n += q[K - 1]
        r.append(float(n) / oracle.step_time(bias, alpha, theta, B, K))
        e.append(n)
    return np.array(r), e


def test_fitted_cost_table_drives_the_scheduler():
    samples = []
    for B in (1, 8, 24, 48):
        inp = pu.make_inputs("sweep_gqa", B=B, V=4000, H=512, ctx=("uniform", 200, 1200))
        for mode in ("static", "compact"):
            step = VerifyStep(inp, mode=mode)
            ms = _step_ms(step)
            samples.append((B, int(step.mm[0].item()), ms))
            del step
    pu.log(f"samples {samples}")
    bs, Ms, ts = (list(x) for x in zip(*samples))
    gamma = 8
    B_max = 48
    coef, alpha_l, theta_l = rv.rv_fit_cost_model(bs, Ms, ts, alpha_len=B_max + 1, theta_len=B_max * gamma + 1)
    coef_o = oracle.fit_cost_model(bs, Ms, ts)
    np.testing.assert_allclose(coef, coef_o, rtol=1e-9, atol=1e-15)
    bias_o, alpha_o, theta_o = oracle.cost_tables(coef_o, B_max + 1, B_max * gamma + 1)
    assert coef_o[2] > 0 and coef_o[1] + coef_o[0] > 0   # a positive step time at every size here
    checked = 0
    for B in (8, 24, 48):
        inp = pu.make_inputs("sweep_gqa", B=B, V=64, H=64, ctx=("uniform", 4, 8))
        conf = inp["conf"]
        r, e = _ratios(conf.cpu().numpy(), gamma, bias_o, alpha_o, theta_o)
        best = int(np.argmax(r))
        # K whose ratio is within what the 1e-9 table difference could move
        # (1e-7 relative, with room): the decision among them is not fixed
        near = [K for K in range(len(r)) if r[K] >= r[best] * (1.0 - 1e-7)]
        i32 = dict(dtype=torch.int32, device="cuda")
        wc, wv, ks = torch.zeros(B, **i32), torch.zeros(B, **i32), torch.zeros(1, **i32)
        es = torch.zeros(1, dtype=torch.float64, device="cuda")
        ws = torch.zeros(rv.rv_workspace_size(B, gamma), dtype=torch.uint8, device="cuda")
        al = torch.tensor(alpha_l, dtype=torch.float64, device="cuda")
        th = torch.tensor(theta_l, dtype=torch.float64, device="cuda")
        rv.rv_schedule(conf, gamma, "compact", coef[0], al, th, wc, wv, ks, es, ws)
        torch.cuda.synchronize()
        want = oracle.schedule(conf.cpu().numpy(), gamma, oracle.COMPACT, bias_o, alpha_o, theta_o)
        if len(near) == 1:
            assert np.array_equal(pu.npi(wv), want[1]) and int(ks.item()) == want[2], B
            np.testing.assert_allclose(float(es.item()), want[3], rtol=1e-12)
        else:
            # a near tie: any of the near-best K, with its exact E(K)
            k_gpu = int(ks.item())
            assert k_gpu in near, (B, k_gpu, near)
            assert float(es.item()) == e[k_gpu] / 2.0 ** 40, B
            pu.log(f"B={B}: near tie among K={near}, GPU chose {k_gpu}")
        pu.log(f"B={B}: K*={want[2]} windows {np.bincount(want[1], minlength=gamma + 1)[1:].tolist()}")
        checked += 1
    assert checked == 3
