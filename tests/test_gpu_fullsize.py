"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (VerifyStep, no logits output unless the rule needs them).

Integer outputs are compared in full (schedule, pack, every row's argmax
against the planted target, accept lengths, bonus tokens, scatter); float
outputs on sampled rows the oracle can afford one by one.
"""

import numpy as np
import pytest
import torch

import oracle
import parity_util as pu
from ragged_verification_amd.pipeline import VerifyStep

pytestmark = pytest.mark.gpu


def _sample_rows(ref, ctx, k_random=4, seed=0):
    M = ref["M"]
    rr = ref["row_req"][:M]
    longest = int(np.argmax(ctx))
    shortest = int(np.argmin(ctx))
    rows = {int(np.nonzero(rr == longest)[0][-1]), int(np.nonzero(rr == shortest)[0][0]), M - 1, 0}
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.choice(M, size=k_random, replace=False))
    return sorted(rows)


def _block_rows(M, seed=1, block=32):
    """One random row in every 32-row block of the packed rows (so every row
    block of every 128-row LM tile holds a compared row), the first row and
    the last real row."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1}
    for b0 in range(0, M, block):
        rows.add(int(rng.integers(b0, min(b0 + block, M))))
    return sorted(rows)


def _planted_accept(inp, ref):
    """Greedy accept lengths known from the planting: leading drafts equal to
    the planted target, capped by the verify and commit windows."""
    correct = inp["correct"].cpu().numpy()
    targets = pu.npi(inp["targets"])
    B = inp["B"]
    acc = np.zeros(B, dtype=np.int64)
    ceil = np.zeros(B, dtype=np.int64)
    for i in range(B):
        lead = 0
        while lead < ref["w_verify"][i] - 1 and correct[i, lead]:
            lead += 1
        ceil[i] = lead
        acc[i] = min(lead, ref["w_commit"][i] - 1)
    bonus = targets[np.arange(B), acc]
    return acc, bonus, ceil


def _greedy_full(name, mode, B=None, attn_rows=6):
    inp = pu.make_inputs(name, B=B, gen_on_gpu=True)
    pu.log(f"full {name} B={inp['B']} mode={mode}")
    ref = pu.oracle_schedule_pack(inp, mode)
    step = VerifyStep(inp, mode=mode)
    step.run()
    torch.cuda.synchronize()
    assert step.status() == 0
    pu.check_schedule_pack(step, ref)
    M, M_pad = ref["M"], ref["M_pad"]
    ctx = pu.npi(inp["ctx"])
    rows = _sample_rows(ref, ctx, k_random=attn_rows)
    worst = pu.check_attention(step, inp, ref, rows, "bf16")
    pu.log(f"attention rows {rows} max err {worst:.3g}")

    # every row's argmax equals the planted target (independent of any GEMM)
    bidx = pu.packed_block_index(ref, inp["gamma"])
    targets = pu.npi(inp["targets"]).reshape(-1)[bidx]
    pred = pu.npi(step.pred)
    assert np.array_equal(pred[:M], targets)
    assert np.all(pred[M:M_pad] == -1)
    # logits of a row in every 32-row block against the oracle's fp64 logits
    lr = _block_rows(M)
    z = pu.oracle_logits_rows(inp, ref, lr)
    pu.check_pred_gap(z)
    assert np.array_equal(oracle.lm_head_pred(z), pred[lr])
    # the logits themselves (same kernel with the logits store on)
    with_l = VerifyStep(inp, mode=mode, with_logits=True)
    with_l.run()
    torch.cuda.synchronize()
    zg = with_l.logits.cpu().numpy()[lr]
    rel = np.max(np.abs(zg - z), axis=1) / np.max(np.abs(z), axis=1)
    assert np.all(rel <= pu.LOGIT_TOL["bf16"]), rel
    assert np.array_equal(pu.npi(with_l.pred), pred)
    del with_l

    acc, bonus, ceil = _planted_accept(inp, ref)
    assert np.array_equal(pu.npi(step.accept), acc)
    assert np.array_equal(pu.npi(step.ceiling), ceil)
    assert np.array_equal(pu.npi(step.bonus), bonus)
    B = inp["B"]
    sc = oracle.compact_scatter(ref["cu"], ref["w_verify"], acc, bonus, pu.npi(inp["drafts"]), ref["slot"],
                                ctx, pu.npi(inp["anchor"]), pu.npi(step.req_to_token0),
                                pu.npi(step.hist0), pu.npi(step.hist_len0))
    n = int(sc["commit_cu"][-1])
    assert np.array_equal(pu.npi(step.commit_cu), sc["commit_cu"])
    assert np.array_equal(pu.npi(step.commit_tok)[:n], sc["commit_tok"])
    assert np.array_equal(pu.npi(step.commit_slot)[:n], sc["commit_slot"])
    nf = int(step.free_count.item())
    assert np.array_equal(pu.npi(step.free_slots)[:nf], sc["free_slots"])
    assert np.array_equal(pu.npi(step.ctx), sc["ctx"])
    assert np.array_equal(pu.npi(step.anchor), sc["anchor"])
    assert np.array_equal(pu.npi(step.req_to_token), sc["req_to_token"])
    assert np.array_equal(pu.npi(step.hist), sc["hist"])
    pu.log(f"ok M={M} M_pad={M_pad} logits rel {rel.max():.3g}")


def test_full_mla_compact():
    """The benchmark's workload and launch configuration."""
    _greedy_full("mla_bf16", "compact")


def test_full_mla_static():
    _greedy_full("mla_bf16", "static", attn_rows=3)


def test_full_gqa_compact():
    _greedy_full("gqa_bf16", "compact")


@pytest.mark.parametrize("B", [1, 32, 256])
def test_full_sweep_cap_accept(B):
    _greedy_full("sweep_gqa", "cap_accept", B=B, attn_rows=3)


def test_full_rejection():
    inp = pu.make_inputs("rejection_bf16", gen_on_gpu=True)
    mode = "compact"
    ref = pu.oracle_schedule_pack(inp, mode)
    step = VerifyStep(inp, mode=mode)
    step.run()
    torch.cuda.synchronize()
    assert step.status() == 0
    pu.check_schedule_pack(step, ref)
    ctx = pu.npi(inp["ctx"])
    rows = _sample_rows(ref, ctx, k_random=3)
    worst = pu.check_attention(step, inp, ref, rows, "bf16")
    pu.log(f"attention rows {rows} max err {worst:.3g}")
    M = ref["M"]
    cu = ref["cu"]
    # logits of a row in every 32-row block
    lr = _block_rows(M)
    z = pu.oracle_logits_rows(inp, ref, lr)
    rel = np.max(np.abs(step.logits.cpu().numpy()[lr] - z), axis=1) / np.max(np.abs(z), axis=1)
    assert np.all(rel <= pu.LOGIT_TOL["bf16"]), rel
    # acceptance for 16 requests spread over the batch plus the longest
    # context: all their rows' logits from the oracle
    B = inp["B"]
    reqs = sorted({int(x) for x in np.linspace(0, B - 1, 16).round()} | {int(np.argmax(ctx))})
    rows = [r for i in reqs for r in range(cu[i], cu[i + 1])]
    z = pu.oracle_logits_rows(inp, ref, rows)
    zg = step.logits.cpu().numpy()[rows]
    rel = np.max(np.abs(zg - z), axis=1) / np.max(np.abs(z), axis=1)
    assert np.all(rel <= pu.LOGIT_TOL["bf16"]), rel
    diag = {}
    sub_cu = np.zeros(len(reqs) + 1, dtype=np.int64)
    for j, i in enumerate(reqs):
        sub_cu[j + 1] = sub_cu[j] + (cu[i + 1] - cu[i])
    acc, bonus, ceil = oracle.accept_rejection(
        z, sub_cu, ref["w_commit"][reqs], ref["w_verify"][reqs], pu.npi(inp["drafts"])[reqs],
        pu.np64(inp["q_rows"][reqs]), pu.np64(inp["u"][reqs]), pu.np64(inp["u_bonus"][reqs]), diag=diag)
    for m in diag["decision_margin"]:
        assert all(x >= 1e-4 for x in m), "accept decision too close to call"
    ga, gb, gc = pu.npi(step.accept)[reqs], pu.npi(step.bonus)[reqs], pu.npi(step.ceiling)[reqs]
    assert np.array_equal(ga, acc) and np.array_equal(gc, ceil)
    moved = pu.check_bonus(gb, bonus, diag)
    pu.log(f"ok rejection: {len(reqs)} requests, accepts {ga.tolist()}, bonus moved across a CDF step "
           f"for {len(moved)}")
    # the sampled requests' scatter entries against the oracle's accepts
    ccu, ctok, cslot = pu.npi(step.commit_cu), pu.npi(step.commit_tok), pu.npi(step.commit_slot)
    r2t, ctx_new, anc = pu.npi(step.req_to_token), pu.npi(step.ctx), pu.npi(step.anchor)
    drafts = pu.npi(inp["drafts"])
    for j, i in enumerate(reqs):
        a = int(acc[j])
        b = int(gb[j]) if j in moved else int(bonus[j])
        assert ccu[i + 1] - ccu[i] == a + 1
        assert ctok[ccu[i]:ccu[i + 1]].tolist() == drafts[i, :a].tolist() + [b]
        assert cslot[ccu[i]:ccu[i + 1]].tolist() == ref["slot"][cu[i]:cu[i] + a + 1].tolist()
        assert r2t[i, ctx[i]:ctx[i] + a + 1].tolist() == ref["slot"][cu[i]:cu[i] + a + 1].tolist()
        assert ctx_new[i] == ctx[i] + a + 1 and anc[i] == b
    # scatter invariants at full size
    a_all = pu.npi(step.accept)
    assert int(step.commit_cu[-1].item()) == int((a_all + 1).sum())
    got = np.concatenate([pu.npi(step.commit_slot)[:int((a_all + 1).sum())],
                          pu.npi(step.free_slots)[:int(step.free_count.item())]])
    assert sorted(got.tolist()) == sorted(ref["slot"][:M].tolist())
