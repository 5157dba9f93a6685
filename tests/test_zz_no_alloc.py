"""The LM head + accept through the no-alloc entry point (static scratch in
the library instead of a caller workspace) against rv_lm_head_accept with a
workspace, on the same inputs: every output equal, on two calls in a row, the
second with a smaller batch (the scratch keeps the first call's contents)."""

import pytest
import torch

import parity_util as pu
from ragged_verification_amd import rv
from ragged_verification_amd.pipeline import VerifyStep

pytestmark = pytest.mark.gpu

OUTS = ("pred", "accept", "bonus", "ceiling", "logits")


def _outputs(step):
    return {n: getattr(step, n).clone() for n in OUTS}


def _noalloc(step, status):
    for n in OUTS:
        getattr(step, n).fill_(-7)
    i = step.inp
    rv.rv_lm_head_accept_noalloc(step.hidden, i["W"], step.mm, step.cu, step.w_commit, step.w_verify, i["drafts"],
                                 step.rule, step.pred, step.accept, step.bonus, step.ceiling, status=status,
                                 logits=step.logits, q_rows=i.get("q_rows"), u=i.get("u"),
                                 u_bonus=i.get("u_bonus"), W_tiled=step.W_tiled)


@pytest.mark.parametrize("name,kw,B1,B2", [
    ("rejection_bf16", dict(V=3000, H=256, ctx=("lognormal", 200, 1.0, 600)), 12, 5),
    ("mla_bf16", dict(V=1000, H=512, ctx=("uniform", 60, 700)), 40, 3),
])
def test_noalloc_equals_workspace_entry_point(name, kw, B1, B2):
    status = torch.zeros(256, dtype=torch.uint8, device="cuda")
    for B in (B1, B2):
        pu.log(f"noalloc {name} B={B}")
        inp = pu.make_inputs(name, B=B, **kw)
        step = VerifyStep(inp, mode="compact", with_logits=True)
        step.schedule()
        step.pack()
        step.stage_payload()
        step.lm()
        torch.cuda.synchronize()
        assert step.status() == 0
        want = _outputs(step)
        M = int(step.mm[0].item())
        for st in (status, None):
            _noalloc(step, st)
            torch.cuda.synchronize()
            got = _outputs(step)
            for n in ("accept", "bonus", "ceiling"):
                assert torch.equal(got[n], want[n]), (B, n)
            assert torch.equal(got["pred"][:M], want["pred"][:M])
            assert torch.equal(got["logits"][:M], want["logits"][:M])
            if st is not None:
                assert rv.rv_device_status(st) == 0


def test_noalloc_reports_device_errors_in_the_callers_status_word():
    inp = pu.make_inputs("gqa_bf16", B=4, V=500, H=128, ctx=("uniform", 10, 60))
    inp["drafts"] = inp["drafts"].clone()
    inp["drafts"][1, 0] = 10_000        # token outside [0, V)
    step = VerifyStep(inp, mode="static", with_logits=True)
    step.schedule()
    step.pack()
    step.stage_payload()
    status = torch.zeros(256, dtype=torch.uint8, device="cuda")
    _noalloc(step, status)
    assert rv.rv_device_status(status) == 6          # BAD_TOKEN
    assert int(step.accept[1].item()) == 0
