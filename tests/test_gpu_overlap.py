"""The overlapped loop (OverlapLoop: step s+1's schedule on a side stream
during step s's attention and LM head, ordered by device events) against the
same loop run in order on one stream: every output of every step and the
final state equal bit for bit.  The windows of each step equal the oracle's
schedule on the relayed confidences (those of two steps back)."""

import numpy as np
import pytest
import torch

import oracle
import parity_util as pu
from ragged_verification_amd import synth
from ragged_verification_amd.pipeline import OverlapLoop

pytestmark = pytest.mark.gpu

OUTS = ("cu", "mm", "row_req", "slot", "o", "lse", "pred", "accept", "bonus", "ceiling", "commit_cu", "commit_tok",
        "commit_slot", "free_count", "ctx", "anchor")


def _loop(inp, steps, overlap, n_steps, gamma):
    return OverlapLoop(inp, steps, overlap=overlap, hist_cap=(n_steps + 1) * gamma, r2t_extra=(n_steps + 2) * gamma)


def _run(inp, steps, overlap, n_steps, gamma):
    loop = _loop(inp, steps, overlap, n_steps, gamma)
    snaps = []

    def snap(s):
        d = {k: getattr(loop.vs, k).clone() for k in OUTS}
        d["w_verify"] = loop.window(s)[1].clone()
        d["k_star"] = loop.window(s)[2].clone()
        snaps.append(d)

    loop.run(after_step=snap)
    torch.cuda.synchronize()
    assert loop.status() == 0
    final = {k: getattr(loop.vs, k).clone() for k in ("ctx", "anchor", "hist", "hist_len", "req_to_token")}
    return snaps, final


def _compare(B):
    gamma, n = 8, 7
    inp = pu.make_inputs("sweep_gqa", B=B, V=2000, H=256, tiers=(), ctx=("uniform", 100, 600),
                         spare_tokens=(n + 2) * gamma)
    wl = inp["workload"]
    seq = synth.target_sequences(wl, B, int(inp["ctx"].max()) + (n + 2) * gamma + 2, seed=11)
    # per-step inputs along the target continuation, drawn at the context the
    # in-order loop reaches (both loops then verify the same drafts)
    steps = []
    ctx = inp["ctx"].clone()
    for s in range(n):
        steps.append(synth.trajectory_step(wl, inp["W"], ctx, seq, seed=900 + s, device="cuda"))
        ctx = ctx + 1          # drafts are planted relative to a context; any context keeps them well formed
    a, fa = _run(inp, steps, False, n, gamma)
    b, fb = _run(inp, steps, True, n, gamma)
    for s in range(n):
        for k, t in a[s].items():
            assert torch.equal(t, b[s][k]), (s, k)
        # windows: the oracle's schedule on the relayed confidences
        conf = steps[max(s - 2, 0)]["conf"].cpu().numpy()
        want = oracle.schedule(conf, gamma, oracle.COMPACT, inp["cost_bias"], inp["cost_alpha"].cpu().numpy(),
                               inp["cost_theta"].cpu().numpy())
        assert np.array_equal(pu.npi(a[s]["w_verify"]), want[1]) and int(a[s]["k_star"].item()) == want[2], s
    for k, t in fa.items():
        assert torch.equal(t, fb[k]), k
    pu.log(f"B={B}: {n} steps, committed {int(pu.npi(fa['hist_len']).sum())} tokens, overlapped == in order")
    return inp, steps, fa


@pytest.mark.parametrize("B", [1, 8, 32])
def test_overlap_equals_in_order_loop(B):
    _compare(B)


@pytest.mark.parametrize("B", [8])
def test_overlap_graph_replays_equal_eager(B):
    """The overlapped loop captured into one graph (both streams): every
    replay, with eager work and synchronisations between them, ends in the
    state of the eager in-order loop."""
    gamma, n = 8, 7
    inp, steps, fa = _compare(B)
    loop = _loop(inp, steps, True, n, gamma)
    loop.capture()
    for r in range(3):
        loop.vs.restore()
        torch.cuda.synchronize()
        loop.replay()
        torch.cuda.synchronize()
        assert loop.status() == 0
        for k in ("ctx", "anchor", "hist", "hist_len", "req_to_token"):
            assert torch.equal(getattr(loop.vs, k), fa[k]), (r, k)
        torch.zeros(1 << 20, device="cuda").sum().item()   # eager work between replays
    pu.log(f"B={B}: graph of {n} overlapped steps, 3 replays == eager")
