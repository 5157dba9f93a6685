"""Seeded synthetic inputs for the verify step (shared by tests and bench).

This module draws inputs only: it holds none of the verify step's arithmetic
(no survival products, cost evaluation, packing, attention, logits-argmax,
acceptance or scatter).  Both the CPU oracle and the HIP library consume what
it returns; neither is imported here.

The pages benchmark on gsm8k / arena-hard / poetry traffic and a frontier
prompt file with trained DeepSeek-V4 models (DSpark-in-SGLang page, §A4); none
of that is available, so these seeded workloads stand in for it, with the
shapes and value distributions listed in ``WORKLOADS``:

* confidences: U(0.3, 0.99), Beta(a, b), or three Beta classes mixed by
  ``request mod 3`` (high Beta(9,1) / mid Beta(3,2) / low Beta(2,3));
* context lengths: uniform integers, or log-normal (median, sigma=1) capped;
* a paged KV cache whose page table is a random permutation of all pages;
* greedy workloads plant each row's target token ``t`` in the hidden state
  (``h = x + beta * W[t] / |W[t]|`` with ``x ~ N(0,1)``) and draw each draft as
  ``t`` with probability equal to its confidence, else a uniform other token,
  so the greedy accept length is known by construction;
* the rejection workload defines the draft distribution as the softmax of the
  target logits plus N(0,1) noise (the workload's own definition; the logits
  for that are formed here with a plain fp32 ``torch.matmul``), samples the
  drafts from it, sets each confidence to the exact per-position acceptance
  probability ``sum_v min(p_v, q_v)`` (a perfectly calibrated confidence), and
  draws the acceptance uniforms away from their decision boundary.
"""

from dataclasses import dataclass, field, replace
import math

import torch

COST_BIAS_MS = 1.0
COST_ALPHA_MS_PER_REQ = 0.01
COST_THETA_MS_PER_TOKEN = 0.004


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    gamma: int
    Hq: int
    Hkv: int
    Dqk: int
    Dv: int
    page_size: int
    H: int
    V: int
    dtype: str               # "f32" or "bf16"
    rule: str                # "greedy" or "rejection"
    tiers: tuple             # capture tiers, () = none, "pow2" = power of two
    conf: tuple              # ("uniform", lo, hi) | ("beta", a, b) | ("classes", ...) | ("overlap",)
    ctx: tuple               # ("uniform", lo, hi) | ("lognormal", median, sigma, cap)
    latent: bool = False     # MLA-style: value = first Dv entries of the key row
    contiguous: bool = False  # one page per request, identity page table
    plant_beta: float = 14.0
    plant_power: float = 1.0  # a draft matches its target with probability conf ** plant_power
    spare_tokens: int = 0     # KV pages for this many positions past ctx + gamma (multi-step runs)
    seed: int = 1000
    modes: tuple = ("static", "compact")


WORKLOADS = {
    "tiny_f32": Workload(
        name="tiny_f32", B=4, gamma=4, Hq=4, Hkv=1, Dqk=64, Dv=64,
        page_size=128, H=128, V=512, dtype="f32", rule="greedy", tiers=(),
        conf=("uniform", 0.3, 0.99), ctx=("uniform", 16, 64), contiguous=True,
        seed=1001),
    "gqa_bf16": Workload(
        name="gqa_bf16", B=32, gamma=8, Hq=32, Hkv=8, Dqk=128, Dv=128,
        page_size=16, H=4096, V=32000, dtype="bf16", rule="greedy",
        tiers=(64, 128, 256), conf=("beta", 4.0, 2.0),
        ctx=("uniform", 512, 4096), seed=1002),
    "rejection_bf16": Workload(
        name="rejection_bf16", B=128, gamma=8, Hq=64, Hkv=8, Dqk=128, Dv=128,
        page_size=64, H=4096, V=151936, dtype="bf16", rule="rejection",
        tiers=(128, 256, 512, 1024), conf=("overlap",),
        ctx=("lognormal", 4096, 1.0, 16384), seed=1003),
    "mla_bf16": Workload(
        name="mla_bf16", B=256, gamma=8, Hq=128, Hkv=1, Dqk=576, Dv=512,
        page_size=64, H=7168, V=129280, dtype="bf16", rule="greedy",
        tiers=(256, 512, 1024, 2048), conf=("beta", 4.0, 2.0),
        ctx=("uniform", 1024, 32768), latent=True, seed=1004),
    "sweep_gqa": Workload(
        name="sweep_gqa", B=256, gamma=8, Hq=32, Hkv=8, Dqk=128, Dv=128,
        page_size=16, H=4096, V=32000, dtype="bf16", rule="greedy",
        tiers="pow2", conf=("classes", (9.0, 1.0), (3.0, 2.0), (2.0, 3.0)),
        ctx=("uniform", 512, 4096), seed=1005,
        modes=("static", "compact", "cap_accept")),
}

SWEEP_BATCHES = (1, 8, 16, 32, 64, 96, 128, 160, 192, 256)


def workload(name, **overrides):
    """A named workload, optionally with some fields replaced (smaller sizes
    for tests)."""
    return replace(WORKLOADS[name], **overrides)


def tiers_for(wl, B=None):
    B = wl.B if B is None else B
    if wl.tiers == "pow2":
        t, out = 1, []
        while t < B * wl.gamma:
            out.append(t)
            t *= 2
        out.append(t)
        return tuple(out)
    return tuple(wl.tiers)


def cost_tables(B_max, M_max):
    """Cost table entries: bias, alpha[bs] for bs=0..B_max, theta[M] for
    M=0..M_max (ms, fp64).  Coefficients of the mixed-confidence sweep
    workload, used for every workload."""
    alpha = torch.arange(B_max + 1, dtype=torch.float64) * COST_ALPHA_MS_PER_REQ
    theta = torch.arange(M_max + 1, dtype=torch.float64) * COST_THETA_MS_PER_TOKEN
    return COST_BIAS_MS, alpha, theta


class _Seeds:
    """Independent torch generators per named tensor, derived from one seed."""

    def __init__(self, seed, device):
        self.seed, self.device = int(seed), torch.device(device)

    def gen(self, name):
        h = 0
        for ch in name:
            h = (h * 131 + ord(ch)) % 1000003
        g = torch.Generator(device=self.device)
        g.manual_seed(self.seed * 1000003 + h)
        return g


def _beta(a, b, shape, g, device):
    # Beta(a, b) from two gammas; torch has no seeded beta sampler.
    x = torch._standard_gamma(torch.full(shape, float(a), dtype=torch.float64, device=device), generator=g)
    y = torch._standard_gamma(torch.full(shape, float(b), dtype=torch.float64, device=device), generator=g)
    return x / (x + y)


def _confidences(wl, B, g, device):
    kind = wl.conf[0]
    shape = (B, wl.gamma - 1)
    if kind == "uniform":
        lo, hi = wl.conf[1], wl.conf[2]
        c = lo + (hi - lo) * torch.rand(shape, dtype=torch.float64, generator=g, device=device)
    elif kind == "beta":
        c = _beta(wl.conf[1], wl.conf[2], shape, g, device)
    elif kind == "classes":
        classes = wl.conf[1:]
        c = torch.empty(shape, dtype=torch.float64, device=device)
        for j, (a, b) in enumerate(classes):
            if j >= B:
                break
            idx = torch.arange(j, B, len(classes), device=device)
            if len(idx):
                c[idx] = _beta(a, b, (len(idx), wl.gamma - 1), g, device)
    else:
        raise ValueError(kind)
    return c.clamp(0.0, 1.0).to(torch.float32)


def _contexts(wl, B, g, device):
    kind = wl.ctx[0]
    if kind == "uniform":
        lo, hi = wl.ctx[1], wl.ctx[2]
        return torch.randint(lo, hi + 1, (B,), generator=g, device=device, dtype=torch.int64)
    if kind == "lognormal":
        median, sigma, cap = wl.ctx[1], wl.ctx[2], wl.ctx[3]
        n = torch.randn((B,), generator=g, device=device, dtype=torch.float64)
        x = torch.round(median * torch.exp(sigma * n))
        return x.clamp(1, cap).to(torch.int64)
    raise ValueError(kind)


def _dtype(wl):
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


def topk_indices(ctx, gamma, K, seed, device="cpu"):
    """Synthetic sparse-attention key lists, block-major int32 [B, gamma, K]:
    block position k of request i (sequence position p = ctx_i + k) lists
    min(K, p + 1) distinct positions drawn uniformly from 0..p, ascending,
    padded with -1.  (The pages name the sparse-MLA path of DeepSeek-V4 but
    not how its selector picks keys; uniform draws stand in for it.)"""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    ctx = ctx.to("cpu").to(torch.int64)
    B = ctx.numel()
    out = torch.full((B, gamma, K), -1, dtype=torch.int32)
    for i in range(B):
        for k in range(gamma):
            p = int(ctx[i]) + k
            n = min(K, p + 1)
            sel = torch.randperm(p + 1, generator=g)[:n].sort().values
            out[i, k, :n] = sel.to(torch.int32)
    return out.to(device)


def _plant(wl, W, x, conf, targets, gd):
    """Hidden states whose target argmax at block position k is targets[:, k]
    (h = x + beta * W[t] / |W[t]|), and drafts d_j equal to targets[:, j-1]
    with probability conf (or conf ** plant_power), else a uniform other
    token."""
    B, gamma = targets.shape
    V, H = W.shape
    Wt = W[targets.reshape(-1)].to(torch.float32)
    unit = Wt / Wt.norm(dim=1, keepdim=True)
    hidden = (x.reshape(B * gamma, H) + wl.plant_beta * unit).reshape(B, gamma, H).to(W.dtype)
    coin = torch.rand((B, gamma - 1), generator=gd, device=W.device, dtype=torch.float64)
    match_p = conf.to(torch.float64)
    if wl.plant_power != 1.0:   # miscalibrated confidences (observability tests)
        match_p = match_p ** wl.plant_power
    correct = coin < match_p
    other = torch.randint(0, V - 1, (B, gamma - 1), generator=gd, device=W.device, dtype=torch.int64)
    t_prev = targets[:, :gamma - 1]
    other = other + (other >= t_prev).to(torch.int64)
    drafts = torch.where(correct, t_prev, other)
    return hidden, drafts, correct


def target_sequences(wl, B, length, seed):
    """A fixed target continuation per request (int64 [B, length]): the token
    the target predicts at every absolute position, for multi-step greedy
    trajectories in which truncated and full-block verification see the same
    target (token at position P = seq[i, P])."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randint(0, wl.V, (B, length), generator=g, dtype=torch.int64)


def trajectory_step(wl, W, ctx, seq, seed, device="cpu"):
    """Greedy step inputs on a target continuation: confidences, drafts
    d_j (proposals for positions ctx + j, equal to seq with probability conf)
    and hidden states planted so that block position k predicts
    seq[i, ctx_i + k + 1].  Returns a dict of conf (f32), drafts (i32),
    hidden_block and targets [B, gamma]."""
    B = ctx.numel()
    gamma = wl.gamma
    S = _Seeds(seed, device)
    c = ctx.to("cpu").to(torch.int64)
    idx = c[:, None] + 1 + torch.arange(gamma)[None, :]
    targets = torch.gather(seq, 1, idx).to(device)
    conf = _confidences(wl, B, S.gen("conf"), device)
    x = torch.randn((B, gamma, wl.H), generator=S.gen("hidden"), device=device, dtype=torch.float32)
    hidden, drafts, _ = _plant(wl, W, x, conf, targets, S.gen("drafts"))
    return {"conf": conf.contiguous(), "drafts": drafts.to(torch.int32).contiguous(), "hidden_block": hidden,
            "targets": targets}


def make_inputs(wl, device="cpu", B=None, seed=None):
    """Draw every input of one verify step for workload ``wl``.

    Returns a dict of tensors on ``device`` (integers as int32 unless noted).
    Block-major payloads ``q_block`` [B, gamma, Hq, Dqk] and ``hidden_block``
    [B, gamma, H] stand in for the model layers that would produce the packed
    rows.
    """
    B = wl.B if B is None else int(B)
    seed = wl.seed if seed is None else int(seed)
    dev = torch.device(device)
    S = _Seeds(seed, dev)
    gamma, V, H, P = wl.gamma, wl.V, wl.H, wl.page_size
    dt = _dtype(wl)
    out = {"workload": wl, "B": B, "gamma": gamma, "sm_scale": 1.0 / math.sqrt(wl.Dqk)}

    ctx = _contexts(wl, B, S.gen("ctx"), dev)
    if wl.contiguous:
        if int(ctx.max()) + gamma > P:
            raise ValueError("contiguous layout needs ctx + gamma <= page_size")
        pages_per = torch.ones(B, dtype=torch.int64, device=dev)
    else:
        pages_per = (ctx + gamma + wl.spare_tokens + P - 1) // P
    num_pages = int(pages_per.sum())
    max_pages = int(pages_per.max())
    if wl.contiguous:
        perm = torch.arange(num_pages, device=dev)
    else:
        perm = torch.randperm(num_pages, generator=S.gen("pages"), device=dev)
    page_table = torch.full((B, max_pages), -1, dtype=torch.int64, device=dev)
    offs = torch.cumsum(pages_per, 0) - pages_per
    for i in range(B):  # B is at most a few hundred
        n = int(pages_per[i])
        o = int(offs[i])
        page_table[i, :n] = perm[o:o + n]

    kshape = (num_pages, P, wl.Hkv, wl.Dqk)
    k_cache = torch.randn(kshape, generator=S.gen("k"), device=dev, dtype=torch.float32).to(dt)
    v_cache = None
    if not wl.latent:
        vshape = (num_pages, P, wl.Hkv, wl.Dv)
        v_cache = torch.randn(vshape, generator=S.gen("v"), device=dev, dtype=torch.float32).to(dt)
    q_block = torch.randn((B, gamma, wl.Hq, wl.Dqk), generator=S.gen("q"), device=dev,
                          dtype=torch.float32).to(dt)

    W = (0.02 * torch.randn((V, H), generator=S.gen("W"), device=dev, dtype=torch.float32)).to(dt)
    anchor = torch.randint(0, V, (B,), generator=S.gen("anchor"), device=dev, dtype=torch.int64)
    x = torch.randn((B, gamma, H), generator=S.gen("hidden"), device=dev, dtype=torch.float32)

    if wl.rule == "greedy":
        conf = _confidences(wl, B, S.gen("conf"), dev)
        targets = torch.randint(0, V, (B, gamma), generator=S.gen("targets"), device=dev,
                                dtype=torch.int64)
        hidden, drafts, correct = _plant(wl, W, x, conf, targets, S.gen("drafts"))
        out.update(targets=targets, correct=correct)
    else:
        hidden = x.to(dt)
        z = torch.matmul(hidden.reshape(B * gamma, H).to(torch.float32),
                         W.to(torch.float32).t()).reshape(B, gamma, V)
        p = torch.softmax(z[:, :gamma - 1].to(torch.float64), dim=-1)
        noise = torch.randn((B, gamma - 1, V), generator=S.gen("qnoise"), device=dev,
                            dtype=torch.float32)
        q_rows = torch.softmax((z[:, :gamma - 1] + noise).to(torch.float64), dim=-1)
        gd = S.gen("drafts")
        drafts = torch.multinomial(q_rows.reshape(-1, V).to(torch.float32), 1,
                                   generator=gd).reshape(B, gamma - 1)
        conf = torch.minimum(p, q_rows).sum(-1).clamp(0.0, 1.0).to(torch.float32)
        q_rows = q_rows.to(torch.float32)
        pd = torch.gather(p, 2, drafts.unsqueeze(-1)).squeeze(-1)
        qd = torch.gather(q_rows.to(torch.float64), 2, drafts.unsqueeze(-1)).squeeze(-1)
        gu = S.gen("u")
        u = torch.rand((B, gamma - 1), generator=gu, device=dev, dtype=torch.float64)
        for _ in range(64):  # keep u * q(d) away from p(d)
            bad = (u * qd - pd).abs() < 2e-3 * pd
            if not bool(bad.any()):
                break
            u = torch.where(bad, torch.rand(u.shape, generator=gu, device=dev,
                                            dtype=torch.float64), u)
        u_bonus = torch.rand((B,), generator=S.gen("ubonus"), device=dev, dtype=torch.float64)
        out.update(q_rows=q_rows, u=u.to(torch.float32), u_bonus=u_bonus.to(torch.float32))
        del z, p, noise

    B_max = max(B, 1)
    bias, alpha, theta = cost_tables(B_max, B_max * gamma)
    i32 = torch.int32
    out.update(
        conf=conf.contiguous(), ctx=ctx.to(i32), anchor=anchor.to(i32),
        drafts=drafts.to(i32).contiguous(), page_table=page_table.to(i32),
        num_pages=num_pages, max_pages=max_pages, page_size=P,
        k_cache=k_cache, v_cache=v_cache, q_block=q_block, hidden_block=hidden,
        W=W, cost_bias=bias, cost_alpha=alpha.to(dev), cost_theta=theta.to(dev),
        tiers=tiers_for(wl, B),
    )
    return out
