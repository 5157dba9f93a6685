"""Benchmark of the ragged, confidence-driven verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mla_bf16]

A step is one pass of the five stages (schedule, pack, verify attention, LM
head + accept, compact scatter) over one batch of seeded synthetic input.  The
default workload is the latent-attention batch of 256 requests with block
width 8 (128 query heads over a 576/512 latent KV cache, contexts uniform in
[1024, 32768], hidden 7168, vocabulary 129280, greedy acceptance, capture
tiers 256/512/1024/2048).  Compact mode is the headline; static mode runs on
identical inputs for comparison.

Reported: packed verify tokens/s (real packed rows per second of five-stage
time) as ``value``, accepted tokens/s, per-stage times, the roofline position
of the dominant kernel (timed with HIP events on the stream it runs on), and
the CPU oracle's rate on a bounded sample of the same workload.
"""

import argparse
import gc
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from ragged_verification_amd import rv, synth  # noqa: E402
from ragged_verification_amd.pipeline import OverlapLoop, VerifyStep  # noqa: E402

METRIC = "packed verify tok/s + accepted tok/s at B=256,γ=8; % of HBM/MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def _json_default(o):
    return o.item() if hasattr(o, "item") else str(o)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class StageTimer:
    """HIP events on torch's current stream (the stream every call uses);
    read back once after the timed region has been synchronised.  The events
    of ``count`` records per stage are created up front, so the timed region
    only records them."""

    def __init__(self, names, count=0):
        self.names = names
        self.pairs = {n: [] for n in names}
        self.acc = {n: 0.0 for n in names}
        self.pool = [torch.cuda.Event(enable_timing=True) for _ in range((len(names) + 1) * count)]

    def _event(self):
        return self.pool.pop() if self.pool else torch.cuda.Event(enable_timing=True)

    def start(self, n):
        e = self._event()
        e.record()
        self.pairs[n].append([e, None])

    def stop(self, n):
        e = self._event()
        e.record()
        self.pairs[n][-1][1] = e

    def switch(self, a, b):
        """Stage a ends where stage b starts: one event for both (a record
        costs about 4 us of host time, as much as a small stage's work)."""
        e = self._event()
        e.record()
        self.pairs[a][-1][1] = e
        self.pairs[b].append([e, None])

    def collect(self):
        pass

    def finish(self):
        torch.cuda.synchronize()
        for n in self.names:
            self.acc[n] = sum(a.elapsed_time(b) for a, b in self.pairs[n])


STAGES = ["schedule", "pack", "attn", "lm_accept", "scatter"]


ROTATE_MIN_BYTES = 1 << 30
ROTATE_MAX_COPIES = 8


def heavy_bytes(inp):
    """Bytes of the inputs a step streams from HBM: the KV caches and the
    LM-head weight (its tiled copy when the step reads that)."""
    n = inp["k_cache"].numel() * inp["k_cache"].element_size()
    if inp.get("v_cache") is not None:
        n += inp["v_cache"].numel() * inp["v_cache"].element_size()
    n += inp["W"].numel() * inp["W"].element_size()
    return n


def rotation_inputs(inp, min_bytes=ROTATE_MIN_BYTES):
    """Input sets for timed steps that rotate through copies of the KV caches
    and the LM-head weight (everything else shared), enough copies that the
    rotated bytes reach min_bytes (at most ROTATE_MAX_COPIES sets):
    consecutive steps then cannot be served from the 256 MB last-level
    cache, as a serving loop's would not be.  One set (no copy) when one copy
    is already that large."""
    per = heavy_bytes(inp)
    n = min(max(1, -(-min_bytes // per)), ROTATE_MAX_COPIES) if per < min_bytes else 1
    sets = [inp]
    for _ in range(n - 1):
        c = dict(inp)
        c["k_cache"] = inp["k_cache"].clone()
        if inp.get("v_cache") is not None:
            c["v_cache"] = inp["v_cache"].clone()
        c["W"] = inp["W"].clone()
        if inp.get("W_tiled") is not None:
            c["W_tiled"] = inp["W_tiled"].clone()
        sets.append(c)
    return sets


def use_inputs(step, inp):
    """Point a built step at another input set of the same shapes."""
    step.inp = inp
    if step.W_tiled is not None:
        step.W_tiled = inp["W_tiled"]


def run_steps(step, n, timer=None, sets=None):
    for s in range(n):
        if sets is not None and len(sets) > 1:
            use_inputs(step, sets[s % len(sets)])
        step.restore()
        if timer:
            timer.start("schedule")
        step.schedule()
        if timer:
            timer.switch("schedule", "pack")
        step.pack()
        if timer:
            timer.switch("pack", "staging")
        step.stage_payload()
        if timer:
            timer.switch("staging", "attn")
        step.attn()
        if timer:
            timer.switch("attn", "lm_accept")
        step.lm()
        if timer:
            timer.switch("lm_accept", "scatter")
        step.scatter()
        if timer:
            timer.stop("scatter")
            timer.collect()


def attn_flops(ctx, w, Hq, Dqk, Dv, window=0):
    """Algorithmic attention flops of one launch: every real row r of request
    i at position ctx_i + k sees ctx_i + k + 1 keys (at most `window` with a
    sliding window), each costing a Dqk-wide dot product and a Dv-wide
    accumulation per query head."""
    tot = 0
    for c, wi in zip(ctx, w):
        keys = sum(min(c + k + 1, window) if window else c + k + 1 for k in range(wi))
        tot += 2 * Hq * (Dqk + Dv) * keys
    return tot


def attn_bytes(ctx, w, wl, elem=2, window=0):
    """Algorithmic attention bytes: each request's visible KV once (keys
    max(0, ctx_i - window + 1) .. ctx_i + w_i - 1 with a sliding window) plus
    the packed queries and outputs."""
    kv_row = wl.Hkv * (wl.Dqk + (0 if wl.latent else wl.Dv)) * elem
    kv = sum((c + wi - (max(0, c - window + 1) if window else 0)) * kv_row for c, wi in zip(ctx, w))
    M = sum(w)
    return kv + M * wl.Hq * (wl.Dqk + wl.Dv) * elem


def lm_flops(M, H, V):
    return 2 * M * H * V


def measure(step, steps, warmup, sets=None):
    # the stages' argument structs of every rotated input set are built up
    # front (host work only, as a serving loop on fixed buffers has them)
    if sets is not None and len(sets) > 1:
        for inp in sets:
            use_inputs(step, inp)
            step.prime()
    run_steps(step, warmup, sets=sets)
    torch.cuda.synchronize()
    timer = StageTimer(STAGES + ["staging"], steps)
    gc.collect()
    gc.disable()   # no collector pause inside the timed steps
    try:
        t0 = time.perf_counter()
        run_steps(step, steps, timer, sets=sets)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    finally:
        gc.enable()
    timer.finish()
    assert step.status() == 0, f"device status {rv.DEV_NAMES.get(step.status())}"
    per = {k: v / steps for k, v in timer.acc.items()}
    five = sum(per[s] for s in STAGES)
    M = int(step.mm[0].item())
    M_pad = int(step.mm[1].item())
    committed = int((step.accept.to(torch.int64) + 1).sum().item())
    return dict(per_stage_ms=per, five_stage_ms=five, wall_ms=wall * 1e3 / steps, M=M, M_pad=M_pad,
                committed=committed)


def measure_graph(step, steps, warmup, sets=None):
    """The same step replayed from its HIP graphs (VerifyStep.capture): front
    (schedule, pack) and back (attention, LM head + accept, scatter) timed
    with HIP events around each replay; staging and state restore between
    them are not counted, as in the eager timing.  With rotated input sets
    one graph pair is captured per set and the steps cycle through them."""
    sets = sets if sets else [step.inp]
    graphs = []
    for inp in sets:
        use_inputs(step, inp)
        step.capture()
        graphs.append((step.g_front, step.g_back))
    for w in range(warmup):
        use_inputs(step, sets[w % len(sets)])
        step.restore()
        graphs[w % len(sets)][0].replay()
        step.stage_payload()
        graphs[w % len(sets)][1].replay()
    torch.cuda.synchronize()
    timer = StageTimer(["front", "staging", "back"], steps)
    gc.collect()
    gc.disable()
    try:
        for k in range(steps):
            g_front, g_back = graphs[k % len(sets)]
            use_inputs(step, sets[k % len(sets)])
            step.restore()
            timer.start("front")
            g_front.replay()
            timer.switch("front", "staging")
            step.stage_payload()
            timer.switch("staging", "back")
            g_back.replay()
            timer.stop("back")
    finally:
        gc.enable()
    timer.finish()
    assert step.status() == 0, f"device status {rv.DEV_NAMES.get(step.status())}"
    per = {k: v / steps for k, v in timer.acc.items()}
    return {"ms_per_step": per["front"] + per["back"], "front_ms": per["front"], "back_ms": per["back"],
            "staging_ms": per["staging"]}


def sweep(steps, warmup):
    """The mixed-confidence sweep: GQA shapes at each batch size of the sweep
    list; request i has confidence class i mod 3.  Static, compact and
    cap-accept run on identical inputs.  One JSON line per batch size: per mode
    the five-stage time, packed rows and committed tokens per step, and (for
    compact and cap-accept) the mean window and committed tokens per class;
    cap-accept also reports its ceiling utilisation (tokens committed over the
    tokens the verified full blocks would allow).  Also the verify-attention
    call's HBM fraction in compact mode."""
    for B in synth.SWEEP_BATCHES:
        wl = synth.workload("sweep_gqa", B=B)
        inp = synth.make_inputs(wl, device="cuda", B=B)
        cls = np.arange(B) % 3
        out = {"workload": "sweep_gqa", "B": B}
        sets = None
        for mode in ("static", "compact", "cap_accept"):
            step = VerifyStep(inp, mode=mode)
            if sets is None:
                sets = rotation_inputs(inp)
                out["rotated_copies"] = len(sets)
            r = measure(step, steps, warmup, sets)
            rec = {"ms_per_step": r["five_stage_ms"], "packed_rows": r["M"], "tier_rows": r["M_pad"],
                   "committed_per_step": r["committed"], "stages_ms": {k: round(v, 4) for k, v in r["per_stage_ms"].items()}}
            wc = step.w_commit.cpu().numpy()
            acc = step.accept.cpu().numpy().astype(np.int64)
            if mode != "static":
                rec["mean_window_by_class"] = [float(wc[cls == k].mean()) if (cls == k).any() else None for k in range(3)]
                rec["committed_by_class"] = [int((acc[cls == k] + 1).sum()) for k in range(3)]
            if mode == "cap_accept":
                ceil = step.ceiling.cpu().numpy().astype(np.int64)
                rec["ceiling_utilisation"] = float((acc + 1).sum() / (ceil + 1).sum())
            if mode == "compact":
                g = measure_graph(step, steps, warmup, sets)
                rec["graph"] = {"ms_per_step": g["ms_per_step"], "front_ms": round(g["front_ms"], 4),
                                "back_ms": round(g["back_ms"], 4)}
                w = step.w_verify.cpu().numpy().astype(np.int64)
                ctx = inp["ctx"].cpu().numpy().astype(np.int64)
                gbs = attn_bytes(ctx, w, wl) / (r["per_stage_ms"]["attn"] / 1e3) / 1e9
                rec["attn_hbm"] = {"achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS}
            out[mode] = rec
            del step
        print(json.dumps(out, default=_json_default), flush=True)
        del inp
        torch.cuda.empty_cache()


def fit_cost(steps, warmup, out_path=None):
    """Cost-table profiling on this GPU: the mixed-confidence workload at every
    batch size of the sweep, static and compact (the sweep's cost table), gives
    samples (bs, M, five-stage ms); rv_fit_cost_model fits
    T = bias + a*bs + th*M; compact then runs again with the fitted tables.
    One JSON line per batch size (measured against predicted time, and the
    committed tokens per ms of static, compact with the sweep's table and
    compact with the fitted table), then one line with the fit."""
    samples, runs = [], {}
    for B in synth.SWEEP_BATCHES:
        wl = synth.workload("sweep_gqa", B=B)
        inp = synth.make_inputs(wl, device="cuda", B=B)
        for mode in ("static", "compact"):
            step = VerifyStep(inp, mode=mode)
            r = measure(step, steps, warmup)
            samples.append((B, r["M"], r["five_stage_ms"]))
            runs[(B, mode)] = r
            del step
        del inp
        torch.cuda.empty_cache()
    bs, Ms, ts = zip(*samples)
    B_max = max(synth.SWEEP_BATCHES)
    gamma = synth.workload("sweep_gqa").gamma
    coef, alpha, theta = rv.rv_fit_cost_model(bs, Ms, ts, alpha_len=B_max + 1, theta_len=B_max * gamma + 1)
    resid = [t - (coef[0] + coef[1] * b + coef[2] * m) for b, m, t in samples]
    for B in synth.SWEEP_BATCHES:
        wl = synth.workload("sweep_gqa", B=B)
        inp = synth.make_inputs(wl, device="cuda", B=B)
        inp["cost_bias"] = coef[0]
        inp["cost_alpha"] = torch.tensor(alpha, dtype=torch.float64, device="cuda")
        inp["cost_theta"] = torch.tensor(theta, dtype=torch.float64, device="cuda")
        step = VerifyStep(inp, mode="compact")
        r = measure(step, steps, warmup)
        cls = np.arange(B) % 3
        wc = step.w_commit.cpu().numpy()
        pred = lambda m: coef[0] + coef[1] * B + coef[2] * m
        out = {"workload": "sweep_gqa", "B": B, "fit": "cost_table"}
        for mode in ("static", "compact"):
            q = runs[(B, mode)]
            out[mode] = {"ms_per_step": q["five_stage_ms"], "predicted_ms": pred(q["M"]), "packed_rows": q["M"],
                         "committed_per_ms": q["committed"] / q["five_stage_ms"]}
        out["compact_fitted"] = {"ms_per_step": r["five_stage_ms"], "predicted_ms": pred(r["M"]),
                                 "packed_rows": r["M"], "committed_per_ms": r["committed"] / r["five_stage_ms"],
                                 "mean_window_by_class": [float(wc[cls == k].mean()) if (cls == k).any() else None
                                                          for k in range(3)]}
        print(json.dumps(out, default=_json_default), flush=True)
        del step, inp
        torch.cuda.empty_cache()
    fit = {"bias_ms": coef[0], "alpha_ms_per_request": coef[1], "theta_ms_per_row": coef[2],
           "samples": len(samples), "rms_residual_ms": float(np.sqrt(np.mean(np.square(resid)))),
           "max_abs_residual_ms": float(np.max(np.abs(resid)))}
    print(json.dumps({"fit": fit}), flush=True)
    if out_path:
        # the recorded samples, the fit and the scheduler's tables, for
        # --cost-table to load
        with open(out_path, "w") as f:
            json.dump({"workload": "sweep_gqa", "device": torch.cuda.get_device_name(0),
                       "samples": [{"bs": b, "M": m, "ms": t} for b, m, t in samples], "fit": fit,
                       "bias": coef[0], "alpha": alpha, "theta": theta}, f)
        log(f"cost table written to {out_path}")


def load_cost_table(path, inp):
    """Replace the workload's cost table with one written by --fit-cost."""
    d = json.load(open(path))
    B, gamma = inp["B"], inp["gamma"]
    if len(d["alpha"]) <= B or len(d["theta"]) <= B * gamma:
        raise SystemExit(f"{path}: tables cover bs < {len(d['alpha'])}, M < {len(d['theta'])}; "
                         f"this workload needs bs = {B}, M up to {B * gamma}")
    inp["cost_bias"] = float(d["bias"])
    inp["cost_alpha"] = torch.tensor(d["alpha"], dtype=torch.float64, device="cuda")
    inp["cost_theta"] = torch.tensor(d["theta"], dtype=torch.float64, device="cuda")


def overlap_bench(steps, warmup, batches=(1, 8, 32, 256)):
    """Steps per second of a multi-step loop with the scheduler overlapped
    (OverlapLoop: the next step's schedule on a side stream during this
    step's attention and LM head) against the same loop in order on one
    stream, at several batch sizes of the GQA sweep shapes, eager and from one
    captured graph (which leaves only the device's critical path).  The step
    inputs cycle through four draws along a target continuation.  One JSON
    line per batch size."""
    gamma = 8
    for B in batches:
        n = warmup + steps
        wl = synth.workload("sweep_gqa", B=B, spare_tokens=(n + 2) * gamma, tiers=())
        inp = synth.make_inputs(wl, device="cuda", B=B)
        seq = synth.target_sequences(wl, B, int(inp["ctx"].max()) + (n + 2) * gamma + 2, seed=3)
        draws = [synth.trajectory_step(wl, inp["W"], inp["ctx"], seq, seed=40 + k, device="cuda") for k in range(4)]
        per_step = [draws[s % 4] for s in range(n)]
        out = {"workload": "sweep_gqa", "B": B, "steps": steps}
        for overlap in (False, True):
            loop = OverlapLoop(inp, per_step, overlap=overlap, hist_cap=(n + 1) * gamma, r2t_extra=(n + 2) * gamma)
            loop.run(n=warmup)
            torch.cuda.synchronize()
            r = {}
            for how in ("eager", "graph"):
                if how == "graph":
                    loop.capture(n=steps)
                loop.vs.restore()
                torch.cuda.synchronize()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                t0 = time.perf_counter()
                a.record()
                if how == "graph":
                    loop.replay()
                else:
                    loop.run(n=steps)
                b.record()
                t_issue = time.perf_counter() - t0
                torch.cuda.synchronize()
                assert loop.status() == 0
                r[how] = {"ms_per_step": a.elapsed_time(b) / steps, "host_issue_ms_per_step": 1e3 * t_issue / steps}
            out["overlapped" if overlap else "in_order"] = r
            del loop
        out["speedup_graph"] = out["in_order"]["graph"]["ms_per_step"] / out["overlapped"]["graph"]["ms_per_step"]
        out["speedup_eager"] = out["in_order"]["eager"]["ms_per_step"] / out["overlapped"]["eager"]["ms_per_step"]
        print(json.dumps(out), flush=True)
        del inp
        torch.cuda.empty_cache()


def cpu_baseline(inp, step, n_req=130):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    schedule and pack for the whole batch, then attention, LM head, accept and
    scatter for the rows of ``n_req`` requests."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:
        blas_threads = None
    wl = inp["workload"]
    gamma = inp["gamma"]
    conf = inp["conf"].cpu().numpy()
    ctx = inp["ctx"].cpu().numpy().astype(np.int64)
    pt = inp["page_table"].cpu().numpy().astype(np.int64)
    drafts = inp["drafts"].cpu().numpy().astype(np.int64)
    anchor = inp["anchor"].cpu().numpy().astype(np.int64)
    alpha = inp["cost_alpha"].cpu().numpy()
    theta = inp["cost_theta"].cpu().numpy()
    n_req = min(n_req, int(inp["B"]))
    reqs = list(range(n_req))
    # host copies of what the sample touches (not timed: data movement)
    pages = sorted({int(p) for r in reqs for p in pt[r] if p >= 0})
    remap = {p: j for j, p in enumerate(pages)}
    kc = inp["k_cache"].index_select(0, torch.tensor(pages, device=inp["k_cache"].device)).float().cpu().numpy()
    vc = None if inp["v_cache"] is None else inp["v_cache"].index_select(
        0, torch.tensor(pages, device=inp["v_cache"].device)).float().cpu().numpy()
    pt2 = np.full_like(pt, -1)
    for r in reqs:
        pt2[r] = [remap[int(p)] if p >= 0 else -1 for p in pt[r]]
    qb = inp["q_block"][:n_req].float().cpu().numpy()
    hb = inp["hidden_block"][:n_req].float().cpu().numpy()
    W = inp["W"].float().cpu().numpy()
    if wl.rule == "rejection":
        q_rows = inp["q_rows"][:n_req].double().cpu().numpy()
        u_acc = inp["u"][:n_req].double().cpu().numpy()
        u_bonus = inp["u_bonus"][:n_req].double().cpu().numpy()

    t0 = time.perf_counter()
    wc, wv, k_star, e_star = oracle.schedule(conf, gamma, oracle.COMPACT, inp["cost_bias"], alpha, theta)
    cu, M, M_pad, row_req, row_pos, tok, slot = oracle.pack(wv, anchor, drafts, ctx, pt, inp["page_size"],
                                                            inp["tiers"])
    rows = [r for r in range(M) if row_req[r] in reqs]
    q = np.stack([qb[row_req[r], r - cu[row_req[r]]] for r in rows])
    o, lse = oracle.verify_attention(q, kc, vc, pt2, inp["page_size"], row_req[rows], row_pos[rows],
                                     len(rows), inp["sm_scale"], Dv=wl.Dv)
    x = np.stack([hb[row_req[r], r - cu[row_req[r]]] for r in rows])
    z = oracle.lm_head_logits(x, W)
    pred = oracle.lm_head_pred(z)
    cu_s = np.concatenate([[0], np.cumsum(wv[:n_req])])
    if wl.rule == "rejection":
        acc, bonus, ceil = oracle.accept_rejection(z, cu_s, wc[:n_req], wv[:n_req], drafts[:n_req], q_rows, u_acc,
                                                   u_bonus)
    else:
        acc, bonus, ceil = oracle.accept_greedy(pred, cu_s, wc[:n_req], wv[:n_req], drafts[:n_req])
    r2t = np.full((n_req, int(ctx[:n_req].max()) + gamma), -1)
    oracle.compact_scatter(cu_s, wv[:n_req], acc, bonus, drafts[:n_req], slot[rows], ctx[:n_req],
                           anchor[:n_req], r2t)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": len(rows) / dt, "unit": "tok/s", "cores": blas_threads or cores, "kind": "oracle",
            "sample": f"schedule+pack of all {inp['B']} requests, then attention, LM head, {wl.rule} accept "
                      f"and scatter for the {len(rows)} packed rows of the first {n_req} requests "
                      f"(numpy fp64, {dt:.1f} s, host has {cores} cores available)",
            "seconds": dt}


COUNTERS_MD = os.path.join(ROOT, "profiles", "verify_attn_latent_bf16_B256_counters.md")
COUNTERS_GQA_MD = os.path.join(ROOT, "profiles", "verify_attn_gqa_bf16_counters.md")
ATTN_SRC = os.path.join(ROOT, "ragged_verification_amd", "csrc", "k_attn.hip")


def measured_traffic(path=None, key="k_attn_mla"):
    """HBM bytes per launch of an attention kernel (``key``: the kernel, and
    for GQA the workload) from a committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE scaled by a copy kernel of known size), or None
    when that summary was taken on another version of the kernel source (its
    recorded sha256 differs from the file's)."""
    try:
        text = open(path or COUNTERS_MD).read()
        src = open(ATTN_SRC, "rb").read()
    except OSError:
        return None
    m_bytes = re.search(r"traffic_bytes_per_launch \(" + re.escape(key) + r"\): (\d+)", text)
    m_hash = re.search(r"source_sha256 \(ragged_verification_amd/csrc/k_attn.hip\): ([0-9a-f]{64})", text)
    if not m_bytes or not m_hash or m_hash.group(1) != hashlib.sha256(src).hexdigest():
        return None
    return int(m_bytes.group(1))


def copy_calibration(mib):
    """A plain device copy of known size (reads and writes ``mib`` MiB per
    launch): profiled under the same counters as the verify kernels, it gives
    the factor between FETCH_SIZE / WRITE_SIZE and bytes actually moved."""
    n = mib * (1 << 20) // 2
    src = torch.randn(n, device="cuda").to(torch.bfloat16)
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 2, "copy_calibration_bytes_written": n * 2,
                      "launches": 5}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mla_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-static", action="store_true")
    ap.add_argument("--topk", type=int, default=0,
                    help="latent workloads: sparse attention over per-row key lists of this many entries")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding-window attention of this many keys (0: full causal)")
    ap.add_argument("--graph", action="store_true",
                    help="also time each mode replayed from HIP graphs (VerifyStep.capture)")
    ap.add_argument("--fit-cost", action="store_true",
                    help="only run cost-table profiling: fit the step-time model on this GPU and rerun compact with it")
    ap.add_argument("--cost-table-out", default=None, metavar="PATH",
                    help="with --fit-cost: write the samples, the fit and the scheduler's tables to PATH (JSON)")
    ap.add_argument("--cost-table", default=None, metavar="PATH",
                    help="schedule with a cost table written by --fit-cost --cost-table-out")
    ap.add_argument("--overlap", action="store_true",
                    help="only time the multi-step loop with the scheduler overlapped against in order (batch 1, 8, 32)")
    ap.add_argument("--overlap-batches", default="1,8,32,256", help="batch sizes for --overlap")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the mixed-confidence batch sweep (one JSON line per batch size)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB five times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU layout is a design "
              f"note, not built", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    rv.load()
    if args.sweep:
        sweep(args.steps, args.warmup)
        return
    if args.fit_cost:
        fit_cost(args.steps, args.warmup, args.cost_table_out)
        return
    if args.overlap:
        overlap_bench(args.steps, args.warmup, tuple(int(b) for b in args.overlap_batches.split(",")))
        return
    wl = synth.workload(args.workload)
    t0 = time.time()
    inp = synth.make_inputs(wl, device="cuda")
    torch.cuda.synchronize()
    if args.cost_table:
        load_cost_table(args.cost_table, inp)
    log(f"inputs for {wl.name} (B={wl.B}) in {time.time() - t0:.1f}s, "
        f"KV {inp['k_cache'].numel() * 2 / 1e9:.2f} GB, W {inp['W'].numel() * 2 / 1e9:.2f} GB")

    results = {}
    sets = None
    for mode in ["compact"] + ([] if args.no_static else ["static"]):
        step = VerifyStep(inp, mode=mode, window=args.window, topk=args.topk)
        if sets is None:
            sets = rotation_inputs(inp)   # after the step made the tiled weight
            if len(sets) > 1:
                log(f"rotating {len(sets)} copies of KV and weights ({heavy_bytes(inp) * len(sets) / 1e9:.2f} GB)")
        r = measure(step, args.steps, args.warmup, sets)
        w = step.w_verify.cpu().numpy().astype(np.int64)
        ctx = inp["ctx"].cpu().numpy().astype(np.int64)
        if args.topk:
            # each row reads its own listed keys: min(topk, p + 1) per row
            keys = sum(min(args.topk, c + k + 1) for c, wi in zip(ctx, w) for k in range(wi))
            r["attn_flops"] = 2 * wl.Hq * (wl.Dqk + wl.Dv) * keys
            r["attn_bytes"] = keys * wl.Dqk * 2 + int(w.sum()) * wl.Hq * (wl.Dqk + wl.Dv) * 2
        else:
            r["attn_flops"] = attn_flops(ctx, w, wl.Hq, wl.Dqk, wl.Dv, args.window)
            r["attn_bytes"] = attn_bytes(ctx, w, wl, window=args.window)
        r["lm_flops"] = lm_flops(r["M"], wl.H, wl.V)
        if args.graph:
            r["graph"] = measure_graph(step, args.steps, args.warmup, sets)
        if wl.rule == "greedy":   # observability, after the timed steps
            cal = step.calibration(10)
            r["calibration"] = {"ece_10_bins": float(cal["ece"].item()),
                                "verified_drafts": int(cal["req_verified"].sum().item()),
                                "matched_drafts": int(cal["req_matched"].sum().item())}
        results[mode] = r
        log(f"{mode}: M={r['M']} M_pad={r['M_pad']} five-stage {r['five_stage_ms']:.3f} ms "
            f"stages {({k: round(v, 4) for k, v in r['per_stage_ms'].items()})}")
        del step
        torch.cuda.empty_cache()

    c = results["compact"]
    t_s = c["five_stage_ms"] / 1e3
    attn_ms = c["per_stage_ms"]["attn"]
    lm_ms = c["per_stage_ms"]["lm_accept"]
    if wl.latent:
        dom, achieved = "verify_attn (latent, bf16 MFMA)", c["attn_flops"] / (attn_ms / 1e3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None if (args.window or args.topk) else measured_traffic(),
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "algorithmic_per_launch": c["attn_flops"], "algorithmic_bytes_per_launch": c["attn_bytes"],
                "launch_ms": attn_ms}
    else:
        achieved = c["attn_bytes"] / (attn_ms / 1e3) / 1e9
        roof = {"kernel": "verify_attn (GQA, bf16)", "bound": "hbm", "achieved": achieved,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "traffic": None if args.window else measured_traffic(COUNTERS_GQA_MD, f"k_attn_gqa, {wl.name}"),
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "algorithmic_per_launch": c["attn_bytes"], "launch_ms": attn_ms}
    lm_tflops = c["lm_flops"] / (lm_ms / 1e3) / 1e12
    # the LM head streams the weight once per launch: below the ridge point
    # (bf16 peak flops per HBM byte) its bound is HBM, above it the MFMAs
    lm_bytes = 2 * wl.V * wl.H + 2 * c["M"] * wl.H + 16 * c["M"] * -(-wl.V // 64)
    if c["lm_flops"] / lm_bytes < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        lm_gbs = lm_bytes / (lm_ms / 1e3) / 1e9
        lm_roof = {"bound": "hbm", "achieved": lm_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                   "frac": lm_gbs / PEAK_HBM_GBS, "algorithmic_bytes_per_launch": lm_bytes, "launch_ms": lm_ms}
    else:
        lm_roof = {"bound": "mfma", "achieved": lm_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                   "frac": lm_tflops / PEAK_BF16_TFLOPS, "algorithmic_per_launch": c["lm_flops"],
                   "launch_ms": lm_ms}
    line = {
        "metric": METRIC,
        "value": c["M"] / t_s,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": c["five_stage_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; stands in for the pages' datasets and trained models)",
        "config": {"workload": f"{wl.name}: B={wl.B}, gamma={wl.gamma}, Hq={wl.Hq}, Hkv={wl.Hkv}, "
                               f"Dqk={wl.Dqk}, Dv={wl.Dv}, page={wl.page_size}, ctx={wl.ctx}, H={wl.H}, "
                               f"V={wl.V}, {wl.rule}, tiers={wl.tiers}",
                   "mode": "compact", "B": wl.B, "gamma": wl.gamma, "window": args.window,
                   "topk": args.topk},
        "accepted_tok_s": c["committed"] / t_s,
        "rotated_input_copies": len(sets),
        "packed_rows": c["M"], "tier_rows": c["M_pad"], "committed_per_step": c["committed"],
        "stages_ms": {k: round(v, 4) for k, v in c["per_stage_ms"].items()},
        "wall_ms_per_step_incl_staging_restore": round(c["wall_ms"], 3),
        "lm_head": lm_roof,
        "roofline": roof,
    }
    if "calibration" in c:
        line["calibration"] = {m: results[m]["calibration"] for m in results}
    if "graph" in c:
        g = c["graph"]
        line["graph"] = {"ms_per_step": g["ms_per_step"], "packed_tok_s": c["M"] / (g["ms_per_step"] / 1e3),
                         "accepted_tok_s": c["committed"] / (g["ms_per_step"] / 1e3),
                         "front_ms": round(g["front_ms"], 4), "back_ms": round(g["back_ms"], 4)}
    if "static" in results:
        s = results["static"]
        line["static"] = {"packed_rows": s["M"], "ms_per_step": s["five_stage_ms"],
                          "packed_tok_s": s["M"] / (s["five_stage_ms"] / 1e3),
                          "accepted_tok_s": s["committed"] / (s["five_stage_ms"] / 1e3),
                          "stages_ms": {k: round(v, 4) for k, v in s["per_stage_ms"].items()}}
        if "graph" in s:
            line["static"]["graph_ms_per_step"] = s["graph"]["ms_per_step"]
        line["compact_vs_static"] = {"row_ratio": c["M"] / s["M"],
                                     "time_ratio": c["five_stage_ms"] / s["five_stage_ms"]}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(inp, None)
    print(json.dumps(line, default=_json_default), flush=True)


if __name__ == "__main__":
    main()
