"""One verify step through the five C-ABI calls, with its device buffers.

``VerifyStep`` owns the buffers of a workload on the GPU (torch allocates
them; the HIP library computes everything) and runs

    rv_schedule -> rv_pack -> [payload staging] -> rv_verify_attn
    -> rv_lm_head_accept -> rv_compact_scatter

Payload staging gathers the block-major query / hidden-state payloads into
the packed row order.  In a serving stack the target model's layers produce
packed rows directly; here it stands in for them and is kept outside the
five-stage timing.  ``restore()`` resets the state the scatter mutates (ctx,
anchor, req_to_token, history) so repeated steps see identical inputs.
"""

import torch

from . import rv, synth


class VerifyStep:
    def __init__(self, inp, mode="compact", with_logits=False, rows_cap=None, r2t_extra=64,
                 hist_cap=64, stream=None, w_layout="tiled", window=0, topk=0, fused_plan=True):
        wl = inp["workload"]
        self.inp, self.wl = inp, wl
        # the stages' C-ABI argument structs, rebuilt only when an input
        # tensor is replaced (the step's own buffers never are)
        self._abi = rv.ArgCache()
        self.mode = mode
        # fused_plan: the pack launch also builds the attention call's plan
        # (rv_pack_plan); an attention call right after such a pack skips its
        # own plan launch (rv_verify_attn_planned).  The plan is single use:
        # the attention kernels advance its work counters, and the LM head's
        # scratch shares the workspace.
        self.fused_plan = fused_plan
        self._plan_ready = False
        dev = inp["conf"].device
        if dev.type != "cuda":
            raise ValueError("VerifyStep needs inputs on the GPU")
        B, gamma = inp["B"], inp["gamma"]
        self.B, self.gamma = B, gamma
        tiers = list(inp["tiers"])
        self.tiers = tuple(tiers)   # immutable: the argument cache compares it by identity
        self.rows_cap = rows_cap or max([B * gamma] + tiers)
        i32 = dict(dtype=torch.int32, device=dev)
        R = self.rows_cap
        self.rule = rv.RV_REJECTION if wl.rule == "rejection" else rv.RV_GREEDY
        self.dtype = torch.float32 if wl.dtype == "f32" else torch.bfloat16

        # stage 1
        self.w_commit = torch.zeros(B, **i32)
        self.w_verify = torch.zeros(B, **i32)
        self.k_star = torch.zeros(1, **i32)
        self.e_star = torch.zeros(1, dtype=torch.float64, device=dev)
        # stage 2
        self.cu = torch.zeros(B + 1, **i32)
        self.mm = torch.zeros(2, **i32)
        self.row_req = torch.full((R,), -1, **i32)
        self.row_pos = torch.full((R,), -1, **i32)
        self.tok = torch.full((R,), -1, **i32)
        self.slot = torch.full((R,), -1, **i32)
        # stage 3
        self.q = torch.zeros((R, wl.Hq, wl.Dqk), dtype=self.dtype, device=dev)
        self.o = torch.zeros((R, wl.Hq, wl.Dv), dtype=self.dtype, device=dev)
        self.lse = torch.zeros((R, wl.Hq), dtype=torch.float32, device=dev)
        # stage 4
        self.hidden = torch.zeros((R, wl.H), dtype=self.dtype, device=dev)
        self.pred = torch.zeros(R, **i32)
        self.accept = torch.zeros(B, **i32)
        self.bonus = torch.zeros(B, **i32)
        self.ceiling = torch.zeros(B, **i32)
        need_logits = with_logits or self.rule == rv.RV_REJECTION
        self.logits = torch.zeros((R, wl.V), dtype=torch.float32, device=dev) if need_logits else None
        # stage 5 state (mutated in place) and its pristine copies
        self.ctx0 = inp["ctx"].clone()
        self.anchor0 = inp["anchor"].clone()
        self.ctx = self.ctx0.clone()
        self.anchor = self.anchor0.clone()
        r2t_len = int(self.ctx0.max()) + gamma + r2t_extra
        self.req_to_token0 = torch.full((B, r2t_len), -1, **i32)
        self.req_to_token = self.req_to_token0.clone()
        self.hist0 = torch.full((B, hist_cap), -1, **i32)
        self.hist_len0 = torch.zeros(B, **i32)
        self.hist = self.hist0.clone()
        self.hist_len = self.hist_len0.clone()
        self.commit_cu = torch.zeros(B + 1, **i32)
        self.commit_tok = torch.zeros(B * gamma, **i32)
        self.commit_slot = torch.zeros(B * gamma, **i32)
        self.free_slots = torch.zeros(B * gamma, **i32)
        self.free_count = torch.zeros(1, **i32)

        ws = rv.rv_workspace_size(B, gamma, wl.Hq, wl.Hkv, wl.Dqk, wl.Dv, wl.V,
                                  rv.RV_F32 if wl.dtype == "f32" else rv.RV_BF16)
        self.workspace = torch.zeros(ws, dtype=torch.uint8, device=dev)
        self.q_flat = inp["q_block"].reshape(B * gamma, wl.Hq, wl.Dqk)
        self.h_flat = inp["hidden_block"].reshape(B * gamma, wl.H)
        self.stream = stream
        self.window = window   # sliding-window attention (keys), 0 = full causal
        # sparse latent attention: block-major key lists (inp["topk_block"],
        # [B, gamma, topk]) gathered into packed order with the payload
        self.topk_idx = None
        if topk:
            if inp.get("topk_block") is None or inp["topk_block"].shape[2] != topk:
                inp["topk_block"] = synth.topk_indices(inp["ctx"], gamma, topk, inp["workload"].seed + 77,
                                                       device=dev)
            self.topk_flat = inp["topk_block"].reshape(B * gamma, topk)
            self.topk_idx = torch.full((R, topk), -1, **i32)
        # LM-head weight in MFMA fragment order, made once per weight (a
        # serving system does this when it loads the model); bf16 with
        # H % 128 == 0 only, otherwise the row-major weight is read
        self.W_tiled = None
        if w_layout == "tiled" and self.dtype == torch.bfloat16 and wl.H % 128 == 0:
            if inp.get("W_tiled") is None:
                inp["W_tiled"] = rv.rv_lm_tile_weight(inp["W"], stream=stream)
            self.W_tiled = inp["W_tiled"]

    # ---- stages ------------------------------------------------------------------
    def schedule(self):
        self._plan_ready = False   # this stage may write the workspace
        i = self.inp
        rv.rv_schedule(i["conf"], self.gamma, self.mode, i["cost_bias"], i["cost_alpha"], i["cost_theta"],
                       self.w_commit, self.w_verify, self.k_star, self.e_star, self.workspace, self.stream,
                       cache=self._abi)

    def _pack_kw(self):
        i = self.inp
        return dict(w_verify=self.w_verify, anchor=self.anchor, drafts=i["drafts"], ctx=self.ctx,
                    page_table=i["page_table"], page_size=i["page_size"], num_pages=i["num_pages"],
                    tiers=self.tiers, cu=self.cu, mm=self.mm, row_req=self.row_req, row_pos=self.row_pos,
                    tok=self.tok, slot=self.slot, workspace=self.workspace)

    def _attn_kw(self):
        i = self.inp
        return dict(q=self.q, k_cache=i["k_cache"], v_cache=i["v_cache"], page_table=i["page_table"],
                    page_size=i["page_size"], num_pages=i["num_pages"], ctx=self.ctx, cu=self.cu, mm=self.mm,
                    gamma=self.gamma, sm_scale=i["sm_scale"], o=self.o, lse=self.lse, workspace=self.workspace,
                    window=self.window, topk_idx=self.topk_idx)

    def pack(self):
        if self.fused_plan:
            rv.rv_pack_plan(self._pack_kw(), self._attn_kw(), self.stream, cache=self._abi)
            self._plan_ready = True
        else:
            rv.rv_pack(**self._pack_kw(), stream=self.stream)

    def stage_payload(self):
        """Gather block-major payload rows into packed order (harness work)."""
        req = self.row_req.long()
        valid = req >= 0
        k = self.row_pos.long() - self.ctx[req.clamp(min=0)].long()
        src = torch.where(valid, req.clamp(min=0) * self.gamma + k.clamp(0, self.gamma - 1),
                          torch.zeros_like(req))
        torch.index_select(self.q_flat, 0, src, out=self.q)
        torch.index_select(self.h_flat, 0, src, out=self.hidden)
        if self.topk_idx is not None:
            torch.index_select(self.topk_flat, 0, src, out=self.topk_idx)

    def attn(self):
        if self._plan_ready:
            rv.rv_verify_attn_planned(**self._attn_kw(), stream=self.stream, cache=self._abi)
        else:
            rv.rv_verify_attn(**self._attn_kw(), stream=self.stream, cache=self._abi)
        self._plan_ready = False

    def lm(self):
        self._plan_ready = False   # this stage may write the workspace
        i = self.inp
        rv.rv_lm_head_accept(self.hidden, i["W"], self.mm, self.cu, self.w_commit, self.w_verify, i["drafts"],
                             self.rule, self.pred, self.accept, self.bonus, self.ceiling, self.workspace,
                             logits=self.logits, q_rows=i.get("q_rows"), u=i.get("u"), u_bonus=i.get("u_bonus"),
                             stream=self.stream, W_tiled=self.W_tiled, cache=self._abi)

    def scatter(self):
        self._plan_ready = False   # this stage may write the workspace
        i = self.inp
        rv.rv_compact_scatter(self.cu, self.w_verify, self.accept, self.bonus, i["drafts"], self.slot, self.ctx,
                              self.anchor, self.req_to_token, self.commit_cu, self.commit_tok, self.commit_slot,
                              self.free_slots, self.free_count, self.workspace, hist=self.hist,
                              hist_len=self.hist_len, stream=self.stream, cache=self._abi)

    def prime(self):
        """Build (and cache) the five stages' argument structs for the
        current inputs without launching anything."""
        i = self.inp
        rv.rv_schedule(i["conf"], self.gamma, self.mode, i["cost_bias"], i["cost_alpha"], i["cost_theta"],
                       self.w_commit, self.w_verify, self.k_star, self.e_star, self.workspace, self.stream,
                       cache=self._abi, launch=False)
        if self.fused_plan:
            rv.rv_pack_plan(self._pack_kw(), self._attn_kw(), self.stream, cache=self._abi, launch=False)
        rv.rv_verify_attn(**self._attn_kw(), stream=self.stream, cache=self._abi, launch=False)
        rv.rv_lm_head_accept(self.hidden, i["W"], self.mm, self.cu, self.w_commit, self.w_verify, i["drafts"],
                             self.rule, self.pred, self.accept, self.bonus, self.ceiling, self.workspace,
                             logits=self.logits, q_rows=i.get("q_rows"), u=i.get("u"), u_bonus=i.get("u_bonus"),
                             stream=self.stream, W_tiled=self.W_tiled, cache=self._abi, launch=False)
        rv.rv_compact_scatter(self.cu, self.w_verify, self.accept, self.bonus, i["drafts"], self.slot, self.ctx,
                              self.anchor, self.req_to_token, self.commit_cu, self.commit_tok, self.commit_slot,
                              self.free_slots, self.free_count, self.workspace, hist=self.hist,
                              hist_len=self.hist_len, stream=self.stream, cache=self._abi, launch=False)

    def restore(self):
        self.ctx.copy_(self.ctx0)
        self.anchor.copy_(self.anchor0)
        self.req_to_token.copy_(self.req_to_token0)
        self.hist.copy_(self.hist0)
        self.hist_len.copy_(self.hist_len0)

    def run(self):
        """All five stages plus staging, in order, on the current stream."""
        self.schedule()
        self.pack()
        self.stage_payload()
        self.attn()
        self.lm()
        self.scatter()

    # ---- observability -----------------------------------------------------------
    def calibration(self, n_bins=10):
        self._plan_ready = False   # this stage may write the workspace
        """Confidence calibration of this step's verified drafts (rv_calibration,
        after lm()): returns the device tensors (bin_count, bin_match,
        bin_conf_fx, ece, req_verified, req_matched)."""
        dev = self.w_verify.device
        if getattr(self, "_calib_bins", None) != n_bins:
            i64 = dict(dtype=torch.int64, device=dev)
            self.calib = dict(bin_count=torch.zeros(n_bins, **i64), bin_match=torch.zeros(n_bins, **i64),
                              bin_conf_fx=torch.zeros(n_bins, **i64),
                              ece=torch.zeros(1, dtype=torch.float64, device=dev),
                              req_verified=torch.zeros(self.B, dtype=torch.int32, device=dev),
                              req_matched=torch.zeros(self.B, dtype=torch.int32, device=dev))
            self._calib_bins = n_bins
        c = self.calib
        rv.rv_calibration(self.inp["conf"], self.inp["drafts"], self.pred, self.cu, self.w_verify, n_bins,
                          c["bin_count"], c["bin_match"], c["bin_conf_fx"], c["ece"], self.workspace,
                          req_verified=c["req_verified"], req_matched=c["req_matched"], stream=self.stream)
        return c

    def block_accept_estimate(self, state):
        self._plan_ready = False   # this stage may write the workspace
        """One step of the block-accept estimator (rv_block_accept_estimate),
        between lm() and scatter(): ``state`` is a zero-filled uint8 tensor of
        rv.rv_estimator_state_bytes(B, gamma) bytes kept across steps."""
        i = self.inp
        rv.rv_block_accept_estimate(self.cu, self.w_verify, self.accept, i["drafts"], self.ctx, self.rule, state,
                                    self.workspace, pred=self.pred if self.rule == rv.RV_GREEDY else None,
                                    logits=self.logits, q_rows=i.get("q_rows"), stream=self.stream)

    # ---- HIP graphs ------------------------------------------------------------
    def capture(self):
        """Record the step into two HIP graphs on a side stream: ``front``
        (schedule, pack) and ``back`` (verify attention, LM head + accept,
        compact scatter); the staging gather stays outside them (harness
        work).  One pair of graphs serves every capture tier: the kernels
        read the packed counts (M, M_pad) on the device and size their grids
        by host-known capacities, so nothing in a launch depends on the tier.
        Replays see the device buffers as they are at replay time; the mutated
        state (ctx, anchors, req_to_token, history) is restored outside."""
        if self.stream is not None:
            raise ValueError("capture records on torch's current stream; build the step without stream=")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):   # warm-up outside capture: sets kernel attributes once
            self.restore()
            self.run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.restore()
        torch.cuda.synchronize()
        self.g_front = torch.cuda.CUDAGraph()
        self.g_back = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g_front, capture_error_mode="thread_local"):
            self.schedule()
            self.pack()
        with torch.cuda.graph(self.g_back, capture_error_mode="thread_local"):
            self.attn()
            self.lm()
            self.scatter()
        torch.cuda.synchronize()

    def replay(self):
        """One step from the captured graphs (capture() first)."""
        self.g_front.replay()
        self.stage_payload()
        self.g_back.replay()

    def status(self):
        return rv.rv_device_status(self.workspace, self.stream)


class OverlapLoop:
    """A multi-step verify loop that hides the scheduler behind the forward
    pass (DSpark-in-SGLang page, §A2 "zero-overhead scheduling" and Fig. 5:
    the next step's scheduling overlaps the current forward pass on its own
    stream, cross-iteration order comes from device-side barriers, and no
    step synchronises with the host).

    Step s runs pack, payload staging, verify attention, LM head + accept
    and compact scatter on the current stream.  With ``overlap`` the
    schedule of step s+1 runs on a side stream of the same priority,
    enqueued after step s's attention so that it overlaps attention and LM
    head.  Device events order the two streams: pack(s+1) waits for
    schedule(s+1), and schedule(s+1) waits until step s-1, which used the
    same one of the two window buffers, has finished with it.  Without
    ``overlap`` the same work runs in order on one stream.

    Confidence relay: because schedule(s+1) runs while step s is still in
    flight, it cannot wait for confidences produced alongside step s; step s
    is scheduled on the confidences of step s-2 (step 0 and 1 on step 0's),
    the pages' two-step-back relay.  ``steps`` is a list of per-step inputs
    (``conf``, ``drafts``, ``hidden_block`` on the GPU, shaped as
    ``make_inputs`` returns them); everything else comes from ``inp``.
    """

    def __init__(self, inp, steps, mode="compact", overlap=True, **kw):
        self.vs = VerifyStep(inp, mode=mode, **kw)
        self.inp, self.steps, self.mode, self.overlap = inp, steps, mode, overlap
        vs = self.vs
        dev = vs.w_verify.device
        i32 = dict(dtype=torch.int32, device=dev)
        self.win = [(torch.zeros(vs.B, **i32), torch.zeros(vs.B, **i32), torch.zeros(1, **i32),
                     torch.zeros(1, dtype=torch.float64, device=dev)) for _ in range(2)]
        # the side stream's schedule keeps its status word apart
        self.ws_side = torch.zeros(rv.rv_workspace_size(vs.B, vs.gamma), dtype=torch.uint8, device=dev)
        self.side = torch.cuda.Stream()

    def relay_conf(self, s):
        return self.steps[max(s - 2, 0)]["conf"]

    def _schedule(self, s, stream):
        i, vs = self.inp, self.vs
        wc, wv, ks, es = self.win[s % 2]
        rv.rv_schedule(self.relay_conf(s), vs.gamma, self.mode, i["cost_bias"], i["cost_alpha"], i["cost_theta"],
                       wc, wv, ks, es, self.ws_side, stream)

    def _step_rest(self, s, after_attn=None):
        """Pack .. scatter of step s on the current stream; ``after_attn``
        runs between attention and the LM head (where the next schedule is
        enqueued)."""
        i, vs = self.inp, self.vs
        st = self.steps[s]
        wc, wv, _, _ = self.win[s % 2]
        drafts = st["drafts"]
        rv.rv_pack(wv, vs.anchor, drafts, vs.ctx, i["page_table"], i["page_size"], i["num_pages"], vs.tiers,
                   vs.cu, vs.mm, vs.row_req, vs.row_pos, vs.tok, vs.slot, vs.workspace)
        req = vs.row_req.long()
        k = vs.row_pos.long() - vs.ctx[req.clamp(min=0)].long()
        src = torch.where(req >= 0, req.clamp(min=0) * vs.gamma + k.clamp(0, vs.gamma - 1), torch.zeros_like(req))
        torch.index_select(vs.q_flat, 0, src, out=vs.q)
        torch.index_select(st["hidden_block"].reshape(vs.B * vs.gamma, -1), 0, src, out=vs.hidden)
        rv.rv_verify_attn(vs.q, i["k_cache"], i["v_cache"], i["page_table"], i["page_size"], i["num_pages"], vs.ctx,
                          vs.cu, vs.mm, vs.gamma, i["sm_scale"], vs.o, vs.lse, vs.workspace)
        if after_attn is not None:
            after_attn()
        rv.rv_lm_head_accept(vs.hidden, i["W"], vs.mm, vs.cu, wc, wv, drafts, vs.rule, vs.pred, vs.accept, vs.bonus,
                             vs.ceiling, vs.workspace, logits=vs.logits, q_rows=i.get("q_rows"), u=i.get("u"),
                             u_bonus=i.get("u_bonus"), W_tiled=vs.W_tiled)
        rv.rv_compact_scatter(vs.cu, wv, vs.accept, vs.bonus, drafts, vs.slot, vs.ctx, vs.anchor, vs.req_to_token,
                              vs.commit_cu, vs.commit_tok, vs.commit_slot, vs.free_slots, vs.free_count,
                              vs.workspace, hist=vs.hist, hist_len=vs.hist_len)

    def run(self, n=None, after_step=None):
        """Run steps 0..n-1 (default: all); ``after_step(s)`` is called after
        step s is enqueued on the current stream (before its window buffer can
        be reused), e.g. to copy outputs."""
        n = len(self.steps) if n is None else n
        main = torch.cuda.current_stream()
        if not self.overlap:
            for s in range(n):
                self._schedule(s, main)
                self._step_rest(s)
                if after_step is not None:
                    after_step(s)
            return
        e_sched = [torch.cuda.Event() for _ in range(n)]
        e_done = [torch.cuda.Event() for _ in range(n)]
        self.side.wait_stream(main)            # the inputs are resident before anything reads them
        self._schedule(0, self.side)
        e_sched[0].record(self.side)
        for s in range(n):
            main.wait_event(e_sched[s])

            def next_schedule(s=s):
                if s + 1 < n:
                    if s >= 1:
                        self.side.wait_event(e_done[s - 1])   # step s-1 is done with this window buffer
                    self._schedule(s + 1, self.side)
                    e_sched[s + 1].record(self.side)

            self._step_rest(s, after_attn=next_schedule)
            if after_step is not None:
                after_step(s)
            e_done[s].record(main)
        main.wait_stream(self.side)

    def capture(self, n=None):
        """Record steps 0..n-1 (both streams, their event edges included) into
        one HIP graph; ``replay()`` then runs them with no host work between
        launches.  The mutated state is restored before capture and must be
        restored (``self.vs.restore()``) before each replay."""
        n = len(self.steps) if n is None else n
        warm = torch.cuda.Stream()
        warm.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(warm):   # warm-up outside capture: sets kernel attributes once
            self.run(n=min(n, 2))
        torch.cuda.current_stream().wait_stream(warm)
        torch.cuda.synchronize()
        self.vs.restore()
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, capture_error_mode="thread_local"):
            self.run(n=n)
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()

    def window(self, s):
        """The window buffers step s used (valid until step s+2 is scheduled)."""
        return self.win[s % 2]

    def status(self):
        return rv.rv_device_status(self.vs.workspace) or rv.rv_device_status(self.ws_side)
