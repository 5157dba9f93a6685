"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer outputs (windows, K*, E*, cu_seqlens, tiers, row metadata, argmax,
accept lengths, bonus tokens, scatter indices) must match bit for bit;
attention output within 2e-2 max-abs (bf16) / 1e-4 (fp32), LM-head logits
within 1e-2 relative to the row's largest logit (bf16) / 1e-5 (fp32).
Reduced-size cases compare every element; full-size cases run the bench's
launch configuration and compare sampled rows plus properties that hold at
any size.
"""

import numpy as np
import pytest
import torch

import oracle
import parity_util as pu
from ragged_verification_amd import rv
from ragged_verification_amd.pipeline import VerifyStep

pytestmark = pytest.mark.gpu


def _oracle_full(inp, ref, mode, window=0, topk=0):
    """Oracle stages 3-5 on every real row (small cases only)."""
    wl = inp["workload"]
    gamma = inp["gamma"]
    M = ref["M"]
    bidx = pu.packed_block_index(ref, gamma)
    q = pu.np64(inp["q_block"].reshape(-1, wl.Hq, wl.Dqk))[bidx]
    o, lse = oracle.verify_attention(q, pu.np64(inp["k_cache"]), pu.np64(inp["v_cache"]),
                                     pu.npi(inp["page_table"]), inp["page_size"], ref["row_req"],
                                     ref["row_pos"], ref["M_pad"], inp["sm_scale"], Dv=wl.Dv, window=window,
                                     topk_idx=pu.npi(inp["topk_block"].reshape(-1, topk))[bidx] if topk else None)
    x = pu.np64(inp["hidden_block"].reshape(-1, wl.H))[bidx]
    z = oracle.lm_head_logits(x, pu.np64(inp["W"]))
    pred = oracle.lm_head_pred(z)
    drafts = pu.npi(inp["drafts"])
    diag = {}
    if wl.rule == "greedy":
        acc, bonus, ceil = oracle.accept_greedy(pred, ref["cu"], ref["w_commit"], ref["w_verify"], drafts)
    else:
        acc, bonus, ceil = oracle.accept_rejection(z, ref["cu"], ref["w_commit"], ref["w_verify"], drafts,
                                                   pu.np64(inp["q_rows"]), pu.np64(inp["u"]),
                                                   pu.np64(inp["u_bonus"]), diag=diag)
    B = inp["B"]
    r2t = np.full((B, int(pu.npi(inp["ctx"]).max()) + gamma + 64), -1)
    hist = np.full((B, 64), -1)
    sc = oracle.compact_scatter(ref["cu"], ref["w_verify"], acc, bonus, drafts, ref["slot"], pu.npi(inp["ctx"]),
                                pu.npi(inp["anchor"]), r2t, hist, np.zeros(B, dtype=np.int64))
    return dict(o=o, lse=lse, z=z, pred=pred, accept=acc, bonus=bonus, ceiling=ceil, scatter=sc, diag=diag)


def _full_parity(inp, mode, dtype, w_layout="tiled", window=0, topk=0):
    pu.log(f"case {inp['workload'].name} B={inp['B']} mode={mode} weight={w_layout} window={window} topk={topk}")
    ref = pu.oracle_schedule_pack(inp, mode)
    step = pu.run_gpu(inp, mode, with_logits=True, w_layout=w_layout, window=window, topk=topk)
    assert step.status() == 0
    pu.check_schedule_pack(step, ref)
    want = _oracle_full(inp, ref, mode, window=window, topk=topk)
    M, M_pad = ref["M"], ref["M_pad"]
    o = step.o.float().cpu().numpy()
    err = np.max(np.abs(o[:M] - want["o"][:M]))
    assert err <= pu.ATTN_TOL[dtype], err
    assert np.all(o[M:M_pad] == 0)
    lse = step.lse.cpu().numpy()
    np.testing.assert_allclose(lse[:M], want["lse"][:M], rtol=1e-3, atol=1e-3)
    z = step.logits.cpu().numpy()[:M]
    rel = np.max(np.abs(z - want["z"]), axis=1) / np.max(np.abs(want["z"]), axis=1)
    assert np.all(rel <= pu.LOGIT_TOL[dtype]), rel.max()
    pu.check_pred_gap(want["z"]) if inp["workload"].rule == "greedy" else None
    pred = pu.npi(step.pred)
    if inp["workload"].rule == "greedy":
        assert np.array_equal(pred[:M], want["pred"])
    assert np.all(pred[M:M_pad] == -1)
    assert np.array_equal(pu.npi(step.accept), want["accept"])
    assert np.array_equal(pu.npi(step.ceiling), want["ceiling"])
    if inp["workload"].rule == "greedy":
        assert np.array_equal(pu.npi(step.bonus), want["bonus"])
        pu.check_scatter(step, want["scatter"], inp["B"])
    else:
        for m in want["diag"]["decision_margin"]:
            assert all(x >= 1e-4 for x in m), "accept decision too close to call"
        moved = pu.check_bonus(pu.npi(step.bonus), want["bonus"], want["diag"])
        pu.check_scatter(step, want["scatter"], inp["B"], moved)
    pu.log(f"ok attn max err {err:.3g}, logits rel {rel.max():.3g}, M={M}, M_pad={M_pad}")
    return step, ref, want


@pytest.mark.parametrize("mode", ["static", "compact", "cap_accept"])
def test_tiny_f32(mode):
    inp = pu.make_inputs("tiny_f32")
    _full_parity(inp, mode, "f32")


@pytest.mark.parametrize("mode", ["compact", "static"])
def test_gqa_reduced(mode):
    inp = pu.make_inputs("gqa_bf16", B=6, V=1000, H=256, ctx=("uniform", 40, 900))
    _full_parity(inp, mode, "bf16")


@pytest.mark.parametrize("mode", ["compact", "static"])
def test_mla_reduced(mode):
    inp = pu.make_inputs("mla_bf16", B=3, V=1000, H=512, ctx=("uniform", 60, 700))
    _full_parity(inp, mode, "bf16")


@pytest.mark.parametrize("mode", ["compact", "cap_accept"])
def test_rejection_reduced(mode):
    inp = pu.make_inputs("rejection_bf16", B=6, V=3000, H=256, ctx=("lognormal", 200, 1.0, 600))
    _full_parity(inp, mode, "bf16")


def test_rejection_odd_vocab():
    """A vocabulary that is neither a multiple of 4 nor of 64: the logits
    rows are not 16-byte aligned (scalar stores in the GEMM epilogue, scalar
    loads in the bonus draw) and the last slab and segment are partial."""
    inp = pu.make_inputs("rejection_bf16", B=5, V=4229, H=128, ctx=("lognormal", 150, 1.0, 500))
    _full_parity(inp, "compact", "bf16")


def test_lm_row_major_weight():
    """The LM head reading W [V][H] row-major (w_layout RV_W_ROWS) instead of
    its tiled copy; V = 4229 leaves a partial last slab."""
    inp = pu.make_inputs("rejection_bf16", B=5, V=4229, H=256, ctx=("lognormal", 150, 1.0, 500))
    _full_parity(inp, "compact", "bf16", w_layout="rows")
    inp = pu.make_inputs("mla_bf16", B=3, V=1000, H=512, ctx=("uniform", 60, 700))
    _full_parity(inp, "static", "bf16", w_layout="rows")


@pytest.mark.parametrize("window", [1, 37, 200])
def test_sliding_window_latent(window):
    """Sliding-window attention on the latent kernel: windows inside the
    first tile of a chunk, across chunks, and one key (W = 1)."""
    inp = pu.make_inputs("mla_bf16", B=3, V=1000, H=512, ctx=("uniform", 60, 700))
    _full_parity(inp, "compact", "bf16", window=window)


@pytest.mark.parametrize("window", [1, 64, 100])
def test_sliding_window_gqa(window):
    """GQA balanced schedule with a sliding window (64: super-tile aligned)."""
    inp = pu.make_inputs("gqa_bf16", B=6, V=1000, H=256, ctx=("uniform", 40, 900))
    _full_parity(inp, "static", "bf16", window=window)


def test_sliding_window_split_and_chunked():
    """A window on long split requests (partials of ranges that lie wholly
    below some rows' windows merge as empty), on the chunked GQA plan, on
    pages that are not a power of two (per-row DMA addressing) and on the
    fp32 kernel."""
    inp = pu.make_inputs("gqa_bf16", B=2, Hq=64, V=700, H=128, ctx=("uniform", 2500, 3000))
    _full_parity(inp, "compact", "bf16", window=700)
    inp = pu.make_inputs("gqa_bf16", B=130, Hq=64, Hkv=64, V=200, H=64, tiers=(1024,), ctx=("uniform", 0, 60))
    _full_parity(inp, "compact", "bf16", window=17)
    inp = pu.make_inputs("mla_bf16", B=2, Hq=64, V=500, H=256, ctx=("uniform", 3000, 5000))
    _full_parity(inp, "compact", "bf16", window=1500)
    inp = pu.make_inputs("mla_bf16", B=3, V=500, H=256, page_size=48, ctx=("uniform", 100, 600))
    _full_parity(inp, "static", "bf16", window=130)
    inp = pu.make_inputs("gqa_bf16", B=4, V=500, H=256, page_size=12, ctx=("uniform", 100, 600))
    _full_parity(inp, "static", "bf16", window=77)
    inp = pu.make_inputs("tiny_f32")
    _full_parity(inp, "static", "f32", window=3)


@pytest.mark.parametrize("topk", [1, 64, 300])
def test_sparse_latent(topk):
    """Sparse latent attention over per-row key lists (ascending positions
    drawn from 0..p, -1 padded where p + 1 < topk)."""
    inp = pu.make_inputs("mla_bf16", B=3, V=1000, H=512, ctx=("uniform", 60, 700))
    _full_parity(inp, "compact", "bf16", topk=topk)


def test_sparse_latent_split_and_empty_rows():
    """2048-entry lists over long contexts (chunks split and merged); then
    lists whose entries all lie past their rows (nothing visible: o = 0 and
    lse = -inf, also through the split merge)."""
    inp = pu.make_inputs("mla_bf16", B=2, Hq=64, V=500, H=256, ctx=("uniform", 3000, 5000))
    _full_parity(inp, "static", "bf16", topk=2048)
    inp = pu.make_inputs("mla_bf16", B=2, Hq=64, V=500, H=256, ctx=("uniform", 100, 300))
    blk = torch.full((2, inp["gamma"], 600), 10**6, dtype=torch.int32, device="cuda")
    blk[0, 0, 5] = 3   # one visible key for one row
    inp["topk_block"] = blk
    step, ref, want = _full_parity(inp, "static", "bf16", topk=600)
    M = ref["M"]
    o = step.o.float().cpu().numpy()
    assert np.all(o[1:M] == 0) and np.all(np.isneginf(step.lse.cpu().numpy()[1:M]))


def test_sparse_latent_row_kernel_lists():
    """128 heads (the one-workgroup-per-row kernel): 2048-entry lists over
    long contexts (the list split into chunks and merged), with -1 entries,
    positions past the row and repeated positions scattered through each list
    (the kernel compacts the visible entries of its chunk in list order; a
    repeat counts once per entry); then lists with nothing visible."""
    inp = pu.make_inputs("mla_bf16", B=2, V=500, H=256, ctx=("uniform", 3000, 5000))
    g = torch.Generator().manual_seed(7)
    gamma, K = inp["gamma"], 2048
    ctx = inp["ctx"].cpu()
    blk = torch.empty((2, gamma, K), dtype=torch.int32)
    for b in range(2):
        for k in range(gamma):
            p_ = int(ctx[b]) + k
            lst = torch.randint(0, p_ + 1, (K,), generator=g, dtype=torch.int32)
            u = torch.rand(K, generator=g)
            lst[u < 0.1] = -1                                   # pads inside the list
            lst[(u >= 0.1) & (u < 0.2)] = p_ + 1 + (lst[(u >= 0.1) & (u < 0.2)] % 50)   # past the row
            lst[1::97] = lst[0::97][: lst[1::97].numel()]       # repeats
            blk[b, k] = lst
    inp["topk_block"] = blk.to("cuda")
    _full_parity(inp, "static", "bf16", topk=K)
    _full_parity(inp, "compact", "bf16", topk=K)
    inp = pu.make_inputs("mla_bf16", B=2, V=500, H=256, ctx=("uniform", 100, 300))
    blk = torch.full((2, inp["gamma"], 600), 10**6, dtype=torch.int32, device="cuda")
    blk[0, 0, 5] = 3   # one visible key for one row
    inp["topk_block"] = blk
    step, ref, want = _full_parity(inp, "static", "bf16", topk=600)
    M = ref["M"]
    o = step.o.float().cpu().numpy()
    assert np.all(o[1:M] == 0) and np.all(np.isneginf(step.lse.cpu().numpy()[1:M]))


@pytest.mark.parametrize("B", [1, 4])
def test_lm_few_rows_odd_vocab(B):
    """At most 32 packed rows take the one-wave weight-streaming kernel; with
    V = 4229 its last tile's second column block lies past the tiled
    weight's end (read as zeros, masked)."""
    inp = pu.make_inputs("mla_bf16", B=B, V=4229, H=256, ctx=("uniform", 60, 300))
    _full_parity(inp, "static", "bf16")


@pytest.mark.parametrize("H", [128, 256])
@pytest.mark.parametrize("B,V", [(3, 900), (6, 900), (11, 900), (17, 900), (32, 900), (50, 40000)])
def test_lm_row_blocks_of_last_tile(B, V, H):
    """Static windows of 8 give 8*B packed rows.  With H = 128 the 128-row
    tiled kernel runs for every count: 24, 48 and 88 rows use one, two and
    four 32-row blocks of their single row tile; 136 and 256 rows over four
    vocabulary tiles run in one round, so both row tiles compute all four
    blocks; 400 rows over 79 tiles of 512 columns take two rounds, so the
    last tile's 16 rows compute one block.  With H = 256, 24 rows take the
    one-wave kernel, 48, 88 and 136 rows the all-rows kernel (two, three
    and five 32-row blocks; 900 columns end inside its last 128-column
    tile), and 256 rows that kernel's two-tile branch.  Every row's logits
    are compared."""
    inp = pu.make_inputs("gqa_bf16", B=B, V=V, H=H, tiers=(), ctx=("uniform", 10, 60))
    _full_parity(inp, "static", "bf16")


def test_tiled_weight_layout():
    """rv_lm_tile_weight against the layout written out with torch view
    operations: lane l of fragment f of block cb holds
    W[32*cb + l%32][16*f + 8*(l//32) .. +7]; rows past V are zero."""
    from ragged_verification_amd import rv
    g = torch.Generator().manual_seed(7)
    for V, H in ((1000, 256), (4229, 128), (64, 384)):
        W = torch.randn(V, H, generator=g).to(torch.bfloat16)
        t = rv.rv_lm_tile_weight(W.cuda())
        torch.cuda.synchronize()
        Vp = (V + 31) // 32 * 32
        Wp = torch.zeros(Vp, H, dtype=torch.bfloat16)
        Wp[:V] = W
        want = Wp.view(Vp // 32, 32, H // 16, 2, 8).permute(0, 2, 3, 1, 4).contiguous()
        got = t.cpu().view(torch.bfloat16).view(Vp // 32, H // 16, 2, 32, 8)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (V, H)


def test_gqa_many_tiles_chunked_plan():
    """One query head per KV head and 64 KV heads: 64 tiles per request, so
    130 requests need more partial slots than the balanced GQA schedule may
    claim (workers + tiles > 8192) and the chunked item plan runs instead."""
    inp = pu.make_inputs("gqa_bf16", B=130, Hq=64, Hkv=64, V=200, H=64, tiers=(1024,),
                         ctx=("uniform", 0, 60))
    _full_parity(inp, "compact", "bf16")


def test_gqa_group8_and_split_kv():
    """Eight query heads per KV head (64 query vectors per tile) and one long
    request so the key range is split and merged."""
    inp = pu.make_inputs("gqa_bf16", B=2, Hq=64, V=700, H=128, ctx=("uniform", 2500, 3000))
    _full_parity(inp, "compact", "bf16")


def test_sweep_classes_cap_accept_equals_compact():
    inp = pu.make_inputs("sweep_gqa", B=24, V=800, H=128, ctx=("uniform", 30, 300))
    s_c, ref_c, want_c = _full_parity(inp, "compact", "bf16")
    c_tok = pu.npi(s_c.commit_tok).copy()
    c_cu = pu.npi(s_c.commit_cu).copy()
    c_slot = pu.npi(s_c.commit_slot).copy()
    s_a, ref_a, want_a = _full_parity(inp, "cap_accept", "bf16")
    assert np.array_equal(pu.npi(s_a.commit_cu), c_cu)
    n = int(c_cu[-1])
    assert np.array_equal(pu.npi(s_a.commit_tok)[:n], c_tok[:n])
    assert np.array_equal(pu.npi(s_a.commit_slot)[:n], c_slot[:n])
    assert np.all(pu.npi(s_a.ceiling) >= pu.npi(s_a.accept))


def test_static_rows_equal_compact_rows():
    """By causality a compact row equals the static row of the same block
    position (attention output and prediction)."""
    inp = pu.make_inputs("mla_bf16", B=4, V=600, H=256, ctx=("uniform", 100, 400))
    st = pu.run_gpu(inp, "static")
    so, sp = st.o.float().cpu().numpy(), pu.npi(st.pred)
    co_step = pu.run_gpu(inp, "compact")
    co, cp = co_step.o.float().cpu().numpy(), pu.npi(co_step.pred)
    cu = pu.npi(co_step.cu)
    g = inp["gamma"]
    for i in range(inp["B"]):
        for k in range(cu[i + 1] - cu[i]):
            assert np.max(np.abs(co[cu[i] + k] - so[i * g + k])) <= 2e-2
            assert cp[cu[i] + k] == sp[i * g + k]


def test_edge_cases():
    """One request, anchor-only windows (huge theta), zero context (the only
    visible key is the anchor's own), block width 2."""
    inp = pu.make_inputs("tiny_f32", B=1, gamma=2, ctx=("uniform", 0, 0))
    _full_parity(inp, "compact", "f32")
    inp = pu.make_inputs("gqa_bf16", B=3, V=300, H=64, ctx=("uniform", 0, 5))
    inp["cost_theta"] = inp["cost_theta"] * 1e6
    step, ref, _ = _full_parity(inp, "compact", "bf16")
    assert np.all(pu.npi(step.w_verify) == 1)


def test_maximum_sizes():
    """The scheduler's limit (4095 of at most 4096 candidates: 273 requests
    of block width 16) in compact mode, the row limit (8192 rows: 512 x 16) in
    static mode, and one candidate past the limit, which the host rejects."""
    from ragged_verification_amd import rv
    small = dict(Hq=8, Hkv=2, V=600, H=128, ctx=("uniform", 0, 40), tiers=(), gamma=16)
    inp = pu.make_inputs("gqa_bf16", B=273, **small)
    _full_parity(inp, "compact", "bf16")
    inp = pu.make_inputs("gqa_bf16", B=512, **small)
    _full_parity(inp, "static", "bf16")
    inp = pu.make_inputs("gqa_bf16", B=274, **small)     # 274 * 15 = 4110 candidates
    with pytest.raises(rv.RVError):
        pu.run_gpu(inp, "compact")


def test_multi_step_state():
    """Three verify steps in a row with the state carried on the device (ctx,
    anchors, req_to_token, history): each step's packing, argmax, accepts and
    scatter equal the oracle run step by step on the oracle's own state."""
    from ragged_verification_amd.pipeline import VerifyStep
    inp = pu.make_inputs("mla_bf16", B=4, V=1000, H=512, ctx=("uniform", 60, 400), spare_tokens=3 * 8)
    gamma, B = inp["gamma"], inp["B"]
    step = VerifyStep(inp, mode="compact", with_logits=True)
    conf = inp["conf"].cpu().numpy()
    drafts = pu.npi(inp["drafts"])
    pt = pu.npi(inp["page_table"])
    ctx, anchor = pu.npi(inp["ctx"]), pu.npi(inp["anchor"])
    r2t = np.full(tuple(step.req_to_token.shape), -1)
    hist = np.full(tuple(step.hist.shape), -1)
    hist_len = np.zeros(B, dtype=np.int64)
    wl = inp["workload"]
    for s_ in range(3):
        step.run()
        torch.cuda.synchronize()
        assert step.status() == 0
        wc, wv, k_star, e_star = oracle.schedule(conf, gamma, oracle.COMPACT, inp["cost_bias"],
                                                 inp["cost_alpha"].cpu().numpy(), inp["cost_theta"].cpu().numpy())
        cu, M, M_pad, row_req, row_pos, tok, slot = oracle.pack(wv, anchor, drafts, ctx, pt, inp["page_size"],
                                                                inp["tiers"])
        assert np.array_equal(pu.npi(step.cu), cu)
        assert np.array_equal(pu.npi(step.tok)[:M_pad], tok) and np.array_equal(pu.npi(step.slot)[:M_pad], slot)
        ref = dict(M=M, row_req=row_req, cu=cu)
        bidx = pu.packed_block_index(ref, gamma)
        q = pu.np64(inp["q_block"].reshape(-1, wl.Hq, wl.Dqk))[bidx]
        o, _ = oracle.verify_attention(q, pu.np64(inp["k_cache"]), None, pt, inp["page_size"], row_req[:M],
                                       row_pos[:M], M, inp["sm_scale"], Dv=wl.Dv)
        assert np.max(np.abs(step.o[:M].float().cpu().numpy() - o)) <= pu.ATTN_TOL["bf16"]
        z = oracle.lm_head_logits(pu.np64(inp["hidden_block"].reshape(-1, wl.H))[bidx], pu.np64(inp["W"]))
        pred = oracle.lm_head_pred(z)
        assert np.array_equal(pu.npi(step.pred)[:M], pred)
        acc, bonus, ceil = oracle.accept_greedy(pred, cu, wc, wv, drafts)
        assert np.array_equal(pu.npi(step.accept), acc) and np.array_equal(pu.npi(step.bonus), bonus)
        sc = oracle.compact_scatter(cu, wv, acc, bonus, drafts, slot, ctx, anchor, r2t, hist, hist_len)
        pu.check_scatter(step, sc, B)
        ctx, anchor, r2t, hist, hist_len = sc["ctx"], sc["anchor"], sc["req_to_token"], sc["hist"], sc["hist_len"]
    assert int(hist_len.min()) >= 3


def test_device_status_errors():
    """Bad data found on the device raises the sticky status and keeps every
    access in bounds."""
    from ragged_verification_amd import rv
    inp = pu.make_inputs("tiny_f32")
    step = pu.run_gpu(inp, "compact")
    assert step.status() == 0
    bad = dict(inp)
    bad["conf"] = inp["conf"].clone()
    bad["conf"][0, 0] = 1.5
    s2 = pu.run_gpu(bad, "compact")
    assert s2.status() == 1                      # BAD_CONF
    rv.rv_clear_status(s2.workspace)
    assert s2.status() == 0
    bad = dict(inp)
    bad["tiers"] = (4,)                          # M > 4 always here: overflow
    s3 = pu.run_gpu(bad, "static")
    assert s3.status() == 4
    assert pu.npi(s3.mm).tolist() == [16, 16]
    bad = dict(inp)
    bad["page_table"] = inp["page_table"].clone()
    bad["page_table"][1, 0] = 10_000             # out of range page id
    s4 = pu.run_gpu(bad, "static")
    assert s4.status() == 5


def test_deterministic_replay():
    inp = pu.make_inputs("mla_bf16", B=3, V=500, H=128, ctx=("uniform", 300, 900))
    a = pu.run_gpu(inp, "compact", with_logits=True)
    o1, z1 = a.o.clone(), a.logits.clone()
    a.restore()
    a.run()
    torch.cuda.synchronize()
    assert torch.equal(a.o, o1) and torch.equal(a.logits, z1)


def _outputs(step):
    names = ("w_commit", "w_verify", "k_star", "e_star", "cu", "mm", "row_req", "row_pos", "tok", "slot", "o",
             "lse", "pred", "accept", "bonus", "ceiling", "logits", "ctx", "anchor", "req_to_token", "hist",
             "hist_len", "commit_cu", "commit_tok", "commit_slot", "free_slots", "free_count")
    return {n: getattr(step, n).clone() for n in names}


@pytest.mark.parametrize("wl,kw,step_kw", [
    ("mla_bf16", dict(B=3, V=1000, H=512, ctx=("uniform", 60, 700)), {}),
    ("mla_bf16", dict(B=3, V=1000, H=512, ctx=("uniform", 600, 2000)), dict(window=200)),
    ("mla_bf16", dict(B=2, V=500, H=256, ctx=("uniform", 3000, 5000)), dict(topk=2048)),
    ("mla_bf16", dict(B=3, Hq=64, V=1000, H=512, ctx=("uniform", 60, 700)), {}),
    ("gqa_bf16", dict(B=6, V=1000, H=256, ctx=("uniform", 40, 900)), {}),
    ("tiny_f32", dict(B=4), {}),
])
def test_fused_pack_plan_equals_separate_launches(wl, kw, step_kw):
    """The pack launch that also builds the attention plan (rv_pack_plan +
    rv_verify_attn_planned) gives every output of the step bit for bit as
    the separate pack and plan launches do: latent row kernel dense, windowed
    and with key lists, the 64-head latent kernel, the balanced GQA plan, and
    the fp32 path (no plan)."""
    inp = pu.make_inputs(wl, **kw)
    outs = []
    for fused in (True, False):
        step = VerifyStep(inp, mode="compact", with_logits=True, fused_plan=fused, **step_kw)
        step.run()
        torch.cuda.synchronize()
        assert step.status() == 0
        outs.append(_outputs(step))
        del step
    for n in outs[0]:
        assert torch.equal(outs[0][n], outs[1][n]), n


def test_cached_argument_structs_equal_fresh_ones():
    """The binding's argument cache (VerifyStep's default) gives the same
    outputs bit for bit as building every struct afresh, over several steps
    in which the inputs switch between two sets (new tensor objects for the
    KV caches, the weight and the drafts) and back, and the mode changes."""
    inp = pu.make_inputs("gqa_bf16", B=6, V=1000, H=256, ctx=("uniform", 40, 900))
    inp["W_tiled"] = rv.rv_lm_tile_weight(inp["W"])
    inp2 = dict(inp)
    for k in ("k_cache", "v_cache", "W", "drafts", "conf"):
        inp2[k] = inp[k].clone()
    inp2["k_cache"].mul_(0.5)
    inp2["conf"] = inp2["conf"].flip(0).contiguous()
    inp2["W_tiled"] = rv.rv_lm_tile_weight(inp2["W"])
    plan = [(inp, "compact"), (inp2, "compact"), (inp, "compact"), (inp2, "static"), (inp, "compact")]
    outs = []
    for cached in (True, False):
        step = VerifyStep(inp, mode="compact", with_logits=True)
        assert step.W_tiled is not None
        if not cached:
            step._abi = None
        got = []
        for src, mode in plan:
            step.inp = src
            step.mode = mode
            step.W_tiled = src["W_tiled"]
            step.restore()
            step.run()
            torch.cuda.synchronize()
            assert step.status() == 0
            got.append(_outputs(step))
        outs.append(got)
        del step
    for a, b in zip(*outs):
        for n in a:
            assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("wl,kw", [("mla_bf16", dict(B=3, V=1000, H=512, ctx=("uniform", 60, 700))),
                                   ("rejection_bf16", dict(B=6, V=3000, H=256,
                                                           ctx=("lognormal", 200, 1.0, 600)))])
def test_graph_replay_equals_eager(wl, kw):
    """The step captured in HIP graphs: every replay, with the program's own
    eager work and synchronisations between replays, equals the eager step
    bit for bit (every output buffer, including the mutated state)."""
    inp = pu.make_inputs(wl, **kw)
    ref = pu.run_gpu(inp, "compact", with_logits=True)
    want = _outputs(ref)
    step = VerifyStep(inp, mode="compact", with_logits=True)
    step.capture()
    for rep in range(3):
        step.restore()
        step.replay()
        torch.cuda.synchronize()
        got = _outputs(step)
        for n, t in want.items():
            assert torch.equal(got[n], t), (rep, n)
        assert step.status() == 0
        # eager work between replays: the reference step again, and torch ops
        ref.restore()
        ref.run()
        torch.cuda.synchronize()
        _ = (inp["q_block"].float() * 2).sum().item()
        assert torch.equal(ref.o, want["o"])


def _check_calibration(step, inp, n_bins):
    c = step.calibration(n_bins)
    torch.cuda.synchronize()
    assert step.status() == 0
    want = oracle.calibration(inp["conf"].cpu().numpy(), pu.npi(inp["drafts"]), pu.npi(step.pred), pu.npi(step.cu), pu.npi(step.w_verify),
                              n_bins)
    cnt, match, cfx, ece, rver, rmat = want
    assert c["bin_count"].cpu().tolist() == cnt
    assert c["bin_match"].cpu().tolist() == match
    assert c["bin_conf_fx"].cpu().tolist() == cfx
    assert float(c["ece"].item()) == ece
    assert c["req_verified"].cpu().tolist() == rver
    assert c["req_matched"].cpu().tolist() == rmat
    return ece


@pytest.mark.parametrize("mode", ["compact", "cap_accept", "static"])
def test_calibration_matches_oracle(mode):
    """Bins, fixed-point confidence sums, ECE and per-request counts, bit for
    bit; under compact only the scheduled window is counted."""
    inp = pu.make_inputs("gqa_bf16", B=40, V=1000, H=256, ctx=("uniform", 40, 300), tiers=(512,))
    step = pu.run_gpu(inp, mode)
    for n_bins in (10, 1, 37):
        _check_calibration(step, inp, n_bins)
    if mode != "compact":
        assert step.calib["req_verified"].sum().item() == 40 * (inp["gamma"] - 1)


def test_calibration_separates_miscalibrated_drafts():
    """Drafts planted with probability conf (calibrated) against conf^2
    (overconfident), all positions verified (cap-accept): the GPU's ECE equals
    the oracle's, and the overconfident batch's is the larger."""
    eces = []
    for power in (1.0, 2.0):
        inp = pu.make_inputs("gqa_bf16", B=256, V=500, H=128, ctx=("uniform", 8, 40), plant_power=power,
                             tiers=(2048,))
        step = pu.run_gpu(inp, "cap_accept")
        eces.append(_check_calibration(step, inp, 10))
    assert eces[1] > eces[0] + 0.05, eces


def test_mla_two_rows_per_tile_and_long_split():
    """64 latent heads (one head block per row) and one long request whose
    key range is split into chunks and merged."""
    inp = pu.make_inputs("mla_bf16", B=2, Hq=64, V=500, H=256, ctx=("uniform", 3000, 5000))
    _full_parity(inp, "compact", "bf16")


def test_mla_late_score_jump_reruns_exactly():
    """A key late in the context whose score exceeds every earlier one by far
    more than the kernel's fixed softmax reference allows: the workgroup must
    rerun the item with the true maximum and still match the oracle."""
    inp = pu.make_inputs("mla_bf16", B=2, V=400, H=128, ctx=("uniform", 600, 900))
    pt = inp["page_table"].cpu()
    P = inp["page_size"]
    c0 = int(inp["ctx"][0])
    pos = c0 - 40                         # well after the first 32-key tile
    page = int(pt[0, pos // P])
    q0 = inp["q_block"][0, 0, 5].float()  # request 0, block row 0, head 5
    inp["k_cache"][page, pos % P, 0] = (2.0 * q0).to(inp["k_cache"].dtype)
    step, ref, want = _full_parity(inp, "compact", "bf16")
    # the planted key dominates head 5 of request 0's first row
    lse = step.lse.cpu().numpy()
    assert lse[0, 5] > 40.0


@pytest.mark.parametrize("B", [14, 22, 27, 29])
def test_lm_all_rows_block_counts(B):
    """The all-rows LM kernel at every row-block count it picks on the device
    and in its two-tile branch with a partly filled second tile: static
    windows of 8 give 112, 176, 216 and 232 packed rows (four, six and seven
    32-row blocks; 232 rows switch to two 128-row tiles whose second tile
    holds 104 rows and reads clamped padding rows).  Every row's logits are
    compared."""
    inp = pu.make_inputs("gqa_bf16", B=B, V=900, H=256, tiers=(), ctx=("uniform", 10, 60))
    _full_parity(inp, "static", "bf16")


def _theta_tables(M_max, B_max):
    """Cost tables that are not linear in M: convex, concave, a step at every
    power of two (a tier-shaped cost), seeded random increments (monotone) and
    seeded random values (not monotone), with a convex alpha."""
    m = np.arange(M_max + 1, dtype=np.float64)
    b = np.arange(B_max + 1, dtype=np.float64)
    rng = np.random.default_rng(20260703)
    pow2 = np.where(m > 0, 2.0 ** np.ceil(np.log2(np.maximum(m, 1.0))), 0.0)
    return {
        "convex": (0.5, 0.01 * b, 0.002 * m + 2e-6 * m * m),
        "concave": (1.0, 0.01 * b, 0.06 * np.sqrt(m)),
        "tier_steps": (1.0, 0.01 * b, 0.004 * pow2),
        "random_increments": (0.8, 0.01 * b + 1e-5 * b * b, np.cumsum(rng.uniform(0.0, 0.01, M_max + 1))),
        "random_values": (2.0, 0.02 * b, rng.uniform(0.0, 3.0, M_max + 1)),
    }


@pytest.mark.parametrize("B", [32, 256, 512])
def test_schedule_nonlinear_theta(B):
    """rv_schedule against the oracle on cost tables that are not linear in M
    (the scheduler's objective must evaluate the table at every K, not assume
    a slope): windows, K* and E* bit for bit, compact and cap-accept."""
    from ragged_verification_amd import rv
    gamma = 8
    wl_inp = pu.make_inputs("sweep_gqa", B=B, V=64, H=64, ctx=("uniform", 4, 8))
    conf = wl_inp["conf"]
    ks = set()
    for name, (bias, alpha, theta) in _theta_tables(B * gamma, B).items():
        al = torch.tensor(alpha, dtype=torch.float64, device="cuda")
        th = torch.tensor(theta, dtype=torch.float64, device="cuda")
        for mode in ("compact", "cap_accept"):
            i32 = dict(dtype=torch.int32, device="cuda")
            wc, wv, ks_t = torch.zeros(B, **i32), torch.zeros(B, **i32), torch.zeros(1, **i32)
            es = torch.zeros(1, dtype=torch.float64, device="cuda")
            ws = torch.zeros(rv.rv_workspace_size(B, gamma), dtype=torch.uint8, device="cuda")
            rv.rv_schedule(conf, gamma, mode, bias, al, th, wc, wv, ks_t, es, ws)
            torch.cuda.synchronize()
            assert rv.rv_device_status(ws) == 0
            want = oracle.schedule(conf.cpu().numpy(), gamma, pu.MODE_CODES[mode], bias, alpha, theta)
            assert np.array_equal(pu.npi(wc), want[0]), (name, mode)
            assert np.array_equal(pu.npi(wv), want[1]), (name, mode)
            assert int(ks_t.item()) == want[2], (name, mode)
            assert float(es.item()) == want[3], (name, mode)
            ks.add(want[2])
    pu.log(f"B={B} K* over the tables: {sorted(ks)}")
    assert len(ks) >= 3   # the tables move the optimum


def test_no_trim_equals_static():
    """no-trim (compact's ragged path without a cost table: full windows)
    against the oracle, and equal to static mode output for output."""
    inp = pu.make_inputs("gqa_bf16", B=6, V=1000, H=256, ctx=("uniform", 40, 900))
    nt, _, _ = _full_parity(inp, "no_trim", "bf16")
    st, _, _ = _full_parity(inp, "static", "bf16")
    for n in ("w_commit", "w_verify", "k_star", "e_star", "cu", "mm", "row_req", "row_pos", "tok", "slot", "o",
              "lse", "pred", "accept", "bonus", "ceiling", "logits", "ctx", "anchor", "req_to_token",
              "commit_cu", "commit_tok", "commit_slot", "free_count"):
        assert torch.equal(getattr(nt, n), getattr(st, n)), n


def test_negative_zero_confidence():
    """A confidence of -0.0 is a valid zero: the scheduler must rank its
    zero survivals with the other zeros (by request, then position), not
    ahead of every positive survival."""
    inp = pu.make_inputs("sweep_gqa", B=24, V=800, H=128, ctx=("uniform", 30, 300))
    conf = inp["conf"].clone()
    conf[3, 0] = -0.0
    conf[10, 2] = -0.0
    conf[17, :] = -0.0
    inp["conf"] = conf
    assert torch.signbit(inp["conf"][3, 0])
    for mode in ("compact", "cap_accept"):
        step, ref, _ = _full_parity(inp, mode, "bf16")
        assert int(pu.npi(step.w_commit)[17]) == 1


def test_mla_negative_scale():
    """A negative softmax scale (any finite scale is valid): the latent row
    kernel's largest scaled score then comes from the smallest raw score."""
    inp = pu.make_inputs("mla_bf16", B=3, V=500, H=256, ctx=("uniform", 60, 700))
    inp["sm_scale"] = -inp["sm_scale"]
    _full_parity(inp, "compact", "bf16")


def test_mla_256_heads_two_head_blocks():
    """256 query heads: each packed row is two 128-head tiles of the latent
    row kernel, one of them on a split key range."""
    inp = pu.make_inputs("mla_bf16", B=2, Hq=256, V=500, H=256, ctx=("uniform", 1500, 3000))
    _full_parity(inp, "compact", "bf16")
