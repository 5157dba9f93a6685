"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, its structs match the binding, and host-side validation rejects bad
arguments before anything is enqueued."""

import ctypes
import os
import re

import pytest

from ragged_verification_amd import rv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rv.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:rv_status|const char\*|int32_t)\s+(rv_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rv.LIB_PATH):
        pytest.fail("librv.so is not built (run __graft_entry__.build())")
    return rv.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert set(names) == set(rv.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layouts_match(lib):
    for which, st in enumerate(rv.STRUCTS):
        c_layout = rv.abi_layout(lib, which)
        assert c_layout[0] == ctypes.sizeof(st)
        assert c_layout[1:] == [getattr(st, f[0]).offset for f in st._fields_]
    assert lib.rv_abi_layout(99, None, 0) == -1


def test_version_and_workspace(lib):
    assert "gfx950" in rv.rv_version()
    small = rv.rv_workspace_size(4, 4, V=512, dtype=rv.RV_F32)
    assert small >= 256
    big = rv.rv_workspace_size(256, 8, 128, 1, 576, 512, 129280, rv.RV_BF16)
    assert big > small
    d = rv.Dims(-1, 4, 0, 0, 0, 0, 0, 0)
    out = ctypes.c_size_t(0)
    assert lib.rv_workspace_size(ctypes.byref(d), ctypes.byref(out)) == rv.RV_ERR_INVALID_ARG
    assert lib.rv_workspace_size(None, ctypes.byref(out)) == rv.RV_ERR_INVALID_ARG


def _fake(n=1):
    # host addresses that are never dereferenced: validation fails first
    return ctypes.c_void_p(0x1000 * n)


def test_schedule_validation(lib):
    a = rv.ScheduleArgs()
    assert lib.rv_schedule(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    assert lib.rv_schedule(None, None) == rv.RV_ERR_INVALID_ARG
    for f in ("conf", "cost_alpha", "cost_theta", "w_commit", "w_verify", "k_star", "e_star"):
        setattr(a, f, _fake())
    a.B, a.gamma, a.mode, a.alpha_len, a.theta_len, a.cost_bias = 4, 4, rv.RV_COMPACT, 5, 17, 1.0
    assert lib.rv_schedule(ctypes.byref(a), None) == rv.RV_ERR_WORKSPACE
    a.gamma = 1
    assert lib.rv_schedule(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    a.gamma = 17
    assert lib.rv_schedule(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    a.gamma, a.theta_len = 4, 16   # theta must cover M = B*gamma
    assert lib.rv_schedule(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    a.theta_len, a.mode = 17, 7
    assert lib.rv_schedule(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    a.mode, a.B, a.gamma, a.alpha_len, a.theta_len = rv.RV_COMPACT, 1000, 8, 1001, 8001
    assert lib.rv_schedule(ctypes.byref(a), None) == rv.RV_ERR_UNSUPPORTED  # > 4096 candidates


def test_pack_validation(lib):
    a = rv.PackArgs()
    for f in ("w_verify", "anchor", "drafts", "ctx", "page_table", "cu", "mm", "row_req", "row_pos",
              "tok", "slot"):
        setattr(a, f, _fake())
    a.B, a.gamma, a.max_pages, a.page_size, a.num_pages, a.rows_cap = 4, 4, 1, 16, 4, 16
    assert lib.rv_pack(ctypes.byref(a), None) == rv.RV_ERR_WORKSPACE
    a.rows_cap = 15   # below B*gamma
    assert lib.rv_pack(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    a.rows_cap = 16
    tiers = (ctypes.c_int32 * 3)(8, 8, 16)   # not strictly ascending
    a.n_tiers, a.tiers = 3, ctypes.cast(tiers, ctypes.c_void_p)
    assert lib.rv_pack(ctypes.byref(a), None) == rv.RV_ERR_TIER
    tiers2 = (ctypes.c_int32 * 2)(8, 32)     # largest tier above rows_cap
    a.n_tiers, a.tiers = 2, ctypes.cast(tiers2, ctypes.c_void_p)
    assert lib.rv_pack(ctypes.byref(a), None) == rv.RV_ERR_TIER
    a.n_tiers = 17
    assert lib.rv_pack(ctypes.byref(a), None) == rv.RV_ERR_TIER


def test_attn_validation(lib):
    a = rv.AttnArgs()
    for f in ("q", "k_cache", "v_cache", "page_table", "ctx", "cu", "mm", "o"):
        setattr(a, f, _fake())
    a.B, a.gamma, a.rows_cap, a.max_pages, a.page_size, a.num_pages = 2, 8, 16, 4, 16, 8
    a.Hq, a.Hkv, a.Dqk, a.Dv, a.dtype, a.sm_scale = 32, 8, 128, 128, rv.RV_BF16, 0.088
    assert lib.rv_verify_attn(ctypes.byref(a), None) == rv.RV_ERR_WORKSPACE
    a.Dqk = a.Dv = 96            # no bf16 kernel for this head dim
    assert lib.rv_verify_attn(ctypes.byref(a), None) == rv.RV_ERR_UNSUPPORTED
    a.Dqk = a.Dv = 128
    a.Hq = 30                    # not a multiple of Hkv
    assert lib.rv_verify_attn(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    a.Hq, a.v_cache, a.Hkv = 32, None, 8   # latent layout needs one KV head
    assert lib.rv_verify_attn(ctypes.byref(a), None) == rv.RV_ERR_UNSUPPORTED
    a.sm_scale = float("nan")
    assert lib.rv_verify_attn(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    a.sm_scale, a.window = 0.1, -1        # negative window
    assert lib.rv_verify_attn(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    a.window, a.v_cache = 0, _fake()      # sparse key lists: latent layout only
    a.topk, a.topk_idx = 64, _fake()
    assert lib.rv_verify_attn(ctypes.byref(a), None) == rv.RV_ERR_UNSUPPORTED
    a.v_cache, a.Hkv, a.Hq, a.Dqk, a.Dv = None, 1, 128, 576, 512
    a.topk = 4096                          # past RV_MAX_TOPK
    assert lib.rv_verify_attn(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    a.topk, a.window = 64, 100             # no window with key lists
    assert lib.rv_verify_attn(ctypes.byref(a), None) == rv.RV_ERR_UNSUPPORTED
    a.window = 0
    assert lib.rv_verify_attn(ctypes.byref(a), None) == rv.RV_ERR_WORKSPACE


def test_pack_plan_validation(lib):
    """rv_pack_plan checks both argument sets, then that the attention call
    reads the pack's own cu, mm and ctx for the same B and gamma; the planned
    attention entry checks its arguments as rv_verify_attn does."""
    pk = rv.PackArgs()
    for f in ("w_verify", "anchor", "drafts", "ctx", "page_table", "cu", "mm", "row_req", "row_pos",
              "tok", "slot"):
        setattr(pk, f, _fake())
    pk.B, pk.gamma, pk.max_pages, pk.page_size, pk.num_pages, pk.rows_cap = 2, 8, 4, 64, 8, 16
    at = rv.AttnArgs()
    for f in ("q", "k_cache", "page_table", "o"):
        setattr(at, f, _fake())
    at.ctx, at.cu, at.mm = pk.ctx, pk.cu, pk.mm
    at.B, at.gamma, at.rows_cap, at.max_pages, at.page_size, at.num_pages = 2, 8, 16, 4, 64, 8
    at.Hq, at.Hkv, at.Dqk, at.Dv, at.dtype, at.sm_scale = 128, 1, 576, 512, rv.RV_BF16, 0.04
    fake_ws = (ctypes.c_uint8 * 16)()
    big = 1 << 40
    pk.workspace, pk.workspace_bytes = ctypes.cast(fake_ws, ctypes.c_void_p), big
    assert lib.rv_pack_plan(ctypes.byref(pk), ctypes.byref(at), None) == rv.RV_ERR_WORKSPACE   # attention's
    assert lib.rv_verify_attn_planned(ctypes.byref(at), None) == rv.RV_ERR_WORKSPACE
    at.workspace, at.workspace_bytes = ctypes.cast(fake_ws, ctypes.c_void_p), big
    at.cu = _fake(7)                      # not the pack's cu
    assert lib.rv_pack_plan(ctypes.byref(pk), ctypes.byref(at), None) == rv.RV_ERR_INVALID_ARG
    at.cu, at.B = pk.cu, 1                # another batch
    assert lib.rv_pack_plan(ctypes.byref(pk), ctypes.byref(at), None) == rv.RV_ERR_INVALID_ARG
    at.B, pk.rows_cap = 2, 15             # the pack's own check
    assert lib.rv_pack_plan(ctypes.byref(pk), ctypes.byref(at), None) == rv.RV_ERR_INVALID_ARG
    pk.rows_cap, at.Hkv = 16, 2           # the attention's own check (latent: one KV head)
    assert lib.rv_pack_plan(ctypes.byref(pk), ctypes.byref(at), None) == rv.RV_ERR_UNSUPPORTED
    assert lib.rv_verify_attn_planned(ctypes.byref(at), None) == rv.RV_ERR_UNSUPPORTED


def test_tiled_weight_size_and_validation(lib):
    n = ctypes.c_size_t(0)
    # V rounded up to 32 rows, 2 bytes per element
    assert lib.rv_lm_tiled_weight_bytes(1000, 256, rv.RV_BF16, ctypes.byref(n)) == rv.RV_OK
    assert n.value == 1024 * 256 * 2
    assert lib.rv_lm_tiled_weight_bytes(129280, 7168, rv.RV_BF16, ctypes.byref(n)) == rv.RV_OK
    assert n.value == 129280 * 7168 * 2
    assert lib.rv_lm_tiled_weight_bytes(1000, 192, rv.RV_BF16, ctypes.byref(n)) == rv.RV_ERR_INVALID_ARG
    assert lib.rv_lm_tiled_weight_bytes(1000, 256, rv.RV_F32, ctypes.byref(n)) == rv.RV_ERR_UNSUPPORTED
    assert lib.rv_lm_tiled_weight_bytes(0, 256, rv.RV_BF16, ctypes.byref(n)) == rv.RV_ERR_INVALID_ARG
    assert lib.rv_lm_tile_weight(None, _fake(), 1000, 256, rv.RV_BF16, None) == rv.RV_ERR_INVALID_ARG
    assert lib.rv_lm_tile_weight(_fake(), _fake(), 1000, 64, rv.RV_BF16, None) == rv.RV_ERR_INVALID_ARG
    assert lib.rv_lm_tile_weight(_fake(), _fake(), 1000, 256, rv.RV_F32, None) == rv.RV_ERR_UNSUPPORTED


def test_lm_and_scatter_validation(lib):
    a = rv.LmArgs()
    for f in ("hidden", "W", "mm", "cu", "w_commit", "w_verify", "drafts", "pred", "accept", "bonus",
              "ceiling"):
        setattr(a, f, _fake())
    a.B, a.gamma, a.rows_cap, a.H, a.V, a.dtype, a.rule = 2, 4, 8, 128, 1000, rv.RV_BF16, rv.RV_GREEDY
    assert lib.rv_lm_head_accept(ctypes.byref(a), None) == rv.RV_ERR_WORKSPACE
    a.H = 100                    # bf16 GEMM needs H % 64 == 0
    assert lib.rv_lm_head_accept(ctypes.byref(a), None) == rv.RV_ERR_UNSUPPORTED
    a.H, a.rule = 128, rv.RV_REJECTION   # rejection needs q_rows, u, u_bonus, logits
    assert lib.rv_lm_head_accept(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    a.rule, a.w_layout = rv.RV_GREEDY, 7      # unknown weight layout
    assert lib.rv_lm_head_accept(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    a.w_layout, a.H = rv.RV_W_TILED, 192      # tiled weight needs H % 128 == 0
    assert lib.rv_lm_head_accept(ctypes.byref(a), None) == rv.RV_ERR_UNSUPPORTED
    a.H, a.dtype = 128, rv.RV_F32             # tiled weight is bf16 only
    assert lib.rv_lm_head_accept(ctypes.byref(a), None) == rv.RV_ERR_UNSUPPORTED
    s = rv.ScatterArgs()
    for f in ("cu", "w_verify", "accept", "bonus", "drafts", "slot", "ctx", "anchor", "req_to_token",
              "commit_cu", "commit_tok", "commit_slot", "free_slots", "free_count"):
        setattr(s, f, _fake())
    s.B, s.gamma, s.r2t_stride = 2, 4, 64
    assert lib.rv_compact_scatter(ctypes.byref(s), None) == rv.RV_ERR_WORKSPACE
    s.hist = _fake()             # hist without hist_len
    assert lib.rv_compact_scatter(ctypes.byref(s), None) == rv.RV_ERR_INVALID_ARG


def test_lm_noalloc_rejects_beyond_its_scratch(lib):
    """The no-alloc LM head refuses, before any device work, a problem whose
    slab partials exceed its static scratch (64 MiB), a status buffer under
    256 bytes, and whatever rv_lm_head_accept refuses."""
    a = rv.LmArgs()
    assert lib.rv_lm_head_accept_noalloc(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG
    for f in ("hidden", "W", "mm", "cu", "w_commit", "w_verify", "drafts", "pred", "accept", "bonus", "ceiling"):
        setattr(a, f, _fake())
    a.B, a.gamma, a.rows_cap, a.H, a.dtype, a.rule, a.w_layout = 64, 8, 512, 256, rv.RV_BF16, rv.RV_GREEDY, 0
    a.V = 1 << 21        # 512 rows x 32768 slabs x 16 bytes: 256 MiB
    assert lib.rv_lm_head_accept_noalloc(ctypes.byref(a), None) == rv.RV_ERR_SCRATCH
    a.B, a.rows_cap, a.V = 256, 2048, 131072 + 64   # 2048 rows x 2049 slabs: 64 MiB + 32 KiB
    assert lib.rv_lm_head_accept_noalloc(ctypes.byref(a), None) == rv.RV_ERR_SCRATCH
    a.workspace, a.workspace_bytes = _fake(), 255
    assert lib.rv_lm_head_accept_noalloc(ctypes.byref(a), None) == rv.RV_ERR_WORKSPACE
    a.rule = 9
    assert lib.rv_lm_head_accept_noalloc(ctypes.byref(a), None) == rv.RV_ERR_INVALID_ARG


def test_arg_cache_reuses_and_rebuilds():
    """ArgCache hands back the same built structs while the tensor arguments
    are the same objects and the other arguments the same values, rebuilds
    on any change, and keeps its tensors alive (so their ids stay theirs)."""
    import gc
    import torch
    from ragged_verification_amd import rv
    c = rv.ArgCache()
    built = []

    def build():
        built.append(object())
        return built[-1]

    t1, t2 = torch.zeros(4), torch.zeros(4)
    a = c.get("x", (t1, 3, None), build)
    assert c.get("x", (t1, 3, None), build) is a and len(built) == 1
    c.get("x", (t2, 3, None), build)            # another tensor object
    assert len(built) == 2
    c.get("x", (t2, 4, None), build)            # another scalar
    assert len(built) == 3
    c.get("y", (t2, 4, None), build)            # entries are per call name
    assert len(built) == 4
    assert c.get("x", (t2, 4, None), build) is built[2]
    assert c.get("x", (t1, 3, None), build) is built[0]   # earlier sets are kept too
    tiers = (64, 128)
    assert c.get("x", (t1, 3, tiers), build) is c.get("x", (t1, 3, tiers), build)
    n_built = len(built)
    c.get("x", (t1, 3, (64, 256)), build)       # another object: rebuilt
    assert len(built) == n_built + 1
    small = rv.ArgCache(per_call=2)
    for n in range(3):
        small.get("z", (n,), build)
    n_built = len(built)
    small.get("z", (0,), build)                  # evicted: rebuilt
    assert len(built) == n_built + 1
    # the cached entry holds t2: dropping the caller's reference does not let
    # a new tensor take its id while the entry lives
    ident = id(t2)
    del t2
    gc.collect()
    fresh = [torch.zeros(4) for _ in range(64)]
    assert all(id(f) != ident for f in fresh)
