"""Thin ctypes binding of librv (include/rv.h): argument marshalling only.

Each ``rv_*`` function here has the name and arguments of the C entry point;
tensors are passed as device pointers (``data_ptr``), the stream is torch's
current HIP stream unless one is given.  All arithmetic happens in the HIP
kernels; torch only provides device memory and streams.  If the shared
library is missing, ``load()`` raises: there is no fallback.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librv.so")

RV_OK, RV_ERR_INVALID_ARG, RV_ERR_UNSUPPORTED, RV_ERR_TIER, RV_ERR_WORKSPACE, RV_ERR_HIP = 0, -1, -2, -3, -4, -5
RV_ERR_SCRATCH = -6
STATUS_NAMES = {0: "RV_OK", -1: "RV_ERR_INVALID_ARG", -2: "RV_ERR_UNSUPPORTED", -3: "RV_ERR_TIER",
                -4: "RV_ERR_WORKSPACE", -5: "RV_ERR_HIP", -6: "RV_ERR_SCRATCH"}
DEV_NAMES = {0: "RV_DEV_OK", 1: "RV_DEV_BAD_CONF", 2: "RV_DEV_BAD_COST", 3: "RV_DEV_BAD_WINDOW",
             4: "RV_DEV_TIER_OVERFLOW", 5: "RV_DEV_BAD_PAGE", 6: "RV_DEV_BAD_TOKEN",
             7: "RV_DEV_HIST_OVERFLOW"}
RV_STATIC, RV_COMPACT, RV_CAP_ACCEPT, RV_NO_TRIM = 0, 1, 2, 3
MODES = {"static": RV_STATIC, "compact": RV_COMPACT, "cap_accept": RV_CAP_ACCEPT, "no_trim": RV_NO_TRIM}
RV_GREEDY, RV_REJECTION = 0, 1
RV_F32, RV_BF16 = 0, 1
RV_W_ROWS, RV_W_TILED = 0, 1
RV_MAX_GAMMA, RV_MAX_TIERS, RV_MAX_ROWS = 16, 16, 8192
RV_NOALLOC_SCRATCH_BYTES = 64 << 20

_vp, _i32, _f32, _f64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_size_t


class Dims(ctypes.Structure):
    _fields_ = [("B", _i32), ("gamma", _i32), ("Hq", _i32), ("Hkv", _i32), ("Dqk", _i32),
                ("Dv", _i32), ("V", _i32), ("dtype", _i32)]


class ScheduleArgs(ctypes.Structure):
    _fields_ = [("conf", _vp), ("B", _i32), ("gamma", _i32), ("mode", _i32), ("alpha_len", _i32),
                ("theta_len", _i32), ("_pad0", _i32), ("cost_bias", _f64), ("cost_alpha", _vp),
                ("cost_theta", _vp), ("w_commit", _vp), ("w_verify", _vp), ("k_star", _vp),
                ("e_star", _vp), ("workspace", _vp), ("workspace_bytes", _sz)]


class PackArgs(ctypes.Structure):
    _fields_ = [("w_verify", _vp), ("anchor", _vp), ("drafts", _vp), ("ctx", _vp), ("page_table", _vp),
                ("B", _i32), ("gamma", _i32), ("max_pages", _i32), ("page_size", _i32),
                ("num_pages", _i32), ("n_tiers", _i32), ("tiers", _vp), ("rows_cap", _i32),
                ("_pad0", _i32), ("cu", _vp), ("mm", _vp), ("row_req", _vp), ("row_pos", _vp),
                ("tok", _vp), ("slot", _vp), ("workspace", _vp), ("workspace_bytes", _sz)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("k_cache", _vp), ("v_cache", _vp), ("page_table", _vp), ("ctx", _vp),
                ("cu", _vp), ("mm", _vp), ("B", _i32), ("gamma", _i32), ("rows_cap", _i32),
                ("max_pages", _i32), ("page_size", _i32), ("num_pages", _i32), ("Hq", _i32),
                ("Hkv", _i32), ("Dqk", _i32), ("Dv", _i32), ("dtype", _i32), ("sm_scale", _f32),
                ("window", _i32), ("topk", _i32), ("topk_idx", _vp), ("o", _vp), ("lse", _vp), ("workspace", _vp), ("workspace_bytes", _sz)]


class LmArgs(ctypes.Structure):
    _fields_ = [("hidden", _vp), ("W", _vp), ("mm", _vp), ("cu", _vp), ("w_commit", _vp),
                ("w_verify", _vp), ("drafts", _vp), ("q_rows", _vp), ("u", _vp), ("u_bonus", _vp),
                ("B", _i32), ("gamma", _i32), ("rows_cap", _i32), ("H", _i32), ("V", _i32),
                ("dtype", _i32), ("rule", _i32), ("w_layout", _i32), ("pred", _vp), ("accept", _vp),
                ("bonus", _vp), ("ceiling", _vp), ("logits", _vp), ("workspace", _vp),
                ("workspace_bytes", _sz)]


class ScatterArgs(ctypes.Structure):
    _fields_ = [("cu", _vp), ("w_verify", _vp), ("accept", _vp), ("bonus", _vp), ("drafts", _vp),
                ("slot", _vp), ("B", _i32), ("gamma", _i32), ("r2t_stride", _i32),
                ("hist_stride", _i32), ("ctx", _vp), ("anchor", _vp), ("req_to_token", _vp),
                ("hist", _vp), ("hist_len", _vp), ("commit_cu", _vp), ("commit_tok", _vp),
                ("commit_slot", _vp), ("free_slots", _vp), ("free_count", _vp), ("workspace", _vp),
                ("workspace_bytes", _sz)]


class CalibArgs(ctypes.Structure):
    _fields_ = [("conf", _vp), ("drafts", _vp), ("pred", _vp), ("cu", _vp), ("w_verify", _vp), ("B", _i32),
                ("gamma", _i32), ("rows_cap", _i32), ("n_bins", _i32), ("bin_count", _vp), ("bin_match", _vp),
                ("bin_conf_fx", _vp), ("ece", _vp), ("req_verified", _vp), ("req_matched", _vp),
                ("workspace", _vp), ("workspace_bytes", _sz)]


class EstimateArgs(ctypes.Structure):
    _fields_ = [("cu", _vp), ("w_verify", _vp), ("accept", _vp), ("drafts", _vp), ("ctx", _vp), ("pred", _vp),
                ("logits", _vp), ("q_rows", _vp), ("B", _i32), ("gamma", _i32), ("rows_cap", _i32), ("V", _i32),
                ("rule", _i32), ("_pad0", _i32), ("state", _vp), ("workspace", _vp), ("workspace_bytes", _sz)]


STRUCTS = [ScheduleArgs, PackArgs, AttnArgs, LmArgs, ScatterArgs, Dims, CalibArgs, EstimateArgs]
EXPORTS = ["rv_version", "rv_workspace_size", "rv_device_status", "rv_clear_status", "rv_schedule",
           "rv_pack", "rv_verify_attn", "rv_lm_head_accept", "rv_compact_scatter", "rv_abi_layout",
           "rv_lm_tiled_weight_bytes", "rv_lm_tile_weight", "rv_fit_cost_model", "rv_calibration",
           "rv_lm_head_accept_noalloc", "rv_estimator_state_bytes", "rv_block_accept_estimate",
           "rv_pack_plan", "rv_verify_attn_planned"]

_LIB = None


class RVError(RuntimeError):
    def __init__(self, call, code):
        super().__init__(f"{call} returned {STATUS_NAMES.get(code, code)}")
        self.code = code


def load(path=LIB_PATH):
    """Load librv.so and check that the ctypes structs match the C layout."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m ragged_verification_amd.build`")
    lib = ctypes.CDLL(path)
    lib.rv_version.restype = ctypes.c_char_p
    lib.rv_version.argtypes = []
    lib.rv_workspace_size.restype = _i32
    lib.rv_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(_sz)]
    lib.rv_device_status.restype = _i32
    lib.rv_device_status.argtypes = [_vp, ctypes.POINTER(_i32), _vp]
    lib.rv_clear_status.restype = _i32
    lib.rv_clear_status.argtypes = [_vp, _vp]
    for name, st in (("rv_schedule", ScheduleArgs), ("rv_pack", PackArgs), ("rv_verify_attn", AttnArgs),
                     ("rv_lm_head_accept", LmArgs), ("rv_compact_scatter", ScatterArgs),
                     ("rv_calibration", CalibArgs), ("rv_lm_head_accept_noalloc", LmArgs),
                     ("rv_block_accept_estimate", EstimateArgs)):
        fn = getattr(lib, name)
        fn.restype = _i32
        fn.argtypes = [ctypes.POINTER(st), _vp]
    lib.rv_verify_attn_planned.restype = _i32
    lib.rv_verify_attn_planned.argtypes = [ctypes.POINTER(AttnArgs), _vp]
    lib.rv_pack_plan.restype = _i32
    lib.rv_pack_plan.argtypes = [ctypes.POINTER(PackArgs), ctypes.POINTER(AttnArgs), _vp]
    lib.rv_estimator_state_bytes.restype = _i32
    lib.rv_estimator_state_bytes.argtypes = [_i32, _i32, ctypes.POINTER(_sz)]
    lib.rv_lm_tiled_weight_bytes.restype = _i32
    lib.rv_lm_tiled_weight_bytes.argtypes = [_i32, _i32, _i32, ctypes.POINTER(_sz)]
    lib.rv_lm_tile_weight.restype = _i32
    lib.rv_lm_tile_weight.argtypes = [_vp, _vp, _i32, _i32, _i32, _vp]
    _pd = ctypes.POINTER(_f64)
    lib.rv_fit_cost_model.restype = _i32
    lib.rv_fit_cost_model.argtypes = [_pd, _pd, _pd, _i32, _pd, _pd, _i32, _pd, _i32]
    lib.rv_abi_layout.restype = _i32
    lib.rv_abi_layout.argtypes = [_i32, ctypes.POINTER(ctypes.c_int64), _i32]
    for which, st in enumerate(STRUCTS):
        c_layout = abi_layout(lib, which)
        py_layout = [ctypes.sizeof(st)] + [getattr(st, f[0]).offset for f in st._fields_]
        if c_layout != py_layout:
            raise RuntimeError(f"struct {st.__name__} layout mismatch: C {c_layout} vs ctypes {py_layout}")
    _LIB = lib
    return lib


def abi_layout(lib, which):
    buf = (ctypes.c_int64 * 64)()
    n = lib.rv_abi_layout(which, buf, 64)
    if n < 0:
        raise RuntimeError(f"rv_abi_layout({which}) failed")
    return list(buf[:n])


# ---- marshalling helpers ------------------------------------------------------
class ArgCache:
    """The argument structs of calls a caller repeats on the same buffers
    (one verify step after another), built once: an entry is reused when
    every argument is the very same object as before (compared by identity:
    equal values in new objects only cost a rebuild).  Up to ``per_call``
    argument sets are kept per call (a caller that rotates among a few input
    copies hits after the first round).  Entries hold their arguments, so
    those objects stay alive and their ids unique.  While cached, tensors
    must keep their storage (no ``resize_`` or ``set_``) and containers
    (tiers) must not change in place.  Building a struct validates and
    converts some 15-30 tensors, about 1 us each on the host; the identity
    key costs a few tens of nanoseconds per argument."""

    def __init__(self, per_call=16):
        self._e = {}
        self._n = per_call

    def get(self, name, args, build):
        key = tuple(map(id, args))
        d = self._e.setdefault(name, {})
        e = d.get(key)
        if e is not None:
            return e[0]
        val = build()
        if len(d) >= self._n:
            d.pop(next(iter(d)))   # the oldest entry
        d[key] = (val, args)
        return val


def _cached(cache, name, args, build):
    return build() if cache is None else cache.get(name, args, build)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be device memory (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(call, code):
    if code != RV_OK:
        raise RVError(call, code)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return RV_F32
    if t.dtype == torch.bfloat16:
        return RV_BF16
    raise TypeError(f"unsupported payload dtype {t.dtype}")


# ---- entry points ---------------------------------------------------------------
def rv_version():
    return load().rv_version().decode()


def rv_workspace_size(B, gamma, Hq=0, Hkv=0, Dqk=0, Dv=0, V=0, dtype=RV_BF16):
    d = Dims(B, gamma, Hq, Hkv, Dqk, Dv, V, dtype)
    out = _sz(0)
    _check("rv_workspace_size", load().rv_workspace_size(ctypes.byref(d), ctypes.byref(out)))
    return out.value


def rv_device_status(workspace, stream=None):
    code = _i32(0)
    _check("rv_device_status", load().rv_device_status(_ptr(workspace, name="workspace"),
                                                       ctypes.byref(code), _stream(stream)))
    return code.value


def rv_clear_status(workspace, stream=None):
    _check("rv_clear_status", load().rv_clear_status(_ptr(workspace, name="workspace"), _stream(stream)))


def rv_schedule(conf, gamma, mode, cost_bias, cost_alpha, cost_theta, w_commit, w_verify, k_star,
                e_star, workspace, stream=None, cache=None, launch=True):
    args = (conf, gamma, mode, cost_bias, cost_alpha, cost_theta, w_commit, w_verify, k_star, e_star, workspace)
    a = _cached(cache, "rv_schedule", args, lambda: _schedule_args(*args))
    if not launch:   # only fill the cache
        return
    _check("rv_schedule", load().rv_schedule(ctypes.byref(a), _stream(stream)))


def _schedule_args(conf, gamma, mode, cost_bias, cost_alpha, cost_theta, w_commit, w_verify, k_star, e_star,
                   workspace):
    B = conf.shape[0]
    return ScheduleArgs(conf=_ptr(conf, torch.float32, "conf"), B=B, gamma=gamma,
                     mode=MODES[mode] if isinstance(mode, str) else mode,
                     alpha_len=cost_alpha.numel(), theta_len=cost_theta.numel(), cost_bias=float(cost_bias),
                     cost_alpha=_ptr(cost_alpha, torch.float64, "cost_alpha"),
                     cost_theta=_ptr(cost_theta, torch.float64, "cost_theta"),
                     w_commit=_ptr(w_commit, torch.int32, "w_commit"),
                     w_verify=_ptr(w_verify, torch.int32, "w_verify"),
                     k_star=_ptr(k_star, torch.int32, "k_star"), e_star=_ptr(e_star, torch.float64, "e_star"),
                     workspace=_ptr(workspace, name="workspace"), workspace_bytes=workspace.numel() * workspace.element_size())


def _pack_args(w_verify, anchor, drafts, ctx, page_table, page_size, num_pages, tiers, cu, mm, row_req,
               row_pos, tok, slot, workspace):
    """PackArgs and the host tier array it points to (keep both alive)."""
    B, g1 = drafts.shape
    tiers = list(tiers or ())
    tarr = (ctypes.c_int32 * max(1, len(tiers)))(*tiers)
    a = PackArgs(w_verify=_ptr(w_verify, torch.int32, "w_verify"), anchor=_ptr(anchor, torch.int32, "anchor"),
                 drafts=_ptr(drafts, torch.int32, "drafts"), ctx=_ptr(ctx, torch.int32, "ctx"),
                 page_table=_ptr(page_table, torch.int32, "page_table"), B=B, gamma=g1 + 1,
                 max_pages=page_table.shape[1], page_size=page_size, num_pages=num_pages,
                 n_tiers=len(tiers), tiers=ctypes.cast(tarr, ctypes.c_void_p) if tiers else None,
                 rows_cap=row_req.numel(), cu=_ptr(cu, torch.int32, "cu"), mm=_ptr(mm, torch.int32, "mm"),
                 row_req=_ptr(row_req, torch.int32, "row_req"), row_pos=_ptr(row_pos, torch.int32, "row_pos"),
                 tok=_ptr(tok, torch.int32, "tok"), slot=_ptr(slot, torch.int32, "slot"),
                 workspace=_ptr(workspace, name="workspace"), workspace_bytes=workspace.numel() * workspace.element_size())
    return a, tarr


def rv_pack(w_verify, anchor, drafts, ctx, page_table, page_size, num_pages, tiers, cu, mm, row_req,
            row_pos, tok, slot, workspace, stream=None):
    a, _keep = _pack_args(w_verify, anchor, drafts, ctx, page_table, page_size, num_pages, tiers, cu, mm, row_req,
                          row_pos, tok, slot, workspace)
    _check("rv_pack", load().rv_pack(ctypes.byref(a), _stream(stream)))


def _attn_args(q, k_cache, v_cache, page_table, page_size, num_pages, ctx, cu, mm, gamma, sm_scale,
               o, lse, workspace, window=0, topk_idx=None):
    rows_cap, Hq, Dqk = q.shape
    Hkv = k_cache.shape[2]
    Dv = o.shape[2]
    dt = _dtype_code(q)
    a = AttnArgs(q=_ptr(q, q.dtype, "q"), k_cache=_ptr(k_cache, q.dtype, "k_cache"),
                 v_cache=_ptr(v_cache, q.dtype, "v_cache"), page_table=_ptr(page_table, torch.int32, "page_table"),
                 ctx=_ptr(ctx, torch.int32, "ctx"), cu=_ptr(cu, torch.int32, "cu"), mm=_ptr(mm, torch.int32, "mm"),
                 B=ctx.numel(), gamma=gamma, rows_cap=rows_cap, max_pages=page_table.shape[1],
                 page_size=page_size, num_pages=num_pages, Hq=Hq, Hkv=Hkv, Dqk=Dqk, Dv=Dv, dtype=dt,
                 sm_scale=float(sm_scale), window=int(window),
                 topk=0 if topk_idx is None else topk_idx.shape[1], topk_idx=_ptr(topk_idx, torch.int32, "topk_idx"),
                 o=_ptr(o, q.dtype, "o"), lse=_ptr(lse, torch.float32, "lse"),
                 workspace=_ptr(workspace, name="workspace"), workspace_bytes=workspace.numel() * workspace.element_size())
    return a


def rv_verify_attn(q, k_cache, v_cache, page_table, page_size, num_pages, ctx, cu, mm, gamma, sm_scale,
                   o, lse, workspace, stream=None, window=0, topk_idx=None, cache=None, launch=True):
    args = (q, k_cache, v_cache, page_table, page_size, num_pages, ctx, cu, mm, gamma, sm_scale, o, lse, workspace,
            window, topk_idx)
    a = _cached(cache, "attn", args, lambda: _attn_args(*args))
    if not launch:
        return
    _check("rv_verify_attn", load().rv_verify_attn(ctypes.byref(a), _stream(stream)))


def rv_verify_attn_planned(q, k_cache, v_cache, page_table, page_size, num_pages, ctx, cu, mm, gamma, sm_scale,
                           o, lse, workspace, stream=None, window=0, topk_idx=None, cache=None):
    """Stage 3 after rv_pack_plan (the plan is already in the workspace)."""
    args = (q, k_cache, v_cache, page_table, page_size, num_pages, ctx, cu, mm, gamma, sm_scale, o, lse, workspace,
            window, topk_idx)
    a = _cached(cache, "attn", args, lambda: _attn_args(*args))
    _check("rv_verify_attn_planned", load().rv_verify_attn_planned(ctypes.byref(a), _stream(stream)))


def rv_pack_plan(pack, attn, stream=None, cache=None, launch=True):
    """Stage 2 and the plan of stage 3 in one launch.  ``pack``: the keyword
    arguments of rv_pack (without stream); ``attn``: those of rv_verify_attn."""
    args = (*pack.keys(), *pack.values(), *attn.keys(), *attn.values())
    pa, _keep, aa = _cached(cache, "pack_plan", args, lambda: _pack_args(**pack) + (_attn_args(**attn),))
    if not launch:
        return
    _check("rv_pack_plan", load().rv_pack_plan(ctypes.byref(pa), ctypes.byref(aa), _stream(stream)))


def rv_calibration(conf, drafts, pred, cu, w_verify, n_bins, bin_count, bin_match, bin_conf_fx, ece, workspace,
                   req_verified=None, req_matched=None, stream=None):
    B, g1 = drafts.shape
    a = CalibArgs(conf=_ptr(conf, torch.float32, "conf"), drafts=_ptr(drafts, torch.int32, "drafts"),
                  pred=_ptr(pred, torch.int32, "pred"), cu=_ptr(cu, torch.int32, "cu"),
                  w_verify=_ptr(w_verify, torch.int32, "w_verify"), B=B, gamma=g1 + 1, rows_cap=pred.numel(),
                  n_bins=n_bins, bin_count=_ptr(bin_count, torch.int64, "bin_count"),
                  bin_match=_ptr(bin_match, torch.int64, "bin_match"),
                  bin_conf_fx=_ptr(bin_conf_fx, torch.int64, "bin_conf_fx"), ece=_ptr(ece, torch.float64, "ece"),
                  req_verified=_ptr(req_verified, torch.int32, "req_verified"),
                  req_matched=_ptr(req_matched, torch.int32, "req_matched"),
                  workspace=_ptr(workspace, name="workspace"), workspace_bytes=workspace.numel() * workspace.element_size())
    _check("rv_calibration", load().rv_calibration(ctypes.byref(a), _stream(stream)))


def rv_estimator_state_bytes(B, gamma):
    n = _sz(0)
    _check("rv_estimator_state_bytes", load().rv_estimator_state_bytes(B, gamma, ctypes.byref(n)))
    return n.value


def estimator_state_views(state, B, gamma):
    """Views of the estimator state buffer (uint8 tensor) by field, per the
    layout rv_block_accept_estimate documents."""
    G = gamma - 1
    i32 = lambda off, n: state[off:off + 4 * n].view(torch.int32)
    f32 = lambda off, n: state[off:off + 4 * n].view(torch.float32)
    return {"pos": i32(0, B), "left": i32(4 * B, B), "done": i32(8 * B, B), "base": i32(12 * B, B),
            "count": i32(16 * B, B), "S": f32(20 * B, B), "E": f32(24 * B, B), "last": f32(28 * B, B),
            "sum": state[32 * B:40 * B].view(torch.float64), "tok": i32(40 * B, B * G).view(B, G),
            "lq": f32(40 * B + 4 * B * G, B * G).view(B, G)}


def rv_block_accept_estimate(cu, w_verify, accept, drafts, ctx, rule, state, workspace, pred=None, logits=None,
                             q_rows=None, stream=None):
    B, g1 = drafts.shape
    rows_cap = pred.numel() if pred is not None else logits.shape[0]
    V = logits.shape[1] if logits is not None else 1
    a = EstimateArgs(cu=_ptr(cu, torch.int32, "cu"), w_verify=_ptr(w_verify, torch.int32, "w_verify"),
                     accept=_ptr(accept, torch.int32, "accept"), drafts=_ptr(drafts, torch.int32, "drafts"),
                     ctx=_ptr(ctx, torch.int32, "ctx"), pred=_ptr(pred, torch.int32, "pred"),
                     logits=_ptr(logits, torch.float32, "logits"), q_rows=_ptr(q_rows, torch.float32, "q_rows"),
                     B=B, gamma=g1 + 1, rows_cap=rows_cap, V=V, rule=rule, state=_ptr(state, name="state"),
                     workspace=_ptr(workspace, name="workspace"),
                     workspace_bytes=workspace.numel() * workspace.element_size())
    _check("rv_block_accept_estimate", load().rv_block_accept_estimate(ctypes.byref(a), _stream(stream)))


def rv_fit_cost_model(bs, M, t, alpha_len=0, theta_len=0):
    """Least-squares fit of the step-time model from host samples (sequences
    of numbers).  Returns (coef [bias, a, th], alpha table, theta table) as
    Python lists; the tables are empty when their length is 0."""
    n = len(bs)
    arr = lambda xs: (_f64 * max(len(xs), 1))(*[float(x) for x in xs])
    coef = (_f64 * 3)()
    al = (_f64 * max(alpha_len, 1))()
    th = (_f64 * max(theta_len, 1))()
    _check("rv_fit_cost_model", load().rv_fit_cost_model(arr(bs), arr(M), arr(t), n, coef,
                                                         al if alpha_len else None, alpha_len,
                                                         th if theta_len else None, theta_len))
    return list(coef), list(al[:alpha_len]), list(th[:theta_len])


def rv_lm_tiled_weight_bytes(V, H, dtype=RV_BF16):
    n = _sz(0)
    _check("rv_lm_tiled_weight_bytes", load().rv_lm_tiled_weight_bytes(V, H, dtype, ctypes.byref(n)))
    return n.value


def rv_lm_tile_weight(W, W_tiled=None, stream=None):
    """Write the tiled copy of W [V][H] (bf16) made for w_layout=RV_W_TILED;
    allocates it with torch when W_tiled is None.  Returns W_tiled."""
    V, H = W.shape
    n = rv_lm_tiled_weight_bytes(V, H, _dtype_code(W))
    if W_tiled is None:
        W_tiled = torch.empty(n, dtype=torch.uint8, device=W.device)
    if W_tiled.numel() * W_tiled.element_size() < n:
        raise ValueError(f"W_tiled holds {W_tiled.numel() * W_tiled.element_size()} bytes, needs {n}")
    _check("rv_lm_tile_weight", load().rv_lm_tile_weight(_ptr(W, W.dtype, "W"), _ptr(W_tiled, name="W_tiled"),
                                                         V, H, _dtype_code(W), _stream(stream)))
    return W_tiled


def _lm_args(hidden, W, mm, cu, w_commit, w_verify, drafts, rule, pred, accept, bonus, ceiling, workspace,
             logits, q_rows, u, u_bonus, W_tiled):
    rows_cap, H = hidden.shape
    V = W.shape[0]
    B, g1 = drafts.shape
    Wp = _ptr(W, hidden.dtype, "W") if W_tiled is None else _ptr(W_tiled, name="W_tiled")
    return LmArgs(hidden=_ptr(hidden, hidden.dtype, "hidden"), W=Wp,
                  mm=_ptr(mm, torch.int32, "mm"), cu=_ptr(cu, torch.int32, "cu"),
                  w_commit=_ptr(w_commit, torch.int32, "w_commit"), w_verify=_ptr(w_verify, torch.int32, "w_verify"),
                  drafts=_ptr(drafts, torch.int32, "drafts"), q_rows=_ptr(q_rows, torch.float32, "q_rows"),
                  u=_ptr(u, torch.float32, "u"), u_bonus=_ptr(u_bonus, torch.float32, "u_bonus"),
                  B=B, gamma=g1 + 1, rows_cap=rows_cap, H=H, V=V, dtype=_dtype_code(hidden), rule=rule,
                  w_layout=RV_W_ROWS if W_tiled is None else RV_W_TILED,
                  pred=_ptr(pred, torch.int32, "pred"), accept=_ptr(accept, torch.int32, "accept"),
                  bonus=_ptr(bonus, torch.int32, "bonus"), ceiling=_ptr(ceiling, torch.int32, "ceiling"),
                  logits=_ptr(logits, torch.float32, "logits"),
                  workspace=_ptr(workspace, name="workspace"),
                  workspace_bytes=0 if workspace is None else workspace.numel() * workspace.element_size())


def rv_lm_head_accept(hidden, W, mm, cu, w_commit, w_verify, drafts, rule, pred, accept, bonus, ceiling,
                      workspace, logits=None, q_rows=None, u=None, u_bonus=None, stream=None, W_tiled=None,
                      cache=None, launch=True):
    """W [V][H] gives the vocabulary size; with W_tiled (rv_lm_tile_weight of
    W) the kernel reads the tiled copy instead."""
    args = (hidden, W, mm, cu, w_commit, w_verify, drafts, rule, pred, accept, bonus, ceiling, workspace,
            logits, q_rows, u, u_bonus, W_tiled)
    a = _cached(cache, "lm", args, lambda: _lm_args(*args))
    if not launch:
        return
    _check("rv_lm_head_accept", load().rv_lm_head_accept(ctypes.byref(a), _stream(stream)))


def rv_lm_head_accept_noalloc(hidden, W, mm, cu, w_commit, w_verify, drafts, rule, pred, accept, bonus, ceiling,
                              status=None, logits=None, q_rows=None, u=None, u_bonus=None, stream=None,
                              W_tiled=None):
    """rv_lm_head_accept with the library's static scratch instead of a
    workspace; ``status`` (optional, at least 256 bytes of device memory)
    receives the sticky device status."""
    a = _lm_args(hidden, W, mm, cu, w_commit, w_verify, drafts, rule, pred, accept, bonus, ceiling, status,
                 logits, q_rows, u, u_bonus, W_tiled)
    _check("rv_lm_head_accept_noalloc", load().rv_lm_head_accept_noalloc(ctypes.byref(a), _stream(stream)))


def rv_compact_scatter(cu, w_verify, accept, bonus, drafts, slot, ctx, anchor, req_to_token, commit_cu,
                       commit_tok, commit_slot, free_slots, free_count, workspace, hist=None, hist_len=None,
                       stream=None, cache=None, launch=True):
    args = (cu, w_verify, accept, bonus, drafts, slot, ctx, anchor, req_to_token, commit_cu, commit_tok,
            commit_slot, free_slots, free_count, workspace, hist, hist_len)
    a = _cached(cache, "scatter", args, lambda: _scatter_args(*args))
    if not launch:
        return
    _check("rv_compact_scatter", load().rv_compact_scatter(ctypes.byref(a), _stream(stream)))


def _scatter_args(cu, w_verify, accept, bonus, drafts, slot, ctx, anchor, req_to_token, commit_cu, commit_tok,
                  commit_slot, free_slots, free_count, workspace, hist, hist_len):
    B, g1 = drafts.shape
    return ScatterArgs(cu=_ptr(cu, torch.int32, "cu"), w_verify=_ptr(w_verify, torch.int32, "w_verify"),
                    accept=_ptr(accept, torch.int32, "accept"), bonus=_ptr(bonus, torch.int32, "bonus"),
                    drafts=_ptr(drafts, torch.int32, "drafts"), slot=_ptr(slot, torch.int32, "slot"),
                    B=B, gamma=g1 + 1, r2t_stride=req_to_token.shape[1],
                    hist_stride=hist.shape[1] if hist is not None else 0,
                    ctx=_ptr(ctx, torch.int32, "ctx"), anchor=_ptr(anchor, torch.int32, "anchor"),
                    req_to_token=_ptr(req_to_token, torch.int32, "req_to_token"),
                    hist=_ptr(hist, torch.int32, "hist"), hist_len=_ptr(hist_len, torch.int32, "hist_len"),
                    commit_cu=_ptr(commit_cu, torch.int32, "commit_cu"),
                    commit_tok=_ptr(commit_tok, torch.int32, "commit_tok"),
                    commit_slot=_ptr(commit_slot, torch.int32, "commit_slot"),
                    free_slots=_ptr(free_slots, torch.int32, "free_slots"),
                    free_count=_ptr(free_count, torch.int32, "free_count"),
                    workspace=_ptr(workspace, name="workspace"), workspace_bytes=workspace.numel() * workspace.element_size())
