"""Thin Python binding of libmoonep_hip.so (the MoonEP hot path on gfx950).

Argument marshalling only: every step runs in the HIP library.  Functions
carry the C entry points' names and take torch tensors that live on the GPU
(torch is used for device memory and the current stream).  The library must
have been built (``python -m moe_expert_load_amd.build``); without it every
call raises -- there is no CPU fallback.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoonep_hip.so")

MOE_OK, MOE_EINVAL, MOE_EHIP, MOE_ELIMIT = 0, -1, -2, -3
MODE_TRAIN, MODE_INFER = 0, 1
STATUS_BAD_ID, STATUS_UNBALANCED, STATUS_CAPACITY, STATUS_INTERNAL = 1, 2, 4, 8
PLAN_ASCENDING, PLAN_LARGEST_FIRST = 0, 1
PLAN_FIELDS = ("counts", "load0", "route", "cu_seqlens", "slot_expert",
               "n_redundant", "src_rank", "moves", "status", "workspace")
ENTRY_POINTS = ("moe_plan_sizes", "moe_plan_run", "moe_plan_run_policy", "moe_prefetch_weight",
                "moe_dispatch", "moe_gemm_workspace_size", "moe_grouped_gemm",
                "moe_grouped_gemm_noalloc",
                "moe_combine", "moe_grouped_gemm_wgrad", "moe_reduce_grad",
                "moe_combine_backward", "moe_grouped_gemm_dgrad",
                "moe_dispatch_backward", "moe_route_encode", "moe_dispatch_dedup",
                "moe_grouped_gemm_swiglu", "moe_swiglu_backward", "moe_strerror")


class MoeError(RuntimeError):
    def __init__(self, code, where):
        super().__init__("%s failed: %s (%d)" % (where, moe_strerror(code), code))
        self.code = code


class moe_cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("R", "S", "E", "K", "H", "Hp", "B", "mode")]

    def __repr__(self):
        return "moe_cfg(%s)" % ", ".join("%s=%d" % (n, getattr(self, n)) for n, _ in self._fields_)


class moe_plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in PLAN_FIELDS]


_lib = None


def load(path=None):
    """Load (once) and return the library; raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("MoonEP HIP library not built: %s is missing "
                           "(run python -m moe_expert_load_amd.build)" % p)
    lib = ctypes.CDLL(p)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    C = ctypes.POINTER(moe_cfg)
    PL = ctypes.POINTER(moe_plan)
    sig = {
        "moe_plan_sizes": [C, ctypes.POINTER(SZ)],
        "moe_plan_run": [C, P, PL, P],
        "moe_plan_run_policy": [C, P, PL, I32, P],
        "moe_prefetch_weight": [C, PL, P, P, P],
        "moe_dispatch": [C, PL, P, P, P],
        "moe_gemm_workspace_size": [C, ctypes.POINTER(SZ)],
        "moe_grouped_gemm": [C, P, P, P, P, P, I32, I32, P, P],
        "moe_grouped_gemm_noalloc": [C, P, P, P, P, P, I32, I32, P],
        "moe_combine": [C, PL, P, P, P, P],
        "moe_grouped_gemm_wgrad": [C, PL, P, P, P, P, P, P],
        "moe_reduce_grad": [C, PL, P, P, P],
        "moe_combine_backward": [C, PL, P, P, P, P, P, P],
        "moe_grouped_gemm_dgrad": [C, P, P, P, P, P, I32, I32, P, P],
        "moe_dispatch_backward": [C, PL, P, P, P],
        "moe_route_encode": [C, PL, P, P],
        "moe_dispatch_dedup": [C, P, P, P, P],
        "moe_grouped_gemm_swiglu": [C, P, P, P, P, P, P, I32, I32, P, P],
        "moe_swiglu_backward": [C, P, P, P, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.moe_strerror.argtypes = [ctypes.c_int]
    lib.moe_strerror.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def make_cfg(R, S, E, K, H, Hp, B, mode=MODE_TRAIN):
    return moe_cfg(R, S, E, K, H, Hp, B, mode)


def _check(code, where):
    if code != MOE_OK:
        raise MoeError(code, where)


def _ptr(t, dtype, numel=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if numel is not None and t.numel() < numel:
        raise ValueError("%s holds %d elements, needs %d" % (name, t.numel(), numel))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def moe_strerror(code):
    return load().moe_strerror(int(code)).decode()


def moe_plan_sizes(cfg):
    out = (ctypes.c_size_t * 10)()
    _check(load().moe_plan_sizes(ctypes.byref(cfg), out), "moe_plan_sizes")
    return [int(v) for v in out]


def moe_gemm_workspace_size(cfg):
    out = ctypes.c_size_t()
    _check(load().moe_gemm_workspace_size(ctypes.byref(cfg), ctypes.byref(out)),
           "moe_gemm_workspace_size")
    return int(out.value)


class Plan:
    """Device arrays of one moe_plan, allocated with torch (int32 + bytes)."""

    def __init__(self, cfg, device="cuda"):
        sizes = moe_plan_sizes(cfg)
        self.cfg = cfg
        self.arrays = {}
        for name, nbytes in zip(PLAN_FIELDS, sizes):
            if name == "workspace":
                self.arrays[name] = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            else:
                self.arrays[name] = torch.empty(max(nbytes // 4, 1), dtype=torch.int32, device=device)
        self._c = moe_plan(*[ctypes.c_void_p(self.arrays[n].data_ptr()) for n in PLAN_FIELDS])

    def __getattr__(self, name):
        arrays = self.__dict__.get("arrays")
        if arrays is not None and name in arrays:
            return arrays[name]
        raise AttributeError(name)

    @property
    def c(self):
        return ctypes.byref(self._c)

    # shaped views of the outputs
    def views(self):
        c = self.cfg
        a = self.arrays
        st = a["status"][:4]
        return {
            "counts": a["counts"][:c.E],
            "load0": a["load0"][:c.R],
            "route": a["route"][:c.R * c.S * c.K],
            "cu_seqlens": a["cu_seqlens"][:c.R * (c.E + c.B + 1)].view(c.R, c.E + c.B + 1),
            "slot_expert": a["slot_expert"][:c.R * c.B].view(c.R, c.B),
            "n_redundant": a["n_redundant"][:c.R],
            "src_rank": a["src_rank"][:c.R],
            "moves": a["moves"][:4 * (c.E + c.R - 1)].view(-1, 4),
            "status": st,
        }


def moe_plan_run(cfg, topk_ids, plan, stream=None):
    n = cfg.R * cfg.S * cfg.K
    ids = _ptr(topk_ids, torch.int32, n, "topk_ids") if n else None
    _check(load().moe_plan_run(ctypes.byref(cfg), ids, plan.c, _stream(stream)), "moe_plan_run")


def moe_plan_run_policy(cfg, topk_ids, plan, policy, stream=None):
    n = cfg.R * cfg.S * cfg.K
    ids = _ptr(topk_ids, torch.int32, n, "topk_ids") if n else None
    _check(load().moe_plan_run_policy(ctypes.byref(cfg), ids, plan.c, int(policy),
                                      _stream(stream)), "moe_plan_run_policy")


def moe_prefetch_weight(cfg, plan, w_home, w_pref, stream=None):
    hh = cfg.H * cfg.Hp
    a = _ptr(w_home, torch.bfloat16, cfg.E * hh, "w_home")
    b = _ptr(w_pref, torch.bfloat16, cfg.R * cfg.B * hh, "w_pref") if cfg.B else None
    _check(load().moe_prefetch_weight(ctypes.byref(cfg), plan.c, a, b, _stream(stream)),
           "moe_prefetch_weight")


def moe_dispatch(cfg, plan, x, xperm, stream=None):
    a = _ptr(x, torch.bfloat16, cfg.R * cfg.S * cfg.H, "x")
    b = _ptr(xperm, torch.bfloat16, cfg.R * cfg.S * cfg.K * cfg.H, "xperm")
    _check(load().moe_dispatch(ctypes.byref(cfg), plan.c, a, b, _stream(stream)), "moe_dispatch")


def moe_grouped_gemm(cfg, xperm, w_home, w_pref, cu_seqlens, y, rank_begin, rank_end,
                     workspace, stream=None):
    SK = cfg.S * cfg.K
    hh = cfg.H * cfg.Hp
    args = (ctypes.byref(cfg),
            _ptr(xperm, torch.bfloat16, cfg.R * SK * cfg.H, "xperm"),
            _ptr(w_home, torch.bfloat16, cfg.E * hh, "w_home"),
            _ptr(w_pref, torch.bfloat16, cfg.R * cfg.B * hh, "w_pref") if cfg.B else None,
            _ptr(cu_seqlens, torch.int32, cfg.R * (cfg.E + cfg.B + 1), "cu_seqlens"),
            _ptr(y, torch.bfloat16, cfg.R * SK * cfg.Hp, "y"),
            int(rank_begin), int(rank_end),
            _ptr(workspace, torch.uint8, moe_gemm_workspace_size(cfg), "workspace"),
            _stream(stream))
    _check(load().moe_grouped_gemm(*args), "moe_grouped_gemm")


def moe_grouped_gemm_noalloc(cfg, xperm, w_home, w_pref, cu_seqlens, y, rank_begin, rank_end,
                             stream=None):
    SK = cfg.S * cfg.K
    hh = cfg.H * cfg.Hp
    args = (ctypes.byref(cfg),
            _ptr(xperm, torch.bfloat16, cfg.R * SK * cfg.H, "xperm"),
            _ptr(w_home, torch.bfloat16, cfg.E * hh, "w_home"),
            _ptr(w_pref, torch.bfloat16, cfg.R * cfg.B * hh, "w_pref") if cfg.B else None,
            _ptr(cu_seqlens, torch.int32, cfg.R * (cfg.E + cfg.B + 1), "cu_seqlens"),
            _ptr(y, torch.bfloat16, cfg.R * SK * cfg.Hp, "y"),
            int(rank_begin), int(rank_end), _stream(stream))
    _check(load().moe_grouped_gemm_noalloc(*args), "moe_grouped_gemm_noalloc")


def moe_combine(cfg, plan, y, gates, out, stream=None):
    ntok = cfg.R * cfg.S
    a = _ptr(y, torch.bfloat16, ntok * cfg.K * cfg.Hp, "y")
    g = _ptr(gates, torch.float32, ntok * cfg.K, "gates")
    o = _ptr(out, torch.bfloat16, ntok * cfg.Hp, "out")
    _check(load().moe_combine(ctypes.byref(cfg), plan.c, a, g, o, _stream(stream)), "moe_combine")


def moe_grouped_gemm_wgrad(cfg, plan, xperm, dy, grad_home, grad_pref, workspace, stream=None):
    SK = cfg.S * cfg.K
    hh = cfg.H * cfg.Hp
    args = (ctypes.byref(cfg), plan.c,
            _ptr(xperm, torch.bfloat16, cfg.R * SK * cfg.H, "xperm"),
            _ptr(dy, torch.bfloat16, cfg.R * SK * cfg.Hp, "dy"),
            _ptr(grad_home, torch.float32, cfg.E * hh, "grad_home"),
            _ptr(grad_pref, torch.float32, cfg.R * cfg.B * hh, "grad_pref") if cfg.B else None,
            _ptr(workspace, torch.uint8, moe_gemm_workspace_size(cfg), "workspace"),
            _stream(stream))
    _check(load().moe_grouped_gemm_wgrad(*args), "moe_grouped_gemm_wgrad")


def moe_combine_backward(cfg, plan, dout, y, gates, dy, dgates, stream=None):
    ntok = cfg.R * cfg.S
    args = (ctypes.byref(cfg), plan.c,
            _ptr(dout, torch.bfloat16, ntok * cfg.Hp, "dout"),
            _ptr(y, torch.bfloat16, ntok * cfg.K * cfg.Hp, "y"),
            _ptr(gates, torch.float32, ntok * cfg.K, "gates"),
            _ptr(dy, torch.bfloat16, ntok * cfg.K * cfg.Hp, "dy"),
            _ptr(dgates, torch.float32, ntok * cfg.K, "dgates"),
            _stream(stream))
    _check(load().moe_combine_backward(*args), "moe_combine_backward")


def moe_grouped_gemm_dgrad(cfg, dy, w_home, w_pref, cu_seqlens, dxperm, rank_begin, rank_end,
                           workspace, stream=None):
    SK = cfg.S * cfg.K
    hh = cfg.H * cfg.Hp
    args = (ctypes.byref(cfg),
            _ptr(dy, torch.bfloat16, cfg.R * SK * cfg.Hp, "dy"),
            _ptr(w_home, torch.bfloat16, cfg.E * hh, "w_home"),
            _ptr(w_pref, torch.bfloat16, cfg.R * cfg.B * hh, "w_pref") if cfg.B else None,
            _ptr(cu_seqlens, torch.int32, cfg.R * (cfg.E + cfg.B + 1), "cu_seqlens"),
            _ptr(dxperm, torch.bfloat16, cfg.R * SK * cfg.H, "dxperm"),
            int(rank_begin), int(rank_end),
            _ptr(workspace, torch.uint8, moe_gemm_workspace_size(cfg), "workspace"),
            _stream(stream))
    _check(load().moe_grouped_gemm_dgrad(*args), "moe_grouped_gemm_dgrad")


def moe_grouped_gemm_swiglu(cfg, xperm, w13_home, w13_pref, cu_seqlens, act, h13, rank_begin,
                            rank_end, workspace, stream=None):
    """cfg.Hp is the intermediate size H'; W13 rows are [H][2H'] (gate | up)."""
    SK = cfg.S * cfg.K
    hh = cfg.H * 2 * cfg.Hp
    args = (ctypes.byref(cfg),
            _ptr(xperm, torch.bfloat16, cfg.R * SK * cfg.H, "xperm"),
            _ptr(w13_home, torch.bfloat16, cfg.E * hh, "w13_home"),
            _ptr(w13_pref, torch.bfloat16, cfg.R * cfg.B * hh, "w13_pref") if cfg.B else None,
            _ptr(cu_seqlens, torch.int32, cfg.R * (cfg.E + cfg.B + 1), "cu_seqlens"),
            _ptr(act, torch.bfloat16, cfg.R * SK * cfg.Hp, "act"),
            _ptr(h13, torch.bfloat16, cfg.R * SK * 2 * cfg.Hp, "h13"),
            int(rank_begin), int(rank_end),
            _ptr(workspace, torch.uint8, moe_gemm_workspace_size(cfg), "workspace"),
            _stream(stream))
    _check(load().moe_grouped_gemm_swiglu(*args), "moe_grouped_gemm_swiglu")


def moe_swiglu_backward(cfg, h13, dact, dh13, stream=None):
    rows = cfg.R * cfg.S * cfg.K
    args = (ctypes.byref(cfg),
            _ptr(h13, torch.bfloat16, rows * 2 * cfg.Hp, "h13"),
            _ptr(dact, torch.bfloat16, rows * cfg.Hp, "dact"),
            _ptr(dh13, torch.bfloat16, rows * 2 * cfg.Hp, "dh13"),
            _stream(stream))
    _check(load().moe_swiglu_backward(*args), "moe_swiglu_backward")


def moe_dispatch_backward(cfg, plan, dxperm, dx, stream=None):
    ntok = cfg.R * cfg.S
    a = _ptr(dxperm, torch.bfloat16, ntok * cfg.K * cfg.H, "dxperm")
    o = _ptr(dx, torch.bfloat16, ntok * cfg.H, "dx")
    _check(load().moe_dispatch_backward(ctypes.byref(cfg), plan.c, a, o, _stream(stream)),
           "moe_dispatch_backward")


def moe_route_encode(cfg, plan, route_enc, stream=None):
    e = _ptr(route_enc, torch.int32, cfg.R * cfg.S * cfg.K, "route_enc")
    _check(load().moe_route_encode(ctypes.byref(cfg), plan.c, e, _stream(stream)),
           "moe_route_encode")


def moe_dispatch_dedup(cfg, route_enc, x, xperm, stream=None):
    ntok = cfg.R * cfg.S
    args = (ctypes.byref(cfg),
            _ptr(route_enc, torch.int32, ntok * cfg.K, "route_enc"),
            _ptr(x, torch.bfloat16, ntok * cfg.H, "x"),
            _ptr(xperm, torch.bfloat16, ntok * cfg.K * cfg.H, "xperm"),
            _stream(stream))
    _check(load().moe_dispatch_dedup(*args), "moe_dispatch_dedup")


def moe_reduce_grad(cfg, plan, grad_home, grad_pref, stream=None):
    hh = cfg.H * cfg.Hp
    a = _ptr(grad_home, torch.float32, cfg.E * hh, "grad_home")
    b = _ptr(grad_pref, torch.float32, cfg.R * cfg.B * hh, "grad_pref") if cfg.B else None
    _check(load().moe_reduce_grad(ctypes.byref(cfg), plan.c, a, b, _stream(stream)),
           "moe_reduce_grad")
