"""MI355X (gfx950) sparse-MoE FFN forward of GLM-4.5 / GLM-5: Python binding of libmoe.so.

Argument marshalling only: every step of the layer runs in the HIP kernels behind the C ABI declared in
include/moe.h (moe_route, moe_dispatch, moe_forward, moe_workspace_size, moe_status_str). Tensors are
torch device tensors; the binding checks their device, dtype, shape and contiguity, passes raw pointers
and the current HIP stream, and raises MoeError on any status other than MOE_OK. There is no fallback:
without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_ROUTE_SCORES_IN, MOE_ROUTE_SCORES_OUT, MOE_ROUTE_PREPARED = 1, 2, 4

EXPORTED = ["moe_check_config", "moe_workspace_size", "moe_dispatch_workspace_size", "moe_router_prepared_size",
            "moe_router_prepare", "moe_route", "moe_dispatch", "moe_forward", "moe_forward_routed",
            "moe_forward_noalloc", "moe_noalloc_scratch_bytes", "moe_dense_workspace_size", "moe_dense_forward",
            "moe_status_str", "moe_profile_begin",
            "moe_profile_begin_mask", "moe_profile_end", "moe_stage_name", "moe_stage_count"]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {moe_status_str(status)}")
        self.status = status


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("hidden_size", ctypes.c_int32),
        ("n_routed_experts", ctypes.c_int32),
        ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("num_experts_per_tok", ctypes.c_int32),
        ("moe_intermediate_size", ctypes.c_int32),
        ("n_shared_experts", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float),
        ("norm_topk_prob", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("alpha_on_output", ctypes.c_int32),
        ("swiglu_limit", ctypes.c_float),
    ]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_router", "e_bias", "gate_up", "down", "sh_gate", "sh_up", "sh_down",
                                               "w_router_prepared")]


_lib = None


def lib():
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
        cp = ctypes.POINTER(MoeConfig)
        L.moe_check_config.argtypes = [cp]
        L.moe_check_config.restype = ctypes.c_int
        L.moe_workspace_size.argtypes = [cp, i64]
        L.moe_workspace_size.restype = ctypes.c_size_t
        L.moe_dispatch_workspace_size.argtypes = [cp, i64]
        L.moe_dispatch_workspace_size.restype = ctypes.c_size_t
        L.moe_router_prepared_size.argtypes = [cp]
        L.moe_router_prepared_size.restype = ctypes.c_size_t
        L.moe_router_prepare.argtypes = [cp, vp, vp, ctypes.c_size_t, vp]
        L.moe_router_prepare.restype = ctypes.c_int
        L.moe_route.argtypes = [cp, i64, vp, vp, vp, vp, u32, vp, vp, vp, ctypes.c_size_t, vp]
        L.moe_route.restype = ctypes.c_int
        L.moe_dispatch.argtypes = [cp, i64, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.moe_dispatch.restype = ctypes.c_int
        L.moe_forward.argtypes = [cp, i64, vp, ctypes.POINTER(MoeWeights), vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.moe_forward_routed.argtypes = [cp, i64, vp, ctypes.POINTER(MoeWeights), vp, vp, vp, vp, vp,
                                         ctypes.c_size_t, vp]
        L.moe_forward_noalloc.argtypes = [cp, i64, vp, ctypes.POINTER(MoeWeights), vp, vp, vp, vp, vp]
        L.moe_forward_noalloc.restype = ctypes.c_int
        L.moe_noalloc_scratch_bytes.argtypes = []
        L.moe_noalloc_scratch_bytes.restype = ctypes.c_size_t
        L.moe_dense_workspace_size.argtypes = [i64, i32, i32, i32]
        L.moe_dense_workspace_size.restype = ctypes.c_size_t
        L.moe_dense_forward.argtypes = [i64, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                        vp]
        L.moe_forward.restype = ctypes.c_int
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_profile_begin.argtypes = []
        L.moe_profile_begin_mask.argtypes = [u32]
        L.moe_profile_begin.restype = ctypes.c_int
        L.moe_profile_end.argtypes = [vp, vp, i32]
        L.moe_profile_end.restype = ctypes.c_int
        L.moe_stage_name.argtypes = [i32]
        L.moe_stage_name.restype = ctypes.c_char_p
        L.moe_stage_count.argtypes = []
        L.moe_stage_count.restype = i32
        _lib = L
    return _lib


def make_config(D, E, G, TG, k, d, n_shared=1, alpha=1.0, norm=True, eps=1e-20, dtype="bf16",
                alpha_on_output=False, limit=0.0) -> MoeConfig:
    """moe_config from the pages' config fields (hidden_size, n_routed_experts, n_group, topk_group,
    num_experts_per_tok, moe_intermediate_size, n_shared_experts, routed_scaling_factor, norm_topk_prob),
    where alpha goes, and the SwiGLU clamp bound (0: none)."""
    dt = {"bf16": MOE_BF16, "f32": MOE_F32}[dtype] if isinstance(dtype, str) else int(dtype)
    return MoeConfig(D, E, G, TG, k, d, n_shared, float(alpha), int(bool(norm)), float(eps), dt,
                     int(bool(alpha_on_output)), float(limit))


def config_of(w) -> MoeConfig:
    """moe_config from an object with fields D, E, G, TG, k, d, n_shared, alpha, norm, eps, dtype (and
    optionally alpha_on_output, limit)."""
    return make_config(w.D, w.E, w.G, w.TG, w.k, w.d, w.n_shared, w.alpha, w.norm, w.eps, w.dtype,
                       getattr(w, "alpha_on_output", False), getattr(w, "limit", 0.0))


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def _ptr(t, name, dtype=None, shape=None, required=True):
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    import torch

    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _act_dtype(cfg: MoeConfig):
    import torch

    return torch.float32 if cfg.dtype == MOE_F32 else torch.bfloat16


def _check(status, what):
    if status != MOE_OK:
        raise MoeError(status, what)


def moe_check_config(cfg: MoeConfig) -> int:
    return lib().moe_check_config(ctypes.byref(cfg))


def moe_workspace_size(cfg: MoeConfig, N: int) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(cfg), int(N)))


def alloc_workspace(cfg: MoeConfig, N: int, device="cuda"):
    import torch

    n = moe_workspace_size(cfg, N)
    if n == 0 and N > 0:
        _check(moe_check_config(cfg) or MOE_ERR_INVALID_ARG, "moe_workspace_size")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_dispatch_workspace_size(cfg: MoeConfig, N: int) -> int:
    return int(lib().moe_dispatch_workspace_size(ctypes.byref(cfg), int(N)))


def moe_router_prepared_size(cfg: MoeConfig) -> int:
    return int(lib().moe_router_prepared_size(ctypes.byref(cfg)))


def moe_router_prepare(cfg: MoeConfig, w_router, prepared=None, stream=None):
    """The [3, E, D] bf16 pieces of w_router (bf16 layers), for moe_weights.w_router_prepared or moe_route
    with MOE_ROUTE_PREPARED. Returns `prepared` (allocated here as a bf16 tensor when None)."""
    import torch

    E, D = cfg.n_routed_experts, cfg.hidden_size
    if prepared is None:
        prepared = torch.empty((3, E, D), dtype=torch.bfloat16, device=w_router.device)
    st = lib().moe_router_prepare(ctypes.byref(cfg), _ptr(w_router, "w_router", torch.float32, (E, D)),
                                  _ptr(prepared, "prepared"), prepared.numel() * prepared.element_size(),
                                  _stream(stream))
    _check(st, "moe_router_prepare")
    return prepared


def moe_route(cfg: MoeConfig, N: int, x, w_router, e_bias, scores, topk_idx, topk_w, flags: int = 0,
              workspace=None, stream=None):
    """Router on the GPU. With flags = MOE_ROUTE_SCORES_IN, `scores` [N, E] is read and x / w_router /
    workspace are ignored; otherwise `workspace` (uint8, moe_workspace_size bytes) is required, `scores`
    is written with MOE_ROUTE_SCORES_OUT (else it may be None), and with MOE_ROUTE_PREPARED `w_router` is
    the output of moe_router_prepare."""
    import torch

    E, D, k = cfg.n_routed_experts, cfg.hidden_size, cfg.num_experts_per_tok
    scores_in = bool(flags & MOE_ROUTE_SCORES_IN)
    prepared = bool(flags & MOE_ROUTE_PREPARED)
    need_scores = scores_in or bool(flags & MOE_ROUTE_SCORES_OUT)
    st = lib().moe_route(
        ctypes.byref(cfg), int(N),
        _ptr(x, "x", _act_dtype(cfg), (N, D), required=not scores_in),
        _ptr(w_router, "w_router", torch.bfloat16 if prepared else torch.float32, (3, E, D) if prepared else (E, D),
             required=not scores_in),
        _ptr(e_bias, "e_bias", torch.float32, (E,)),
        _ptr(scores, "scores", torch.float32, (N, E), required=need_scores),
        int(flags),
        _ptr(topk_idx, "topk_idx", torch.int32, (N, k)),
        _ptr(topk_w, "topk_w", torch.float32, (N, k)),
        _ptr(workspace, "workspace", torch.uint8, required=not scores_in),
        0 if workspace is None else workspace.numel(),
        _stream(stream))
    _check(st, "moe_route")


def moe_dispatch(cfg: MoeConfig, N: int, topk_idx, counts, offsets, sorted_pair, inv_row, workspace=None,
                 stream=None):
    """Dispatch on the GPU; `workspace` (uint8, moe_dispatch_workspace_size bytes) may be None when that
    size is 0."""
    import torch

    E, k = cfg.n_routed_experts, cfg.num_experts_per_tok
    st = lib().moe_dispatch(
        ctypes.byref(cfg), int(N),
        _ptr(topk_idx, "topk_idx", torch.int32, (N, k)),
        _ptr(counts, "counts", torch.int32, (E,)),
        _ptr(offsets, "offsets", torch.int32, (E + 1,)),
        _ptr(sorted_pair, "sorted_pair", torch.int32, (N * k,)),
        _ptr(inv_row, "inv_row", torch.int32, (N * k,)),
        _ptr(workspace, "workspace", torch.uint8, required=False),
        0 if workspace is None else workspace.numel(),
        _stream(stream))
    _check(st, "moe_dispatch")


def weights_struct(cfg: MoeConfig, w: dict) -> MoeWeights:
    """MoeWeights from a dict of device tensors: w_router, e_bias, gate_up, down, sh_gate, sh_up, sh_down and
    optionally w_router_prepared (the router pair may be absent for moe_forward_routed)."""
    import torch

    E, D, d = cfg.n_routed_experts, cfg.hidden_size, cfg.moe_intermediate_size
    dsh = d * cfg.n_shared_experts
    adt = _act_dtype(cfg)
    sh = cfg.n_shared_experts > 0
    prep = w.get("w_router_prepared")
    return MoeWeights(
        _ptr(w.get("w_router"), "w_router", torch.float32, (E, D), required=False),
        _ptr(w.get("e_bias"), "e_bias", torch.float32, (E,), required=False),
        _ptr(w["gate_up"], "gate_up", adt, (E, 2 * d, D)),
        _ptr(w["down"], "down", adt, (E, D, d)),
        _ptr(w.get("sh_gate"), "sh_gate", adt, (dsh, D), required=sh) if sh else None,
        _ptr(w.get("sh_up"), "sh_up", adt, (dsh, D), required=sh) if sh else None,
        _ptr(w.get("sh_down"), "sh_down", adt, (D, dsh), required=sh) if sh else None,
        _ptr(prep, "w_router_prepared", torch.bfloat16, (3, E, D), required=False),
    )


def moe_forward(cfg: MoeConfig, N: int, x, weights, y, workspace, topk_idx_out=None, topk_w_out=None,
                counts_out=None, stream=None):
    """The whole layer on the GPU; `weights` is a MoeWeights or a dict accepted by weights_struct."""
    import torch

    E, D, k = cfg.n_routed_experts, cfg.hidden_size, cfg.num_experts_per_tok
    ws = weights if isinstance(weights, MoeWeights) else weights_struct(cfg, weights)
    adt = _act_dtype(cfg)
    st = lib().moe_forward(
        ctypes.byref(cfg), int(N),
        _ptr(x, "x", adt, (N, D)),
        ctypes.byref(ws),
        _ptr(y, "y", adt, (N, D)),
        _ptr(topk_idx_out, "topk_idx_out", torch.int32, (N, k), required=False),
        _ptr(topk_w_out, "topk_w_out", torch.float32, (N, k), required=False),
        _ptr(counts_out, "counts_out", torch.int32, (E,), required=False),
        _ptr(workspace, "workspace", torch.uint8),
        workspace.numel(),
        _stream(stream))
    _check(st, "moe_forward")


def moe_forward_routed(cfg: MoeConfig, N: int, x, weights, topk_idx, topk_w, y, workspace, counts_out=None,
                       stream=None):
    """The layer with routing given by the caller: topk_idx [N, k] int32 (id E = empty slot), topk_w [N, k]
    float32 used as given."""
    import torch

    E, D, k = cfg.n_routed_experts, cfg.hidden_size, cfg.num_experts_per_tok
    ws = weights if isinstance(weights, MoeWeights) else weights_struct(cfg, weights)
    adt = _act_dtype(cfg)
    st = lib().moe_forward_routed(
        ctypes.byref(cfg), int(N),
        _ptr(x, "x", adt, (N, D)),
        ctypes.byref(ws),
        _ptr(topk_idx, "topk_idx", torch.int32, (N, k)),
        _ptr(topk_w, "topk_w", torch.float32, (N, k)),
        _ptr(y, "y", adt, (N, D)),
        _ptr(counts_out, "counts_out", torch.int32, (E,), required=False),
        _ptr(workspace, "workspace", torch.uint8),
        workspace.numel(),
        _stream(stream))
    _check(st, "moe_forward_routed")


def _dtype_code(dtype) -> int:
    return {"bf16": MOE_BF16, "f32": MOE_F32}[dtype] if isinstance(dtype, str) else int(dtype)


def moe_dense_workspace_size(N: int, D: int, dff: int, dtype="bf16") -> int:
    return int(lib().moe_dense_workspace_size(int(N), int(D), int(dff), _dtype_code(dtype)))


def moe_dense_forward(N: int, x, gate, up, down, y, workspace, limit: float = 0.0, stream=None):
    """Dense SwiGLU FFN y = down (SiLU(gate x) * up x); gate, up [dff, D], down [D, dff]."""
    import torch

    dff, D = gate.shape
    dt = _dtype_code("f32" if x.dtype == torch.float32 else "bf16")
    adt = torch.float32 if dt == MOE_F32 else torch.bfloat16
    st = lib().moe_dense_forward(
        int(N), int(D), int(dff), dt, float(limit),
        _ptr(x, "x", adt, (N, D)), _ptr(gate, "gate", adt, (dff, D)), _ptr(up, "up", adt, (dff, D)),
        _ptr(down, "down", adt, (D, dff)), _ptr(y, "y", adt, (N, D)),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
    _check(st, "moe_dense_forward")


def stage_names() -> list:
    L = lib()
    return [L.moe_stage_name(i).decode() for i in range(L.moe_stage_count())]


def profile_begin(stages=None) -> None:
    """Start per-stage timing; `stages` (stage names) limits it to those stages."""
    if stages is None:
        _check(lib().moe_profile_begin(), "moe_profile_begin")
        return
    names = stage_names()
    mask = 0
    for st in stages:
        mask |= 1 << names.index(st)
    _check(lib().moe_profile_begin_mask(mask), "moe_profile_begin_mask")


def profile_end() -> dict:
    """{stage name: (total ms, launches)} for the launches since profile_begin()."""
    import numpy as np

    names = stage_names()
    ms = np.zeros(len(names), np.float64)
    n = np.zeros(len(names), np.int32)
    _check(lib().moe_profile_end(ms.ctypes.data, n.ctypes.data, len(names)), "moe_profile_end")
    return {names[i]: (float(ms[i]), int(n[i])) for i in range(len(names))}
