"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

Every tensor is a pure function of (seed, tensor id, element index): see
``synth_core.h`` for the Philox4x32-10 stream and the Irwin-Hall(8) normal
stand-in. The host library (gcc) and the device library (hipcc) compile the
same header and produce identical bits, so a test may generate a slice on the
host and compare it with the full tensor generated in HBM.

This module holds the five workloads' shapes and value recipes and nothing of
the MoE method itself.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

# Tensor ids (the Philox key's second word).
ID_X, ID_WG, ID_BIAS, ID_GATE_UP, ID_DOWN, ID_SH_GATE, ID_SH_UP, ID_SH_DOWN, ID_SKEW, ID_X_DECODE = range(1, 11)
ID_DENSE_GATE, ID_DENSE_UP, ID_DENSE_DOWN = range(11, 14)


@dataclass(frozen=True)
class Workload:
    """One MoE-layer configuration: the router/expert config fields plus the input recipe."""

    name: str
    N: int  # tokens (batch x positions, flattened)
    D: int  # hidden size
    E: int  # routed experts
    G: int  # n_group
    TG: int  # topk_group
    k: int  # num_experts_per_tok
    d: int  # moe_intermediate_size
    n_shared: int = 1
    alpha: float = 2.5  # routed_scaling_factor
    norm: bool = True  # norm_topk_prob
    eps: float = 1e-20
    dtype: str = "bf16"  # activations / expert weights; router weight and bias are always fp32
    seed: int = 0
    skew: float = 0.0  # std of the per-expert offset added to every element of a router row
    x_id: int = ID_X
    limit: float = 0.0  # SwiGLU clamp bound (0: plain SwiGLU)
    alpha_on_output: bool = False  # alpha scales the routed sum instead of the weights
    outlier_every: int = 0  # every outlier_every-th token (0: none) is scaled by outlier_scale
    outlier_scale: float = 32.0  # a power of two, so the scaled bf16 values stay exact

    @property
    def d_sh(self) -> int:
        return self.d * self.n_shared

    def with_tokens(self, N: int) -> "Workload":
        return replace(self, N=N)


WORKLOADS = {
    # Tiny fp32 layer with a live group stage.
    "tiny_fp32": Workload("tiny_fp32", N=64, D=256, E=16, G=4, TG=2, k=4, d=128, alpha=2.5, dtype="f32"),
    # GLM-4.5-Air-shaped layer.
    "air_prefill": Workload("air_prefill", N=4096, D=4096, E=128, G=1, TG=1, k=8, d=1408, alpha=1.0),
    # GLM-4.5-shaped prefill with skewed router rows (uneven expert load).
    "glm45_prefill_skewed": Workload("glm45_prefill_skewed", N=8192, D=5120, E=160, G=1, TG=1, k=8, d=1536,
                                     alpha=2.5, skew=0.5),
    # The same shape with offsets small enough that no sigmoid score saturates (logit std ~1.7 against ~35
    # above): the load is still uneven (largest expert ~7x the mean, the top 16 experts ~40% of the rows),
    # but every score carries the gate product.
    "glm45_prefill_mild_skew": Workload("glm45_prefill_mild_skew", N=8192, D=5120, E=160, G=1, TG=1, k=8,
                                        d=1536, alpha=2.5, skew=0.02),
    # GLM-5-shaped prefill with the group stage live.
    "glm5_prefill": Workload("glm5_prefill", N=8192, D=6144, E=256, G=8, TG=4, k=8, d=2048, alpha=2.5),
    # GLM-5-shaped decode step: the prefill weights, 32 fresh tokens.
    "glm5_decode": Workload("glm5_decode", N=32, D=6144, E=256, G=8, TG=4, k=8, d=2048, alpha=2.5,
                            x_id=ID_X_DECODE),
    # The 288-expert shape with the clamped SwiGLU (bound 10): a batch of 32 decode requests, and a prefill.
    "glm53_flash_decode": Workload("glm53_flash_decode", N=32, D=4096, E=288, G=1, TG=1, k=8, d=2048, alpha=2.5,
                                   limit=10.0, x_id=ID_X_DECODE),
    "glm53_flash_prefill": Workload("glm53_flash_prefill", N=8192, D=4096, E=288, G=1, TG=1, k=8, d=2048,
                                    alpha=2.5, limit=10.0),
}
WORKLOAD_ORDER = ["tiny_fp32", "air_prefill", "glm45_prefill_skewed", "glm5_prefill", "glm5_decode",
                  "glm53_flash_decode", "glm53_flash_prefill", "glm45_prefill_mild_skew"]



@dataclass(frozen=True)
class DenseWorkload:
    """A dense SwiGLU FFN (the layers before the MoE ones) and its input recipe."""

    name: str
    N: int
    D: int
    dff: int  # intermediate width (not on the pages: chosen, see the design notes)
    dtype: str = "bf16"
    seed: int = 0
    limit: float = 0.0
    outlier_every: int = 0
    outlier_scale: float = 32.0
    x_id: int = ID_X

    def with_tokens(self, N: int) -> "DenseWorkload":
        return replace(self, N=N)


DENSE_WORKLOADS = {
    # GLM-4.5-shaped dense prefix FFN: hidden 5120, intermediate width 12288.
    "glm45_dense_ffn": DenseWorkload("glm45_dense_ffn", N=8192, D=5120, dff=12288),
}

# ---------------------------------------------------------------------------------------------
_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        path = os.path.join(_HERE, "libsynth_host.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        u32, u64, i64, dbl, vp = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        for fn in ("synth_normal_f64", "synth_normal_f32", "synth_normal_bf16"):
            getattr(lib, fn).argtypes = [u32, u32, u64, i64, dbl, vp]
            getattr(lib, fn).restype = None
        lib.synth_uniform_f32.argtypes = [u32, u32, u64, i64, dbl, dbl, vp]
        lib.synth_uniform_f32.restype = None
        lib.synth_philox_block.argtypes = [u32, u32, vp, vp]
        lib.synth_philox_block.restype = None
        lib.synth_f32_to_bf16_array.argtypes = [vp, i64, vp]
        lib.synth_f32_to_bf16_array.restype = None
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        path = os.path.join(_HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        u32, u64, i64, dbl, vp = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        for fn in ("synth_dev_normal_bf16", "synth_dev_normal_f32"):
            getattr(lib, fn).argtypes = [u32, u32, u64, i64, dbl, vp, vp]
            getattr(lib, fn).restype = ctypes.c_int
        _dev = lib
    return _dev


def philox_block(k0: int, k1: int, ctr) -> list:
    """Raw Philox4x32-10 output block for a 4-word counter and 2-word key."""
    c = np.asarray(ctr, dtype=np.uint32)
    o = np.empty(4, dtype=np.uint32)
    _host_lib().synth_philox_block(k0, k1, c.ctypes.data, o.ctypes.data)
    return [int(v) for v in o]


def normal(seed: int, tid: int, offset: int, count: int, std: float, dtype: str) -> np.ndarray:
    """Elements offset..offset+count of stream (seed, tid), as float64, float32 or bf16 bits (uint16)."""
    lib = _host_lib()
    if dtype == "f64":
        out = np.empty(count, np.float64)
        lib.synth_normal_f64(seed, tid, offset, count, std, out.ctypes.data)
    elif dtype == "f32":
        out = np.empty(count, np.float32)
        lib.synth_normal_f32(seed, tid, offset, count, std, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(count, np.uint16)
        lib.synth_normal_bf16(seed, tid, offset, count, std, out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out


def uniform_f32(seed: int, tid: int, offset: int, count: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(count, np.float32)
    _host_lib().synth_uniform_f32(seed, tid, offset, count, lo, hi, out.ctypes.data)
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    _host_lib().synth_f32_to_bf16_array(a.ctypes.data, a.size, out.ctypes.data)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits (uint16) to float32."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------------------------
# Value recipes. x ~ N(0,1); router rows ~ N(0, 1/D) (+ a per-expert offset ~ N(0, skew^2) added to
# every element of the row when skew > 0); b ~ U(-0.05, 0.05); gate/up ~ N(0, 1/D);
# routed down ~ N(0, 1/d); shared down ~ N(0, 1/d_sh).


def x_host(w: Workload, first: int = 0, count: int | None = None) -> np.ndarray:
    """Tokens first..first+count of x, shape [count, D] (float32, or bf16 bits). Outlier tokens (every
    outlier_every-th, counting from token 0) are multiplied by outlier_scale, a power of two."""
    count = w.N - first if count is None else count
    x = normal(w.seed, w.x_id, first * w.D, count * w.D, 1.0, w.dtype).reshape(count, w.D)
    if w.outlier_every > 0:
        rows = [i for i in range(count) if (first + i) % w.outlier_every == 0]
        if rows:
            if w.dtype == "bf16":
                x[rows] = f32_to_bf16(bf16_to_f32(x[rows]) * np.float32(w.outlier_scale))
            else:
                x[rows] = x[rows] * np.float32(w.outlier_scale)
    return x


def router_host(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """(W_g [E, D] float32, b [E] float32)."""
    wg = normal(w.seed, ID_WG, 0, w.E * w.D, 1.0 / math.sqrt(w.D), "f32").reshape(w.E, w.D)
    if w.skew > 0.0:
        off = normal(w.seed, ID_SKEW, 0, w.E, w.skew, "f32")
        wg = (wg + off[:, None]).astype(np.float32)  # one float32 add per element
    b = uniform_f32(w.seed, ID_BIAS, 0, w.E, -0.05, 0.05)
    return wg, b


def expert_host(w: Workload, e: int) -> tuple[np.ndarray, np.ndarray]:
    """Routed expert e: (gate_up [2d, D], down [D, d]) in the workload dtype."""
    n_gu, n_dn = 2 * w.d * w.D, w.D * w.d
    gu = normal(w.seed, ID_GATE_UP, e * n_gu, n_gu, 1.0 / math.sqrt(w.D), w.dtype).reshape(2 * w.d, w.D)
    dn = normal(w.seed, ID_DOWN, e * n_dn, n_dn, 1.0 / math.sqrt(w.d), w.dtype).reshape(w.D, w.d)
    return gu, dn


def shared_host(w: Workload):
    """Shared expert: (gate [d_sh, D], up [d_sh, D], down [D, d_sh]) in the workload dtype; None without one."""
    if w.n_shared == 0:
        return None
    n = w.d_sh * w.D
    g = normal(w.seed, ID_SH_GATE, 0, n, 1.0 / math.sqrt(w.D), w.dtype).reshape(w.d_sh, w.D)
    u = normal(w.seed, ID_SH_UP, 0, n, 1.0 / math.sqrt(w.D), w.dtype).reshape(w.d_sh, w.D)
    dn = normal(w.seed, ID_SH_DOWN, 0, n, 1.0 / math.sqrt(w.d_sh), w.dtype).reshape(w.D, w.d_sh)
    return g, u, dn


def all_experts_host(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """All routed experts at once: (gate_up [E, 2d, D], down [E, D, d])."""
    n_gu, n_dn = 2 * w.d * w.D, w.D * w.d
    gu = normal(w.seed, ID_GATE_UP, 0, w.E * n_gu, 1.0 / math.sqrt(w.D), w.dtype).reshape(w.E, 2 * w.d, w.D)
    dn = normal(w.seed, ID_DOWN, 0, w.E * n_dn, 1.0 / math.sqrt(w.d), w.dtype).reshape(w.E, w.D, w.d)
    return gu, dn


def dense_host(w: DenseWorkload):
    """Dense FFN weights: (gate [dff, D], up [dff, D], down [D, dff]); gate/up ~ N(0, 1/D), down ~ N(0, 1/dff)."""
    n = w.dff * w.D
    g = normal(w.seed, ID_DENSE_GATE, 0, n, 1.0 / math.sqrt(w.D), w.dtype).reshape(w.dff, w.D)
    u = normal(w.seed, ID_DENSE_UP, 0, n, 1.0 / math.sqrt(w.D), w.dtype).reshape(w.dff, w.D)
    dn = normal(w.seed, ID_DENSE_DOWN, 0, n, 1.0 / math.sqrt(w.dff), w.dtype).reshape(w.D, w.dff)
    return g, u, dn


# ---------------------------------------------------------------------------------------------
# Device fill (torch tensors in HBM), bit-identical to the host recipes above.

def _dev_fill(t, seed: int, tid: int, offset: int, std: float) -> None:
    import torch

    lib = _dev_lib()
    stream = torch.cuda.current_stream(t.device).cuda_stream
    if t.dtype == torch.bfloat16:
        rc = lib.synth_dev_normal_bf16(seed, tid, offset, t.numel(), std, t.data_ptr(), stream)
    elif t.dtype == torch.float32:
        rc = lib.synth_dev_normal_f32(seed, tid, offset, t.numel(), std, t.data_ptr(), stream)
    else:
        raise ValueError(t.dtype)
    if rc != 0:
        raise RuntimeError(f"device generator launch failed: hip error {rc}")


def experts_device(w: Workload, device="cuda") -> dict:
    """All expert weights generated directly in HBM: gate_up [E,2d,D], down [E,D,d], sh_gate, sh_up, sh_down."""
    import torch

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {
        "gate_up": torch.empty((w.E, 2 * w.d, w.D), dtype=dt, device=device),
        "down": torch.empty((w.E, w.D, w.d), dtype=dt, device=device),
    }
    _dev_fill(out["gate_up"], w.seed, ID_GATE_UP, 0, 1.0 / math.sqrt(w.D))
    _dev_fill(out["down"], w.seed, ID_DOWN, 0, 1.0 / math.sqrt(w.d))
    if w.n_shared > 0:
        out["sh_gate"] = torch.empty((w.d_sh, w.D), dtype=dt, device=device)
        out["sh_up"] = torch.empty((w.d_sh, w.D), dtype=dt, device=device)
        out["sh_down"] = torch.empty((w.D, w.d_sh), dtype=dt, device=device)
        _dev_fill(out["sh_gate"], w.seed, ID_SH_GATE, 0, 1.0 / math.sqrt(w.D))
        _dev_fill(out["sh_up"], w.seed, ID_SH_UP, 0, 1.0 / math.sqrt(w.D))
        _dev_fill(out["sh_down"], w.seed, ID_SH_DOWN, 0, 1.0 / math.sqrt(w.d_sh))
    return out


def dense_device(w: DenseWorkload, device="cuda") -> dict:
    """Dense FFN weights generated directly in HBM: gate [dff, D], up [dff, D], down [D, dff]."""
    import torch

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {"gate": torch.empty((w.dff, w.D), dtype=dt, device=device),
           "up": torch.empty((w.dff, w.D), dtype=dt, device=device),
           "down": torch.empty((w.D, w.dff), dtype=dt, device=device)}
    _dev_fill(out["gate"], w.seed, ID_DENSE_GATE, 0, 1.0 / math.sqrt(w.D))
    _dev_fill(out["up"], w.seed, ID_DENSE_UP, 0, 1.0 / math.sqrt(w.D))
    _dev_fill(out["down"], w.seed, ID_DENSE_DOWN, 0, 1.0 / math.sqrt(w.dff))
    return out
