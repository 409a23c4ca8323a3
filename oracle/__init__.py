"""CPU oracle of the GLM-4.5 / GLM-5 sparse-MoE FFN forward (ctypes wrapper around moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline leg are the
only users. The GPU library never imports, links or runs anything here, and nothing here imports the
GPU library. Scope, sources and the readings of open points are in moe_oracle.h.

Pinned by tests/test_oracle_*.py against brute-force enumeration, library routines, closed forms,
invariants and the parameter counts the pages print. The gate dot product and the sigmoid are pinned
only by sanity cases (one-hot rows, sigma(0) = 1/2, sigma(-r) = 1 - sigma(r)): beyond the definition
itself their parity is unpinned.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
F32, BF16 = 0, 1


class OracleCfg(ctypes.Structure):
    _fields_ = [
        ("D", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("G", ctypes.c_int32),
        ("TG", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("n_shared", ctypes.c_int32),
        ("alpha", ctypes.c_float),
        ("norm", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("limit", ctypes.c_float),
        ("alpha_on_output", ctypes.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        cp = ctypes.POINTER(OracleCfg)
        L.oracle_check_cfg.argtypes = [cp]
        L.oracle_logits.argtypes = [cp, i64, vp, i32, vp, vp]
        L.oracle_sigmoid.argtypes = [i64, vp, vp]
        L.oracle_sigmoid.restype = None
        L.oracle_select.argtypes = [cp, i64, vp, vp, vp, vp, vp]
        L.oracle_select_margin.argtypes = [cp, i64, vp, vp, vp]
        L.oracle_dispatch.argtypes = [cp, i64, vp, vp, vp, vp, vp]
        L.oracle_swiglu.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp, vp, i32, ctypes.c_double, vp, vp]
        L.oracle_swiglu.restype = None
        L.oracle_forward_tokens.argtypes = [cp, i64, vp, vp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp]
        L.oracle_forward_expert_loop.argtypes = [cp, i64, vp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp]
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_param_count.argtypes = [cp, vp]
        L.oracle_param_count.restype = None
        _lib = L
    return _lib


def cfg_of(w) -> OracleCfg:
    """Oracle config from any object with the fields D, E, G, TG, k, d, n_shared, alpha, norm, eps (and
    optionally limit, alpha_on_output)."""
    return OracleCfg(w.D, w.E, w.G, w.TG, w.k, w.d, w.n_shared, float(w.alpha), int(bool(w.norm)), float(w.eps),
                     float(getattr(w, "limit", 0.0)), int(bool(getattr(w, "alpha_on_output", False))))


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bf16 bits (uint16), got {a.dtype}")


def _c(a, dtype=None):
    return np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid configuration or input")


def check_cfg(w) -> bool:
    c = cfg_of(w)
    return lib().oracle_check_cfg(ctypes.byref(c)) == 0


def logits(w, x: np.ndarray, wg: np.ndarray) -> np.ndarray:
    x = _c(x)
    wg = _c(wg, np.float32)
    N = x.shape[0]
    r = np.empty((N, w.E), np.float32)
    c = cfg_of(w)
    _check(lib().oracle_logits(ctypes.byref(c), N, x.ctypes.data, _dt(x), wg.ctypes.data, r.ctypes.data), "logits")
    return r


def sigmoid(r: np.ndarray) -> np.ndarray:
    r = _c(r, np.float32)
    s = np.empty_like(r)
    lib().oracle_sigmoid(r.size, r.ctypes.data, s.ctypes.data)
    return s


def scores(w, x, wg) -> np.ndarray:
    return sigmoid(logits(w, x, wg))


def select(w, s: np.ndarray, b: np.ndarray, want_kept: bool = False):
    s = _c(s, np.float32)
    b = _c(b, np.float32)
    N = s.shape[0]
    idx = np.empty((N, w.k), np.int32)
    wt = np.empty((N, w.k), np.float32)
    kept = np.empty((N, w.G), np.uint8) if want_kept else None
    c = cfg_of(w)
    _check(
        lib().oracle_select(ctypes.byref(c), N, s.ctypes.data, b.ctypes.data, idx.ctypes.data, wt.ctypes.data,
                            None if kept is None else kept.ctypes.data),
        "select",
    )
    return (idx, wt, kept) if want_kept else (idx, wt)


def select_margin(w, s: np.ndarray, b: np.ndarray) -> np.ndarray:
    s = _c(s, np.float32)
    b = _c(b, np.float32)
    m = np.empty(s.shape[0], np.float64)
    c = cfg_of(w)
    _check(lib().oracle_select_margin(ctypes.byref(c), s.shape[0], s.ctypes.data, b.ctypes.data, m.ctypes.data),
           "select_margin")
    return m


def dispatch(w, idx: np.ndarray):
    idx = _c(idx, np.int32)
    N = idx.shape[0]
    counts = np.empty(w.E, np.int32)
    offsets = np.empty(w.E + 1, np.int32)
    sorted_pair = np.empty(N * w.k, np.int32)
    inv_row = np.empty(N * w.k, np.int32)
    c = cfg_of(w)
    _check(lib().oracle_dispatch(ctypes.byref(c), N, idx.ctypes.data, counts.ctypes.data, offsets.ctypes.data,
                                 sorted_pair.ctypes.data, inv_row.ctypes.data), "dispatch")
    return counts, offsets, sorted_pair, inv_row


def swiglu(gate, up, down, x, limit: float = 0.0) -> np.ndarray:
    """One SwiGLU MLP on one token in double: down (SiLU(a) * u), a = gate x, u = up x, clamped as
    a = min(a, limit), u = clip(u, -limit, limit) when limit > 0."""
    gate, up, down = _c(gate), _c(up), _c(down)
    dt = _dt(gate)
    assert _dt(up) == dt and _dt(down) == dt
    dff, D = gate.shape
    xd = _c(x, np.float64)
    out = np.empty(D, np.float64)
    lib().oracle_swiglu(D, dff, gate.ctypes.data, up.ctypes.data, down.ctypes.data, dt, float(limit),
                        xd.ctypes.data, out.ctypes.data)
    return out


class ExpertTable:
    """Host pointers to the routed experts' (gate_up [2d, D], down [D, d]) and the shared MLP.

    Built either from full stacked arrays or from a dict {expert: (gate_up, down)} holding only the
    experts a computation needs; the arrays are kept alive by this object.
    """

    def __init__(self, w, experts, shared):
        self.keep = []
        self.gu = (ctypes.c_void_p * w.E)()
        self.dn = (ctypes.c_void_p * w.E)()
        dts = set()
        if isinstance(experts, dict):
            items = experts.items()
        else:
            gu_all, dn_all = experts
            items = ((e, (gu_all[e], dn_all[e])) for e in range(w.E))
        for e, (gu, dn) in items:
            gu, dn = _c(gu), _c(dn)
            assert gu.shape == (2 * w.d, w.D) and dn.shape == (w.D, w.d), (gu.shape, dn.shape)
            self.keep += [gu, dn]
            self.gu[e] = gu.ctypes.data
            self.dn[e] = dn.ctypes.data
            dts.add(_dt(gu))
            dts.add(_dt(dn))
        self.sh = [None, None, None]
        if shared is not None:
            sg, su, sd = (_c(a) for a in shared)
            self.keep += [sg, su, sd]
            self.sh = [sg.ctypes.data, su.ctypes.data, sd.ctypes.data]
            dts |= {_dt(sg), _dt(su), _dt(sd)}
        assert len(dts) == 1, "all expert weights must share one element type"
        self.wdt = dts.pop()


def forward_tokens(w, tokens, x, table: ExpertTable, idx, wt) -> np.ndarray:
    """y rows (float32) for the listed tokens, per-token form, given routing idx/wt for all tokens."""
    tokens = _c(tokens, np.int64)
    x = _c(x)
    idx = _c(idx, np.int32)
    wt = _c(wt, np.float32)
    y = np.empty((tokens.size, w.D), np.float32)
    c = cfg_of(w)
    _check(
        lib().oracle_forward_tokens(ctypes.byref(c), tokens.size, tokens.ctypes.data, x.ctypes.data, _dt(x),
                                    table.gu, table.dn, table.sh[0], table.sh[1], table.sh[2], table.wdt,
                                    idx.ctypes.data, wt.ctypes.data, y.ctypes.data),
        "forward_tokens",
    )
    return y


def forward_expert_loop(w, x, table: ExpertTable, idx, wt) -> np.ndarray:
    """y [N, D] (float32), per-expert loop form over all N tokens."""
    x = _c(x)
    idx = _c(idx, np.int32)
    wt = _c(wt, np.float32)
    N = x.shape[0]
    y = np.empty((N, w.D), np.float32)
    c = cfg_of(w)
    _check(
        lib().oracle_forward_expert_loop(ctypes.byref(c), N, x.ctypes.data, _dt(x), table.gu, table.dn,
                                         table.sh[0], table.sh[1], table.sh[2], table.wdt, idx.ctypes.data,
                                         wt.ctypes.data, y.ctypes.data),
        "forward_expert_loop",
    )
    return y


def route(w, x, wg, b):
    """Scores, then selection: (s [N,E], idx [N,k], w [N,k])."""
    s = scores(w, x, wg)
    idx, wt = select(w, s, b)
    return s, idx, wt


def forward(w, x, wg, b, experts, shared):
    """The whole layer on the host: routing, then the per-token sum. Returns (y, s, idx, wt)."""
    s, idx, wt = route(w, x, wg, b)
    table = ExpertTable(w, experts, shared)
    y = forward_tokens(w, np.arange(x.shape[0]), x, table, idx, wt)
    return y, s, idx, wt


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def param_count(w) -> dict:
    out = np.zeros(6, np.int64)
    c = cfg_of(w)
    lib().oracle_param_count(ctypes.byref(c), out.ctypes.data)
    keys = ["router", "expert", "routed", "shared", "total", "used_per_token"]
    return {k: int(v) for k, v in zip(keys, out)}
