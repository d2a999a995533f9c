"""Python access to the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this module; the product package never imports it.

Functions take a workload-like object with attributes T, H, F, N, k, capacity,
order, noisy, out_scale, act, wt and numpy arrays x, Wg, Wn, eps, Wgate, Wup,
Wdown (bf16 tensors as uint16 bit patterns, fp32 as float32), and return numpy
arrays.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

H_EXACT, H_F32, H_BF16 = 0, 1, 2


class OracleCfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("F", ctypes.c_int32),
                ("N", ctypes.c_int32), ("k", ctypes.c_int32), ("capacity", ctypes.c_int64),
                ("order", ctypes.c_int32), ("noisy", ctypes.c_int32), ("out_scale", ctypes.c_double),
                ("h_round", ctypes.c_int32), ("x_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32)]


_lib = None


def load(path: str = None):
    """Load liboracle.so (building it first if absent). A custom path loads a
    separately built variant (used by the mutation tests)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or os.environ.get("MOE_ORACLE_LIB") or _LIB_PATH
    if not os.path.exists(p):
        from . import build as _b
        _b.build(out=p)
    lib = ctypes.CDLL(p)
    vp, i32, i64, cfgp = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(OracleCfg)
    lib.oracle_route.argtypes = [cfgp] + [vp] * 9
    lib.oracle_stats.argtypes = [cfgp] + [vp] * 9
    lib.oracle_capacity.argtypes = [cfgp] + [vp] * 6
    lib.oracle_expert_rows.argtypes = [cfgp, vp, vp, vp, vp, i32, vp, i64, i32, vp, vp]
    lib.oracle_combine_tokens.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, vp, vp]
    lib.oracle_combine_rows.argtypes = [cfgp, vp, vp, vp, i64, vp, vp, vp]
    lib.oracle_smooth_load.argtypes = [cfgp] + [vp] * 5
    lib.oracle_residual_combine_rows.argtypes = [cfgp, vp, vp, vp, i64, vp, vp, vp, vp]
    lib.oracle_backward.argtypes = [cfgp] + [vp] * 8 + [ctypes.c_double, i32] + [vp] * 6
    lib.brute_layer.argtypes = [cfgp] + [vp] * 17
    for f in ("oracle_route", "oracle_stats", "oracle_capacity", "oracle_expert_rows",
              "oracle_combine_tokens", "oracle_combine_rows", "oracle_smooth_load", "oracle_residual_combine_rows",
              "oracle_backward", "brute_layer"):
        getattr(lib, f).restype = ctypes.c_int
    for f in ("oracle_round_bf16", "oracle_round_f32", "oracle_silu", "oracle_softplus", "brute_round_bf16"):
        getattr(lib, f).argtypes = [ctypes.c_double]
        getattr(lib, f).restype = ctypes.c_double
    if path is None:
        _lib = lib
    return lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _dt(a):
    return 1 if a.dtype == np.uint16 else 0


def default_h_round(w) -> int:
    return H_BF16 if w.wt == "bf16" else H_F32


def cfg(w, h_round: int = None) -> OracleCfg:
    return OracleCfg(T=w.T, H=w.H, F=w.F, N=w.N, k=w.k, capacity=int(w.capacity), order=int(w.order),
                     noisy=int(bool(w.noisy)), out_scale=float(w.out_scale),
                     h_round=default_h_round(w) if h_round is None else h_round,
                     x_dtype=_dt(w.x), w_dtype=_dt(w.Wgate) if w.Wgate is not None else 0)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (code {rc})")


def route(w, lib=None):
    lib = lib or load()
    c = cfg(w)
    T, N, k = w.T, w.N, w.k
    out = dict(logits=np.zeros((T, N), np.float32), H=np.zeros((T, N), np.float32),
               topk_idx=np.zeros((T, k), np.int32), topk_w=np.zeros((T, k), np.float64),
               min_gap=np.zeros(T, np.float64))
    Wn = w.Wn if w.noisy else None
    eps = w.eps if w.noisy else None
    _check(lib.oracle_route(ctypes.byref(c), _p(w.x), _p(w.Wg), _p(Wn), _p(eps), _p(out["logits"]),
                            _p(out["H"]), _p(out["topk_idx"]), _p(out["topk_w"]), _p(out["min_gap"])),
           "oracle_route")
    return out


def stats(w, r, lib=None):
    lib = lib or load()
    c = cfg(w)
    N = w.N
    out = dict(load=np.zeros(N, np.int64), importance=np.zeros(N), P=np.zeros(N), f=np.zeros(N))
    bal = ctypes.c_double()
    balc = ctypes.c_double()
    _check(lib.oracle_stats(ctypes.byref(c), _p(r["logits"]), _p(r["topk_idx"]), _p(r["topk_w"]),
                            _p(out["load"]), _p(out["importance"]), _p(out["P"]), _p(out["f"]),
                            ctypes.byref(bal), ctypes.byref(balc)), "oracle_stats")
    out["balance"] = bal.value
    out["balance_code"] = balc.value
    return out


def smooth_load(w, lib=None):
    """Smooth gate load [N] of the noisy top-k gate (see moe_oracle.h)."""
    lib = lib or load()
    c = cfg(w)
    out = np.zeros(w.N)
    _check(lib.oracle_smooth_load(ctypes.byref(c), _p(w.x), _p(w.Wg), _p(w.Wn), _p(w.eps), _p(out)),
           "oracle_smooth_load")
    return out


def capacity(w, topk_idx, lib=None):
    lib = lib or load()
    c = cfg(w)
    T, N, k = w.T, w.N, w.k
    topk_idx = np.ascontiguousarray(topk_idx, np.int32)
    out = dict(counts=np.zeros(N, np.int64), kept=np.zeros(N, np.int64), offsets=np.zeros(N + 1, np.int64),
               slot=np.zeros((T, k), np.int64), row_token=np.zeros(T * k, np.int64))
    _check(lib.oracle_capacity(ctypes.byref(c), _p(topk_idx), _p(out["counts"]), _p(out["kept"]),
                               _p(out["offsets"]), _p(out["slot"]), _p(out["row_token"])), "oracle_capacity")
    return out


def expert_rows(w, e, tokens, nthreads=1, want_h=False, h_round=None, lib=None):
    lib = lib or load()
    c = cfg(w, h_round)
    tokens = np.ascontiguousarray(tokens, np.int64)
    n = tokens.size
    E = np.zeros((n, w.H))
    h = np.zeros((n, w.F)) if want_h else None
    _check(lib.oracle_expert_rows(ctypes.byref(c), _p(w.x), _p(w.Wgate), _p(w.Wup), _p(w.Wdown), int(e),
                                  _p(tokens), n, int(nthreads), _p(h), _p(E)), "oracle_expert_rows")
    return (h, E) if want_h else E


def combine_tokens(w, topk_idx, topk_w, slot, tokens, nthreads=1, h_round=None, lib=None):
    lib = lib or load()
    c = cfg(w, h_round)
    tokens = np.ascontiguousarray(tokens, np.int64)
    n = tokens.size
    y64 = np.zeros((n, w.H))
    y32 = np.zeros((n, w.H), np.float32)
    _check(lib.oracle_combine_tokens(ctypes.byref(c), _p(w.x), _p(w.Wgate), _p(w.Wup), _p(w.Wdown),
                                     _p(np.ascontiguousarray(topk_idx, np.int32)),
                                     _p(np.ascontiguousarray(topk_w, np.float64)),
                                     _p(np.ascontiguousarray(slot, np.int64)), _p(tokens), n, int(nthreads),
                                     _p(y64), _p(y32)), "oracle_combine_tokens")
    return y64, y32


def assignment_outputs(w, topk_idx, tokens=None, nthreads=1, h_round=None, lib=None):
    """E [n,k,H]: the output of expert topk_idx[t,j] for token t, for every
    slot j of the listed tokens (all when None), whether or not a capacity
    keeps it. Each expert runs once over the tokens that chose it."""
    tokens = np.arange(w.T, dtype=np.int64) if tokens is None else np.asarray(tokens, np.int64)
    idx = np.asarray(topk_idx)[tokens]
    E = np.zeros((tokens.size, w.k, w.H))
    for e in range(w.N):
        ii, jj = np.nonzero(idx == e)
        if ii.size:
            E[ii, jj] = expert_rows(w, e, tokens[ii], nthreads=nthreads, h_round=h_round, lib=lib)
    return E


def combine_rows(w, topk_w, slot, E, tokens=None, h_round=None, lib=None):
    """The layer output of the listed tokens from expert outputs E [n,k,H]
    (see assignment_outputs) and a capacity setting's slots."""
    lib = lib or load()
    c = cfg(w, h_round)
    tokens = np.arange(w.T, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, np.int64)
    n = tokens.size
    E = np.ascontiguousarray(E, np.float64)
    assert E.shape == (n, w.k, w.H)
    y64 = np.zeros((n, w.H))
    y32 = np.zeros((n, w.H), np.float32)
    _check(lib.oracle_combine_rows(ctypes.byref(c), _p(np.ascontiguousarray(topk_w, np.float64)),
                                   _p(np.ascontiguousarray(slot, np.int64)), _p(tokens), n, _p(E), _p(y64),
                                   _p(y32)), "oracle_combine_rows")
    return y64, y32


def shared_slice(w):
    """The residual layer's shared slice as a one-expert layer (its weights
    [1,Fs,H], [1,Fs,H], [1,H,Fs]), for expert_rows."""
    Sg, Su, Sd = w.shared
    Fs = Sg.shape[0]
    return type(w)(w.name + "_shared", w.T, w.H, Fs, 1, 1, -1, w.order, False, False, 1.0, w.act, w.wt, w.x,
                   None, None, None, Sg[None], Su[None], Sd[None])


def residual_forward(w, tokens=None, nthreads=1, h_round=None, lib=None, E=None, ora=None):
    """The residual (shared-slice) layer: routing and capacity for every
    token, y = shared(x) + s * sum_j w_j E_j(x) for `tokens` (all when None).
    E: expert outputs of every slot of those tokens, if already computed."""
    lib = lib or load()
    r = ora if ora is not None else route(w, lib)
    cap = capacity(w, r["topk_idx"], lib)
    tokens = np.arange(w.T, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, np.int64)
    if E is None:
        E = assignment_outputs(w, r["topk_idx"], tokens, nthreads=nthreads, h_round=h_round, lib=lib)
    R = expert_rows(shared_slice(w), 0, tokens, nthreads=nthreads, h_round=h_round, lib=lib)
    c = cfg(w, h_round)
    n = tokens.size
    y64 = np.zeros((n, w.H))
    y32 = np.zeros((n, w.H), np.float32)
    _check(lib.oracle_residual_combine_rows(ctypes.byref(c), _p(np.ascontiguousarray(r["topk_w"], np.float64)),
                                            _p(np.ascontiguousarray(cap["slot"], np.int64)), _p(tokens), n,
                                            _p(np.ascontiguousarray(E, np.float64)), _p(np.ascontiguousarray(R)),
                                            _p(y64), _p(y32)), "oracle_residual_combine_rows")
    out = dict(r)
    out.update(cap)
    out.update(tokens=tokens, y64=y64, y=y32, R=R)
    return out


def backward(w, dy, d_balance=0.0, h_round=None, lib=None, nthreads=1):
    """Gradients of <dy, y> + d_balance * balance (see moe_oracle.h):
    dict of dx, dWg, dWn, dWgate, dWup, dWdown (double)."""
    lib = lib or load()
    c = cfg(w, h_round)
    T, H, F, N = w.T, w.H, w.F, w.N
    o = dict(dx=np.zeros((T, H)), dWg=np.zeros((H, N)), dWn=np.zeros((H, N)), dWgate=np.zeros((N, F, H)),
             dWup=np.zeros((N, F, H)), dWdown=np.zeros((N, H, F)))
    Wn = w.Wn if w.noisy else None
    eps = w.eps if w.noisy else None
    _check(lib.oracle_backward(ctypes.byref(c), _p(w.x), _p(w.Wg), _p(Wn), _p(eps), _p(w.Wgate), _p(w.Wup),
                               _p(w.Wdown), _p(np.ascontiguousarray(dy, np.float32)), float(d_balance),
                               int(nthreads), _p(o["dx"]),
                               _p(o["dWg"]), _p(o["dWn"]), _p(o["dWgate"]), _p(o["dWup"]), _p(o["dWdown"])),
           "oracle_backward")
    return o


def forward(w, tokens=None, nthreads=1, h_round=None, lib=None):
    """The whole layer: routing and capacity for every token, expert outputs
    for `tokens` (all tokens when None)."""
    r = route(w, lib)
    cap = capacity(w, r["topk_idx"], lib)
    if tokens is None:
        tokens = np.arange(w.T, dtype=np.int64)
    y64, y32 = combine_tokens(w, r["topk_idx"], r["topk_w"], cap["slot"], tokens, nthreads, h_round, lib)
    out = dict(r)
    out.update(cap)
    out.update(tokens=np.asarray(tokens, np.int64), y64=y64, y=y32)
    if getattr(w, "want_stats", False):
        out["stats"] = stats(w, r, lib)
    return out


def brute(w, h_round=None, lib=None):
    lib = lib or load()
    c = cfg(w, h_round)
    T, N, k, H = w.T, w.N, w.k, w.H
    o = dict(topk_idx=np.zeros((T, k), np.int32), topk_w=np.zeros((T, k)), gate=np.zeros((T, N)),
             keep=np.zeros((T, k), np.int32), rank=np.zeros((T, k), np.int64), y64=np.zeros((T, H)),
             load=np.zeros(N, np.int64), importance=np.zeros(N), P=np.zeros(N))
    bal = ctypes.c_double()
    Wn = w.Wn if w.noisy else None
    eps = w.eps if w.noisy else None
    _check(lib.brute_layer(ctypes.byref(c), _p(w.x), _p(w.Wg), _p(Wn), _p(eps), _p(w.Wgate), _p(w.Wup),
                           _p(w.Wdown), _p(o["topk_idx"]), _p(o["topk_w"]), _p(o["gate"]), _p(o["keep"]),
                           _p(o["rank"]), _p(o["y64"]), _p(o["load"]), _p(o["importance"]), _p(o["P"]),
                           ctypes.byref(bal)), "brute_layer")
    o["balance"] = bal.value
    return o


def round_bf16(v: float, lib=None) -> float:
    return (lib or load()).oracle_round_bf16(float(v))
