"""Seeded synthetic workloads for the top-k MoE SwiGLU layer.

Inputs only: this module builds activations, router and expert weights, noise
draws and the neuron permutation that splits a dense FFN into experts. It holds
none of the layer's arithmetic, so both the CPU oracle's tests and the GPU
path's tests and benchmark can draw from it without sharing method code.

Workloads follow the shapes of the pages' models:
  * LLaMA-MoE expert construction by a non-overlapping random split of the
    FFN's intermediate neurons (LLaMA-MoE v2 article, section on independent
    neuron partitioning; LLaMA-MoE summary, section on the non-overlapping
    random split);
  * Llama-3 upcycling, where each expert is a copy of the dense FFN
    ("Llama 3 Meets MoE: Efficient Upcycling" review, section 2), here with a
    small per-copy perturbation so the experts are not bit-identical;
  * activations N(0, 1) and weights N(0, 0.02) stand in for trained hidden
    states and checkpoints, which are not available.

Every tensor is drawn from its own counter stream (see synth.c for the exact
generator), so any config can be rebuilt anywhere from (seed, stream).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_synth.so")
_lib = None

# stream ids
S_X, S_WGATE, S_WUP, S_WDOWN, S_WG, S_WNOISE, S_EPS, S_PERM = 0, 1, 2, 3, 4, 5, 6, 7
S_PERTURB0 = 8          # + expert index
S_SKEW_SET, S_SKEW_DIR = 20, 21

MIXTRAL, ST = 0, 1      # KeepTopK -> softmax ; softmax -> top-k


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
    vp = ctypes.c_void_p
    lib.syn_draw_u64.argtypes = [u64, u64, u64]
    lib.syn_draw_u64.restype = u64
    lib.syn_normal_f32.argtypes = [u64, u64, u64, i64, dbl, vp]
    lib.syn_normal_bf16.argtypes = [u64, u64, u64, i64, dbl, vp]
    lib.syn_perturb_bf16.argtypes = [vp, u64, u64, u64, i64, dbl, vp]
    lib.syn_f32_to_bf16.argtypes = [vp, i64, vp]
    lib.syn_bf16_to_f32.argtypes = [vp, i64, vp]
    lib.syn_permutation.argtypes = [u64, u64, i64, vp]
    for f in ("syn_normal_f32", "syn_normal_bf16", "syn_perturb_bf16", "syn_f32_to_bf16",
              "syn_bf16_to_f32", "syn_permutation"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def normal_f32(seed: int, stream: int, shape, sigma: float = 1.0, offset: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().syn_normal_f32(seed, stream, offset, out.size, sigma, _ptr(out))
    return out


def normal_bf16(seed: int, stream: int, shape, sigma: float = 1.0, offset: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0, sigma^2) draws."""
    out = np.empty(shape, dtype=np.uint16)
    _load().syn_normal_bf16(seed, stream, offset, out.size, sigma, _ptr(out))
    return out


def perturb_bf16(base: np.ndarray, seed: int, stream: int, sigma: float, offset: int = 0) -> np.ndarray:
    base = np.ascontiguousarray(base, dtype=np.float32)
    out = np.empty(base.shape, dtype=np.uint16)
    _load().syn_perturb_bf16(_ptr(base), seed, stream, offset, base.size, sigma, _ptr(out))
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().syn_f32_to_bf16(_ptr(a), a.size, _ptr(out))
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    _load().syn_bf16_to_f32(_ptr(bits), bits.size, _ptr(out))
    return out


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int64)
    _load().syn_permutation(seed, stream, n, _ptr(out))
    return out


@dataclass
class Workload:
    """One MoE-layer problem: shapes, options and input tensors (numpy, host).

    Storage: tensors whose dtype is "bf16" hold uint16 bit patterns; "f32"
    tensors hold float32. x is [T,H]; Wg, Wn are [H,N] fp32; eps is [T,N] fp32;
    Wgate, Wup are [N,F,H]; Wdown is [N,H,F] (nn.Linear [out,in] layout per
    expert).
    """
    name: str
    T: int
    H: int
    F: int
    N: int
    k: int
    capacity: int = -1          # < 0: dropless
    order: int = MIXTRAL
    noisy: bool = False
    want_stats: bool = False
    out_scale: float = 1.0
    act: str = "bf16"
    wt: str = "bf16"
    x: Optional[np.ndarray] = None
    Wg: Optional[np.ndarray] = None
    Wn: Optional[np.ndarray] = None
    eps: Optional[np.ndarray] = None
    Wgate: Optional[np.ndarray] = None
    Wup: Optional[np.ndarray] = None
    Wdown: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)
    shared: Optional[tuple] = None   # residual layer: (gate [Fs,H], up [Fs,H], down [H,Fs]) of the shared slice

    def f32(self, name: str) -> np.ndarray:
        """fp32 values of a tensor (exact upcast for bf16 storage)."""
        a = getattr(self, name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            return bf16_to_f32(a)
        return a


def capacity_from_cf(T: int, N: int, k: int, cf: float, count_assignments: bool = False) -> int:
    """Expert capacity = tokens per batch / N * CF, rounded up (upcycling
    review, section 3, capacity-factor equation). With count_assignments the
    numerator counts (token, expert) assignments, T*k, instead of tokens."""
    num = T * k if count_assignments else T
    return int(np.ceil(cf * num / N - 1e-9))


def _rand_w(seed, stream, shape, sigma, dtype):
    if dtype == "bf16":
        return normal_bf16(seed, stream, shape, sigma)
    return normal_f32(seed, stream, shape, sigma)


def split_dense(Wgate_d: np.ndarray, Wup_d: np.ndarray, Wdown_d: np.ndarray, perm: np.ndarray, N: int):
    """Non-overlapping split of a dense SwiGLU FFN: expert e receives the
    intermediate neurons perm[e*F:(e+1)*F] (rows of gate/up, columns of down)."""
    Ftot = Wgate_d.shape[0]
    assert Ftot % N == 0
    F = Ftot // N
    idx = perm.reshape(N, F)
    Wgate = np.ascontiguousarray(Wgate_d[idx])                     # [N,F,H]
    Wup = np.ascontiguousarray(Wup_d[idx])                         # [N,F,H]
    Wdown = np.ascontiguousarray(np.transpose(Wdown_d[:, idx], (1, 0, 2)))  # [N,H,F]
    return Wgate, Wup, Wdown


def make_split(name, seed, T, H, Ftot, N, k, *, act="bf16", wt="bf16", order=MIXTRAL, noisy=False,
               want_stats=False, out_scale=1.0, capacity=-1, wsig=0.02) -> Workload:
    """A LLaMA-MoE style layer: one dense FFN split into N experts."""
    x = _rand_w(seed, S_X, (T, H), 1.0, act)
    Wgate_d = _rand_w(seed, S_WGATE, (Ftot, H), wsig, wt)
    Wup_d = _rand_w(seed, S_WUP, (Ftot, H), wsig, wt)
    Wdown_d = _rand_w(seed, S_WDOWN, (H, Ftot), wsig, wt)
    perm = permutation(seed, S_PERM, Ftot)
    Wgate, Wup, Wdown = split_dense(Wgate_d, Wup_d, Wdown_d, perm, N)
    Wg = normal_f32(seed, S_WG, (H, N), wsig)
    Wn = normal_f32(seed, S_WNOISE, (H, N), wsig) if noisy else None
    eps = normal_f32(seed, S_EPS, (T, N), 1.0) if noisy else None
    w = Workload(name, T, H, Ftot // N, N, k, capacity, order, noisy, want_stats, out_scale, act, wt,
                 x, Wg, Wn, eps, Wgate, Wup, Wdown)
    w.meta.update(kind="split", seed=seed, perm=perm, dense=(Wgate_d, Wup_d, Wdown_d))
    return w


def make_residual(name, seed, T, H, Ftot, Fs, N, k, *, act="bf16", wt="bf16", order=MIXTRAL, noisy=False,
                  want_stats=False, out_scale=1.0, capacity=-1, wsig=0.02) -> Workload:
    """A residual (shared-neuron, "Inter" mode) LLaMA-MoE layer: one dense FFN
    whose neurons perm[:Fs] form an always-active shared slice and whose other
    Ftot - Fs neurons are split into N experts (LLaMA-MoE hub page, Inter
    mode; LLaMA-MoE v2 article, shared-neuron partitioning). The seeded
    permutation stands in for the gradient-importance choice of the shared
    neurons, which needs a trained model and data."""
    x = _rand_w(seed, S_X, (T, H), 1.0, act)
    Wgate_d = _rand_w(seed, S_WGATE, (Ftot, H), wsig, wt)
    Wup_d = _rand_w(seed, S_WUP, (Ftot, H), wsig, wt)
    Wdown_d = _rand_w(seed, S_WDOWN, (H, Ftot), wsig, wt)
    perm = permutation(seed, S_PERM, Ftot)
    sh, rest = perm[:Fs], perm[Fs:]
    Wgate, Wup, Wdown = split_dense(Wgate_d[rest], Wup_d[rest], Wdown_d[:, rest], np.arange(Ftot - Fs), N)
    shared = (np.ascontiguousarray(Wgate_d[sh]), np.ascontiguousarray(Wup_d[sh]),
              np.ascontiguousarray(Wdown_d[:, sh]))
    Wg = normal_f32(seed, S_WG, (H, N), wsig)
    Wn = normal_f32(seed, S_WNOISE, (H, N), wsig) if noisy else None
    eps = normal_f32(seed, S_EPS, (T, N), 1.0) if noisy else None
    w = Workload(name, T, H, (Ftot - Fs) // N, N, k, capacity, order, noisy, want_stats, out_scale, act, wt,
                 x, Wg, Wn, eps, Wgate, Wup, Wdown, shared=shared)
    w.meta.update(kind="residual", seed=seed, perm=perm, dense=(Wgate_d, Wup_d, Wdown_d))
    return w


def make_inner_shared(name, seed, T, H, Ftot, Fs, N, k, *, act="bf16", wt="bf16", out_scale=1.0,
                      capacity=-1, wsig=0.02) -> Workload:
    """The "Inner" sharing mode: every expert holds the shared neurons
    perm[:Fs] followed by its own share of the rest (experts of Fs +
    (Ftot - Fs)/N neurons; the shared weights are repeated in each expert)."""
    r = make_residual(name, seed, T, H, Ftot, Fs, N, k, act=act, wt=wt, out_scale=out_scale, capacity=capacity,
                      wsig=wsig)
    Sg, Su, Sd = r.shared
    Wgate = np.ascontiguousarray(np.concatenate([np.broadcast_to(Sg, (N,) + Sg.shape), r.Wgate], axis=1))
    Wup = np.ascontiguousarray(np.concatenate([np.broadcast_to(Su, (N,) + Su.shape), r.Wup], axis=1))
    Wdown = np.ascontiguousarray(np.concatenate([np.broadcast_to(Sd, (N,) + Sd.shape), r.Wdown], axis=2))
    w = Workload(name, T, H, Fs + r.F, N, k, capacity, MIXTRAL, False, False, out_scale, act, wt, r.x, r.Wg,
                 None, None, Wgate, Wup, Wdown)
    w.meta.update(kind="inner_shared", seed=seed, residual=r)
    return w


def make_upcycled(name, seed, T, H, F, N, k, *, perturb=1e-3, order=MIXTRAL, capacity=-1, out_scale=1.0,
                  wsig=0.02, keep_base=False) -> Workload:
    """A Llama-3 style upcycled layer: N copies of one dense FFN, each plus an
    independent N(0, perturb^2) perturbation, rounded to bf16 after adding."""
    x = normal_bf16(seed, S_X, (T, H), 1.0)
    bg = normal_f32(seed, S_WGATE, (F, H), wsig)
    bu = normal_f32(seed, S_WUP, (F, H), wsig)
    bd = normal_f32(seed, S_WDOWN, (H, F), wsig)
    n = F * H
    Wgate = np.empty((N, F, H), np.uint16)
    Wup = np.empty((N, F, H), np.uint16)
    Wdown = np.empty((N, H, F), np.uint16)
    for e in range(N):
        if perturb > 0:
            Wgate[e] = perturb_bf16(bg, seed, S_PERTURB0 + e, perturb, 0)
            Wup[e] = perturb_bf16(bu, seed, S_PERTURB0 + e, perturb, n)
            Wdown[e] = perturb_bf16(bd, seed, S_PERTURB0 + e, perturb, 2 * n)
        else:
            Wgate[e] = f32_to_bf16(bg)
            Wup[e] = f32_to_bf16(bu)
            Wdown[e] = f32_to_bf16(bd)
    Wg = normal_f32(seed, S_WG, (H, N), wsig)
    w = Workload(name, T, H, F, N, k, capacity, order, False, False, out_scale, "bf16", "bf16",
                 x, Wg, None, None, Wgate, Wup, Wdown)
    w.meta.update(kind="upcycled", seed=seed, perturb=perturb)
    if keep_base:
        w.meta["base"] = (bg, bu, bd)
    return w


def make_independent(name, seed, T, H, F, N, k, *, act="bf16", wt="bf16", order=MIXTRAL, noisy=False,
                     want_stats=False, out_scale=1.0, capacity=-1, wsig=0.02) -> Workload:
    """N independently drawn experts (no shared dense parent)."""
    x = _rand_w(seed, S_X, (T, H), 1.0, act)
    Wgate = _rand_w(seed, S_WGATE, (N, F, H), wsig, wt)
    Wup = _rand_w(seed, S_WUP, (N, F, H), wsig, wt)
    Wdown = _rand_w(seed, S_WDOWN, (N, H, F), wsig, wt)
    Wg = normal_f32(seed, S_WG, (H, N), wsig)
    Wn = normal_f32(seed, S_WNOISE, (H, N), wsig) if noisy else None
    eps = normal_f32(seed, S_EPS, (T, N), 1.0) if noisy else None
    w = Workload(name, T, H, F, N, k, capacity, order, noisy, want_stats, out_scale, act, wt,
                 x, Wg, Wn, eps, Wgate, Wup, Wdown)
    w.meta.update(kind="independent", seed=seed)
    return w


def apply_skew(w: Workload, n_pref: int, boost: float = 8.0, expert: int = 0):
    """Skew routing so that a seeded set of n_pref tokens prefers `expert`.

    A seeded unit vector u is added to the router column of `expert`; every
    token has its u-component removed, and the chosen tokens get boost*u
    instead, which raises their logit for `expert` by about `boost`.
    """
    seed = w.meta["seed"]
    x = w.f32("x").astype(np.float64)
    u = normal_f32(seed, S_SKEW_DIR, (w.H,), 1.0).astype(np.float64)
    u /= np.linalg.norm(u)
    chosen = np.sort(permutation(seed, S_SKEW_SET, w.T)[:n_pref])
    x = x - np.outer(x @ u, u)
    x[chosen] += boost * u
    xf = x.astype(np.float32)
    w.x = f32_to_bf16(xf) if w.act == "bf16" else xf
    Wg = w.Wg.astype(np.float64)
    Wg[:, expert] += u
    w.Wg = Wg.astype(np.float32)
    w.meta.update(skew_tokens=chosen, skew_expert=expert)
    return w


# ----------------------------------------------------------------------------
# The five named workloads. Seeds are 1000 + config number.
# ----------------------------------------------------------------------------

def c1() -> Workload:
    """Tiny fp32 layer: 256 tokens, hidden 256, intermediate 688 split into
    8 experts of 86, top-2, Mixtral order, no noise, dropless, s = 1."""
    return make_split("C1_tiny_fp32", 1001, 256, 256, 688, 8, 2, act="f32", wt="f32", out_scale=1.0)


def c2(T: int = 4096) -> Workload:
    """LLaMA-MoE-3.5B (2/8) layer: hidden 4096, LLaMA-2-7B intermediate 11008
    split into 8 experts of 1376, top-2, dropless, s = N/k = 4."""
    return make_split("C2_llama_moe_2of8", 1002, T, 4096, 11008, 8, 2, out_scale=4.0)


def c3(T: int = 4096) -> Workload:
    """LLaMA-MoE-3.5B (4/16) layer: 16 experts of 688, top-4, noisy gate,
    stats, dropless, s = N/k = 4."""
    return make_split("C3_llama_moe_4of16_noisy", 1003, T, 4096, 11008, 16, 4, noisy=True,
                      want_stats=True, out_scale=4.0)


def c4(variant: str = "cf4", T: int = 8192) -> Workload:
    """Llama-3-8B upcycled E8T2: 8 perturbed copies of a 14336-wide FFN,
    top-2 Mixtral, s = 1. variant: cf4 | cf1 | dropless | cf1_assign."""
    N, k = 8, 2
    cap = {"cf4": capacity_from_cf(T, N, k, 4.0), "cf1": capacity_from_cf(T, N, k, 1.0),
           "dropless": -1, "cf1_assign": capacity_from_cf(T, N, k, 1.0, count_assignments=True)}[variant]
    w = make_upcycled(f"C4_llama3_e8t2_{variant}", 1004, T, 4096, 14336, N, k, capacity=cap)
    w.meta["variant"] = variant
    return w


def c5() -> Workload:
    """Decode-shaped E8T2: 64 tokens, 8 experts of 14336, top-2, with half of
    the tokens steered to prefer expert 0; dropless, s = 1."""
    w = make_independent("C5_decode_e8t2_skewed", 1005, 64, 4096, 14336, 8, 2)
    return apply_skew(w, n_pref=32)


CONFIGS = {"C1": c1, "C2": c2, "C3": c3, "C4": c4, "C5": c5}
