"""ctypes binding of libmoe.so (the C ABI declared in include/moe.h).

Argument marshalling only: every function here takes torch device tensors,
passes their raw pointers and the HIP stream to the C entry point of the same
name, and raises MoEError on a non-OK status. No computation happens here, and
there is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libmoe_debug.so")  # the same ABI with recorded bounds checks

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_TOPK_THEN_SOFTMAX, MOE_SOFTMAX_THEN_TOPK = 0, 1
(MOE_KERNEL_ROUTER, MOE_KERNEL_HIST, MOE_KERNEL_SCATTER, MOE_KERNEL_GATHER, MOE_KERNEL_GEMM1,
 MOE_KERNEL_GEMM2, MOE_KERNEL_COMBINE, MOE_KERNEL_STATS, MOE_KERNEL_EXPERTS, MOE_KERNEL_BWD_GATE,
 MOE_KERNEL_BWD_DGRAD, MOE_KERNEL_BWD_DX, MOE_KERNEL_BWD_WGRAD, MOE_KERNEL_BWD_ROUTER) = range(14)

EXPORTED = ["moe_capacity", "moe_check", "moe_workspace_bytes", "moe_route", "moe_permute",
            "moe_grouped_swiglu", "moe_combine", "moe_forward", "moe_status_str", "moe_last_error",
            "moe_profile_select", "moe_profile_read", "moe_debug_set_wait", "moe_forward_noalloc",
            "moe_noalloc_scratch_bytes", "moe_forward_residual", "moe_residual_workspace_bytes",
            "moe_train_workspace_bytes", "moe_forward_train", "moe_backward", "moe_debug_build",
            "moe_debug_word_offset"]


class moe_cfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("F", ctypes.c_int32), ("N", ctypes.c_int32),
                ("k", ctypes.c_int32), ("capacity", ctypes.c_int32), ("order", ctypes.c_int32),
                ("noisy", ctypes.c_int32), ("want_stats", ctypes.c_int32), ("out_scale", ctypes.c_float),
                ("act", ctypes.c_int32), ("wt", ctypes.c_int32), ("out", ctypes.c_int32)]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {_status_name(status)}: {message}")
        self.status = status


_lib = None


def load_library(path: Optional[str] = None):
    """Load libmoe.so. Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing; build it with sparse_mixture_experts_05_amd/build.py "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(p)
    vp, i32, i64, f64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
    cfgp = ctypes.POINTER(moe_cfg)
    lib.moe_capacity.argtypes = [i64, i32, i32, f64, i32]
    lib.moe_capacity.restype = i32
    lib.moe_check.argtypes = [cfgp]
    lib.moe_check.restype = i32
    lib.moe_workspace_bytes.argtypes = [cfgp]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_route.argtypes = [cfgp] + [vp] * 12 + [vp, sz, vp]
    lib.moe_route.restype = i32
    lib.moe_permute.argtypes = [cfgp] + [vp] * 7 + [vp, sz, vp]
    lib.moe_permute.restype = i32
    lib.moe_grouped_swiglu.argtypes = [cfgp] + [vp] * 7 + [vp, sz, vp]
    lib.moe_grouped_swiglu.restype = i32
    lib.moe_combine.argtypes = [cfgp] + [vp] * 4 + [vp]
    lib.moe_combine.restype = i32
    lib.moe_forward.argtypes = [cfgp] + [vp] * 16 + [vp, sz, vp]
    lib.moe_forward.restype = i32
    lib.moe_status_str.argtypes = [i32]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_profile_select.argtypes = [i32]
    lib.moe_profile_select.restype = i32
    lib.moe_profile_read.argtypes = [ctypes.POINTER(f64), ctypes.POINTER(i64)]
    lib.moe_profile_read.restype = i32
    lib.moe_forward_noalloc.argtypes = [cfgp] + [vp] * 16 + [vp]
    lib.moe_forward_noalloc.restype = i32
    lib.moe_forward_residual.argtypes = [cfgp, i32] + [vp] * 19 + [vp, sz, vp]
    lib.moe_forward_residual.restype = i32
    lib.moe_residual_workspace_bytes.argtypes = [cfgp, i32]
    lib.moe_residual_workspace_bytes.restype = sz
    lib.moe_train_workspace_bytes.argtypes = [cfgp]
    lib.moe_train_workspace_bytes.restype = sz
    lib.moe_forward_train.argtypes = [cfgp] + [vp] * 14 + [vp, sz, vp]
    lib.moe_forward_train.restype = i32
    lib.moe_backward.argtypes = [cfgp] + [vp] * 8 + [ctypes.c_float] + [vp] * 6 + [vp, sz, vp]
    lib.moe_backward.restype = i32
    lib.moe_noalloc_scratch_bytes.argtypes = []
    lib.moe_noalloc_scratch_bytes.restype = sz
    lib.moe_debug_set_wait.argtypes = [i32, i32]
    lib.moe_debug_set_wait.restype = i32
    lib.moe_debug_build.argtypes = []
    lib.moe_debug_build.restype = i32
    lib.moe_debug_word_offset.argtypes = [cfgp]
    lib.moe_debug_word_offset.restype = sz
    if path is None:
        _lib = lib
    return lib


def _status_name(s: int) -> str:
    return {0: "MOE_OK", 1: "MOE_ERR_INVALID", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
            4: "MOE_ERR_DEVICE"}.get(s, f"status {s}")


def _check(status: int, where: str):
    if status != MOE_OK:
        msg = load_library().moe_last_error().decode(errors="replace")
        raise MoEError(status, where, msg)


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _s(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


_DT = {"f32": MOE_F32, "bf16": MOE_BF16, torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}


@dataclass
class MoEConfig:
    """Python mirror of moe_cfg (see include/moe.h for every field)."""
    T: int
    H: int
    F: int
    N: int
    k: int
    capacity: int = -1
    order: int = MOE_TOPK_THEN_SOFTMAX
    noisy: bool = False
    want_stats: bool = False
    out_scale: float = 1.0
    act: str = "bf16"
    wt: str = "bf16"
    out: str = "f32"

    def c(self) -> moe_cfg:
        return moe_cfg(T=self.T, H=self.H, F=self.F, N=self.N, k=self.k, capacity=int(self.capacity),
                       order=int(self.order), noisy=int(bool(self.noisy)), want_stats=int(bool(self.want_stats)),
                       out_scale=float(self.out_scale), act=_DT[self.act], wt=_DT[self.wt], out=_DT[self.out])


def moe_capacity(T: int, N: int, k: int, cf: float, count_assignments: bool = False) -> int:
    return int(load_library().moe_capacity(T, N, k, cf, int(count_assignments)))


def moe_check(cfg: MoEConfig) -> int:
    c = cfg.c()
    return int(load_library().moe_check(ctypes.byref(c)))


def moe_workspace_bytes(cfg: MoEConfig) -> int:
    c = cfg.c()
    return int(load_library().moe_workspace_bytes(ctypes.byref(c)))


def workspace(cfg: MoEConfig, device="cuda") -> torch.Tensor:
    """A workspace tensor of moe_workspace_bytes(cfg) bytes (at least 256)."""
    n = max(256, moe_workspace_bytes(cfg))
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_route(cfg, x, Wg, Wn, eps, logits, topk_idx, topk_w, load=None, importance=None, P=None, balance=None,
              ws=None, stream=None, smooth_load=None):
    c = cfg.c()
    _check(load_library().moe_route(ctypes.byref(c), _p(x), _p(Wg), _p(Wn), _p(eps), _p(logits), _p(topk_idx),
                                    _p(topk_w), _p(load), _p(importance), _p(P), _p(balance), _p(smooth_load),
                                    _p(ws),
                                    0 if ws is None else ws.numel(), _s(stream)), "moe_route")


def moe_permute(cfg, x, topk_idx, counts, offsets, slot, row_token, x_perm=None, ws=None, stream=None):
    c = cfg.c()
    _check(load_library().moe_permute(ctypes.byref(c), _p(x), _p(topk_idx), _p(counts), _p(offsets), _p(slot),
                                      _p(row_token), _p(x_perm), _p(ws), 0 if ws is None else ws.numel(),
                                      _s(stream)), "moe_permute")


def moe_grouped_swiglu(cfg, x_perm_or_x, row_token, offsets, Wgate, Wup, Wdown, y_perm, ws=None, stream=None):
    c = cfg.c()
    _check(load_library().moe_grouped_swiglu(ctypes.byref(c), _p(x_perm_or_x), _p(row_token), _p(offsets),
                                             _p(Wgate), _p(Wup), _p(Wdown), _p(y_perm), _p(ws),
                                             0 if ws is None else ws.numel(), _s(stream)), "moe_grouped_swiglu")


def moe_combine(cfg, y_perm, slot, topk_w, y, stream=None):
    c = cfg.c()
    _check(load_library().moe_combine(ctypes.byref(c), _p(y_perm), _p(slot), _p(topk_w), _p(y), _s(stream)),
           "moe_combine")


def moe_forward(cfg, x, Wg, Wn, eps, Wgate, Wup, Wdown, y, topk_idx=None, topk_w=None, kept=None, load=None,
                importance=None, P=None, balance=None, ws=None, stream=None, smooth_load=None):
    c = cfg.c()
    _check(load_library().moe_forward(ctypes.byref(c), _p(x), _p(Wg), _p(Wn), _p(eps), _p(Wgate), _p(Wup),
                                      _p(Wdown), _p(y), _p(topk_idx), _p(topk_w), _p(kept), _p(load),
                                      _p(importance), _p(P), _p(balance), _p(smooth_load), _p(ws),
                                      0 if ws is None else ws.numel(), _s(stream)), "moe_forward")


def moe_forward_noalloc(cfg, x, Wg, Wn, eps, Wgate, Wup, Wdown, y, topk_idx=None, topk_w=None, kept=None,
                        load=None, importance=None, P=None, balance=None, stream=None, smooth_load=None):
    c = cfg.c()
    _check(load_library().moe_forward_noalloc(ctypes.byref(c), _p(x), _p(Wg), _p(Wn), _p(eps), _p(Wgate), _p(Wup),
                                              _p(Wdown), _p(y), _p(topk_idx), _p(topk_w), _p(kept), _p(load),
                                              _p(importance), _p(P), _p(balance), _p(smooth_load), _s(stream)),
           "moe_forward_noalloc")


def moe_residual_workspace_bytes(cfg: MoEConfig, F_shared: int) -> int:
    c = cfg.c()
    return int(load_library().moe_residual_workspace_bytes(ctypes.byref(c), int(F_shared)))


def moe_forward_residual(cfg, F_shared, x, Wg, Wn, eps, Wgate, Wup, Wdown, Ws_gate, Ws_up, Ws_down, y, topk_idx=None,
                         topk_w=None, kept=None, load=None, importance=None, P=None, balance=None, smooth_load=None,
                         ws=None, stream=None):
    c = cfg.c()
    _check(load_library().moe_forward_residual(ctypes.byref(c), int(F_shared), _p(x), _p(Wg), _p(Wn), _p(eps),
                                               _p(Wgate), _p(Wup), _p(Wdown), _p(Ws_gate), _p(Ws_up), _p(Ws_down),
                                               _p(y), _p(topk_idx), _p(topk_w), _p(kept), _p(load), _p(importance),
                                               _p(P), _p(balance), _p(smooth_load), _p(ws),
                                               0 if ws is None else ws.numel(), _s(stream)), "moe_forward_residual")


def moe_train_workspace_bytes(cfg: MoEConfig) -> int:
    c = cfg.c()
    return int(load_library().moe_train_workspace_bytes(ctypes.byref(c)))


def moe_forward_train(cfg, x, Wg, Wn, eps, Wgate, Wup, Wdown, y, kept=None, load=None, importance=None, P=None,
                      balance=None, smooth_load=None, ws=None, stream=None):
    c = cfg.c()
    _check(load_library().moe_forward_train(ctypes.byref(c), _p(x), _p(Wg), _p(Wn), _p(eps), _p(Wgate), _p(Wup),
                                            _p(Wdown), _p(y), _p(kept), _p(load), _p(importance), _p(P),
                                            _p(balance), _p(smooth_load), _p(ws), 0 if ws is None else ws.numel(),
                                            _s(stream)), "moe_forward_train")


def moe_backward(cfg, x, Wg, Wn, eps, Wgate, Wup, Wdown, dy, d_balance, dx, dWg, dWn, dWgate, dWup, dWdown, ws=None,
                 stream=None):
    c = cfg.c()
    _check(load_library().moe_backward(ctypes.byref(c), _p(x), _p(Wg), _p(Wn), _p(eps), _p(Wgate), _p(Wup),
                                       _p(Wdown), _p(dy), float(d_balance), _p(dx), _p(dWg), _p(dWn), _p(dWgate),
                                       _p(dWup), _p(dWdown), _p(ws), 0 if ws is None else ws.numel(), _s(stream)),
           "moe_backward")


def moe_noalloc_scratch_bytes() -> int:
    return int(load_library().moe_noalloc_scratch_bytes())


def moe_profile_select(kernel_id: int):
    _check(load_library().moe_profile_select(kernel_id), "moe_profile_select")


def moe_profile_read():
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(load_library().moe_profile_read(ctypes.byref(ms), ctypes.byref(n)), "moe_profile_read")
    return ms.value, n.value


def moe_debug_set_wait(spin_limit: int, wait_extra: int):
    _check(load_library().moe_debug_set_wait(int(spin_limit), int(wait_extra)), "moe_debug_set_wait")


def moe_debug_build() -> bool:
    return bool(load_library().moe_debug_build())


def moe_debug_word_offset(cfg: MoEConfig) -> int:
    return int(load_library().moe_debug_word_offset(ctypes.byref(cfg.c())))


@contextlib.contextmanager
def use_library(path: str):
    """Route every call of this module through the library at `path` (for
    example DEBUG_LIB_PATH) inside the block."""
    global _lib
    saved = load_library()
    _lib = load_library(path)
    try:
        yield _lib
    finally:
        _lib = saved
