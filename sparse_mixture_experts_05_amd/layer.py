"""MoELayer: a convenience holder for one layer's weights and workspace.

Its constructor mirrors the layer interface of the LLaMA-MoE v2 article's code
example (dim, hidden_dim, num_experts, k); forward() calls moe_forward, so all
arithmetic runs in libmoe.so. Inference only (no autograd).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import abi


class MoELayer:
    def __init__(self, dim: int, hidden_dim: int, num_experts: int, k: int = 2, *, capacity: int = -1,
                 order: int = abi.MOE_TOPK_THEN_SOFTMAX, out_scale: float = 1.0, dtype=torch.bfloat16,
                 device="cuda", out_dtype=torch.float32):
        self.H, self.F, self.N, self.k = dim, hidden_dim, num_experts, k
        self.capacity, self.order, self.out_scale = capacity, order, out_scale
        self.dtype, self.out_dtype, self.device = dtype, out_dtype, torch.device(device)
        self.Wg = torch.zeros(dim, num_experts, dtype=torch.float32, device=device)
        self.Wn: Optional[torch.Tensor] = None
        self.Wgate = torch.zeros(num_experts, hidden_dim, dim, dtype=dtype, device=device)
        self.Wup = torch.zeros_like(self.Wgate)
        self.Wdown = torch.zeros(num_experts, dim, hidden_dim, dtype=dtype, device=device)
        self.load_balancing_loss: Optional[torch.Tensor] = None
        self._ws: Optional[torch.Tensor] = None

    def config(self, T: int, noisy: bool, want_stats: bool) -> abi.MoEConfig:
        act = "bf16" if self.dtype == torch.bfloat16 else "f32"
        return abi.MoEConfig(T=T, H=self.H, F=self.F, N=self.N, k=self.k, capacity=self.capacity, order=self.order,
                             noisy=noisy, want_stats=want_stats, out_scale=self.out_scale, act=act, wt=act,
                             out="f32" if self.out_dtype == torch.float32 else "bf16")

    def forward(self, x: torch.Tensor, eps: Optional[torch.Tensor] = None, want_stats: bool = False):
        """x: [..., H]. eps: [T, N] standard-normal draws (turns the noisy gate
        on; needs self.Wn). Returns y with x's leading shape."""
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.H).contiguous()
        T = x2.shape[0]
        noisy = eps is not None
        cfg = self.config(T, noisy, want_stats)
        need = max(256, abi.moe_workspace_bytes(cfg))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        y = torch.empty(T, self.H, dtype=self.out_dtype, device=self.device)
        bal = torch.empty(1, dtype=torch.float32, device=self.device) if want_stats else None
        abi.moe_forward(cfg, x2, self.Wg, self.Wn if noisy else None, eps, self.Wgate, self.Wup, self.Wdown, y,
                        balance=bal, ws=self._ws)
        self.load_balancing_loss = bal
        return y.reshape(*lead, self.H)

    __call__ = forward
