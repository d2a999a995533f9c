"""MoELayer: a convenience holder for one layer's weights and workspace, and
MoEFunction, the layer as a torch.autograd.Function.

MoELayer's constructor mirrors the layer interface of the LLaMA-MoE v2
article's code example (dim, hidden_dim, num_experts, k); forward() calls
moe_forward and forward_train() MoEFunction, so all arithmetic of the layer and
of its gradients runs in libmoe.so.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import abi


class MoEFunction(torch.autograd.Function):
    """One MoE layer for training: forward runs moe_forward_train, backward
    runs moe_backward (continual pre-training, the LLaMA-MoE pages' workload).

    apply(x, Wg, Wn, eps, Wgate, Wup, Wdown, cfg) -> (y, balance):
      x [T,H] and the expert weights as cfg says (bf16 for the training path),
      Wg and Wn [H,N] fp32 (Wn and eps None for the clean gate; eps [T,N]
      carries no gradient); cfg a MoEConfig with want_stats set. y [T,H] fp32;
      balance [1] fp32 is the balance statistic sum_i f_i P_i, and its
      gradient (the loss weight) reaches the router as moe_backward's
      d_balance, read to the host when backward runs.
    The gradients come back in fp32; autograd casts those of bf16 inputs to
    bf16. The training workspace lives from forward to backward."""

    @staticmethod
    def forward(ctx, x, Wg, Wn, eps, Wgate, Wup, Wdown, cfg):
        T = x.shape[0]
        ws = torch.empty(max(256, abi.moe_train_workspace_bytes(cfg)), dtype=torch.uint8, device=x.device)
        y = torch.empty(T, cfg.H, dtype=torch.float32, device=x.device)
        bal = torch.empty(1, dtype=torch.float32, device=x.device)
        abi.moe_forward_train(cfg, x, Wg, Wn, eps, Wgate, Wup, Wdown, y, balance=bal, ws=ws)
        ctx.save_for_backward(x, Wg, Wn, eps, Wgate, Wup, Wdown)
        ctx.ws, ctx.cfg = ws, cfg
        ctx.set_materialize_grads(False)  # an unused balance gives None, and no host read
        return y, bal

    @staticmethod
    def backward(ctx, dy, dbal):
        x, Wg, Wn, eps, Wgate, Wup, Wdown = ctx.saved_tensors
        cfg = ctx.cfg
        T, H, F, N = x.shape[0], cfg.H, cfg.F, cfg.N
        dev = x.device
        d_balance = float(dbal.reshape(-1)[0].item()) if dbal is not None else 0.0
        if dy is None:
            dy = torch.zeros(T, H, dtype=torch.float32, device=dev)
        dy = dy.contiguous()
        f32 = dict(dtype=torch.float32, device=dev)
        dx = torch.empty(T, H, **f32)
        dWg = torch.empty(H, N, **f32)
        dWn = torch.empty(H, N, **f32) if Wn is not None else None
        dWgate, dWup = torch.empty(N, F, H, **f32), torch.empty(N, F, H, **f32)
        dWdown = torch.empty(N, H, F, **f32)
        abi.moe_backward(cfg, x, Wg, Wn, eps, Wgate, Wup, Wdown, dy, d_balance, dx, dWg, dWn, dWgate, dWup, dWdown,
                         ws=ctx.ws)
        ctx.ws = None
        return dx, dWg, dWn, None, dWgate, dWup, dWdown, None


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

    def forward_train(self, x: torch.Tensor, eps: Optional[torch.Tensor] = None):
        """x: [T, H] bf16. Returns (y [T, H] fp32, balance [1]) through
        MoEFunction, so that autograd reaches x and every weight that requires
        a gradient (bf16 experts, F % 8 == 0, more than 48 rows per expert on
        average; otherwise the library reports MOE_ERR_UNSUPPORTED)."""
        noisy = eps is not None
        cfg = self.config(x.shape[0], noisy, True)
        return MoEFunction.apply(x.contiguous(), self.Wg, self.Wn if noisy else None, eps, self.Wgate, self.Wup,
                                 self.Wdown, cfg)
