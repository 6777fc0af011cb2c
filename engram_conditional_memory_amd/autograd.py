"""PyTorch autograd binding of the Engram gate.

The juejin.cn TileKernels page (highlight 5) describes a torch.autograd.Function
around the Engram gate: forward, backward and the weight-gradient reduction.
This module is that wrapper over the C-ABI calls of libtk_engram.so:

    forward   tk_engram_fused_weight    w = wh * we (fp64), once per step
              tk_engram_gate_fwd_fused  out = x + gate * v
    backward  tk_engram_gate_bwd_fused  dx, dk, dv and per-block partials
              tk_engram_grad_w_reduce   dwh, dwe from the partials

The zhichai.net page's section "5. Engram" lists the fused weight as the
weight preprocessing ahead of the gate; the forward and the backward read it
in place of the two RMSNorm weights, and the reduction, which needs the two
separately, takes wh and we.

The gate itself is the formula of the zhichai.net TileKernels page, section
"5. Engram". Inputs of any leading shape [..., H] are flattened to [T, H]
rows; x, k, v are bf16 and the RMSNorm weights wh, we are fp32. Autograd
accumulates the returned gradients into .grad as usual. Every step runs in the
library's HIP kernels; there is no other implementation.
"""

from __future__ import annotations

import torch

from . import _binding as B


def _rows(t: torch.Tensor, H: int) -> torch.Tensor:
    return t.reshape(-1, H).contiguous()


class EngramGateFunction(torch.autograd.Function):
    """out, gate = EngramGateFunction.apply(x, k, v, wh, we, eps, dsqrt_clamp).

    `gate` (fp32, one per token) is returned for inspection and is not
    differentiable; gradients flow through `out` only."""

    @staticmethod
    def forward(ctx, x, k, v, wh, we, eps=B.EPS, dsqrt_clamp=B.DSQRT_CLAMP):
        H = x.shape[-1]
        lead = x.shape[:-1]
        if k.shape != x.shape or v.shape != x.shape:
            raise ValueError(f"x, k, v must have the same shape, got {tuple(x.shape)}, "
                             f"{tuple(k.shape)}, {tuple(v.shape)}")
        x2, k2, v2 = _rows(x, H), _rows(k, H), _rows(v, H)
        wh_c, we_c = wh.contiguous(), we.contiguous()
        w = B.tk_engram_fused_weight(wh_c, we_c)
        out, gate = B.tk_engram_gate_fwd_fused(x2, k2, v2, w, eps=eps)
        ctx.save_for_backward(x2, k2, v2, wh_c, we_c, w)
        ctx.eps, ctx.clamp, ctx.lead, ctx.H = eps, dsqrt_clamp, lead, H
        gate = gate.view(lead)
        ctx.mark_non_differentiable(gate)
        return out.view(*lead, H), gate

    @staticmethod
    def backward(ctx, grad_out, grad_gate):
        x2, k2, v2, wh, we, w = ctx.saved_tensors
        H = ctx.H
        g = _rows(grad_out.to(torch.bfloat16), H)
        dx, dk, dv, ws, P = B.tk_engram_gate_bwd_fused(g, x2, k2, v2, w, eps=ctx.eps,
                                                       dsqrt_clamp=ctx.clamp)
        dwh = dwe = None
        if ctx.needs_input_grad[3] or ctx.needs_input_grad[4]:
            dwh, dwe = B.tk_engram_grad_w_reduce(ws, P, H, wh, we)
        lead = ctx.lead
        return (dx.view(*lead, H), dk.view(*lead, H), dv.view(*lead, H),
                dwh if ctx.needs_input_grad[3] else None,
                dwe if ctx.needs_input_grad[4] else None, None, None)


def engram_gate(x, k, v, wh, we, eps=B.EPS, dsqrt_clamp=B.DSQRT_CLAMP):
    """Functional form: returns (out, gate)."""
    return EngramGateFunction.apply(x, k, v, wh, we, eps, dsqrt_clamp)


class EngramGate(torch.nn.Module):
    """The gate as a module with its two RMSNorm weights as parameters.

    forward(x, k, v) returns x + gate * v; x, k, v are [..., H] bf16
    on the GPU; `last_gate` keeps the most recent per-token gate (fp32)."""

    def __init__(self, hidden_size: int, eps: float = B.EPS,
                 dsqrt_clamp: float = B.DSQRT_CLAMP, device=None):
        super().__init__()
        self.hidden_size = hidden_size
        self.eps = eps
        self.dsqrt_clamp = dsqrt_clamp
        self.wh = torch.nn.Parameter(torch.ones(hidden_size, dtype=torch.float32, device=device))
        self.we = torch.nn.Parameter(torch.ones(hidden_size, dtype=torch.float32, device=device))
        self.last_gate = None

    def forward(self, x, k, v):
        if x.shape[-1] != self.hidden_size:
            raise ValueError(f"last dimension must be {self.hidden_size}, got {x.shape[-1]}")
        out, gate = EngramGateFunction.apply(x, k, v, self.wh, self.we,
                                             self.eps, self.dsqrt_clamp)
        self.last_gate = gate
        return out

    def extra_repr(self) -> str:
        return f"hidden_size={self.hidden_size}, eps={self.eps}, dsqrt_clamp={self.dsqrt_clamp}"
