"""Deterministic backward of the fused linear log-probability.

    grad_hidden, grad_weight, grad_bias = backward(hidden, weight, target, bias,
                                                   lse, grad_logp, grad_lse)
    logp, lse = linear_logp(hidden, weight, target, bias)     # autograd-capable

The forward's first contract (RL-Kernel PR #337, author's annotation on the
``requires_grad`` check) stops at the forward; this module extends it with
the gradients of both outputs, reduced in fixed orders (the deterministic
GEMM layouts of RL-Kernel PR #395, summary):

    dZ[i, v]     = g_lse[i] P[i, v] + g_logp[i] ([v == target[i]] - P[i, v]),
                   P = exp(z - lse), z recomputed tile by tile, dZ kept in bf16
    grad_hidden  = dZ . W          (rows batch-invariant)
    grad_weight  = dZ^T . hidden   (ascending row order)
    grad_bias    = sum_i dZ[i, :]  (ascending row order)

``forward`` keeps the page's fail-closed forward-only contract; training
code calls ``linear_logp`` (or ``backward`` directly).
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from ._binding import bilogp_backward, bilogp_backward_workspace_bytes

__all__ = ["backward", "backward_workspace_for", "linear_logp", "LinearLogp"]

_BAD = (1 << 64) - 1


def backward_workspace_for(N: int, V: int, device) -> torch.Tensor:
    """A uint8 device tensor big enough for ``bilogp_backward`` (it holds dZ^T
    in bf16, [V, N rounded up to 8], and the padded fp32 bias)."""
    nbytes = bilogp_backward_workspace_bytes(N, V)
    if nbytes == _BAD:
        raise ValueError(f"invalid sizes N={N}, V={V} (the backward takes N <= 2^21)")
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def backward(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
             bias: Optional[torch.Tensor], lse: torch.Tensor, grad_logp: torch.Tensor,
             grad_lse: torch.Tensor, *, bias_grad: bool = True,
             workspace: Optional[torch.Tensor] = None
             ) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """(grad_hidden, grad_weight, grad_bias), fp32, shaped like hidden, weight
    and bias (grad_bias None without a bias or with ``bias_grad=False``).

    hidden [..., H] bf16, weight [V, H] bf16, target [...] int64, bias [V]
    bf16 / fp32 or None; lse, grad_logp, grad_lse: fp32 with target's shape
    (lse is the forward's output for these inputs).  A target outside
    [0, V) contributes no one-hot term.
    """
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    if target.dtype != torch.int64:
        raise TypeError("target must be int64")
    if weight.dim() != 2 or hidden.dim() < 1 or hidden.shape[-1] != weight.shape[1]:
        raise ValueError(f"shape mismatch: hidden {tuple(hidden.shape)}, "
                         f"weight {tuple(weight.shape)}")
    lead = tuple(hidden.shape[:-1])
    for name, t in (("target", target), ("lse", lse), ("grad_logp", grad_logp),
                    ("grad_lse", grad_lse)):
        if tuple(t.shape) != lead:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {lead}")
    for name, t in (("lse", lse), ("grad_logp", grad_logp), ("grad_lse", grad_lse)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    V, H = weight.shape
    if bias is not None:
        if bias.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("bias must be bfloat16 or float32")
        if tuple(bias.shape) != (V,):
            raise ValueError(f"bias shape {tuple(bias.shape)} != ({V},)")
    tensors = [hidden, weight, target, lse, grad_logp, grad_lse] + \
        ([bias] if bias is not None else [])
    dev = weight.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors):
        raise ValueError("all tensors must be on the same GPU")

    with torch.no_grad():
        h2 = hidden.reshape(-1, H).contiguous()
        N = h2.shape[0]
        flat = [t.reshape(-1).contiguous() for t in (target, lse, grad_logp, grad_lse)]
        w2 = weight.contiguous()
        b1 = None if bias is None else bias.contiguous()
        gh = torch.empty((N, H), dtype=torch.float32, device=dev)
        gw = torch.empty((V, H), dtype=torch.float32, device=dev)
        gb = torch.empty(V, dtype=torch.float32, device=dev) \
            if (bias is not None and bias_grad) else None
        ws = workspace if workspace is not None else backward_workspace_for(N, V, dev)
        bilogp_backward(h2, w2, flat[0], b1, flat[1], flat[2], flat[3], gh, gw, gb, ws)
    return gh.reshape(hidden.shape), gw, gb


class LinearLogp(torch.autograd.Function):
    """(logp, lse) with the deterministic backward above.  Gradients are
    returned in the inputs' dtypes (fp32 results rounded once)."""

    @staticmethod
    def forward(ctx, hidden, weight, target, bias):
        from . import forward as _forward      # the package's fail-closed forward
        with torch.no_grad():
            logp, lse = _forward(hidden.detach(), weight.detach(), target,
                                 None if bias is None else bias.detach())
        ctx.save_for_backward(hidden, weight, target, bias, lse)
        return logp, lse

    @staticmethod
    def backward(ctx, g_logp, g_lse):
        hidden, weight, target, bias, lse = ctx.saved_tensors
        need_h, need_w, _, need_b = ctx.needs_input_grad
        gh, gw, gb = backward(hidden, weight, target, bias, lse, g_logp.float().contiguous(),
                              g_lse.float().contiguous(), bias_grad=bool(need_b))
        return (gh.to(hidden.dtype) if need_h else None,
                gw.to(weight.dtype) if need_w else None,
                None,
                gb.to(bias.dtype) if (need_b and gb is not None) else None)


def linear_logp(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                bias: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """``forward`` with autograd support through ``backward``."""
    return LinearLogp.apply(hidden, weight, target, bias)
