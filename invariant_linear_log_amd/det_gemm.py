"""Deterministic bf16 GEMM on gfx950 (RL-Kernel PR #395, "feat(musa): add
native deterministic gemm kernel": a fixed ascending contraction order with
fp32 accumulation; the forward [M, K] @ [N, K]^T without materialising the
transposed right-hand side; dA and the [N, K] weight gradient; an autograd
wrapper for ``linear(A, weight[N, K])``).

    C = det_gemm(a, b)               # a [M, K], b [N, K] bf16 -> [M, N]
    C = det_gemm(a, b, out_dtype=torch.float32)
    det_gemm(a, b, out=c32, accumulate=True)      # c32 += a . b^T
    dA = det_gemm_da(dc, b)          # [M, N] . [N, K] -> [M, K]
    dB = det_gemm_db(a, dc)          # [M, N]^T . [M, K] -> [N, K]
    y = DetLinear.apply(a, w)        # differentiable; backward uses dA / dB

Every output element's bits depend only on the two vectors it contracts: the
rows of the forward and of dA do not depend on M.  All work runs in the HIP
library; a missing library raises.
"""

from __future__ import annotations

from typing import Optional

import torch

from ._binding import bilogp_det_gemm_da, bilogp_det_gemm_db, bilogp_det_gemm_fwd


def _check_bf16(*ts):
    for t in ts:
        if t.dtype != torch.bfloat16:
            raise TypeError(f"det_gemm operands must be bfloat16, got {t.dtype}")
        if t.dim() != 2:
            raise ValueError("det_gemm operands must be 2-D")
        if t.device.type != "cuda" or t.device != ts[0].device:
            raise ValueError("det_gemm operands must be on the same GPU")


def _out(shape, dtype, device, out, accumulate):
    if out is None:
        if accumulate:
            raise ValueError("accumulate=True needs an output tensor")
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(out.shape) != tuple(shape) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {tuple(shape)} tensor")
    return out


def det_gemm(a: torch.Tensor, b: torch.Tensor, *, out_dtype=torch.bfloat16,
             out: Optional[torch.Tensor] = None, accumulate: bool = False) -> torch.Tensor:
    """a[M, K] . b[N, K]^T (bf16 in; bf16 or fp32 out; ``accumulate`` adds
    into a float32 ``out``)."""
    _check_bf16(a, b)
    if a.shape[1] != b.shape[1]:
        raise ValueError(f"K mismatch: {tuple(a.shape)} vs {tuple(b.shape)}")
    a, b = a.contiguous(), b.contiguous()
    c = _out((a.shape[0], b.shape[0]), out_dtype, a.device, out, accumulate)
    bilogp_det_gemm_fwd(a, b, c, accumulate)
    return c


def det_gemm_da(dc: torch.Tensor, b: torch.Tensor, *, out_dtype=torch.bfloat16,
                out: Optional[torch.Tensor] = None, accumulate: bool = False) -> torch.Tensor:
    """dc[M, N] . b[N, K]: the input gradient of ``det_gemm``."""
    _check_bf16(dc, b)
    if dc.shape[1] != b.shape[0]:
        raise ValueError(f"N mismatch: {tuple(dc.shape)} vs {tuple(b.shape)}")
    dc, b = dc.contiguous(), b.contiguous()
    da = _out((dc.shape[0], b.shape[1]), out_dtype, dc.device, out, accumulate)
    bilogp_det_gemm_da(dc, b, da, accumulate)
    return da


def det_gemm_db(a: torch.Tensor, dc: torch.Tensor, *, out_dtype=torch.bfloat16,
                out: Optional[torch.Tensor] = None, accumulate: bool = False) -> torch.Tensor:
    """dc[M, N]^T . a[M, K]: the weight gradient of ``det_gemm`` ([N, K])."""
    _check_bf16(a, dc)
    if a.shape[0] != dc.shape[0]:
        raise ValueError(f"M mismatch: {tuple(a.shape)} vs {tuple(dc.shape)}")
    a, dc = a.contiguous(), dc.contiguous()
    db = _out((dc.shape[1], a.shape[1]), out_dtype, a.device, out, accumulate)
    bilogp_det_gemm_db(a, dc, db, accumulate)
    return db


class DetLinear(torch.autograd.Function):
    """y = a . w^T with deterministic kernels in both directions.  The
    gradients are computed from a bf16 copy of the upstream gradient (the
    kernels take bf16 operands), as the page's review asks for fp32 outputs."""

    @staticmethod
    def forward(ctx, a, w, out_fp32: bool = False):
        ctx.save_for_backward(a, w)
        return det_gemm(a, w, out_dtype=torch.float32 if out_fp32 else torch.bfloat16)

    @staticmethod
    def backward(ctx, grad_out):
        a, w = ctx.saved_tensors
        g = grad_out.to(torch.bfloat16).contiguous()
        grad_a = det_gemm_da(g, w) if ctx.needs_input_grad[0] else None
        grad_w = det_gemm_db(a, g) if ctx.needs_input_grad[1] else None
        return grad_a, grad_w, None
