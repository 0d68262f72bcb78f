"""Batch-invariant fused linear log-probability forward for AMD MI355X (gfx950).

    logp, lse = invariant_linear_log_amd.forward(hidden, weight, target, bias=None)

computes, per row of ``hidden[..., H]`` (bf16), the logits ``hidden . W^T
(+ bias)`` over the vocabulary ``W[V, H]`` (bf16) without storing them, and
returns the log-probability of ``target`` and the log-sum-exp of the logits
(fp32, shaped like ``target``).  Output bits never depend on the number of
rows, their order or neighbours, the stream, or the GPU's compute-unit
count.  Forward only: inputs that require grad while autograd is enabled are
rejected (RL-Kernel PR #337, author's annotation on the ``requires_grad``
check: the backward is outside the first contract, so the path fails closed).

``det_gemm``, ``det_gemm_da``, ``det_gemm_db`` and ``DetLinear`` are the
deterministic GEMM (forward, input gradient, [N, K] weight gradient).
``backward`` and the autograd-capable ``linear_logp`` add a deterministic
backward to the forward (gradients of logp and lse with respect to hidden,
weight and bias).

The C entry points of ``include/bilogp.h`` are available under the same
names (``bilogp_forward``, ``bilogp_forward_ex``, ``bilogp_workspace_bytes``,
...), marshalling torch tensors to device pointers and the current stream.
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from ._binding import (  # noqa: F401
    BILOGP_BIAS_BF16,
    BILOGP_BIAS_F32,
    BILOGP_BIAS_NONE,
    BILOGP_E_HIP,
    BILOGP_E_INVALID_ARG,
    BILOGP_E_UNSUPPORTED,
    BILOGP_E_WORKSPACE,
    BILOGP_MAX_THROUGHPUT_SPLITS,
    BILOGP_OK,
    BILOGP_SPLITS_INVARIANT,
    BILOGP_SPLITS_THROUGHPUT,
    BilogpError,
    LIB_PATH,
    BILOGP_GEMM_OUT_BF16,
    BILOGP_GEMM_OUT_F32,
    BILOGP_GEMM_OUT_F32_ACCUM,
    bilogp_abi_version,
    bilogp_bit_contract_version,
    bilogp_backward,
    bilogp_backward_workspace_bytes,
    bilogp_det_gemm_da,
    bilogp_det_gemm_db,
    bilogp_det_gemm_fwd,
    bilogp_forward,
    bilogp_forward_ex,
    bilogp_forward_mode,
    bilogp_forward_noalloc,
    bilogp_last_error,
    bilogp_launch_plan,
    bilogp_launch_schedule,
    bilogp_max_splits,
    bilogp_merge,
    bilogp_noalloc_max_workspace_bytes,
    bilogp_num_vocab_splits,
    bilogp_num_vocab_splits_mode,
    bilogp_partials,
    bilogp_partials_range,
    bilogp_status_string,
    bilogp_vtile_cols,
    bilogp_vtiles_per_split,
    bilogp_vtiles_per_split_mode,
    bilogp_workspace_bytes,
    bilogp_workspace_bytes_mode,
    load_library,
    vocab_split_columns,
)

from .det_gemm import DetLinear, det_gemm, det_gemm_da, det_gemm_db  # noqa: F401,E402
from .grad import LinearLogp, backward, backward_workspace_for, linear_logp  # noqa: F401,E402

__all__ = ["forward", "workspace_for", "device_cu_count", "BilogpError", "load_library",
           "det_gemm", "det_gemm_da", "det_gemm_db", "DetLinear", "backward",
           "backward_workspace_for", "linear_logp", "LinearLogp"]


_SPLIT_MODES = {"invariant": BILOGP_SPLITS_INVARIANT, "throughput": BILOGP_SPLITS_THROUGHPUT}


def device_cu_count(device) -> int:
    """Compute units of a GPU (what the throughput split policy fills)."""
    return torch.cuda.get_device_properties(torch.device(device)).multi_processor_count


def workspace_for(N: int, V: int, device, split_mode: str = "invariant",
                  cu_count: Optional[int] = None) -> Optional[torch.Tensor]:
    """A uint8 device tensor big enough for ``bilogp_forward_ex`` (or, with
    ``split_mode="throughput"``, ``bilogp_forward_mode``); None if N == 0."""
    mode = _SPLIT_MODES[split_mode]
    if mode == BILOGP_SPLITS_THROUGHPUT and cu_count is None:
        cu_count = device_cu_count(device)
    nbytes = bilogp_workspace_bytes_mode(N, V, mode, cu_count or 0)
    if nbytes == (1 << 64) - 1:
        raise ValueError(f"invalid sizes N={N}, V={V}")
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def forward(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
            bias: Optional[torch.Tensor] = None, *, check_targets: bool = True,
            workspace: Optional[torch.Tensor] = None, split_mode: str = "invariant",
            cu_count: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(logp, lse), each fp32 with ``target``'s shape.

    hidden  [..., H] bf16        weight [V, H] bf16
    target  [...] int64 (the leading shape of hidden); a zero-stride
            (expanded) target is accepted and made contiguous
    bias    [V] bf16 or fp32, optional

    ``check_targets`` verifies 0 <= target < V on the host first (one device
    sync); without it an out-of-range target gives NaN for that row.

    ``split_mode="throughput"`` chooses the vocabulary splits from N, V and
    ``cu_count`` (default: the device's compute units) instead of V alone:
    the same accuracy, but a row's bits then depend on the batch it is in.
    It exists to measure what the invariant policy costs.
    """
    if split_mode not in _SPLIT_MODES:
        raise ValueError(f"split_mode must be one of {sorted(_SPLIT_MODES)}")
    if torch.is_grad_enabled() and (hidden.requires_grad or weight.requires_grad or
                                    (bias is not None and bias.requires_grad)):
        raise RuntimeError("batch-invariant linear logp is forward-only: call it under "
                           "torch.no_grad() or with inputs that do not require grad")
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    if target.dtype != torch.int64:
        raise TypeError("target must be int64")
    if weight.dim() != 2 or hidden.dim() < 1 or hidden.shape[-1] != weight.shape[1]:
        raise ValueError(f"shape mismatch: hidden {tuple(hidden.shape)}, "
                         f"weight {tuple(weight.shape)}")
    lead_shape = hidden.shape[:-1]
    if tuple(target.shape) != tuple(lead_shape):
        raise ValueError(f"target shape {tuple(target.shape)} != {tuple(lead_shape)}")
    V, H = weight.shape
    if bias is not None:
        if bias.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("bias must be bfloat16 or float32")
        if tuple(bias.shape) != (V,):
            raise ValueError(f"bias shape {tuple(bias.shape)} != ({V},)")
    tensors = [hidden, weight, target] + ([bias] if bias is not None else [])
    dev = hidden.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors):
        raise ValueError("all tensors must be on the same GPU")

    with torch.no_grad():
        hidden_2d = hidden.reshape(-1, H).contiguous()
        weight_2d = weight.contiguous()
        target_1d = target.reshape(-1).contiguous()
        bias_1d = None if bias is None else bias.contiguous()
        N = hidden_2d.shape[0]
        if check_targets and N > 0:
            # one device-to-host read for both bounds
            lo, hi = torch.stack(torch.aminmax(target_1d)).tolist()
            if lo < 0 or hi >= V:
                raise ValueError(f"target outside [0, {V}): min {lo}, max {hi}")
        logp = torch.empty(N, dtype=torch.float32, device=dev)
        lse = torch.empty(N, dtype=torch.float32, device=dev)
        if N > 0:
            mode = _SPLIT_MODES[split_mode]
            if mode == BILOGP_SPLITS_INVARIANT:
                ws = workspace if workspace is not None else workspace_for(N, V, dev)
                bilogp_forward_ex(hidden_2d, weight_2d, target_1d, bias_1d, logp, lse, ws)
            else:
                cus = device_cu_count(dev) if cu_count is None else int(cu_count)
                ws = workspace if workspace is not None else \
                    workspace_for(N, V, dev, split_mode, cus)
                bilogp_forward_mode(hidden_2d, weight_2d, target_1d, bias_1d, logp, lse, mode,
                                    cus, ws)
    return logp.reshape(lead_shape), lse.reshape(lead_shape)
