"""Seeded synthetic inputs for the fused linear log-probability forward.

This module only draws random numbers and arranges them into inputs.  It holds
none of the arithmetic of the method: no logits, no softmax, no split policy.
Both the CPU oracle and the HIP library receive the tensors made here, so
this is the one piece of code the two sides share.

Workloads (shapes and value distributions of the five standard cases; the
``N(0, s)`` notation means a normal draw scaled by the standard deviation s):

========  =====  ====  ======  ==========================================================
name      N      H     V       inputs
========  =====  ====  ======  ==========================================================
tiny      8      64    1000    hidden N(0,1); W N(0,1/8); no bias; targets include 0, V-1
medium    512    1024  32000   hidden N(0,1); W N(0,1/32); bias fp32 N(0,0.1)
headline  4096   4096  128256  hidden [8,512,H] N(0,1); W N(0,0.02); no bias
sweep     4096   4096  151936  W N(0,0.02); bias bf16 N(0,0.05); targets drawn with
                               repeats from a 512-value pool holding 0, V-1, every
                               2560-column boundary and its neighbours, and the start
                               of the last 256-column tile
peaky     16384  8192  152064  hidden N(0,1) rounded to bf16 then x8 (exact); W
                               N(0,0.02); no bias; a seeded half of the rows is flagged
                               to take its argmax logit as target (filled in by the
                               caller), the rest draw uniformly
========  =====  ====  ======  ==========================================================

Recipe: a ``torch.Generator`` seeded with the workload's seed draws, in this
order, hidden, weight (in blocks of 8192 rows), bias, targets and any extra
fields.  Draws are float32 ``randn`` times the standard deviation, rounded to
bf16 with round-to-nearest-even.  ``tiny``, ``medium`` and the ad-hoc shapes
of ``make_custom`` draw on the CPU; the three large workloads draw on the
device they are built for (their CPU copies are what the oracle reads).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_custom", "make_upstream_grads",
           "peaky_argmax_rows"]


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    H: int
    V: int
    seed: int
    w_std: float
    lead_shape: tuple
    bias: Optional[str] = None          # None | "f32" | "bf16"
    bias_std: float = 0.0
    hidden_scale: float = 1.0           # exact power-of-two scale applied after rounding
    big: bool = False                   # drawn on the target device
    extra: Dict = field(default_factory=dict)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 8, 64, 1000, 0, 1.0 / math.sqrt(64), (8,)),
    "medium": Workload("medium", 512, 1024, 32000, 1, 1.0 / math.sqrt(1024), (512,),
                       bias="f32", bias_std=0.1),
    "headline": Workload("headline", 4096, 4096, 128256, 2, 0.02, (8, 512), big=True),
    "sweep": Workload("sweep", 4096, 4096, 151936, 3, 0.02, (4096,), bias="bf16",
                      bias_std=0.05, big=True,
                      extra={"pool": 512, "boundary_stride": 2560, "last_tile_start": 151808}),
    "peaky": Workload("peaky", 16384, 8192, 152064, 4, 0.02, (16384,), hidden_scale=8.0,
                      big=True, extra={"argmax_fraction": 0.5}),
}


def _randn_bf16(shape, std, gen, device, block_rows=8192):
    """float32 randn * std rounded to bf16, drawn in blocks of ``block_rows`` rows."""
    rows = shape[0]
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    for r0 in range(0, rows, block_rows):
        r1 = min(rows, r0 + block_rows)
        blk = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen, device=device,
                          dtype=torch.float32)
        if std != 1.0:
            blk.mul_(std)
        out[r0:r1] = blk.to(torch.bfloat16)
    return out


def _sweep_targets(wl: Workload, gen, device):
    V = wl.V
    stride = wl.extra["boundary_stride"]
    special = {0, V - 1, wl.extra["last_tile_start"] - 1, wl.extra["last_tile_start"],
               wl.extra["last_tile_start"] + 1}
    for c in range(0, V, stride):
        special.update((c - 1, c, c + 1))
    special = sorted(x for x in special if 0 <= x < V)
    pool_size = wl.extra["pool"]
    fill = torch.randint(0, V, (4 * pool_size,), generator=gen, device=device,
                         dtype=torch.int64).tolist()
    pool = list(special)
    seen = set(pool)
    for x in fill:
        if len(pool) >= pool_size:
            break
        if x not in seen:
            pool.append(x)
            seen.add(x)
    pool_t = torch.tensor(pool, dtype=torch.int64, device=device)
    pick = torch.randint(0, len(pool), (wl.N,), generator=gen, device=device,
                         dtype=torch.int64)
    return pool_t[pick]


def make_inputs(name: str, device="cpu", variant: Optional[str] = None) -> dict:
    """Inputs of a standard workload as a dict with ``hidden`` (lead shape + [H],
    bf16), ``weight`` ([V, H] bf16), ``target`` (lead shape, int64), ``bias``
    ([V] or None) and workload metadata.

    ``variant``: ``None``; ``"w0"`` (weight all zero, the workload's bias kept);
    ``"w0_nobias"`` (weight zero, no bias).
    """
    wl = WORKLOADS[name]
    gen_device = torch.device(device) if wl.big else torch.device("cpu")
    gen = torch.Generator(device=gen_device).manual_seed(wl.seed)

    hidden = _randn_bf16((wl.N, wl.H), 1.0, gen, gen_device)
    if wl.hidden_scale != 1.0:
        hidden.mul_(wl.hidden_scale)               # power of two: exact in bf16
    weight = _randn_bf16((wl.V, wl.H), wl.w_std, gen, gen_device)
    bias = None
    if wl.bias is not None:
        b = torch.randn((wl.V,), generator=gen, device=gen_device, dtype=torch.float32)
        b.mul_(wl.bias_std)
        bias = b if wl.bias == "f32" else b.to(torch.bfloat16)

    out = {"workload": wl}
    if name == "sweep":
        target = _sweep_targets(wl, gen, gen_device)
    else:
        target = torch.randint(0, wl.V, (wl.N,), generator=gen, device=gen_device,
                               dtype=torch.int64)
    if name == "tiny":
        target[0] = 0
        target[-1] = wl.V - 1
    if name == "peaky":
        out["argmax_rows"] = torch.rand((wl.N,), generator=gen, device=gen_device) < \
            wl.extra["argmax_fraction"]

    if variant in ("w0", "w0_nobias"):
        weight = torch.zeros_like(weight)
        if variant == "w0_nobias":
            bias = None
    elif variant is not None:
        raise ValueError(f"unknown variant {variant!r}")

    dev = torch.device(device)
    out["hidden"] = hidden.reshape(*wl.lead_shape, wl.H).to(dev)
    out["weight"] = weight.to(dev)
    out["target"] = target.reshape(wl.lead_shape).to(dev)
    out["bias"] = None if bias is None else bias.to(dev)
    if "argmax_rows" in out:
        out["argmax_rows"] = out["argmax_rows"].to(dev)
    return out


def make_custom(N: int, H: int, V: int, seed: int, w_std: Optional[float] = None,
                bias: Optional[str] = None, bias_std: float = 0.1, hidden_scale: float = 1.0,
                device="cpu") -> dict:
    """Ad-hoc shape with the same recipe (drawn on the CPU, then moved)."""
    gen = torch.Generator().manual_seed(seed)
    w_std = 1.0 / math.sqrt(H) if w_std is None else w_std
    hidden = _randn_bf16((N, H), 1.0, gen, "cpu") if N > 0 else \
        torch.empty((0, H), dtype=torch.bfloat16)
    if hidden_scale != 1.0:
        hidden.mul_(hidden_scale)
    weight = _randn_bf16((V, H), w_std, gen, "cpu")
    b = None
    if bias is not None:
        bb = torch.randn((V,), generator=gen, dtype=torch.float32).mul_(bias_std)
        b = bb if bias == "f32" else bb.to(torch.bfloat16)
    target = torch.randint(0, V, (N,), generator=gen, dtype=torch.int64)
    dev = torch.device(device)
    return {"hidden": hidden.to(dev), "weight": weight.to(dev), "target": target.to(dev),
            "bias": None if b is None else b.to(dev)}


def make_upstream_grads(N: int, seed: int, g_lse_std: float = 0.1, device="cpu") -> dict:
    """Upstream gradients of the forward's two outputs for the backward:
    ``grad_logp`` ~ N(0, 1) (a per-token policy-gradient weight) and
    ``grad_lse`` ~ N(0, g_lse_std^2) (a small log-partition penalty), fp32 [N],
    drawn on the CPU, then moved."""
    gen = torch.Generator().manual_seed(seed)
    g_logp = torch.randn((N,), generator=gen, dtype=torch.float32)
    g_lse = torch.randn((N,), generator=gen, dtype=torch.float32).mul_(g_lse_std)
    dev = torch.device(device)
    return {"grad_logp": g_logp.to(dev), "grad_lse": g_lse.to(dev)}


def peaky_argmax_rows(inputs: dict) -> torch.Tensor:
    """Indices of the rows flagged to take their argmax logit as target."""
    return torch.nonzero(inputs["argmax_rows"].reshape(-1)).reshape(-1)
