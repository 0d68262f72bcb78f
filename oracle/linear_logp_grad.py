"""fp64 CPU oracle of the backward of the fused linear log-probability:
the gradients of logp and lse with respect to hidden, the weight and the
bias.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources.  RL-Kernel PR #337, "feat(linear-logp): add batch-invariant fused
SM90 operator": the forward's definition (walkthrough; description, "Why this
happens": logits hidden . weight^T, the log-sum-exp over the vocabulary and
the target's log-probability) and the author's annotation on the
``requires_grad`` check (the page's first contract stops at the forward, so
the gradients below are the plain derivatives of that forward).  RL-Kernel
PR #395, "feat(musa): add native deterministic gemm kernel", summary: the
input gradient dA = dC . B and the weight gradient in the forward's [N, K]
layout, which fix the layouts of grad_hidden and grad_weight.

Derivation (chain rule on the forward): with P[i, v] = exp(z[i, v] - lse[i]),
d lse[i] / d z[i, v] = P[i, v] and d logp[i] / d z[i, v] = [v == target[i]]
- P[i, v].  For upstream gradients g_logp[i] and g_lse[i]:

    dZ[i, v]     = g_lse[i] P[i, v] + g_logp[i] ([v == target[i]] - P[i, v])
    grad_hidden  = dZ . W          (z = hidden . W^T + bias)
    grad_weight  = dZ^T . hidden   ([V, H], the weight's own layout)
    grad_bias[v] = sum_i dZ[i, v]

Readings where the pages are silent (repeated in the design notes):
  * the backward is handed the forward's lse and uses it as given (it is not
    recomputed), together with the upstream gradients of both outputs;
  * a target outside [0, V) adds no one-hot term (its row's forward logp is
    NaN; a caller masks such rows with g_logp = 0);
  * nothing is rounded: the oracle is the exact derivative in float64, from
    the exact values of the bf16 / fp32 inputs.
"""

from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .linear_logp import _to_i64, to_f64

__all__ = ["softmax_grad", "linear_logp_backward", "grad_hidden_rows", "grad_weight_rows"]


def _inputs(hidden, weight, target, bias, lse, grad_logp, grad_lse):
    h, w, b = to_f64(hidden), to_f64(weight), to_f64(bias)
    t = _to_i64(target)
    lse_, gl, gs = to_f64(lse).reshape(-1), to_f64(grad_logp).reshape(-1), \
        to_f64(grad_lse).reshape(-1)
    if h.ndim != 2 or w.ndim != 2 or h.shape[1] != w.shape[1]:
        raise ValueError(f"shape mismatch: hidden {h.shape}, weight {w.shape}")
    N, V = h.shape[0], w.shape[0]
    for name, x in (("target", t), ("lse", lse_), ("grad_logp", gl), ("grad_lse", gs)):
        if x.shape[0] != N:
            raise ValueError(f"{name} has {x.shape[0]} rows, hidden has {N}")
    if b is not None and b.shape != (V,):
        raise ValueError(f"bias shape {b.shape} != ({V},)")
    return h, w, t, b, lse_, gl, gs


def _dz(h, w, t, b, lse_, gl, gs, rows, cols) -> np.ndarray:
    """dZ[rows][:, cols] from the definition (rows / cols: index arrays)."""
    z = h[rows] @ w[cols].T
    if b is not None:
        z += b[cols]
    p = np.exp(z - lse_[rows][:, None])
    dz = gs[rows][:, None] * p - gl[rows][:, None] * p
    onehot = t[rows][:, None] == cols[None, :]
    dz += np.where(onehot, gl[rows][:, None], 0.0)
    return dz


def softmax_grad(hidden, weight, target, bias, lse, grad_logp, grad_lse,
                 rows: Optional[Sequence[int]] = None,
                 cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """dZ in float64, restricted to ``rows`` x ``cols`` if given (in that
    order)."""
    h, w, t, b, lse_, gl, gs = _inputs(hidden, weight, target, bias, lse, grad_logp, grad_lse)
    r = np.arange(h.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    c = np.arange(w.shape[0]) if cols is None else np.asarray(cols, dtype=np.int64)
    return _dz(h, w, t, b, lse_, gl, gs, r, c)


def linear_logp_backward(hidden, weight, target, bias, lse, grad_logp, grad_lse,
                         row_chunk: int = 128) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(grad_hidden [N, H], grad_weight [V, H], grad_bias [V]) in float64.
    dZ is formed one row chunk at a time; each product is one BLAS dgemm."""
    h, w, t, b, lse_, gl, gs = _inputs(hidden, weight, target, bias, lse, grad_logp, grad_lse)
    N, V = h.shape[0], w.shape[0]
    cols = np.arange(V)
    gh = np.zeros_like(h)
    gw = np.zeros_like(w)
    gb = np.zeros(V, dtype=np.float64)
    for c0 in range(0, N, row_chunk):
        r = np.arange(c0, min(c0 + row_chunk, N))
        dz = _dz(h, w, t, b, lse_, gl, gs, r, cols)
        gh[r] = dz @ w
        gw += dz.T @ h[r]
        gb += dz.sum(axis=0)
    return gh, gw, gb


def grad_hidden_rows(hidden, weight, target, bias, lse, grad_logp, grad_lse,
                     rows: Sequence[int]) -> np.ndarray:
    """grad_hidden[rows] (one dZ row each, over the whole vocabulary)."""
    h, w, t, b, lse_, gl, gs = _inputs(hidden, weight, target, bias, lse, grad_logp, grad_lse)
    r = np.asarray(rows, dtype=np.int64)
    return _dz(h, w, t, b, lse_, gl, gs, r, np.arange(w.shape[0])) @ w


def grad_weight_rows(hidden, weight, target, bias, lse, grad_logp, grad_lse,
                     cols: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """(grad_weight[cols], grad_bias[cols]): one dZ column each, over the
    whole batch."""
    h, w, t, b, lse_, gl, gs = _inputs(hidden, weight, target, bias, lse, grad_logp, grad_lse)
    c = np.asarray(cols, dtype=np.int64)
    dz = _dz(h, w, t, b, lse_, gl, gs, np.arange(h.shape[0]), c)     # [N, len(cols)]
    return dz.T @ h, dz.sum(axis=0)
