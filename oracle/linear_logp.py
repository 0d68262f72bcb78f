"""fp64 CPU oracle: fused linear log-probability (logp of the target token and
the log-sum-exp of the logits), per row.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Source: RL-Kernel PR #337, "feat(linear-logp): add batch-invariant fused SM90
operator".
  * Walkthrough and sequence diagram: the operator takes hidden states, an
    lm-head weight, target ids and an optional bias, and returns the
    log-probability of each row's target together with the log-sum-exp of the
    row's logits; the pull request's own accuracy reference is an FP32
    computation of the same quantity.
  * Description, "Why this happens": the logits are hidden . weight^T over the
    whole vocabulary; the fused kernel never materialises the [N, V] matrix
    and instead merges partial online-softmax states (a running maximum and a
    rescaled sum of exponentials) of contiguous vocabulary chunks.  Different
    groupings of the chunks are equal in real arithmetic.
  * Description, "What this PR changes": the split count is chosen from V
    only, the same contiguous vocabulary splits are used for every N, and the
    partial states are combined in ascending order.
  * Author's annotation on ``select_batch_invariant_vocab_splits``: at most a
    fixed maximum number of non-empty, contiguous ranges of vocabulary tiles.

Readings where the page is silent (each is repeated in the design notes):
  * logits are not rounded to a narrow type before the log-sum-exp; the oracle
    keeps them in float64;
  * the optional bias has shape [V] and is added once to each logit (in
    float64 the order of that one addition is immaterial);
  * "log" is the natural logarithm;
  * a target must lie in [0, V); there is no ignore index.

Every function here reads bf16 / fp32 inputs exactly (a bf16 value is the
upper half of an IEEE binary32 bit pattern) and computes in binary64.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "decode_bf16",
    "to_f64",
    "linear_logp",
    "vocab_splits",
    "vocab_splits_throughput",
    "split_merge_linear_logp",
    "brute_force_linear_logp",
]


# --------------------------------------------------------------------------
# exact input decoding
# --------------------------------------------------------------------------
def decode_bf16(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bf16 tensor, decoded from its bit pattern.

    bfloat16 is the top 16 bits of an IEEE-754 binary32 word, so shifting the
    16-bit pattern left by 16 gives the binary32 word of the same value; the
    binary32 -> binary64 widening is exact.
    """
    if t.dtype != torch.bfloat16:
        raise TypeError(f"decode_bf16 expects a bfloat16 tensor, got {t.dtype}")
    raw = t.detach().to("cpu").contiguous().view(torch.int16).numpy()
    word = raw.view(np.uint16).astype(np.uint32) << np.uint32(16)
    return word.view(np.float32).astype(np.float64)


def to_f64(x) -> Optional[np.ndarray]:
    """float64 view of an input given as a torch tensor (bf16 / fp32 / fp64) or
    a numpy array.  ``None`` passes through.  Never rounds."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        if x.dtype == np.float64:
            return x
        if x.dtype in (np.float32, np.float16):
            return x.astype(np.float64)
        raise TypeError(f"unsupported numpy dtype {x.dtype}")
    if isinstance(x, torch.Tensor):
        if x.dtype == torch.bfloat16:
            return decode_bf16(x)
        if x.dtype in (torch.float32, torch.float64, torch.float16):
            return x.detach().to("cpu").numpy().astype(np.float64)
        raise TypeError(f"unsupported tensor dtype {x.dtype}")
    raise TypeError(f"unsupported input type {type(x)}")


def _to_i64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu").numpy()
    return np.asarray(x, dtype=np.int64).reshape(-1)


def _check(h: np.ndarray, w: np.ndarray, t: np.ndarray, b: Optional[np.ndarray]) -> None:
    if h.ndim != 2 or w.ndim != 2 or h.shape[1] != w.shape[1]:
        raise ValueError(f"shape mismatch: hidden {h.shape}, weight {w.shape}")
    if t.shape[0] != h.shape[0]:
        raise ValueError(f"target has {t.shape[0]} rows, hidden has {h.shape[0]}")
    if b is not None and b.shape != (w.shape[0],):
        raise ValueError(f"bias shape {b.shape} != ({w.shape[0]},)")
    V = w.shape[0]
    if t.size and (t.min() < 0 or t.max() >= V):
        raise ValueError("target outside [0, V)")


# --------------------------------------------------------------------------
# the plain definition
# --------------------------------------------------------------------------
def linear_logp(hidden, weight, target, bias=None, rows: Optional[Sequence[int]] = None,
                row_chunk: int = 128) -> Tuple[np.ndarray, np.ndarray]:
    """(logp, lse) in float64 by the plain definition, row by row:

        z[i, v]  = sum_k hidden[i, k] * W[v, k]  (+ bias[v])
        lse[i]   = max_v z[i, v] + ln( sum_v exp(z[i, v] - max_v z[i, v]) )
        logp[i]  = z[i, target[i]] - lse[i]

    This is the value the fused kernel reaches in real arithmetic (PR #337,
    description, "Why this happens").  The contraction is one BLAS dgemm per
    row chunk; the maximum, exponentials, sum and log are explicit float64
    numpy operations over the full vocabulary.  ``rows`` restricts the
    computation to the listed rows (results in that order).
    """
    h = to_f64(hidden)
    w = to_f64(weight)
    b = to_f64(bias)
    t = _to_i64(target)
    _check(h, w, t, b)
    idx = np.arange(h.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    logp = np.empty(idx.shape[0], dtype=np.float64)
    lse = np.empty(idx.shape[0], dtype=np.float64)
    wt = w.T
    for c0 in range(0, idx.shape[0], row_chunk):
        r = idx[c0:c0 + row_chunk]
        z = h[r] @ wt                                   # [R, V] logits
        if b is not None:
            z += b
        zmax = z.max(axis=1)
        sumexp = np.exp(z - zmax[:, None]).sum(axis=1)
        lse_c = zmax + np.log(sumexp)
        zt = z[np.arange(r.shape[0]), t[r]]
        logp[c0:c0 + r.shape[0]] = zt - lse_c
        lse[c0:c0 + r.shape[0]] = lse_c
    return logp, lse


# --------------------------------------------------------------------------
# the method's own steps (split policy, online partials, ascending combine)
# --------------------------------------------------------------------------
def vocab_splits(V: int, vtile: int, max_splits: int) -> list:
    """Contiguous vocabulary-tile ranges chosen from V alone.

    PR #337, annotation on ``select_batch_invariant_vocab_splits``: keep at
    most ``max_splits`` non-empty contiguous ranges, and let only V decide the
    partition.  The page's formula is cut off after its left-hand side, so this
    takes the plainest reading that yields such ranges: with
    T = ceil(V / vtile) tiles, every split takes ceil(T / max_splits) tiles
    (the last one takes the remainder), giving ceil(T / per_split) splits.
    Returns a list of half-open tile ranges (first_tile, end_tile).
    """
    if V <= 0 or vtile <= 0 or max_splits <= 0:
        raise ValueError("V, vtile and max_splits must be positive")
    tiles = -(-V // vtile)
    per_split = -(-tiles // max_splits)
    n_splits = -(-tiles // per_split)
    return [(k * per_split, min((k + 1) * per_split, tiles)) for k in range(n_splits)]


def vocab_splits_throughput(N: int, V: int, cu_count: int, vtile: int = 256,
                            block_rows: int = 256, max_splits: int = 1024) -> list:
    """Contiguous vocabulary-tile ranges chosen from N, V and the number of
    compute units: the throughput-oriented scheduling that the invariant
    policy replaces.

    PR #337, description ("Why this happens" and its flowchart): the existing
    fused operator's throughput scheduler picks the vocabulary split from N, V
    and the GPU's SM count, so one token row can be reduced as [A][B][C][D]
    inside one batch and as [A B][C D] inside another.  The page does not give
    that scheduler's formula; this is the plainest policy of that kind: enough
    splits that ceil(N / block_rows) row blocks times the split count reach
    the compute-unit count, at most ``max_splits`` and at most one per tile,
    every split (but the last) taking the same number of tiles.  Returns
    half-open tile ranges (first_tile, end_tile).
    """
    if N <= 0 or V <= 0 or cu_count <= 0 or vtile <= 0 or block_rows <= 0 or max_splits <= 0:
        raise ValueError("N, V, cu_count, vtile, block_rows and max_splits must be positive")
    tiles = -(-V // vtile)
    row_blocks = -(-N // block_rows)
    want = min(max(-(-cu_count // row_blocks), 1), tiles, max_splits)
    per_split = -(-tiles // want)
    n_splits = -(-tiles // per_split)
    return [(k * per_split, min((k + 1) * per_split, tiles)) for k in range(n_splits)]


def split_merge_linear_logp(hidden, weight, target, bias=None, vtile: int = 256,
                            max_splits: int = 256,
                            rows: Optional[Sequence[int]] = None,
                            splits: Optional[Sequence[Tuple[int, int]]] = None
                            ) -> Tuple[np.ndarray, np.ndarray]:
    """(logp, lse) in float64 following the method's steps in the page's order
    (PR #337, description, "What this PR changes"):

      1. split policy from V only (``vocab_splits``);
      2. for every split, walk its vocabulary tiles in ascending order and keep
         an online-softmax state per row: running maximum m and the sum s of
         exp(z - m), rescaled by exp(m_old - m_new) whenever the maximum grows;
         the target's logit is taken from the one tile that holds it;
      3. combine the per-split partials (m_k, s_k) in ascending split order:
         M = max_k m_k, Sigma = sum over k = 0, 1, ... of s_k exp(m_k - M),
         lse = M + ln Sigma, logp = z_target - lse.

    In real arithmetic this equals ``linear_logp``; in float64 the two agree to
    rounding, which pins the combine algebra independently of any GPU code.
    ``splits`` replaces step 1 by an explicit list of contiguous tile ranges
    (for instance ``vocab_splits_throughput``); the combine is unchanged.
    """
    h = to_f64(hidden)
    w = to_f64(weight)
    b = to_f64(bias)
    t = _to_i64(target)
    _check(h, w, t, b)
    idx = np.arange(h.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    hr = h[idx]
    tr = t[idx]
    R = idx.shape[0]
    V = w.shape[0]
    if splits is None:
        splits = vocab_splits(V, vtile, max_splits)
    tiles = -(-V // vtile)
    ok = (len(splits) > 0 and splits[0][0] == 0 and splits[-1][1] == tiles
          and all(a < b for a, b in splits)
          and all(splits[i][1] == splits[i + 1][0] for i in range(len(splits) - 1)))
    if not ok:
        raise ValueError("splits must be non-empty contiguous tile ranges covering [0, T)")

    part_m = np.empty((len(splits), R))
    part_s = np.empty((len(splits), R))
    z_target = np.full(R, np.nan)
    for k, (first, end) in enumerate(splits):
        m = np.full(R, -np.inf)
        s = np.zeros(R)
        for tile in range(first, end):
            c0 = tile * vtile
            c1 = min(c0 + vtile, V)
            z = hr @ w[c0:c1].T
            if b is not None:
                z += b[c0:c1]
            hit = (tr >= c0) & (tr < c1)
            z_target[hit] = z[np.nonzero(hit)[0], tr[hit] - c0]
            m_new = np.maximum(m, z.max(axis=1))
            s = s * np.exp(m - m_new) + np.exp(z - m_new[:, None]).sum(axis=1)
            m = m_new
        part_m[k] = m
        part_s[k] = s

    M = part_m.max(axis=0)
    sigma = np.zeros(R)
    for k in range(len(splits)):                    # ascending split order
        sigma = sigma + part_s[k] * np.exp(part_m[k] - M)
    lse = M + np.log(sigma)
    return z_target - lse, lse


# --------------------------------------------------------------------------
# pure-Python brute force for tiny inputs
# --------------------------------------------------------------------------
def brute_force_linear_logp(hidden, weight, target, bias=None) -> Tuple[list, list]:
    """(logp, lse) with plain Python floats and ``math.fsum``; tiny inputs only.

    Each logit is the correctly rounded sum of the exact products (a product
    of two bf16 values is exact in binary64) plus the bias; the sum of
    exponentials is an ``fsum`` as well.  No numpy arithmetic is used, so this
    checks the dgemm / reduction path of ``linear_logp`` independently.
    """
    h = to_f64(hidden).tolist()
    w = to_f64(weight).tolist()
    b = None if bias is None else to_f64(bias).tolist()
    t = _to_i64(target).tolist()
    V = len(w)
    logps, lses = [], []
    for i, row in enumerate(h):
        z = []
        for v in range(V):
            terms = [a * c for a, c in zip(row, w[v])]
            if b is not None:
                terms.append(b[v])
            z.append(math.fsum(terms))
        zmax = max(z)
        lse = zmax + math.log(math.fsum(math.exp(x - zmax) for x in z))
        ti = t[i]
        if not 0 <= ti < V:
            raise ValueError("target outside [0, V)")
        logps.append(z[ti] - lse)
        lses.append(lse)
    return logps, lses
