"""Helpers for the GPU tests: run the HIP library through its C ABI and
compare with the fp64 oracle.  Tolerance: |delta| <= 2e-3 absolute on logp
and lse (the accuracy bar of the method's statement); bit equality
(torch.equal) for every invariance property."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import invariant_linear_log_amd as ila
import oracle
import synth

TOL = 2e-3
DEV = "cuda:0"


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a fault can be placed."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def flat(inp):
    h = inp["hidden"]
    return h.reshape(-1, h.shape[-1]).contiguous(), inp["target"].reshape(-1).contiguous()


def run_ex(hidden2d, weight, target1d, bias=None, stream=None):
    """(logp, lse) from bilogp_forward_ex with a caller workspace."""
    N = hidden2d.shape[0]
    V = weight.shape[0]
    logp = torch.empty(N, dtype=torch.float32, device=hidden2d.device)
    lse = torch.empty(N, dtype=torch.float32, device=hidden2d.device)
    ws = ila.workspace_for(N, V, hidden2d.device)
    ila.bilogp_forward_ex(hidden2d, weight, target1d, bias, logp, lse, ws, stream=stream)
    return logp, lse


def run_inputs(inp, stream=None):
    h, t = flat(inp)
    return run_ex(h, inp["weight"], t, inp["bias"], stream=stream)


def oracle_rows(inp, rows=None):
    h, t = flat(inp)
    b = inp["bias"]
    return oracle.linear_logp(h.cpu(), inp["weight"].cpu(), t.cpu(),
                              None if b is None else b.cpu(), rows=rows)


def assert_parity(logp, lse, ref_logp, ref_lse, rows=None, tol=TOL, what=""):
    lp = logp.double().cpu().numpy()
    ls = lse.double().cpu().numpy()
    if rows is not None:
        lp, ls = lp[rows], ls[rows]
    assert np.all(np.isfinite(lp)) and np.all(np.isfinite(ls)), f"{what}: non-finite output"
    d_lp = float(np.max(np.abs(lp - ref_logp))) if lp.size else 0.0
    d_ls = float(np.max(np.abs(ls - ref_lse))) if ls.size else 0.0
    say(f"{what}: max|dlogp|={d_lp:.3e} max|dlse|={d_ls:.3e} over {lp.size} rows")
    assert d_lp <= tol and d_ls <= tol, f"{what}: |dlogp|={d_lp}, |dlse|={d_ls} > {tol}"


def sample_rows(N: int, k: int, seed: int):
    g = np.random.default_rng(seed)
    rows = set(g.choice(N, size=min(k, N) - 2, replace=False).tolist()) | {0, N - 1}
    return np.array(sorted(rows), dtype=np.int64)


def peaky_with_argmax_targets(device=DEV):
    """The peaky workload with the flagged rows' targets set to the argmax of
    their fp32 logits (torch matmul on the GPU, row chunks; lowest index on
    ties).  Returns (inputs, argmax_row_indices)."""
    inp = synth.make_inputs("peaky", device=device)
    h, t = flat(inp)
    w = inp["weight"]
    rows = synth.peaky_argmax_rows(inp)
    wf = w.float()
    for c0 in range(0, rows.numel(), 1024):
        r = rows[c0:c0 + 1024]
        z = h[r].float() @ wf.T
        t[r] = torch.argmax(z, dim=1)
    del wf
    inp["target"] = t.reshape(inp["target"].shape)
    return inp, rows


def ln(x):
    return math.log(x)
