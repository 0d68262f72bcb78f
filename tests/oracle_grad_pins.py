"""Pins of the backward oracle (oracle/linear_logp_grad.py), each against
something other than the backward oracle itself:

  * central finite differences of L = sum_i g_logp[i] logp[i] + g_lse[i]
    lse[i], with logp and lse from the (separately pinned) forward oracle;
  * torch's float64 autograd through ``log_softmax`` / ``logsumexp`` (a
    library's own derivative of the same forward);
  * the cross-entropy case (g_logp = -1, g_lse = 0): every dZ row sums to 0,
    the target entry is P - 1 < 0 and the rest are P > 0;
  * the uniform case W = 0 without bias: P = 1 / V exactly, so dZ, the bias
    gradient and the weight gradient have closed forms;
  * a constant added to every bias entry (with the lse it implies) changes no
    gradient, while a shift of the given lse alone scales P by exp(-shift);
  * the row / column subset functions agree with the full backward.

Each function takes the backward module under test (the real one, or a
mutant built by the mutation test) as ``grad``; the forward comes from the
real oracle package.
"""

import math

import numpy as np
import torch

import oracle
import synth


class PinFailure(AssertionError):
    pass


def _assert(cond, msg):
    if not cond:
        raise PinFailure(msg)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(1e-300, float(np.max(np.abs(b)))))


def _f64_case(N, H, V, seed, bias=True):
    """Plain float64 inputs (not bf16-valued): finite differences need a
    smooth function of every input."""
    g = np.random.default_rng(seed)
    h = g.standard_normal((N, H))
    w = g.standard_normal((V, H)) / math.sqrt(H)
    b = g.standard_normal(V) * 0.3 if bias else None
    t = g.integers(0, V, N)
    gl = g.standard_normal(N)
    gs = g.standard_normal(N) * 0.5
    return h, w, t, b, gl, gs


def _loss(h, w, t, b, gl, gs):
    logp, lse = oracle.linear_logp(h, w, t, b)
    return float(np.dot(gl, logp) + np.dot(gs, lse))


def pin_finite_differences(grad):
    """Central differences of the forward oracle's loss, every input entry."""
    for seed, bias in ((1, True), (2, False)):
        h, w, t, b, gl, gs = _f64_case(3, 5, 7, seed, bias)
        _, lse = oracle.linear_logp(h, w, t, b)
        gh, gw, gb = grad.linear_logp_backward(h, w, t, b, lse, gl, gs)
        eps = 1e-5

        def fd(arr, idx):
            old = arr[idx]
            arr[idx] = old + eps
            lp = _loss(h, w, t, b, gl, gs)
            arr[idx] = old - eps
            lm = _loss(h, w, t, b, gl, gs)
            arr[idx] = old
            return (lp - lm) / (2 * eps)

        num_h = np.array([[fd(h, (i, k)) for k in range(h.shape[1])] for i in range(h.shape[0])])
        num_w = np.array([[fd(w, (v, k)) for k in range(w.shape[1])] for v in range(w.shape[0])])
        _assert(np.max(np.abs(gh - num_h)) < 1e-7, f"grad_hidden vs finite differences (seed {seed})")
        _assert(np.max(np.abs(gw - num_w)) < 1e-7, f"grad_weight vs finite differences (seed {seed})")
        if b is not None:
            num_b = np.array([fd(b, (v,)) for v in range(b.shape[0])])
            _assert(np.max(np.abs(gb - num_b)) < 1e-7, f"grad_bias vs finite differences (seed {seed})")


def pin_torch_autograd(grad):
    """torch float64 autograd of the same loss on bf16-valued inputs, with and
    without bias, with one target at each vocabulary end."""
    for seed, bias in ((3, "f32"), (4, None), (5, "bf16")):
        inp = synth.make_custom(40, 24, 300, seed, bias=bias)
        inp["target"][0] = 0
        inp["target"][1] = 299
        up = synth.make_upstream_grads(40, seed)
        h = oracle.to_f64(inp["hidden"])
        w = oracle.to_f64(inp["weight"])
        b = oracle.to_f64(inp["bias"])
        t = inp["target"].numpy()
        th = torch.tensor(h, requires_grad=True)
        tw = torch.tensor(w, requires_grad=True)
        tb = torch.tensor(b, requires_grad=True) if b is not None else None
        z = th @ tw.T + (tb if tb is not None else 0.0)
        lse = torch.logsumexp(z, dim=1)
        logp = torch.log_softmax(z, dim=1).gather(1, torch.tensor(t)[:, None])[:, 0]
        gl = oracle.to_f64(up["grad_logp"])
        gs = oracle.to_f64(up["grad_lse"])
        loss = (torch.tensor(gl) * logp + torch.tensor(gs) * lse).sum()
        loss.backward()
        gh, gw, gb = grad.linear_logp_backward(inp["hidden"], inp["weight"], inp["target"],
                                               inp["bias"], lse.detach().numpy(), gl, gs)
        _assert(_rel(gh, th.grad.numpy()) < 1e-12, f"grad_hidden vs autograd (seed {seed})")
        _assert(_rel(gw, tw.grad.numpy()) < 1e-12, f"grad_weight vs autograd (seed {seed})")
        if tb is not None:
            _assert(_rel(gb, tb.grad.numpy()) < 1e-12, f"grad_bias vs autograd (seed {seed})")


def pin_cross_entropy(grad):
    """g_logp = -1, g_lse = 0: dZ = P - onehot, so rows sum to 0, the target
    entry is negative, the others positive, and the bias gradient sums to 0."""
    inp = synth.make_custom(16, 32, 257, 6, bias="f32")
    N, V = 16, 257
    _, lse = oracle.linear_logp(inp["hidden"], inp["weight"], inp["target"], inp["bias"])
    gl, gs = -np.ones(N), np.zeros(N)
    dz = grad.softmax_grad(inp["hidden"], inp["weight"], inp["target"], inp["bias"], lse, gl, gs)
    _assert(dz.shape == (N, V), f"dZ shape {dz.shape}")
    _assert(np.max(np.abs(dz.sum(axis=1))) < 1e-12, "cross-entropy dZ rows must sum to 0")
    t = inp["target"].numpy()
    mask = np.zeros((N, V), dtype=bool)
    mask[np.arange(N), t] = True
    _assert(np.all(dz[mask] < 0) and np.all(dz[~mask] > 0), "signs of P - onehot")
    _, _, gb = grad.linear_logp_backward(inp["hidden"], inp["weight"], inp["target"],
                                         inp["bias"], lse, gl, gs)
    _assert(abs(gb.sum()) < 1e-10, "cross-entropy bias gradient must sum to 0")


def pin_uniform_closed_form(grad):
    """W = 0 and no bias: z = 0, lse = ln V, P = 1 / V."""
    N, H, V = 6, 8, 50
    inp = synth.make_custom(N, H, V, 7)
    w = torch.zeros((V, H), dtype=torch.bfloat16)
    up = synth.make_upstream_grads(N, 7)
    gl = oracle.to_f64(up["grad_logp"])
    gs = oracle.to_f64(up["grad_lse"])
    h = oracle.to_f64(inp["hidden"])
    t = inp["target"].numpy()
    lse = np.full(N, math.log(V))
    gh, gw, gb = grad.linear_logp_backward(inp["hidden"], w, inp["target"], None, lse, gl, gs)
    want_b = np.zeros(V)
    want_w = np.zeros((V, H))
    for i in range(N):
        for v in range(V):
            d = (gs[i] - gl[i]) / V + (gl[i] if v == t[i] else 0.0)
            want_b[v] += d
            want_w[v] += d * h[i]
    _assert(np.max(np.abs(gh)) == 0.0, "grad_hidden must be 0 when W = 0")
    _assert(np.max(np.abs(gb - want_b)) < 1e-12, "uniform bias gradient")
    _assert(np.max(np.abs(gw - want_w)) < 1e-12, "uniform weight gradient")


def pin_shift_invariance(grad):
    """bias + c with lse + c gives the same gradients; lse + d alone scales P
    (g_logp = 0, g_lse = 1: dZ = P) by exp(-d)."""
    inp = synth.make_custom(10, 16, 70, 8, bias="f32")
    up = synth.make_upstream_grads(10, 8)
    _, lse = oracle.linear_logp(inp["hidden"], inp["weight"], inp["target"], inp["bias"])
    b = oracle.to_f64(inp["bias"])
    base = grad.linear_logp_backward(inp["hidden"], inp["weight"], inp["target"], b, lse,
                                     up["grad_logp"], up["grad_lse"])
    c = 3.0
    shifted = grad.linear_logp_backward(inp["hidden"], inp["weight"], inp["target"], b + c,
                                        lse + c, up["grad_logp"], up["grad_lse"])
    for x, y, name in zip(base, shifted, ("hidden", "weight", "bias")):
        _assert(_rel(y, x) < 1e-12, f"bias + c, lse + c changed grad_{name}")
    d = 0.7
    ones, zeros = np.ones(10), np.zeros(10)
    p = grad.softmax_grad(inp["hidden"], inp["weight"], inp["target"], b, lse, zeros, ones)
    q = grad.softmax_grad(inp["hidden"], inp["weight"], inp["target"], b, lse + d, zeros, ones)
    _assert(np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12, "P rows must sum to 1")
    _assert(_rel(q, p * math.exp(-d)) < 1e-12, "the given lse must be used as given")


def pin_subsets(grad):
    """grad_hidden_rows / grad_weight_rows / softmax_grad subsets equal the
    full backward's entries, rows and columns in the order asked."""
    inp = synth.make_custom(30, 16, 90, 9, bias="bf16")
    up = synth.make_upstream_grads(30, 9)
    _, lse = oracle.linear_logp(inp["hidden"], inp["weight"], inp["target"], inp["bias"])
    args = (inp["hidden"], inp["weight"], inp["target"], inp["bias"], lse, up["grad_logp"],
            up["grad_lse"])
    gh, gw, gb = grad.linear_logp_backward(*args, row_chunk=7)
    rows, cols = [29, 0, 13], [89, 4, 0, 50]
    _assert(_rel(grad.grad_hidden_rows(*args, rows=rows), gh[rows]) < 1e-12, "grad_hidden rows")
    sw, sb = grad.grad_weight_rows(*args, cols=cols)
    _assert(_rel(sw, gw[cols]) < 1e-12, "grad_weight rows")
    _assert(_rel(sb, gb[cols]) < 1e-12, "grad_bias entries")
    full = grad.softmax_grad(*args)
    _assert(_rel(grad.softmax_grad(*args, rows=rows, cols=cols), full[np.ix_(rows, cols)]) < 1e-12,
            "dZ subset")


ALL_PINS = [pin_finite_differences, pin_torch_autograd, pin_cross_entropy,
            pin_uniform_closed_form, pin_shift_invariance, pin_subsets]
