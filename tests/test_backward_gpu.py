"""The deterministic backward on MI355X against the fp64 oracle
(oracle/linear_logp_grad.py), and its bit contract.

Tolerance, per element, from the arithmetic (u = 2^-24):
  * z: an fp32 accumulation of H exact products started at the exact bias is
    within dz = (H + 1) u S of the exact logit, S = sum_k |h_k w_k| + |b|;
  * P = exp(z - lse) in fp32 (a subtraction, a scaling by log2(e), the
    hardware exp2): relative error e_P = dz + 4u (|z| + |lse| + dz) + 4u;
  * dZ = P (g_lse - g_logp) (+ g_logp at the target) in fp32, then rounded
    to bf16 (nearest even, relative 2^-8):
        E = |g_lse - g_logp| P (e_P + u) + u |dZ|,  B = E + 2^-8 (|dZ| + E)
    bounds |dZ_kernel - dZ|;
  * plus an absolute 2^-120 (|g_lse - g_logp| + 1) for exponentials that
    fall below fp32's normal range;
  * the products accumulate n = V (grad_hidden) or N (grad_weight,
    grad_bias) terms in fp32: the error is at most B . |W| (or B^T . |h|,
    sum B) plus n u (|dZ| + B) . |W| (or (|dZ| + B)^T . |h|, sum (|dZ| + B)).
The dZ the kernel leaves in the workspace ([V, ldz] bf16, ldz = N rounded up
to 8) is checked against B directly, and the gradients against the exact
products of that dZ within the accumulation term alone.
"""

import numpy as np
import pytest
import torch

import invariant_linear_log_amd as ila
import oracle
import synth
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _inputs(N, H, V, seed, bias=None, hidden_scale=1.0):
    inp = synth.make_custom(N, H, V, seed, bias=bias, hidden_scale=hidden_scale, device=DEV)
    up = synth.make_upstream_grads(N, seed, device=DEV)
    return inp, up


def _run(inp, up, lse, bias_grad=True):
    N = inp["hidden"].shape[0]
    V = inp["weight"].shape[0]
    ws = ila.backward_workspace_for(N, V, DEV)
    gh, gw, gb = ila.backward(inp["hidden"], inp["weight"], inp["target"], inp["bias"], lse,
                              up["grad_logp"], up["grad_lse"], bias_grad=bias_grad,
                              workspace=ws)
    return gh, gw, gb, ws


def _dzt(ws, N, V):
    ldz = (N + 7) // 8 * 8
    return ws[:V * ldz * 2].view(torch.bfloat16).view(V, ldz)[:, :N]


def _bounds(h, w, b, t, lse, gl, gs, rows, cols):
    """(dZ, B) over rows x cols: exact dZ and the bound on the kernel's bf16 dZ."""
    z = h[rows] @ w[cols].T
    S = np.abs(h[rows]) @ np.abs(w[cols]).T
    if b is not None:
        z += b[cols]
        S += np.abs(b[cols])
    H = h.shape[1]
    dzl = (H + 1) * U * S
    ls = lse[rows][:, None]
    P = np.exp(z - ls)
    coef = (gs - gl)[rows][:, None]
    onehot = t[rows][:, None] == cols[None, :]
    dz = coef * P + np.where(onehot, gl[rows][:, None], 0.0)
    e_p = dzl + 4 * U * (np.abs(z) + np.abs(ls) + dzl) + 4 * U
    E = np.abs(coef) * P * (e_p + U) + U * np.abs(dz)
    B = E + 2.0 ** -8 * (np.abs(dz) + E)
    # exp2 results below the normal range may flush to zero
    B += 2.0 ** -120 * (np.abs(coef) + 1.0)
    return dz, B


def _f64(inp, up, lse):
    return (oracle.to_f64(inp["hidden"]), oracle.to_f64(inp["weight"]),
            oracle.to_f64(inp["bias"]), inp["target"].cpu().numpy(), oracle.to_f64(lse),
            oracle.to_f64(up["grad_logp"]), oracle.to_f64(up["grad_lse"]))


def _within(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    say(f"{what}: max|err| {float(err.max()) if err.size else 0:.3e}, worst err/tol {worst:.3f}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    assert np.all(err <= tol), f"{what}: error beyond the derived bound (worst {worst:.3f})"


CASES = [  # (N, H, V, bias, seed)
    (300, 520, 1000, None, 1),        # 2 row blocks (ragged), ragged K and vocabulary tiles
    (257, 264, 777, "bf16", 2),       # N % 8 != 0 (padded dZ^T), V % 8 != 0
    (1, 64, 300, "f32", 3),
    (513, 1024, 4099, "f32", 4),      # 3 row blocks, 17 tiles
    (64, 8, 256, None, 5),            # H = 8, one exact tile
    (70001, 64, 600, "f32", 6),       # long ragged batch: 274 row blocks, dZ^T padded to 70008
    (96, 16384, 520, None, 7),        # wide K: 256 stages per projection tile
]


@pytest.mark.parametrize("N,H,V,bias,seed", CASES)
def test_backward_parity(N, H, V, bias, seed):
    inp, up = _inputs(N, H, V, seed, bias)
    t = inp["target"]
    # targets on tile edges and at both vocabulary ends; one out of range
    for i, tv in enumerate([0, V - 1, min(255, V - 1), min(256, V - 1), -1]):
        if i < N:
            t[i] = tv
    say(f"backward parity N={N} H={H} V={V} bias={bias}")
    with torch.no_grad():
        _, lse = ila.forward(inp["hidden"], inp["weight"], t.clamp(0, V - 1), inp["bias"])
    gh, gw, gb, ws = _run(inp, up, lse)
    dzt = _dzt(ws, N, V)
    torch.cuda.synchronize()
    h, w, b, tt, ls, gl, gs = _f64(inp, up, lse)
    rows, cols = np.arange(N), np.arange(V)
    dz, B = _bounds(h, w, b, tt, ls, gl, gs, rows, cols)
    ref_dz = oracle.softmax_grad(h, w, tt, b, ls, gl, gs)
    # two float64 evaluations of dZ (BLAS blocking may differ): equal to rounding
    assert np.allclose(ref_dz, dz, rtol=1e-12, atol=1e-14)
    _within(oracle.to_f64(dzt).T, ref_dz, B, "dZ (workspace)")
    ref_gh, ref_gw, ref_gb = oracle.linear_logp_backward(h, w, tt, b, ls, gl, gs)
    aW, ah = np.abs(w), np.abs(h)
    big = np.abs(dz) + B
    _within(gh.cpu().numpy(), ref_gh, B @ aW + V * U * (big @ aW), "grad_hidden")
    _within(gw.cpu().numpy(), ref_gw, B.T @ ah + N * U * (big.T @ ah), "grad_weight")
    if bias is not None:
        _within(gb.cpu().numpy(), ref_gb, B.sum(0) + N * U * big.sum(0), "grad_bias")
    else:
        assert gb is None
    # the two products from the kernel's own dZ: accumulation error only
    dzk = oracle.to_f64(dzt).T
    adk = np.abs(dzk)
    _within(gh.cpu().numpy(), dzk @ w, V * U * (adk @ aW) + U * np.abs(dzk @ w), "dZ_k . W")
    _within(gw.cpu().numpy(), dzk.T @ h, N * U * (adk.T @ ah) + U * np.abs(dzk.T @ h),
            "dZ_k^T . hidden")


def test_cross_entropy_gradient():
    """g_logp = -1, g_lse = 0: dZ = softmax - onehot; each row of the kernel's
    dZ sums to 0 within the rounding bound."""
    N, H, V = 200, 256, 3000
    inp, _ = _inputs(N, H, V, 6)
    up = {"grad_logp": -torch.ones(N, device=DEV), "grad_lse": torch.zeros(N, device=DEV)}
    say("backward cross-entropy N=200 V=3000")
    with torch.no_grad():
        _, lse = ila.forward(inp["hidden"], inp["weight"], inp["target"])
    _, _, _, ws = _run(inp, up, lse)
    dzt = _dzt(ws, N, V)
    torch.cuda.synchronize()
    h, w, b, tt, ls, gl, gs = _f64(inp, up, lse)
    dz, B = _bounds(h, w, b, tt, ls, gl, gs, np.arange(N), np.arange(V))
    dzk = oracle.to_f64(dzt).T
    row_sum = dzk.sum(axis=1)
    exact = dz.sum(axis=1)            # 0 up to the fp32 lse handed in
    assert np.all(np.abs(row_sum - exact) <= B.sum(axis=1))
    assert np.all(dzk[np.arange(N), tt] < 0)


def test_empty_batch_zero_weight_gradient():
    V, H = 1000, 64
    w = synth.make_custom(1, H, V, 7, device=DEV)["weight"]
    e = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    z = torch.empty(0, device=DEV)
    bias = torch.randn(V, device=DEV)
    say("backward N=0")
    gh, gw, gb = ila.backward(e, w, torch.empty(0, dtype=torch.int64, device=DEV), bias, z, z, z)
    torch.cuda.synchronize()
    assert gh.shape == (0, H)
    assert torch.equal(gw, torch.zeros_like(gw))
    assert torch.equal(gb, torch.zeros_like(gb))


@pytest.mark.parametrize("N,H,V,chunk", [
    (700, 512, 2100, 1), (700, 512, 2100, 7), (700, 512, 2100, 256), (700, 512, 2100, 300),
    # 64 splits: the full batch runs 256-token row blocks (5 x 64 workgroups), the
    # chunks 128-token blocks (at most 3 x 64 < 256 compute units)
    (1100, 256, 16384, 300), (1100, 256, 16384, 37),
])
def test_grad_hidden_rows_do_not_depend_on_the_batch(N, H, V, chunk):
    """grad_hidden of a row is the same bits in any batch: chunked calls and a
    permuted batch reproduce the full batch's rows exactly."""
    inp, up = _inputs(N, H, V, 8, "bf16")
    say(f"grad_hidden batch invariance N={N} V={V} chunk={chunk}")
    with torch.no_grad():
        _, lse = ila.forward(inp["hidden"], inp["weight"], inp["target"], inp["bias"])
    full, _, _, _ = _run(inp, up, lse)
    parts = []
    for i in range(0, N, chunk):
        sl = slice(i, i + chunk)
        sub = {k: (v[sl] if k in ("hidden", "target") else v) for k, v in inp.items()}
        sup = {k: v[sl] for k, v in up.items()}
        parts.append(_run(sub, sup, lse[sl])[0])
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(chunk)).to(DEV)
    pin = {k: (v[perm] if k in ("hidden", "target") else v) for k, v in inp.items()}
    pup = {k: v[perm] for k, v in up.items()}
    permuted = _run(pin, pup, lse[perm])[0]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts), full)
    assert torch.equal(permuted, full[perm])


def test_split_schedule_with_a_second_launch_keeps_the_bits():
    """N = 1024, H = 1024, V = 20480 on 256 compute units: 4 row blocks x 80
    splits, scheduled as one round of 256 whole tiles plus the last 16 splits
    as 128 half-height pieces in a second launch.  256-row chunks run
    128-token blocks in one launch.  dZ^T (the workspace) and grad_hidden of
    every row are the same bits either way."""
    N, H, V = 1024, 1024, 20480
    S = ila.bilogp_num_vocab_splits(V)
    if ila.device_cu_count(DEV) == 256:
        assert ila.bilogp_launch_schedule(N, H, V, ila.BILOGP_SPLITS_INVARIANT, 256)[1] < S
    inp, up = _inputs(N, H, V, 9, "bf16")
    say(f"backward split schedule N={N} H={H} V={V}")
    with torch.no_grad():
        _, lse = ila.forward(inp["hidden"], inp["weight"], inp["target"], inp["bias"])
    full, _, _, ws = _run(inp, up, lse)
    full_dz = _dzt(ws, N, V).clone()
    for i in range(0, N, 256):
        sl = slice(i, i + 256)
        sub = {k: (v[sl] if k in ("hidden", "target") else v) for k, v in inp.items()}
        sup = {k: v[sl] for k, v in up.items()}
        gh, _, _, wsc = _run(sub, sup, lse[sl])
        torch.cuda.synchronize()
        assert torch.equal(gh, full[sl]), f"grad_hidden rows {i}.. differ"
        assert torch.equal(_dzt(wsc, 256, V), full_dz[:, sl]), f"dZ rows {i}.. differ"


def test_run_to_run_and_streams():
    """Every output, on a second call and on a side stream, is the same bits."""
    N, H, V = 600, 384, 1500
    inp, up = _inputs(N, H, V, 9, "f32")
    say("backward run-to-run and side stream")
    with torch.no_grad():
        _, lse = ila.forward(inp["hidden"], inp["weight"], inp["target"], inp["bias"])
    a = _run(inp, up, lse)[:3]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        b = _run(inp, up, lse)[:3]
    s.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("bias", ["f32", "bf16"])
def test_autograd_linear_logp(bias):
    """linear_logp: the forward's outputs, and gradients equal to backward()'s
    (rounded once to the inputs' dtypes)."""
    N, H, V = 300, 256, 1200
    inp, up = _inputs(N, H, V, 10, bias)
    h = inp["hidden"].clone().requires_grad_(True)
    w = inp["weight"].clone().requires_grad_(True)
    b = inp["bias"].clone().requires_grad_(True)
    say(f"linear_logp autograd, {bias} bias")
    logp, lse = ila.linear_logp(h, w, inp["target"], b)
    (logp * up["grad_logp"] + lse * up["grad_lse"]).sum().backward()
    with torch.no_grad():
        ref_logp, ref_lse = ila.forward(inp["hidden"], inp["weight"], inp["target"], inp["bias"])
        gh, gw, gb = ila.backward(inp["hidden"], inp["weight"], inp["target"], inp["bias"],
                                  ref_lse, up["grad_logp"], up["grad_lse"])
    torch.cuda.synchronize()
    assert torch.equal(logp, ref_logp) and torch.equal(lse, ref_lse)
    assert torch.equal(h.grad, gh.to(torch.bfloat16))
    assert torch.equal(w.grad, gw.to(torch.bfloat16))
    assert b.grad.dtype == b.dtype and torch.equal(b.grad, gb.to(b.dtype))


def test_autograd_partial_requires_grad():
    """Only hidden requires grad (a frozen lm-head): the weight and bias get no
    gradient, and hidden's equals backward()'s."""
    N, H, V = 200, 128, 900
    inp, up = _inputs(N, H, V, 11, "f32")
    h = inp["hidden"].clone().requires_grad_(True)
    say("linear_logp autograd, frozen weight")
    logp, lse = ila.linear_logp(h, inp["weight"], inp["target"], inp["bias"])
    (logp * up["grad_logp"] + lse * up["grad_lse"]).sum().backward()
    with torch.no_grad():
        _, ref_lse = ila.forward(inp["hidden"], inp["weight"], inp["target"], inp["bias"])
        gh, _, _ = ila.backward(inp["hidden"], inp["weight"], inp["target"], inp["bias"],
                                ref_lse, up["grad_logp"], up["grad_lse"])
    torch.cuda.synchronize()
    assert torch.equal(h.grad, gh.to(torch.bfloat16))
    assert inp["weight"].grad is None and inp["bias"].grad is None


def test_headline_sampled_parity():
    """N = 4096, H = 4096, V = 128256 (the benchmark's shape): sampled rows of
    grad_hidden and vocabulary rows of grad_weight / grad_bias against the
    oracle, one by one, within the derived bound."""
    inp = synth.make_inputs("headline", device=DEV)
    h2 = inp["hidden"].reshape(-1, 4096).contiguous()
    t1 = inp["target"].reshape(-1).contiguous()
    N, V = h2.shape[0], inp["weight"].shape[0]
    up = synth.make_upstream_grads(N, 11, device=DEV)
    say("backward headline N=4096 H=4096 V=128256")
    with torch.no_grad():
        _, lse = ila.forward(h2, inp["weight"], t1)
    gh, gw, _ = ila.backward(h2, inp["weight"], t1, None, lse, up["grad_logp"], up["grad_lse"])
    torch.cuda.synchronize()
    h, w, b = oracle.to_f64(h2), oracle.to_f64(inp["weight"]), None
    tt, ls = t1.cpu().numpy(), oracle.to_f64(lse)
    gl, gs = oracle.to_f64(up["grad_logp"]), oracle.to_f64(up["grad_lse"])
    rows = np.array([0, 1, 2047, N - 1])
    vrows = np.unique(np.array([0, 255, 256, int(tt[0]), int(tt[5]), V - 1]))
    ref_h = oracle.grad_hidden_rows(h, w, tt, b, ls, gl, gs, rows=rows)
    dz, B = _bounds(h, w, b, tt, ls, gl, gs, rows, np.arange(V))
    big = np.abs(dz) + B
    aW = np.abs(w)
    _within(gh[torch.as_tensor(rows, device=DEV)].cpu().numpy(), ref_h,
            B @ aW + V * U * (big @ aW), "grad_hidden rows")
    ref_w, _ = oracle.grad_weight_rows(h, w, tt, b, ls, gl, gs, cols=vrows)
    dzc, Bc = _bounds(h, w, b, tt, ls, gl, gs, np.arange(N), vrows)
    bigc = np.abs(dzc) + Bc
    ah = np.abs(h)
    _within(gw[torch.as_tensor(vrows, device=DEV)].cpu().numpy(), ref_w,
            Bc.T @ ah + N * U * (bigc.T @ ah), "grad_weight rows")


def test_buffers_past_4gib():
    """V = 2^19 + 40, N = 4096, H = 2048: dZ^T ([V, 4096] bf16) and grad_weight
    ([V, 2048] fp32) are each just over 2^32 bytes, so the last 40 vocabulary
    rows of both lie past every 32-bit byte offset.  Sampled rows of the
    kernel's dZ^T, of grad_weight (among them rows past the 2^32-byte mark)
    and of grad_hidden against the oracle within the derived bound."""
    N, H, V = 4096, 2048, (1 << 19) + 40
    assert V * N * 2 > 1 << 32 and V * H * 4 > 1 << 32
    inp, up = _inputs(N, H, V, 12)
    t = inp["target"]
    t[0], t[1] = V - 1, V - 20                  # targets past the mark
    say(f"backward buffers past 4 GiB N={N} H={H} V={V}")
    with torch.no_grad():
        _, lse = ila.forward(inp["hidden"], inp["weight"], t)
    gh, gw, _, ws = _run(inp, up, lse, bias_grad=False)
    vrows = np.array([0, 255, 256, V - 41, V - 40, V - 20, V - 1])
    vsel = torch.as_tensor(vrows, device=DEV)
    dzt = _dzt(ws, N, V)[vsel].cpu()
    gw_s = gw[vsel].cpu().numpy()
    rows = np.array([0, 1, 2047, N - 1])
    gh_s = gh[torch.as_tensor(rows, device=DEV)].cpu().numpy()
    torch.cuda.synchronize()
    del ws, gw
    h, w, b, tt, ls, gl, gs = _f64(inp, up, lse)
    ah, aW = np.abs(h), np.abs(w)
    dzc, Bc = _bounds(h, w, b, tt, ls, gl, gs, np.arange(N), vrows)
    _within(oracle.to_f64(dzt).T, dzc, Bc, "dZ^T rows (workspace)")
    ref_w, _ = oracle.grad_weight_rows(h, w, tt, b, ls, gl, gs, cols=vrows)
    bigc = np.abs(dzc) + Bc
    _within(gw_s, ref_w, Bc.T @ ah + N * U * (bigc.T @ ah), "grad_weight rows")
    ref_h = oracle.grad_hidden_rows(h, w, tt, b, ls, gl, gs, rows=rows)
    dz, B = _bounds(h, w, b, tt, ls, gl, gs, rows, np.arange(V))
    big = np.abs(dz) + B
    _within(gh_s, ref_h, B @ aW + V * U * (big @ aW), "grad_hidden rows")
