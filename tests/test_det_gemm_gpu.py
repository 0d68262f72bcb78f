"""The deterministic GEMM on MI355X against the fp64 oracle, plus its bit
contract (RL-Kernel PR #395, summary and tests paragraph: a fixed ascending
K-order reduction with fp32 accumulation; batch and chunk invariance checked
with exact tensor equality).

Tolerance per output element, from the arithmetic: an fp32 accumulation of
n exact products (bf16 x bf16 is exact in fp32) is within n * 2^-24 * S of
the exact sum, S the sum of |products| (``oracle.abs_product``); a bf16
output adds at most 2^-8 |value| (8 significand bits, round to nearest even:
half a spacing), an fp32 output 2^-24 |value|, and an accumulating output one
more fp32 rounding of the sum.
"""

import numpy as np
import pytest
import torch

import invariant_linear_log_amd as ila
import oracle
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16).to(DEV)


def check(got, ref, absref, n_terms, out_dtype, what, extra=None):
    got = got.double().cpu().numpy()
    tol = n_terms * U * absref + (2.0 ** -8 if out_dtype == torch.bfloat16 else U) * np.abs(ref)
    if extra is not None:
        tol = tol + extra
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    say(f"{what}: max|err| {float(err.max()) if err.size else 0:.3e}, worst err/tol {worst:.3f}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    assert np.all(err <= tol), f"{what}: error exceeds the fp32 accumulation bound"


SHAPES = [  # (M, N, K)
    (1, 8, 8),
    (300, 264, 520),        # every dimension ragged against 256 / 64
    (513, 520, 1032),
    (128, 128, 128),        # the page's benchmark shapes, M x K x N
    (256, 512, 512),
    (512, 1024, 1024),
    (2048, 4096, 4096),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_forward_parity(M, N, K):
    a, b = bf16((M, K), 1 + M), bf16((N, K), 2 + N)
    say(f"det_gemm fwd M={M} N={N} K={K}")
    c16 = ila.det_gemm(a, b)
    c32 = ila.det_gemm(a, b, out_dtype=torch.float32)
    init = torch.randn((M, N), generator=torch.Generator().manual_seed(3)).to(DEV)
    acc = init.clone()
    ila.det_gemm(a, b, out=acc, accumulate=True)
    torch.cuda.synchronize()
    ref = oracle.det_gemm_fwd(a.cpu(), b.cpu())
    s = oracle.abs_product("fwd", a.cpu(), b.cpu())
    check(c16, ref, s, K, torch.bfloat16, "fwd bf16")
    check(c32, ref, s, K, torch.float32, "fwd fp32")
    ref_acc = ref + init.double().cpu().numpy()
    check(acc, ref_acc, s, K + 1, torch.float32, "fwd fp32 accumulate",
          extra=U * np.abs(init.double().cpu().numpy()))
    # fp32 output rounded to bf16 is the bf16 output (one rounding, nearest even)
    assert torch.equal(c32.to(torch.bfloat16), c16)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gradients_parity(M, N, K):
    a, b, dc = bf16((M, K), 4 + M), bf16((N, K), 5 + N), bf16((M, N), 6 + K)
    say(f"det_gemm dA / dB M={M} N={N} K={K}")
    da = ila.det_gemm_da(dc, b, out_dtype=torch.float32)
    db = ila.det_gemm_db(a, dc, out_dtype=torch.float32)
    da16 = ila.det_gemm_da(dc, b)
    db16 = ila.det_gemm_db(a, dc)
    torch.cuda.synchronize()
    ref_da = oracle.det_gemm_da(dc.cpu(), b.cpu())
    ref_db = oracle.det_gemm_db(a.cpu(), dc.cpu())
    s_da = oracle.abs_product("da", dc.cpu(), b.cpu())
    s_db = oracle.abs_product("db", a.cpu(), dc.cpu())
    check(da, ref_da, s_da, N, torch.float32, "dA fp32")
    check(db, ref_db, s_db, M, torch.float32, "dB fp32")
    check(da16, ref_da, s_da, N, torch.bfloat16, "dA bf16")
    check(db16, ref_db, s_db, M, torch.bfloat16, "dB bf16")


def test_256_tiles_with_ragged_edges():
    """Products large enough for 256 x 256 tiles on every compute unit (17 x 17
    tiles) with the last tile row and column ragged, in all three layouts and
    all output kinds: the store epilogue of the 256-tile kernels (whole rows
    through LDS; fp32 in two passes) against the fp64 oracle."""
    Mb, Nb, Kc = 4200, 4136, 520
    # forward: C[4200, 4136] = A[4200, 520] . B[4136, 520]^T
    a, b = bf16((Mb, Kc), 31), bf16((Nb, Kc), 32)
    # dA[4200, 4136] = dC[4200, 520] . B2[520, 4136]
    dc, b2 = bf16((Mb, Kc), 33), bf16((Kc, Nb), 34)
    # dB[4200, 4136] = dC3[520, 4200]^T . A3[520, 4136]
    a3, dc3 = bf16((Kc, Nb), 35), bf16((Kc, Mb), 36)
    say("det_gemm 256-tile kernels, ragged edges")
    c16 = ila.det_gemm(a, b)
    c32 = ila.det_gemm(a, b, out_dtype=torch.float32)
    init = torch.randn((Mb, Nb), generator=torch.Generator().manual_seed(37)).to(DEV)
    acc = init.clone()
    ila.det_gemm(a, b, out=acc, accumulate=True)
    da16 = ila.det_gemm_da(dc, b2)
    da32 = ila.det_gemm_da(dc, b2, out_dtype=torch.float32)
    db16 = ila.det_gemm_db(a3, dc3)
    db32 = ila.det_gemm_db(a3, dc3, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.det_gemm_fwd(a.cpu(), b.cpu())
    s = oracle.abs_product("fwd", a.cpu(), b.cpu())
    check(c16, ref, s, Kc, torch.bfloat16, "fwd bf16, 256 tiles")
    check(c32, ref, s, Kc, torch.float32, "fwd fp32, 256 tiles")
    check(acc, ref + init.double().cpu().numpy(), s, Kc + 1, torch.float32,
          "fwd fp32 accumulate, 256 tiles", extra=U * np.abs(init.double().cpu().numpy()))
    ref = oracle.det_gemm_da(dc.cpu(), b2.cpu())
    s = oracle.abs_product("da", dc.cpu(), b2.cpu())
    check(da16, ref, s, Kc, torch.bfloat16, "dA bf16, 256 tiles")
    check(da32, ref, s, Kc, torch.float32, "dA fp32, 256 tiles")
    ref = oracle.det_gemm_db(a3.cpu(), dc3.cpu())
    s = oracle.abs_product("db", a3.cpu(), dc3.cpu())
    check(db16, ref, s, Kc, torch.bfloat16, "dB bf16, 256 tiles")
    check(db32, ref, s, Kc, torch.float32, "dB fp32, 256 tiles")


@pytest.mark.parametrize("chunk", [1, 7, 256, 300])
def test_rows_do_not_depend_on_the_batch(chunk):
    """Forward and dA rows: the full batch equals the concatenation of
    row-chunked calls, bit for bit."""
    M, N, K = 1000, 520, 1032
    a, b, dc = bf16((M, K), 7), bf16((N, K), 8), bf16((M, N), 9)
    say(f"det_gemm batch invariance chunk={chunk}")
    full_c = ila.det_gemm(a, b, out_dtype=torch.float32)
    full_da = ila.det_gemm_da(dc, b, out_dtype=torch.float32)
    parts_c = [ila.det_gemm(a[i:i + chunk], b, out_dtype=torch.float32)
               for i in range(0, M, chunk)]
    parts_da = [ila.det_gemm_da(dc[i:i + chunk], b, out_dtype=torch.float32)
                for i in range(0, M, chunk)]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts_c), full_c)
    assert torch.equal(torch.cat(parts_da), full_da)


def test_run_to_run_and_streams():
    M, N, K = 777, 264, 520
    a, b, dc = bf16((M, K), 10), bf16((N, K), 11), bf16((M, N), 12)
    say("det_gemm run-to-run and side stream")
    ref = [ila.det_gemm(a, b), ila.det_gemm_da(dc, b), ila.det_gemm_db(a, dc)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        again = [ila.det_gemm(a, b), ila.det_gemm_da(dc, b), ila.det_gemm_db(a, dc)]
    s.synchronize()
    for x, y in zip(ref, again):
        assert torch.equal(x, y)


def test_weight_gradient_of_an_empty_batch():
    a = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    dc = torch.empty((0, 72), dtype=torch.bfloat16, device=DEV)
    say("det_gemm dB with M = 0")
    db = ila.det_gemm_db(a, dc, out_dtype=torch.float32)
    keep = torch.randn((72, 64), device=DEV)
    acc = keep.clone()
    ila.det_gemm_db(a, dc, out=acc, accumulate=True)
    c = ila.det_gemm(a, bf16((72, 64), 13))
    torch.cuda.synchronize()
    assert torch.equal(db, torch.zeros_like(db))
    assert torch.equal(acc, keep)
    assert c.shape == (0, 72)


def test_det_linear_autograd():
    M, N, K = 300, 264, 520
    a = bf16((M, K), 14).requires_grad_(True)
    w = bf16((N, K), 15).requires_grad_(True)
    g = bf16((M, N), 16)
    say("DetLinear forward + backward")
    y = ila.DetLinear.apply(a, w)
    y.backward(g)
    torch.cuda.synchronize()
    with torch.no_grad():
        assert torch.equal(y, ila.det_gemm(a, w))
        assert torch.equal(a.grad, ila.det_gemm_da(g, w))
        assert torch.equal(w.grad, ila.det_gemm_db(a, g))
    # fp32 output: the upstream gradient is rounded to bf16 before the kernels
    a2 = a.detach().clone().requires_grad_(True)
    y32 = ila.DetLinear.apply(a2, w.detach(), True)
    assert y32.dtype == torch.float32
    y32.backward(g.float())
    torch.cuda.synchronize()
    assert torch.equal(a2.grad, ila.det_gemm_da(g, w.detach()))


def test_tile_sizes_give_the_same_bits():
    """A full batch with 256 x 256 tiles for every compute unit and row chunks
    small enough for 128 x 128 tiles: the same rows, bit for bit (forward, dA
    and dB; every output is one MFMA chain whatever the tile)."""
    M, N, K = 4096, 4096, 256
    a, b = bf16((M, K), 17), bf16((N, K), 18)
    dc, b2 = bf16((M, 256), 19), bf16((256, 4096), 20)
    say("det_gemm 256- vs 128-tiles")
    full_c = ila.det_gemm(a, b, out_dtype=torch.float32)            # 16 x 16 tiles of 256
    full_da = ila.det_gemm_da(dc, b2, out_dtype=torch.float32)      # 16 x 16 tiles of 256
    parts_c = [ila.det_gemm(a[i:i + 300], b, out_dtype=torch.float32) for i in range(0, M, 300)]
    parts_da = [ila.det_gemm_da(dc[i:i + 300], b2, out_dtype=torch.float32)
                for i in range(0, M, 300)]
    # dB (both operands read transposed): its rows n from column slices of dC
    a3, dc3 = bf16((256, 4096), 21), bf16((256, 4096), 22)
    full_db = ila.det_gemm_db(a3, dc3, out_dtype=torch.float32)   # 16 x 16 tiles of 256
    parts_db = [ila.det_gemm_db(a3, dc3[:, i:i + 296].contiguous(), out_dtype=torch.float32)
                for i in range(0, 4096, 296)]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts_c), full_c)
    assert torch.equal(torch.cat(parts_da), full_da)
    assert torch.equal(torch.cat(parts_db), full_db)
