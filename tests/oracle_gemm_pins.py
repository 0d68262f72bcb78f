"""Pins of the det_gemm oracle (oracle/det_gemm.py), each against something
other than the oracle itself:

  * pure-Python ``math.fsum`` brute force of the forward on tiny shapes;
  * a hand-worked 2 x 3 example (values in tests/golden/det_gemm_worked.txt)
    for the forward, dA and dB;
  * the adjoint identity <dC, A B^T> = <dA, A> = <dB, B> (it ties the three
    products together: a transposed or swapped operand breaks it);
  * the single-row weight gradient is the outer product dC[0]^T A[0];
  * forward symmetry fwd(A, B) = fwd(B, A)^T and the output shapes.
"""

import math
import os

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "det_gemm_worked.txt")


class PinFailure(AssertionError):
    pass


def _assert(cond, msg):
    if not cond:
        raise PinFailure(msg)


def _bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


def pin_brute_force(orc):
    """fsum of exact products equals the float64 forward (tiny shapes)."""
    for j, (M, N, K) in enumerate([(1, 1, 1), (2, 3, 5), (5, 4, 16), (3, 7, 33)]):
        a, b = _bf16((M, K), 10 + j), _bf16((N, K), 20 + j)
        c = orc.det_gemm_fwd(a, b)
        ref = np.array(orc.brute_force_fwd(a, b))
        _assert(c.shape == (M, N), f"fwd shape {c.shape}")
        _assert(np.max(np.abs(c - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref))), f"fsum {j}")


def _read_golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        name, rest = line.split("=", 1)
        vals[name.strip()] = np.array(
            [[float(x) for x in row.split()] for row in rest.split(";")], dtype=np.float64)
    return vals


def pin_worked_example(orc):
    """A 2 x 3, B 2 x 3 (so C is 2 x 2), dC 2 x 2: every value worked by hand."""
    v = _read_golden()
    a = torch.tensor(v["A"], dtype=torch.bfloat16)
    b = torch.tensor(v["B"], dtype=torch.bfloat16)
    dc = torch.tensor(v["dC"], dtype=torch.bfloat16)
    _assert(np.array_equal(orc.det_gemm_fwd(a, b), v["C"]), "worked forward")
    _assert(np.array_equal(orc.det_gemm_da(dc, b), v["dA"]), "worked dA")
    _assert(np.array_equal(orc.det_gemm_db(a, dc), v["dB"]), "worked dB")


def pin_adjoint_identity(orc):
    """<dC, A B^T> = <dC B, A> = <dC^T A, B> for random shapes."""
    for j, (M, N, K) in enumerate([(3, 5, 8), (17, 9, 24), (64, 40, 72)]):
        a, b, dc = _bf16((M, K), 30 + j), _bf16((N, K), 40 + j), _bf16((M, N), 50 + j)
        A, B, G = (x.double().numpy() for x in (a, b, dc))
        c = orc.det_gemm_fwd(a, b)
        da = orc.det_gemm_da(dc, b)
        db = orc.det_gemm_db(a, dc)
        _assert(da.shape == (M, K) and db.shape == (N, K), f"gradient shapes {j}")
        s0 = float(np.sum(G * c))
        s1 = float(np.sum(da * A))
        s2 = float(np.sum(db * B))
        scale = float(np.sum(np.abs(G) * (np.abs(A) @ np.abs(B).T)))
        _assert(abs(s0 - s1) <= 1e-12 * scale and abs(s0 - s2) <= 1e-12 * scale, f"adjoint {j}")


def pin_single_row_outer_product(orc):
    """With M = 1 the weight gradient is the outer product dC[0]^T A[0]."""
    a, dc = _bf16((1, 24), 60), _bf16((1, 9), 61)
    db = orc.det_gemm_db(a, dc)
    ref = np.outer(dc.double().numpy()[0], a.double().numpy()[0])
    _assert(db.shape == (9, 24) and np.array_equal(db, ref), "outer product")


def pin_symmetry_and_abs(orc):
    """fwd(A, B) = fwd(B, A)^T; |terms| sums bound |results| and equal them for
    non-negative operands (forward, dA and dB)."""
    a, b = _bf16((6, 16), 70), _bf16((11, 16), 71)
    _assert(np.array_equal(orc.det_gemm_fwd(a, b), orc.det_gemm_fwd(b, a).T), "symmetry")
    c = orc.det_gemm_fwd(a, b)
    _assert(np.all(np.abs(c) <= orc.abs_product("fwd", a, b) * (1 + 1e-15)), "abs bound")
    pa, pb = a.abs(), b.abs()
    _assert(np.allclose(orc.det_gemm_fwd(pa, pb), orc.abs_product("fwd", pa, pb), rtol=1e-15,
                        atol=0), "abs equal")
    dc = _bf16((6, 11), 72)
    _assert(np.all(np.abs(orc.det_gemm_da(dc, b)) <= orc.abs_product("da", dc, b) * (1 + 1e-15)),
            "abs da")
    _assert(np.all(np.abs(orc.det_gemm_db(a, dc)) <= orc.abs_product("db", a, dc) * (1 + 1e-15)),
            "abs db")
    # with non-negative operands every term is its own absolute value, so the
    # sums of |terms| equal the products exactly (an over-estimate, which
    # would loosen the GPU tolerances built on them, fails here)
    pdc = dc.abs()
    _assert(np.allclose(orc.det_gemm_da(pdc, pb), orc.abs_product("da", pdc, pb), rtol=1e-15,
                        atol=0), "abs da equal")
    _assert(np.allclose(orc.det_gemm_db(pa, pdc), orc.abs_product("db", pa, pdc), rtol=1e-15,
                        atol=0), "abs db equal")


ALL_PINS = [pin_brute_force, pin_worked_example, pin_adjoint_identity,
            pin_single_row_outer_product, pin_symmetry_and_abs]
