"""CPU pins of the det_gemm oracle (tests/oracle_gemm_pins.py), and a mutation
check: each entry plants one plausible mistake (a transposed or swapped
operand, a dropped term, a sign) into a private copy of oracle/det_gemm.py and
the pins must reject every copy.  The real oracle is never modified."""

import os
import types

import pytest

import oracle
import oracle_gemm_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "det_gemm.py")


@pytest.mark.parametrize("pin", oracle_gemm_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_gemm_oracle_pin(pin):
    pin(oracle)


MUTATIONS = {
    "fwd_operands_swapped": ("return A @ B.T", "return B @ A.T"),
    "fwd_no_transpose_k_reversed": ("return A @ B.T", "return A @ B[:, ::-1].T"),
    "da_uses_transpose": ("return G @ B\n", "return G @ B[::-1]\n"),
    "db_transposed_layout": ("return G.T @ A", "return A.T @ G"),
    "db_sign": ("return G.T @ A", "return -(G.T @ A)"),
    "db_drops_first_row": ("return G.T @ A", "return G[1:].T @ A[1:]"),
    "brute_drops_last_term": ("for k in range(K)", "for k in range(K - 1)"),
    # over-estimated error scales (they would only loosen the GPU tolerances)
    "abs_da_doubled": ("        return X @ Y\n", "        return 2 * (X @ Y)\n"),
    "abs_db_plus_one": ("        return Y.T @ X\n", "        return Y.T @ X + 1\n"),
}


def _load_mutant(find, repl):
    with open(SRC) as f:
        src = f.read()
    assert src.count(find) >= 1, f"mutation anchor not found: {find!r}"
    mod = types.ModuleType("oracle.det_gemm_mutant")
    mod.__dict__["__package__"] = "oracle"        # the module's relative import
    exec(compile(src.replace(find, repl), "det_gemm_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_gemm_pins_reject_mutant(name):
    mutant = _load_mutant(*MUTATIONS[name])
    caught = False
    for pin in oracle_gemm_pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception:  # a PinFailure, or a crash caused by the mutation
            caught = True
            break
    assert caught, f"no pin catches mutation {name}"
