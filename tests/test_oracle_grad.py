"""CPU pins of the backward oracle (tests/oracle_grad_pins.py), and a mutation
check: each entry plants one plausible mistake (a dropped or sign-flipped
one-hot term, swapped upstream gradients, a dropped bias, an unnormalised
softmax, a shifted operand, a lost row) into a private copy of
oracle/linear_logp_grad.py and the pins must reject every copy.  The real
oracle is never modified."""

import os
import types

import pytest

import oracle
import oracle_grad_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "linear_logp_grad.py")


@pytest.mark.parametrize("pin", oracle_grad_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_grad_oracle_pin(pin):
    pin(oracle)


MUTATIONS = {
    "onehot_dropped": ("    dz += np.where(onehot, gl[rows][:, None], 0.0)\n", "    pass\n"),
    "onehot_sign": ("np.where(onehot, gl[rows][:, None], 0.0)", "np.where(onehot, -gl[rows][:, None], 0.0)"),
    "upstream_swapped": ("dz = gs[rows][:, None] * p - gl[rows][:, None] * p",
                         "dz = gl[rows][:, None] * p - gs[rows][:, None] * p"),
    "p_term_of_logp_dropped": ("dz = gs[rows][:, None] * p - gl[rows][:, None] * p",
                               "dz = gs[rows][:, None] * p"),
    "bias_dropped": ("        z += b[cols]\n", "        z += 0.0\n"),
    "unnormalised": ("p = np.exp(z - lse_[rows][:, None])", "p = np.exp(z)"),
    "target_off_by_one": ("onehot = t[rows][:, None] == cols[None, :]",
                          "onehot = t[rows][:, None] == cols[None, :] + 1"),
    "grad_hidden_operand_reversed": ("gh[r] = dz @ w", "gh[r] = dz @ w[:, ::-1]"),
    "grad_weight_rows_shifted": ("gw += dz.T @ h[r]", "gw += dz.T @ h[r][::-1]"),
    "grad_bias_first_row_lost": ("gb += dz.sum(axis=0)", "gb += dz[1:].sum(axis=0)"),
    "last_row_lost": ("r = np.arange(c0, min(c0 + row_chunk, N))",
                      "r = np.arange(c0, min(c0 + row_chunk, N - 1))"),
    "rows_fn_wrong_operand": ("np.arange(w.shape[0])) @ w", "np.arange(w.shape[0])) @ w[::-1]"),
    "cols_fn_wrong_operand": ("return dz.T @ h, dz.sum(axis=0)", "return dz.T @ h[::-1], dz.sum(axis=0)"),
}


def _load_mutant(find, repl):
    with open(SRC) as f:
        src = f.read()
    assert src.count(find) >= 1, f"mutation anchor not found: {find!r}"
    mod = types.ModuleType("oracle.linear_logp_grad_mutant")
    mod.__dict__["__package__"] = "oracle"        # the module's relative import
    exec(compile(src.replace(find, repl), "linear_logp_grad_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_grad_pins_reject_mutant(name):
    mutant = _load_mutant(*MUTATIONS[name])
    caught = False
    for pin in oracle_grad_pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception:  # a PinFailure, or a crash caused by the mutation
            caught = True
            break
    assert caught, f"no pin catches mutation {name}"
