"""Mutation check of the oracle's pins: each entry plants one plausible
mistake (a dropped term, a wrong sign, index or operand, a wrong log base, a
missing rescale, a wrong rounding of the split formula) into a private copy of
``oracle/linear_logp.py``, and the pin battery must reject every copy.  The
real oracle is never modified."""

import os
import types

import pytest

import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "linear_logp.py")

MUTATIONS = {
    "sign_of_logp": ("logp[c0:c0 + r.shape[0]] = zt - lse_c", "logp[c0:c0 + r.shape[0]] = lse_c - zt"),
    "bias_dropped": ("        if b is not None:\n            z += b\n", "        pass\n"),
    "log10": ("np.log(sumexp)", "np.log10(sumexp)"),
    "no_max_shift": ("np.exp(z - zmax[:, None])", "np.exp(z) * np.exp(-zmax[:, None]) "),
    "target_off_by_one": ("z[np.arange(r.shape[0]), t[r]]", "z[np.arange(r.shape[0]), (t[r] + 1) % z.shape[1]]"),
    "k_misaligned": ("wt = w.T", "wt = w[:, ::-1].T"),
    "rows_swapped": ("z = h[r] @ wt", "z = h[r[::-1]] @ wt"),
    "bias_twice": ("            z += b\n", "            z += 2 * b\n"),
    "online_rescale_dropped": ("s = s * np.exp(m - m_new) +", "s = s +"),
    "combine_rescale_dropped": ("part_s[k] * np.exp(part_m[k] - M)", "part_s[k]"),
    "tile_dropped": ("for tile in range(first, end):", "for tile in range(first, max(first + 1, end - 1)):"),
    "split_count_floor": ("n_splits = -(-tiles // per_split)", "n_splits = max(1, tiles // per_split)"),
    "per_split_floor_plus_one": ("per_split = -(-tiles // max_splits)", "per_split = tiles // max_splits + 1"),
    "split_bias_dropped": ("z += b[c0:c1]", "z += 0.0"),
    "split_target_offset": ("tr[hit] - c0]", "tr[hit] - c0 - (c1 - c0 > 1)]"),
    "decode_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "combine_max_not_global": ("M = part_m.max(axis=0)", "M = part_m[0]"),
    "brute_no_bias": ("            if b is not None:\n                terms.append(b[v])\n", ""),
    "brute_lse_shift_lost": ("lse = zmax + math.log(", "lse = math.log("),
    "throughput_row_blocks_floor": ("row_blocks = -(-N // block_rows)", "row_blocks = max(1, N // block_rows)"),
    "throughput_cu_floor": ("-(-cu_count // row_blocks)", "(cu_count // row_blocks)"),
    "throughput_no_max_cap": ("want = min(max(-(-cu_count // row_blocks), 1), tiles, max_splits)",
                              "want = min(max(-(-cu_count // row_blocks), 1), tiles)"),
}


def _load_mutant(find, repl):
    with open(SRC) as f:
        src = f.read()
    assert src.count(find) >= 1, f"mutation anchor not found: {find!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(find, repl), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_mutant(name):
    mutant = _load_mutant(*MUTATIONS[name])
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception as e:  # a PinFailure, or a crash caused by the mutation
            failed.append((pin.__name__, type(e).__name__))
            break
    assert failed, f"no pin catches mutation {name}"
