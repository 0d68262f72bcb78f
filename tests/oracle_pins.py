"""The pins of the fp64 oracle, written as a battery of checks against any
object exposing the oracle's functions.  ``tests/test_oracle.py`` runs them on
the real oracle; ``tests/test_oracle_mutations.py`` runs them on copies of the
oracle with a plausible mistake planted, and requires that some pin fails.

Every pin compares the oracle with something other than itself: mpmath closed
forms, pure-Python ``fsum`` brute force, torch's float64 ``log_softmax``, or an
invariant the mathematics fixes.
"""

from __future__ import annotations

import math
import os

import mpmath
import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


class PinFailure(AssertionError):
    pass


def _assert(cond, msg):
    if not cond:
        raise PinFailure(msg)


def _maxabs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise PinFailure(f"shape {a.shape} != {b.shape}")
    if not (np.all(np.isfinite(a)) and np.all(np.isfinite(b))):
        return math.inf
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def _tiny_shapes():
    """Small seeded shapes for the brute-force comparison (with and without bias)."""
    out = [synth.make_inputs("tiny")]
    out.append(synth.make_custom(5, 24, 37, seed=11))
    out.append(synth.make_custom(3, 16, 300, seed=12, bias="f32"))
    out.append(synth.make_custom(4, 8, 257, seed=13, bias="bf16", bias_std=0.5))
    return out


# ---------------------------------------------------------------- pin 0
def pin_decode(orc):
    """bf16 decoding against the IEEE bit-level definition of a few patterns."""
    pats = {0x3F80: 1.0, 0xC000: -2.0, 0x3E00: 0.125, 0x0000: 0.0,
            0x7F7F: float.fromhex("0x1.fep127"), 0x0001: 2.0 ** -133,
            0x4049: float.fromhex("0x1.92p1"), 0xBF01: -float.fromhex("0x1.02p-1")}
    bits = torch.tensor([p - 65536 if p >= 32768 else p for p in pats], dtype=torch.int16)
    got = orc.decode_bf16(bits.view(torch.bfloat16))
    _assert(list(got) == list(pats.values()), f"decode_bf16 wrong: {list(got)}")


# ---------------------------------------------------------------- pin 1
def pin_worked_example(orc):
    """Hand-worked example with closed-form values (tests/golden/worked_example.txt)."""
    kv = {}
    with open(os.path.join(GOLDEN, "worked_example.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=", 1)
                kv[k.strip()] = [[float(x) for x in part.split()] for part in v.split(";")]
    hidden = torch.tensor(kv["hidden"], dtype=torch.bfloat16)
    weight = torch.tensor(kv["weight"], dtype=torch.bfloat16)
    target = torch.tensor([int(x) for x in kv["target"][0]], dtype=torch.int64)
    logp, lse = orc.linear_logp(hidden, weight, target)
    mpmath.mp.dps = 50
    for i in range(2):
        off, exps, poff = kv[f"row{i}"]
        ln_sum = mpmath.log(mpmath.fsum(mpmath.e ** mpmath.mpf(x) for x in exps))
        _assert(abs(lse[i] - float(off[0] + ln_sum)) <= 1e-14, f"worked lse row {i}: {lse[i]}")
        _assert(abs(logp[i] - float(poff[0] - ln_sum)) <= 1e-14, f"worked logp row {i}: {logp[i]}")


# ---------------------------------------------------------------- pin 2
def pin_brute_force(orc):
    """numpy/dgemm oracle vs pure-Python fsum brute force on tiny inputs."""
    for inp in _tiny_shapes():
        h = inp["hidden"].reshape(-1, inp["hidden"].shape[-1])
        t = inp["target"].reshape(-1)
        lp, ls = orc.linear_logp(h, inp["weight"], t, inp["bias"])
        blp, bls = orc.brute_force_linear_logp(h, inp["weight"], t, inp["bias"])
        _assert(_maxabs(lp, blp) <= 1e-12 and _maxabs(ls, bls) <= 1e-12,
                f"oracle vs brute force: {_maxabs(lp, blp)}, {_maxabs(ls, bls)}")


def pin_brute_force_mpmath(orc):
    """The brute force itself vs mpmath at 40 digits on one tiny case."""
    inp = synth.make_custom(2, 8, 20, seed=21, bias="f32")
    blp, bls = orc.brute_force_linear_logp(inp["hidden"], inp["weight"], inp["target"], inp["bias"])
    mpmath.mp.dps = 40
    h = inp["hidden"].double().tolist()
    w = inp["weight"].double().tolist()
    b = inp["bias"].double().tolist()
    for i in range(2):
        z = [mpmath.fsum([mpmath.mpf(x) * mpmath.mpf(y) for x, y in zip(h[i], w[v])]) + b[v]
             for v in range(20)]
        lse = mpmath.log(mpmath.fsum(mpmath.e ** zz for zz in z))
        t = int(inp["target"][i])
        _assert(abs(bls[i] - float(lse)) <= 1e-13, "brute lse vs mpmath")
        _assert(abs(blp[i] - float(z[t] - lse)) <= 1e-13, "brute logp vs mpmath")


# ---------------------------------------------------------------- pin 3
def pin_log_softmax_library(orc, names=("tiny", "medium")):
    """Against torch.log_softmax in float64 (an independent library routine)."""
    for name in names:
        inp = synth.make_inputs(name)
        h = inp["hidden"].reshape(-1, inp["hidden"].shape[-1])
        t = inp["target"].reshape(-1)
        z = h.double() @ inp["weight"].double().T
        if inp["bias"] is not None:
            z = z + inp["bias"].double()
        ref_lse = torch.logsumexp(z, dim=-1)
        ref_lp = torch.log_softmax(z, dim=-1).gather(1, t[:, None])[:, 0]
        lp, ls = orc.linear_logp(h, inp["weight"], t, inp["bias"])
        _assert(_maxabs(lp, ref_lp.numpy()) <= 1e-12 and _maxabs(ls, ref_lse.numpy()) <= 1e-12,
                f"{name}: oracle vs torch.log_softmax {_maxabs(lp, ref_lp.numpy())}")


# ---------------------------------------------------------------- pin 4
def pin_w0_closed_form(orc, Vs=(1000, 32000, 128256, 151936, 152064)):
    """W = 0, no bias: every logit is 0, so logp = -ln V and lse = ln V."""
    mpmath.mp.dps = 30
    for V in Vs:
        N, H = 3, 8
        h = torch.randn(N, H).to(torch.bfloat16)
        w = torch.zeros(V, H, dtype=torch.bfloat16)
        t = torch.tensor([0, V // 2, V - 1])
        lnv = float(mpmath.log(V))
        for fn in (orc.linear_logp, orc.split_merge_linear_logp):
            lp, ls = fn(h, w, t)
            _assert(np.all(np.abs(lp + lnv) <= 1e-12) and np.all(np.abs(ls - lnv) <= 1e-12),
                    f"W=0 V={V}: {lp} {ls} vs {lnv}")


# ---------------------------------------------------------------- pin 5
def pin_w0_bias(orc):
    """W = 0 with bias b: lse_i = LSE(b) for every row and logp_i = b[t_i] - LSE(b)."""
    mpmath.mp.dps = 30
    for name in ("medium",):
        inp = synth.make_inputs(name, variant="w0")
        h = inp["hidden"][:16]
        t = inp["target"][:16]
        b = inp["bias"].double().tolist()
        lse_b = float(mpmath.log(mpmath.fsum(mpmath.e ** mpmath.mpf(x) for x in b)))
        for fn in (orc.linear_logp, orc.split_merge_linear_logp):
            lp, ls = fn(h, inp["weight"], t, inp["bias"])
            exp_lp = np.array([b[int(x)] for x in t]) - lse_b
            _assert(_maxabs(ls, np.full(16, lse_b)) <= 1e-12, f"w0 bias lse {ls[:3]} vs {lse_b}")
            _assert(_maxabs(lp, exp_lp) <= 1e-12, "w0 bias logp")


# ---------------------------------------------------------------- pin 6
def pin_bias_shift(orc):
    """Adding a constant c to every bias entry moves lse by c and leaves logp."""
    inp = synth.make_custom(6, 32, 700, seed=31, bias="f32")
    b1 = inp["bias"].double()
    b2 = b1 + 1.0                    # exact: an fp32 value plus 1 fits in 53 bits
    for fn in (orc.linear_logp, orc.split_merge_linear_logp):
        lp1, ls1 = fn(inp["hidden"], inp["weight"], inp["target"], b1)
        lp2, ls2 = fn(inp["hidden"], inp["weight"], inp["target"], b2)
        _assert(_maxabs(lp1, lp2) <= 1e-12 and _maxabs(ls1 + 1.0, ls2) <= 1e-12, "bias shift")


# ---------------------------------------------------------------- pin 7
def pin_normalisation(orc):
    """Row 0 of the tiny workload replicated V times with targets 0..V-1:
    sum_v exp(logp_v) = 1, and every copy has the same lse."""
    inp = synth.make_inputs("tiny")
    V = inp["weight"].shape[0]
    h = inp["hidden"][:1].expand(V, -1).contiguous()
    t = torch.arange(V)
    for fn in (orc.linear_logp, orc.split_merge_linear_logp):
        lp, ls = fn(h, inp["weight"], t)
        total = math.fsum(math.exp(x) for x in lp)
        _assert(abs(total - 1.0) <= 1e-12, f"sum exp(logp) = {total}")
        _assert(float(np.ptp(ls)) == 0.0, "lse differs across identical rows")


# ---------------------------------------------------------------- pin 8
def pin_sign_and_argmax(orc):
    """logp <= 0 everywhere; for argmax targets -ln V <= logp <= 0 (brute-force argmax)."""
    inp = synth.make_custom(6, 64, 500, seed=41, hidden_scale=8.0, w_std=0.02)
    h, w = inp["hidden"], inp["weight"]
    z = h.double() @ w.double().T
    t_arg = torch.argmax(z, dim=1)
    V = w.shape[0]
    for fn in (orc.linear_logp, orc.split_merge_linear_logp):
        lp, _ = fn(h, w, inp["target"])
        _assert(np.all(lp <= 0.0), "logp > 0")
        lpa, _ = fn(h, w, t_arg)
        _assert(np.all(lpa <= 0.0) and np.all(lpa >= -math.log(V)), f"argmax bounds {lpa}")
        # row 0 with every target: the largest logp is at the argmax target
        lpx, _ = fn(h[:1].expand(V, -1).contiguous(), w, torch.arange(V))
        _assert(int(np.argmax(lpx)) == int(t_arg[0]), "argmax target is not the max logp")


# ---------------------------------------------------------------- pin 9
def pin_large_logits(orc):
    """Logits near 1000 (exp overflows without the max shift): W = 0 with
    bias 1000 + b must give lse = 1000 + LSE(b) (mpmath) and finite values."""
    mpmath.mp.dps = 30
    rng = np.random.default_rng(5)
    b_small = torch.tensor(rng.standard_normal(300), dtype=torch.float32)
    b = b_small + 1000.0
    h = torch.ones(2, 8, dtype=torch.bfloat16)
    w = torch.zeros(300, 8, dtype=torch.bfloat16)
    t = torch.tensor([3, 299])
    bb = b.double().tolist()
    lse_ref = float(mpmath.log(mpmath.fsum(mpmath.e ** mpmath.mpf(x) for x in bb)))
    for fn in (orc.linear_logp, orc.split_merge_linear_logp):
        lp, ls = fn(h, w, t, b)
        _assert(np.all(np.isfinite(lp)) and np.all(np.isfinite(ls)), "non-finite at large logits")
        _assert(_maxabs(ls, [lse_ref, lse_ref]) <= 1e-10, f"large-logit lse {ls} vs {lse_ref}")
        _assert(_maxabs(lp, [bb[3] - lse_ref, bb[299] - lse_ref]) <= 1e-10, "large-logit logp")


def pin_large_logit_spread(orc):
    """Logits of ~0 in the first vocabulary tile and ~800 in the later ones
    (exp(800) overflows binary64): the combine must shift by the global maximum.
    Reference: mpmath at 30 digits."""
    mpmath.mp.dps = 30
    rng = np.random.default_rng(6)
    V = 600
    b = torch.tensor(rng.standard_normal(V), dtype=torch.float64)
    b[256:] += 800.0
    h = torch.ones(2, 8, dtype=torch.bfloat16)
    w = torch.zeros(V, 8, dtype=torch.bfloat16)
    t = torch.tensor([5, 599])
    bb = b.tolist()
    lse_ref = float(mpmath.log(mpmath.fsum(mpmath.e ** mpmath.mpf(x) for x in bb)))
    for fn in (orc.linear_logp, orc.split_merge_linear_logp):
        lp, ls = fn(h, w, t, b)
        _assert(np.all(np.isfinite(lp)) and np.all(np.isfinite(ls)), "non-finite at logit spread")
        _assert(_maxabs(ls, [lse_ref, lse_ref]) <= 1e-10, f"spread lse {ls} vs {lse_ref}")
        _assert(_maxabs(lp, [bb[5] - lse_ref, bb[599] - lse_ref]) <= 1e-10, "spread logp")


# ---------------------------------------------------------------- pin 10
def pin_split_policy(orc):
    """The V-only split policy: ranges contiguous, non-empty, covering all
    tiles, at most max_splits of them; plus worked values of the formula."""
    for V in list(range(1, 3000, 7)) + [16383, 16384, 16385, 32000, 65536, 128256, 151936,
                                         152064, 256 * 64 * 3 + 1, 10 ** 6, 2 ** 31 - 1]:
        for vt, mx in ((256, 256), (256, 64), (128, 8), (64, 1)):
            r = orc.vocab_splits(V, vt, mx)
            tiles = -(-V // vt)
            _assert(r[0][0] == 0 and r[-1][1] == tiles, f"cover V={V}")
            _assert(all(a < b for a, b in r), f"empty split V={V}")
            _assert(all(r[i][1] == r[i + 1][0] for i in range(len(r) - 1)), f"gap V={V}")
            _assert(len(r) <= mx, f"too many splits V={V}")
            sizes = [b - a for a, b in r]
            _assert(all(s == sizes[0] for s in sizes[:-1]) and sizes[-1] <= sizes[0],
                    f"uneven split V={V}")
    # worked, at most 256 splits: V=128256 -> 501 tiles of 256, 2 per split,
    # 251 splits (the last has one tile)
    r = orc.vocab_splits(128256, 256, 256)
    _assert(len(r) == 251 and r[0] == (0, 2) and r[-1] == (500, 501), "V=128256 splits, 256")
    r = orc.vocab_splits(152064, 256, 256)     # 594 tiles -> 3 per split -> 198 splits
    _assert(len(r) == 198 and r[1] == (3, 6) and r[-1] == (591, 594), "V=152064 splits, 256")
    r = orc.vocab_splits(256 * 256, 256, 256)  # 256 tiles -> 256 splits of one tile
    _assert(len(r) == 256 and r[-1] == (255, 256), "V=65536 splits, 256")
    r = orc.vocab_splits(256 * 256 + 1, 256, 256)  # 257 tiles -> 2 per split -> 129
    _assert(len(r) == 129 and r[-1] == (256, 257), "V=65537 splits, 256")
    r = orc.vocab_splits(32000, 256, 256)      # 125 tiles -> 125 splits of one tile
    _assert(len(r) == 125 and r[-1] == (124, 125), "V=32000 splits, 256")
    # worked, at most 64 splits: V=128256 -> 8 per split, 63 splits (last has 5)
    r = orc.vocab_splits(128256, 256, 64)
    _assert(len(r) == 63 and r[0] == (0, 8) and r[-1] == (496, 501), "V=128256 splits")
    r = orc.vocab_splits(151936, 256, 64)      # 594 tiles -> 10 per split -> 60 splits
    _assert(len(r) == 60 and r[-1] == (590, 594), "V=151936 splits")
    r = orc.vocab_splits(1000, 256, 64)        # 4 tiles -> 4 splits of one tile
    _assert(r == [(0, 1), (1, 2), (2, 3), (3, 4)], "V=1000 splits")
    r = orc.vocab_splits(256 * 65, 256, 64)    # 65 tiles -> 2 per split -> 33 splits
    _assert(len(r) == 33 and r[-1] == (64, 65), "V=16640 splits")
    r = orc.vocab_splits(256 * 64, 256, 64)    # 64 tiles -> 64 splits of one tile
    _assert(len(r) == 64 and r[-1] == (63, 64), "V=16384 splits")
    r = orc.vocab_splits(256 * 64 + 1, 256, 64)  # 65 tiles (one column in the last)
    _assert(len(r) == 33 and r[-1] == (64, 65), "V=16385 splits")


def pin_throughput_policy(orc):
    """The N / V / compute-unit split policy: ranges contiguous, non-empty,
    covering all tiles, even-sized, at most min(tiles, 1024) of them, and at
    least half the count that would fill the compute units (per_split =
    ceil(T / want) gives S >= want / 2 whenever T >= want); plus worked values."""
    for N in (1, 8, 255, 256, 257, 512, 4096, 16384, 100000):
        for V in (1, 255, 1000, 32000, 128256, 151936):
            for cu in (1, 3, 80, 256, 304, 5000):
                r = orc.vocab_splits_throughput(N, V, cu)
                tiles, R = -(-V // 256), -(-N // 256)
                _assert(r[0][0] == 0 and r[-1][1] == tiles, f"cover N={N} V={V} cu={cu}")
                _assert(all(a < b for a, b in r), f"empty split N={N} V={V} cu={cu}")
                _assert(all(r[i][1] == r[i + 1][0] for i in range(len(r) - 1)), "gap")
                sizes = [b - a for a, b in r]
                _assert(all(x == sizes[0] for x in sizes[:-1]) and sizes[-1] <= sizes[0], "uneven")
                want = min(-(-cu // R), tiles, 1024)
                _assert(want / 2 <= len(r) <= want, f"count N={N} V={V} cu={cu}: {len(r)} vs {want}")
    # worked values (T = ceil(V / 256), R = ceil(N / 256), want = min(ceil(cu / R), T, 1024))
    r = orc.vocab_splits_throughput(4096, 128256, 256)      # R 16, want 16, 32 per split
    _assert(len(r) == 16 and r[0] == (0, 32) and r[-1] == (480, 501), "N=4096 V=128256")
    r = orc.vocab_splits_throughput(512, 128256, 256)       # R 2, want 128, 4 per split
    _assert(len(r) == 126 and r[-1] == (500, 501), "N=512 V=128256")
    r = orc.vocab_splits_throughput(8, 128256, 256)         # R 1, want 256, 2 per split
    _assert(len(r) == 251 and r[-1] == (500, 501), "N=8 V=128256")
    r = orc.vocab_splits_throughput(8, 1000, 256)           # want capped by the 4 tiles
    _assert(r == [(0, 1), (1, 2), (2, 3), (3, 4)], "N=8 V=1000")
    r = orc.vocab_splits_throughput(16384, 152064, 256)     # R 64, want 4, 149 per split
    _assert(len(r) == 4 and r[-1] == (447, 594), "N=16384 V=152064")
    r = orc.vocab_splits_throughput(16384, 152064, 304)     # R 64, want ceil(4.75) = 5
    _assert(len(r) == 5 and r[0] == (0, 119) and r[-1] == (476, 594), "N=16384 cu=304")
    r = orc.vocab_splits_throughput(1, 2 ** 30, 5000)       # want capped at 1024
    _assert(len(r) == 1024 and r[0] == (0, 4096), "cap 1024")


# ---------------------------------------------------------------- pin 11
def pin_split_merge_equals_plain(orc):
    """The method's split / online / ascending-combine steps equal the plain
    definition (they are equal in real arithmetic) across tails and split counts."""
    cases = [(4, 16, 1000, 256, 64), (3, 32, 2000, 256, 64), (5, 16, 1031, 64, 4),
             (2, 24, 16641, 256, 64), (3, 8, 1, 256, 64), (2, 8, 257, 256, 64),
             (3, 16, 5000, 128, 3), (3, 16, 70001, 256, 256)]
    for j, (N, H, V, vt, mx) in enumerate(cases):
        inp = synth.make_custom(N, H, V, seed=50 + j, bias="f32" if j % 2 else None)
        lp1, ls1 = orc.linear_logp(inp["hidden"], inp["weight"], inp["target"], inp["bias"])
        lp2, ls2 = orc.split_merge_linear_logp(inp["hidden"], inp["weight"], inp["target"],
                                               inp["bias"], vtile=vt, max_splits=mx)
        _assert(_maxabs(lp1, lp2) <= 1e-12 and _maxabs(ls1, ls2) <= 1e-12,
                f"split-merge vs plain case {j}: {_maxabs(lp1, lp2)} {_maxabs(ls1, ls2)}")
    # the same steps over throughput-mode partitions (more, smaller splits)
    for j, (N, H, V, cu) in enumerate([(3, 16, 5000, 64), (2, 8, 70001, 256), (5, 16, 1000, 3)]):
        inp = synth.make_custom(N, H, V, seed=70 + j, bias="bf16" if j % 2 else None)
        lp1, ls1 = orc.linear_logp(inp["hidden"], inp["weight"], inp["target"], inp["bias"])
        lp2, ls2 = orc.split_merge_linear_logp(inp["hidden"], inp["weight"], inp["target"],
                                               inp["bias"],
                                               splits=orc.vocab_splits_throughput(N, V, cu))
        _assert(_maxabs(lp1, lp2) <= 1e-12 and _maxabs(ls1, ls2) <= 1e-12,
                f"throughput split-merge vs plain case {j}")


# ---------------------------------------------------------------- pin 12
def pin_row_subset(orc):
    """``rows=`` gives the same values as the full computation, in the listed order."""
    inp = synth.make_custom(40, 16, 300, seed=61, bias="bf16")
    rows = [39, 0, 17, 17, 5]
    lp, ls = orc.linear_logp(inp["hidden"], inp["weight"], inp["target"], inp["bias"], row_chunk=7)
    lp2, ls2 = orc.linear_logp(inp["hidden"], inp["weight"], inp["target"], inp["bias"], rows=rows)
    lp3, ls3 = orc.split_merge_linear_logp(inp["hidden"], inp["weight"], inp["target"],
                                           inp["bias"], rows=rows)
    _assert(_maxabs(lp[rows], lp2) == 0.0 and _maxabs(ls[rows], ls2) == 0.0, "row subset")
    _assert(_maxabs(lp2, lp3) <= 1e-12 and _maxabs(ls2, ls3) <= 1e-12, "row subset split-merge")


ALL_PINS = [pin_decode, pin_worked_example, pin_brute_force, pin_brute_force_mpmath,
            pin_log_softmax_library, pin_w0_closed_form, pin_w0_bias, pin_bias_shift,
            pin_normalisation, pin_sign_and_argmax, pin_large_logits, pin_large_logit_spread,
            pin_split_policy, pin_throughput_policy,
            pin_split_merge_equals_plain, pin_row_subset]
