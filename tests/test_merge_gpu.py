"""The split merge on hand-made partials (bilogp_merge through the C ABI).

RL-Kernel PR #337, description ("What this PR changes"): the per-split
online-softmax partials are combined in ascending split order.  The library
reads that as one pairwise tree over ascending split index, the same tree for
every row and every N.  With every running max at 0 each term is its sum s_k
exactly, so the tree's fp32 sum can be written out on the host: these tests
check the merge against that tree, show that a left-to-right fold would
give a different answer on the same partials, and check general partials
against a float64 log-sum-exp."""

import numpy as np
import pytest
import torch

import invariant_linear_log_amd as ila
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu

# vocabulary sizes giving 20, 65, 137 and 251 splits (one, two, three and four
# splits per lane of the merge's wave)
VOCABS = (5003, 16385, 70000, 128256)


def _pairwise_f32(terms, leaves):
    """fp32 pairwise tree over ascending index, zero-padded to `leaves`."""
    t = np.zeros(leaves, dtype=np.float32)
    t[:len(terms)] = terms
    while len(t) > 1:
        t = (t[0::2] + t[1::2]).astype(np.float32)
    return float(t[0])


def _fold_f32(terms):
    acc = np.float32(0)
    for x in terms:
        acc = np.float32(acc + np.float32(x))
    return float(acc)


def _run_merge(m, s, V):
    N, S = m.shape
    ws = ila.workspace_for(N, V, DEV)
    ws.zero_()
    part = ws[:N * S * 8].view(torch.float32).view(N, S, 2)
    part[:, :, 0] = torch.from_numpy(m).to(DEV)
    part[:, :, 1] = torch.from_numpy(s).to(DEV)
    off = (N * S * 8 + 255) // 256 * 256
    ws[off:off + 4 * N].view(torch.float32).zero_()      # target logits 0
    target = torch.zeros(N, dtype=torch.int64, device=DEV)
    logp = torch.empty(N, device=DEV)
    lse = torch.empty(N, device=DEV)
    ila.bilogp_merge(target, ws, logp, lse, V)
    torch.cuda.synchronize()
    return logp.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("V", VOCABS)
def test_merge_is_one_pairwise_tree(V):
    S = ila.bilogp_num_vocab_splits(V)
    leaves = 64
    while leaves < S:
        leaves *= 2
    rng = np.random.default_rng(S)
    rows = [
        np.r_[2.0 ** 24, np.ones(S - 1)],                   # a fold loses every 1
        np.r_[np.ones(S - 1), 2.0 ** 24],
        rng.uniform(1.0, 2.0, S),
        2.0 ** rng.uniform(-10, 24, S),
    ]
    s = np.stack(rows).astype(np.float32)
    m = np.zeros_like(s)
    say(f"merge tree V={V} S={S} leaves={leaves}")
    logp, lse = _run_merge(m, s, V)
    tol = 5e-6      # hardware log2 (about 1 ulp at <= 40) times ln 2, then one rounding
    for i, terms in enumerate(s):
        want = np.log(_pairwise_f32(terms, leaves))
        assert abs(lse[i] - want) <= tol, (i, lse[i], want)
        assert logp[i] == -lse[i]
    # with 251 splits the first row separates the tree from a left-to-right
    # fold: the fold drops all 250 ones (1.5e-5 in lse), the tree two of them
    if S > 200:
        fold = np.log(_fold_f32(s[0]))
        assert abs(fold - np.log(_pairwise_f32(s[0], leaves))) > 2 * tol
        assert abs(lse[0] - fold) > tol


@pytest.mark.parametrize("V", VOCABS)
def test_merge_matches_float64(V):
    S = ila.bilogp_num_vocab_splits(V)
    rng = np.random.default_rng(1000 + S)
    N = 37
    m = rng.uniform(-30.0, 30.0, (N, S)).astype(np.float32)
    s = rng.uniform(1.0, 300.0, (N, S)).astype(np.float32)
    m[3, :] = -np.inf                                   # a split with no columns cannot occur,
    s[3, :] = 0.0                                       # but one finite split must carry the row
    m[3, S // 2], s[3, S // 2] = 4.0, 1.0
    say(f"merge vs float64 V={V} S={S}")
    logp, lse = _run_merge(m, s, V)
    m64, s64 = m.astype(np.float64), s.astype(np.float64)
    M = m64.max(axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):
        terms = np.where(s64 > 0, s64 * np.exp(m64 - M), 0.0)
    want = M[:, 0] + np.log(terms.sum(axis=1))
    err = np.abs(lse - want) / np.maximum(1.0, np.abs(want))
    assert float(err.max()) <= 2e-5, (int(err.argmax()), float(err.max()))
    np.testing.assert_array_equal(logp, -lse)
    assert lse[3] == pytest.approx(4.0, abs=1e-6)
