"""One GPU's share of a vocabulary-sharded forward (bilogp_partials_range):
ranks holding contiguous split ranges of the full V, each with only its own
weight and bias columns, write their partials into the workspace, and the
ascending merge then reproduces bilogp_forward_ex bit for bit (RL-Kernel PR
#337, description: split boundaries from V only, ascending combine).  The
exchange between ranks is replaced here by calls on one device into one
workspace."""

import numpy as np
import pytest
import torch

import invariant_linear_log_amd as ila
import synth
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu


def _ranges(S, cuts):
    bounds = [0] + [c for c in cuts if 0 < c < S] + [S]
    return [(a, b) for a, b in zip(bounds[:-1], bounds[1:])]


CASES = [  # N, H, V, bias, seed, cut points (split indices)
    (300, 520, 5003, None, 1, [3, 11]),          # 20 splits of one tile, vocabulary tail
    (257, 264, 70000, "bf16", 2, [1, 27, 54, 100]),   # 137 splits of 2 tiles, last tile partial
    (1, 4096, 16385, "f32", 3, [16, 32]),        # 65 splits, last split one column
    (4096, 4096, 128256, None, 4, [32, 64, 96, 128, 160, 192, 224]),   # 8-way share of the headline
    # on 256 compute units the full forward and both ranges end with a second,
    # 128-token launch (16 x 198, 16 x 100 and 16 x 98 splits); bf16 bias read in place
    (4096, 1024, 151936, "bf16", 5, [100]),
]


@pytest.mark.parametrize("N,H,V,bias,seed,cuts", CASES)
def test_ranges_compose_to_the_full_forward(N, H, V, bias, seed, cuts):
    inp = synth.make_custom(N, H, V, seed, bias=bias, device=DEV)
    h, w, t, b = inp["hidden"], inp["weight"], inp["target"], inp["bias"]
    S = ila.bilogp_num_vocab_splits(V)
    say(f"vocabulary shards N={N} H={H} V={V} bias={bias} S={S} cuts={cuts}")
    logp = torch.empty(N, device=DEV)
    lse = torch.empty(N, device=DEV)
    ws = ila.workspace_for(N, V, DEV)
    ila.bilogp_forward_ex(h, w, t, b, logp, lse, ws)
    ws2 = ila.workspace_for(N, V, DEV)
    ws2.fill_(0xFF)                                   # NaN everywhere until written
    for (a, e) in reversed(_ranges(S, cuts)):         # any order
        c0, c1 = ila.vocab_split_columns(V, a, e)
        w_slice = w[c0:c1].clone()                    # the rank's own copy
        b_slice = None if b is None else b[c0:c1].clone()
        ila.bilogp_partials_range(h, w_slice, t, b_slice, V, a, e, ws2)
    lp2 = torch.empty(N, device=DEV)
    ls2 = torch.empty(N, device=DEV)
    ila.bilogp_merge(t, ws2, lp2, ls2, V)
    torch.cuda.synchronize()
    assert torch.equal(lp2, logp) and torch.equal(ls2, lse)
    assert torch.equal(ws2[:8 * N * S], ws[:8 * N * S])


def test_a_range_writes_only_its_columns():
    N, H, V = 300, 256, 70000
    inp = synth.make_custom(N, H, V, 5, bias="f32", device=DEV)
    h, w, t, b = inp["hidden"], inp["weight"], inp["target"], inp["bias"]
    S = ila.bilogp_num_vocab_splits(V)
    a, e = 20, 31
    c0, c1 = ila.vocab_split_columns(V, a, e)
    t[:50] = torch.randint(c0, c1, (50,), device=DEV)          # some targets inside the range
    say(f"one vocabulary shard writes only its columns: splits [{a}, {e}) of {S}")
    ws = ila.workspace_for(N, V, DEV)
    ws.fill_(0x5A)
    ila.bilogp_partials_range(h, w[c0:c1].clone(), t, b[c0:c1].clone(), V, a, e, ws)
    torch.cuda.synchronize()
    part_bytes = 8 * N * S
    part = ws[:part_bytes].view(N, S, 8).cpu()
    untouched = torch.full((8,), 0x5A, dtype=torch.uint8)
    outside = torch.cat([part[:, :a], part[:, e:]], dim=1)
    assert bool((outside == untouched).all())
    assert not bool((part[:, a:e] == untouched).all(dim=-1).any())   # every own column written
    tl_off = (part_bytes + 255) // 256 * 256
    tl = ws[tl_off:tl_off + 4 * N].view(torch.float32).cpu()
    tt = t.cpu().numpy()
    inside = (tt >= c0) & (tt < c1)
    raw = ws[tl_off:tl_off + 4 * N].view(N, 4).cpu()
    assert bool((raw[torch.from_numpy(~inside)] == 0x5A).all())
    assert bool(torch.isfinite(tl[torch.from_numpy(inside)]).all())
