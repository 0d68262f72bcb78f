"""Bitwise batch invariance of the HIP path (torch.equal, never allclose):
the full batch equals every concatenation of row-chunked runs; a row's bits do
not depend on its slot, its neighbours, the tensor layout, the stream or the
run.  RL-Kernel PR #337, description (tests paragraph and "What this PR
changes"): same row + same V -> same arithmetic order and bits; the
annotation on the chunk test: full-batch bits equal concatenated chunk bits.
The sweep workload's full batch runs 256-token row blocks and its chunks of up
to 1000 rows 128-token blocks (too few 256-token blocks to fill the device),
so the chunk comparison also holds the two block heights to the same bits.
On 256 compute units the full batch's schedule also has a second launch: 12
whole rounds of 256-token tiles, and the last 6 splits as 128-token pieces.
"""

import pytest
import torch

import invariant_linear_log_amd as ila
import synth
from gpu_common import DEV, flat, run_ex, run_inputs, say

pytestmark = pytest.mark.gpu

_CACHE = {}


def sweep_inputs():
    if "sweep" not in _CACHE:
        inp = synth.make_inputs("sweep", device=DEV)
        logp, lse = run_inputs(inp)
        torch.cuda.synchronize()
        _CACHE["sweep"] = (inp, logp, lse)
    return _CACHE["sweep"]


@pytest.mark.parametrize("chunk", [1, 7, 64, 1000, 4096])
def test_chunked_equals_full(chunk):
    inp, full_lp, full_ls = sweep_inputs()
    h, t = flat(inp)
    N = h.shape[0]
    V = inp["weight"].shape[0]
    if ila.device_cu_count(DEV) == 256:
        sa, st = ila.bilogp_launch_schedule(N, h.shape[1], V, ila.BILOGP_SPLITS_INVARIANT, 256)
        assert st < ila.bilogp_num_vocab_splits(V), "the full batch has no second launch"
    say(f"sweep chunk={chunk}")
    lps, lss = [], []
    for c0 in range(0, N, chunk):
        lp, ls = run_ex(h[c0:c0 + chunk], inp["weight"], t[c0:c0 + chunk], inp["bias"])
        lps.append(lp)
        lss.append(ls)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(lps), full_lp), f"chunk {chunk} changed logp bits"
    assert torch.equal(torch.cat(lss), full_ls), f"chunk {chunk} changed lse bits"


def test_run_to_run():
    inp, full_lp, full_ls = sweep_inputs()
    say("sweep run-to-run x3")
    for _ in range(3):
        lp, ls = run_inputs(inp)
        torch.cuda.synchronize()
        assert torch.equal(lp, full_lp) and torch.equal(ls, full_ls)


def test_side_stream():
    inp, full_lp, full_ls = sweep_inputs()
    s = torch.cuda.Stream()
    say("sweep on a side stream")
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lp, ls = run_inputs(inp, stream=s)
    s.synchronize()
    assert torch.equal(lp, full_lp) and torch.equal(ls, full_ls)


def test_row_position():
    """One row placed at every slot of a 256-row block (and at slot 0 of the
    next block, N = 257) gives the bits it has inside the full batch."""
    inp, full_lp, full_ls = sweep_inputs()
    h, t = flat(inp)
    for r in (0, 1234, 4095):
        hh = h[r:r + 1].expand(257, -1).contiguous()
        tt = t[r:r + 1].expand(257).contiguous()
        say(f"row position r={r}")
        lp, ls = run_ex(hh, inp["weight"], tt, inp["bias"])
        torch.cuda.synchronize()
        assert torch.equal(lp, full_lp[r].expand(257)), f"row {r}: logp depends on slot"
        assert torch.equal(ls, full_ls[r].expand(257)), f"row {r}: lse depends on slot"


def test_neighbours():
    """Replacing every other row by fresh random rows leaves the kept rows' bits."""
    inp, full_lp, full_ls = sweep_inputs()
    h, t = flat(inp)
    g = torch.Generator(device=DEV).manual_seed(1234)
    h2 = torch.randn(h.shape, generator=g, device=DEV).to(torch.bfloat16)
    t2 = torch.randint(0, inp["weight"].shape[0], t.shape, generator=g, device=DEV)
    keep = torch.arange(0, h.shape[0], 3, device=DEV)
    h2[keep] = h[keep]
    t2[keep] = t[keep]
    say("neighbours replaced")
    lp, ls = run_ex(h2, inp["weight"], t2, inp["bias"])
    torch.cuda.synchronize()
    assert torch.equal(lp[keep], full_lp[keep]) and torch.equal(ls[keep], full_ls[keep])


def test_layouts():
    """[8, 512, H] input vs its [4096, H] reshape vs a strided view made
    contiguous by the wrapper: identical bits (headline workload)."""
    inp = synth.make_inputs("headline", device=DEV)
    h3, w, t2 = inp["hidden"], inp["weight"], inp["target"]
    say("layouts headline")
    lp3, ls3 = ila.forward(h3, w, t2, check_targets=False)
    lp2, ls2 = run_ex(h3.reshape(-1, h3.shape[-1]), w, t2.reshape(-1))
    wide = torch.zeros(h3.shape[0], h3.shape[1], h3.shape[2] + 64, dtype=torch.bfloat16,
                       device=DEV)
    wide[..., 32:32 + h3.shape[2]] = h3
    view = wide[..., 32:32 + h3.shape[2]]
    assert not view.is_contiguous()
    lpv, lsv = ila.forward(view, w, t2.expand(8, 512), check_targets=False)
    # a zero-stride (expanded) target is accepted
    t_exp = t2[:, :1].expand(8, 512)
    lpe, _ = ila.forward(h3, w, t_exp, check_targets=False)
    lpe2, _ = run_ex(h3.reshape(-1, h3.shape[-1]), w, t_exp.reshape(-1).contiguous())
    torch.cuda.synchronize()
    assert lp3.shape == (8, 512)
    assert torch.equal(lp3.reshape(-1), lp2) and torch.equal(ls3.reshape(-1), ls2)
    assert torch.equal(lpv, lp3) and torch.equal(lsv, ls3)
    assert torch.equal(lpe.reshape(-1), lpe2)


_HEAD = {}


def headline_full():
    if "headline" not in _HEAD:
        inp = synth.make_inputs("headline", device=DEV)
        logp, lse = run_inputs(inp)
        torch.cuda.synchronize()
        _HEAD["headline"] = (inp, logp.reshape(-1), lse.reshape(-1))
    return _HEAD["headline"]


@pytest.mark.parametrize("rows", [768, 1280, 1792])
def test_odd_row_block_counts_keep_the_bits(rows):
    """V = 128256 (2 tiles per split).  The full 4096-row batch launches 16 row
    blocks with runs of 2 splits; the first `rows` rows alone make an odd number
    of 256-token blocks (3, 5, 7), for which whole rounds of the grid call for
    runs of 1 split; 256-row chunks run 128-token blocks with three LDS
    buffers.  Every one of them gives the full batch's bits."""
    inp, full_lp, full_ls = headline_full()
    h, t = flat(inp)
    say(f"headline first {rows} rows: alone and in 256-row chunks vs the full batch")
    lp, ls = run_ex(h[:rows], inp["weight"], t[:rows], inp["bias"])
    lps, lss = [], []
    for c0 in range(0, rows, 256):
        a, b = run_ex(h[c0:c0 + 256], inp["weight"], t[c0:c0 + 256], inp["bias"])
        lps.append(a)
        lss.append(b)
    torch.cuda.synchronize()
    assert torch.equal(lp, full_lp[:rows]) and torch.equal(ls, full_ls[:rows])
    assert torch.equal(torch.cat(lps), full_lp[:rows])
    assert torch.equal(torch.cat(lss), full_ls[:rows])


CU_COUNTS = [1, 8, 32, 80, 128, 256, 304, 1024, 4096, 65536]


@pytest.mark.parametrize("n", [1, 7, 300, 4096])
def test_compute_unit_count_never_changes_bits(n):
    """The bits never depend on the number of compute units (RL-Kernel PR
    #337, description, "Why this happens": the SM count is the input that
    made the scheduler it replaces change a row's reduction).  The launch is
    scheduled for each count in turn - row-block height and splits per
    workgroup differ (checked on the host plan) - on the sweep workload (bf16
    bias, 128-column vocabulary tail), and every result equals
    bilogp_forward_ex's bit for bit."""
    inp, full_lp, full_ls = sweep_inputs()
    h, t = flat(inp)
    h, t = h[:n].contiguous(), t[:n].contiguous()
    w, b = inp["weight"], inp["bias"]
    V = w.shape[0]
    ref_lp, ref_ls = run_ex(h, w, t, b)
    plans = set()
    for cu in CU_COUNTS:
        plans.add(ila.bilogp_launch_plan(n, h.shape[1], V, ila.BILOGP_SPLITS_INVARIANT, cu))
        say(f"sweep n={n} cu_count={cu}")
        lp = torch.empty(n, device=DEV)
        ls = torch.empty(n, device=DEV)
        ws = ila.workspace_for(n, V, DEV)
        ila.bilogp_forward_mode(h, w, t, b, lp, ls, ila.BILOGP_SPLITS_INVARIANT, cu, ws)
        torch.cuda.synchronize()
        assert torch.equal(lp, ref_lp) and torch.equal(ls, ref_ls), f"bits differ at cu={cu}"
        assert torch.equal(lp, full_lp[:n]) and torch.equal(ls, full_ls[:n])
    assert len(plans) >= 2, f"the counts gave one plan only: {plans}"
