"""The no-allocation forward (bilogp_forward_noalloc) against bilogp_forward_ex.

Same kernels and arguments, so the bar is bit equality: two calls in a row on
the shared per-GPU scratch array, the second smaller (its results must not
depend on what the first left there), plus the size limit, which is checked
before any device work."""

import pytest
import torch

import invariant_linear_log_amd as ila
from invariant_linear_log_amd import _binding as B

DEV = torch.device("cuda:0")


def _inputs(N, H, V, seed, bias_dtype):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(N, H, generator=g).to(torch.bfloat16)
    w = (torch.randn(V, H, generator=g) / H ** 0.5).to(torch.bfloat16)
    t = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
    t[0], t[-1] = 0, V - 1
    b = None if bias_dtype is None else (torch.randn(V, generator=g) * 0.1).to(bias_dtype)
    return [x if x is None else x.to(DEV) for x in (h, w, t, b)]


def _reference(h, w, t, b):
    N, V = h.shape[0], w.shape[0]
    lp = torch.empty(N, device=DEV)
    ls = torch.empty(N, device=DEV)
    ila.bilogp_forward_ex(h, w, t, b, lp, ls, ila.workspace_for(N, V, DEV))
    return lp, ls


def _noalloc_raw(h, w, t, b):
    """Through the C ABI directly (pointers, sizes, the current stream)."""
    N, H = h.shape
    V = w.shape[0]
    lp = torch.full((N,), float("nan"), device=DEV)
    ls = torch.full((N,), float("nan"), device=DEV)
    lib = ila.load_library()
    bd = B.BILOGP_BIAS_NONE if b is None else (
        B.BILOGP_BIAS_BF16 if b.dtype == torch.bfloat16 else B.BILOGP_BIAS_F32)
    st = lib.bilogp_forward_noalloc(h.data_ptr(), w.data_ptr(), t.data_ptr(),
                                    None if b is None else b.data_ptr(), bd, lp.data_ptr(),
                                    ls.data_ptr(), N, H, V,
                                    torch.cuda.current_stream(DEV).cuda_stream)
    assert st == B.BILOGP_OK, ila.bilogp_last_error()
    return lp, ls


@pytest.mark.gpu
def test_noalloc_matches_forward_ex_on_consecutive_calls():
    # first call: 4096 rows x V = 32000 (2 MB of scratch), fp32 bias
    a = _inputs(4096, 1024, 32000, 31, torch.float32)
    lp1, ls1 = _noalloc_raw(*a)
    # second call, smaller: 300 rows x a ragged V = 50003 with bf16 bias; the
    # scratch still holds the first call's partials
    b = _inputs(300, 512, 50003, 32, torch.bfloat16)
    lp2, ls2 = _noalloc_raw(*b)
    torch.cuda.synchronize()
    r1 = _reference(*a)
    r2 = _reference(*b)
    torch.cuda.synchronize()
    assert torch.equal(lp1, r1[0]) and torch.equal(ls1, r1[1])
    assert torch.equal(lp2, r2[0]) and torch.equal(ls2, r2[1])
    # and once more through the Python wrapper, no bias
    c = _inputs(64, 256, 1000, 33, None)
    lp3 = torch.empty(64, device=DEV)
    ls3 = torch.empty(64, device=DEV)
    ila.bilogp_forward_noalloc(*c, lp3, ls3)
    r3 = _reference(*c)
    torch.cuda.synchronize()
    assert torch.equal(lp3, r3[0]) and torch.equal(ls3, r3[1])


@pytest.mark.gpu
def test_noalloc_empty_batch_is_a_noop():
    h, w, t, _ = _inputs(1, 64, 1000, 34, None)
    lib = ila.load_library()
    st = lib.bilogp_forward_noalloc(h.data_ptr(), w.data_ptr(), t.data_ptr(), None, 0,
                                    h.data_ptr(), h.data_ptr(), 0, 64, 1000, None)
    assert st == B.BILOGP_OK


def test_noalloc_rejects_sizes_beyond_its_array():
    lib = ila.load_library()
    cap = lib.bilogp_noalloc_max_workspace_bytes()
    assert cap == 64 << 20
    V = 128256
    N = 1
    while ila.bilogp_workspace_bytes(N, V) <= cap:
        N *= 2
    fake = 0x10000
    st = lib.bilogp_forward_noalloc(fake, fake + 0x100000, fake + 0x200000, None, 0,
                                    fake + 0x300000, fake + 0x400000, N, 4096, V, None)
    assert st == B.BILOGP_E_WORKSPACE
    assert "at most" in ila.bilogp_last_error()
