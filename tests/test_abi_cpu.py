"""CPU checks of the C ABI (no kernel launches): the library loads, exports
every function include/bilogp.h declares, its V-only split policy agrees with
the oracle's independent reading of the page, and every fail-closed argument
check fires before any device work."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import invariant_linear_log_amd as ila
import oracle
from invariant_linear_log_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bilogp.h")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bilogp_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ila.load_library()
    names = _header_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), f"{name} declared in bilogp.h but not exported"
        assert name in B.SIGNATURES, f"{name} has no binding signature"
    assert set(B.SIGNATURES) == set(names)


def test_constants_and_version():
    # ABI 2 added bilogp_bit_contract_version and the scheduling compute-unit
    # count of the invariant mode; ABI 3 added H to bilogp_launch_plan; ABI 4
    # added bilogp_launch_schedule.  Bit contract 2: tiles of 256 columns, at
    # most 256 splits, the merge tree over consecutive per-lane split blocks
    # (contract 1 had at most 64 splits and lane-strided pre-sums).  Bit
    # contract 3: K in 32-wide steps of the 16 x 16 x 32 bf16 MFMA, per-token
    # sums over (lane group, register) of that tile layout.  Bit contract 4:
    # the deterministic GEMM and the backward's products on that MFMA too.
    assert ila.bilogp_abi_version() == 4
    assert ila.bilogp_bit_contract_version() == 4
    assert ila.bilogp_vtile_cols() == 256
    assert ila.bilogp_max_splits() == 256
    for s in range(5):
        assert ila.bilogp_status_string(s) != "unknown status"
    assert ila.bilogp_status_string(99) == "unknown status"


def _policy_values():
    vs = list(range(1, 5000, 13)) + [16383, 16384, 16385, 32000, 65536, 128256, 151936, 152064,
                                      256 * 64 * 7 + 1, 256 * 256, 256 * 256 + 1, 256 * 512 + 1,
                                      10 ** 6, 2 ** 30]
    return vs


def test_split_policy_matches_oracle():
    vt, mx = ila.bilogp_vtile_cols(), ila.bilogp_max_splits()
    for V in _policy_values():
        ranges = oracle.vocab_splits(V, vt, mx)
        assert ila.bilogp_num_vocab_splits(V) == len(ranges), V
        assert ila.bilogp_vtiles_per_split(V) == ranges[0][1] - ranges[0][0], V


def test_throughput_policy_matches_oracle():
    inv, tp = B.BILOGP_SPLITS_INVARIANT, B.BILOGP_SPLITS_THROUGHPUT
    for N in (1, 8, 255, 256, 257, 512, 1000, 4096, 16384, 2 ** 20):
        for V in (1, 255, 1000, 5003, 32000, 70001, 128256, 151936, 2 ** 30):
            for cu in (1, 3, 80, 256, 304, 5000):
                ranges = oracle.vocab_splits_throughput(N, V, cu, vtile=256, block_rows=256,
                                                        max_splits=B.BILOGP_MAX_THROUGHPUT_SPLITS)
                assert ila.bilogp_num_vocab_splits_mode(N, V, tp, cu) == len(ranges), (N, V, cu)
                assert ila.bilogp_vtiles_per_split_mode(N, V, tp, cu) == \
                    ranges[0][1] - ranges[0][0], (N, V, cu)
            # the invariant mode ignores N and the compute units
            assert ila.bilogp_num_vocab_splits_mode(N, V, inv, 7) == ila.bilogp_num_vocab_splits(V)
            assert ila.bilogp_vtiles_per_split_mode(N, V, inv, 0) == ila.bilogp_vtiles_per_split(V)


def test_throughput_policy_invalid():
    tp = B.BILOGP_SPLITS_THROUGHPUT
    for N, V, mode, cu in [(0, 1000, tp, 256), (-1, 1000, tp, 256), (8, 0, tp, 256),
                           (8, 1000, tp, 0), (8, 1000, 2, 256), (8, 1000, -1, 256),
                           (8, 2 ** 30 + 1, tp, 256)]:
        assert ila.bilogp_num_vocab_splits_mode(N, V, mode, cu) == 0, (N, V, mode, cu)
        assert ila.bilogp_vtiles_per_split_mode(N, V, mode, cu) == 0, (N, V, mode, cu)


def test_workspace_bytes_mode():
    def up(x):
        return (x + 255) // 256 * 256
    tp = B.BILOGP_SPLITS_THROUGHPUT
    for N, V, cu in [(1, 1000, 256), (8, 128256, 256), (512, 128256, 256), (4096, 128256, 80)]:
        S = len(oracle.vocab_splits_throughput(N, V, cu))
        padded = (V + 255) // 256 * 256
        assert ila.bilogp_workspace_bytes_mode(N, V, tp, cu) == up(8 * N * S) + up(4 * N) + \
            up(4 * padded)
        assert ila.bilogp_workspace_bytes_mode(N, V, B.BILOGP_SPLITS_INVARIANT, cu) == \
            ila.bilogp_workspace_bytes(N, V)
    big = (1 << 64) - 1
    assert ila.bilogp_workspace_bytes_mode(0, 1000, tp, 256) == 0
    assert ila.bilogp_workspace_bytes_mode(8, 1000, tp, 0) == big
    assert ila.bilogp_workspace_bytes_mode(8, 1000, 5, 256) == big


def test_split_policy_out_of_range():
    for V in (0, -1, 2 ** 30 + 1, 2 ** 40):
        assert ila.bilogp_num_vocab_splits(V) == 0
        assert ila.bilogp_vtiles_per_split(V) == 0


def test_workspace_bytes():
    def up(x):
        return (x + 255) // 256 * 256
    for N, V in [(1, 1000), (8, 1000), (4096, 128256), (4097, 151936), (16384, 152064)]:
        S = ila.bilogp_num_vocab_splits(V)
        padded = (V + 255) // 256 * 256
        assert ila.bilogp_workspace_bytes(N, V) == up(8 * N * S) + up(4 * N) + up(4 * padded)
    assert ila.bilogp_workspace_bytes(0, 1000) == 0
    big = (1 << 64) - 1
    assert ila.bilogp_workspace_bytes(-1, 1000) == big
    assert ila.bilogp_workspace_bytes(8, 0) == big


# ------------------------------------------------------------- fail-closed checks
FAKE = 0x10000          # aligned, never dereferenced: the checks below fail first


def _call_ex(hidden=FAKE, weight=FAKE + 0x100000, target=FAKE + 0x200000, bias=None,
             bias_dtype=0, logp=FAKE + 0x300000, lse=FAKE + 0x400000, N=8, H=64, V=1000,
             ws=FAKE + 0x500000, ws_bytes=1 << 20):
    lib = ila.load_library()
    return lib.bilogp_forward_ex(hidden, weight, target, bias, bias_dtype, logp, lse, N, H, V,
                                 ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=None), B.BILOGP_E_INVALID_ARG),
    (dict(weight=None), B.BILOGP_E_INVALID_ARG),
    (dict(target=None), B.BILOGP_E_INVALID_ARG),
    (dict(logp=None), B.BILOGP_E_INVALID_ARG),
    (dict(lse=None), B.BILOGP_E_INVALID_ARG),
    (dict(N=-1), B.BILOGP_E_INVALID_ARG),
    (dict(H=0), B.BILOGP_E_INVALID_ARG),
    (dict(H=(1 << 20) + 8), B.BILOGP_E_INVALID_ARG),
    (dict(V=0), B.BILOGP_E_INVALID_ARG),
    (dict(V=(1 << 30) + 1), B.BILOGP_E_INVALID_ARG),
    (dict(bias_dtype=7, bias=FAKE + 0x600000), B.BILOGP_E_UNSUPPORTED),
    (dict(bias_dtype=2), B.BILOGP_E_INVALID_ARG),            # dtype without pointer
    (dict(bias=FAKE + 0x600000), B.BILOGP_E_INVALID_ARG),    # pointer without dtype
    (dict(H=60), B.BILOGP_E_UNSUPPORTED),                     # H % 8 != 0
    (dict(hidden=FAKE + 8), B.BILOGP_E_UNSUPPORTED),          # misaligned
    (dict(weight=FAKE + 0x100004), B.BILOGP_E_UNSUPPORTED),
    (dict(target=FAKE + 0x200004), B.BILOGP_E_UNSUPPORTED),
    (dict(bias_dtype=2, bias=FAKE + 0x600002), B.BILOGP_E_UNSUPPORTED),
    (dict(logp=FAKE + 0x300002), B.BILOGP_E_UNSUPPORTED),
    (dict(lse=FAKE + 0x300000), B.BILOGP_E_INVALID_ARG),      # outputs alias
    (dict(lse=FAKE + 0x300010), B.BILOGP_E_INVALID_ARG),      # outputs overlap
    (dict(logp=FAKE), B.BILOGP_E_INVALID_ARG),                # output aliases hidden
    (dict(logp=FAKE + 0x200000), B.BILOGP_E_INVALID_ARG),     # output aliases target
    (dict(logp=FAKE + 0x500000), B.BILOGP_E_INVALID_ARG),     # output aliases workspace
    (dict(ws=None), B.BILOGP_E_WORKSPACE),
    (dict(ws_bytes=100), B.BILOGP_E_WORKSPACE),
    (dict(ws=FAKE + 0x500010), B.BILOGP_E_WORKSPACE),         # misaligned workspace
    (dict(ws=FAKE), B.BILOGP_E_INVALID_ARG),                  # workspace over hidden
    (dict(ws=FAKE + 0x100000), B.BILOGP_E_INVALID_ARG),       # workspace over weight
    (dict(ws=FAKE + 0x1fff00), B.BILOGP_E_INVALID_ARG),       # workspace over target
    (dict(bias_dtype=2, bias=FAKE + 0x600000, ws=FAKE + 0x5fff00,
          ws_bytes=0x2000), B.BILOGP_E_INVALID_ARG),          # workspace over bias
])
def test_forward_ex_fails_closed(kw, status):
    st = _call_ex(**kw)
    assert st == status, (st, ila.bilogp_last_error())
    assert ila.bilogp_last_error() != ""


@pytest.mark.parametrize("mode,cu,status", [
    (2, 256, B.BILOGP_E_INVALID_ARG),           # unknown mode
    (-1, 256, B.BILOGP_E_INVALID_ARG),
    (B.BILOGP_SPLITS_THROUGHPUT, 0, B.BILOGP_E_INVALID_ARG),   # no compute units
    (B.BILOGP_SPLITS_THROUGHPUT, -5, B.BILOGP_E_INVALID_ARG),
])
def test_forward_mode_fails_closed(mode, cu, status):
    lib = ila.load_library()
    st = lib.bilogp_forward_mode(FAKE, FAKE + 0x100000, FAKE + 0x200000, None, 0, FAKE + 0x300000,
                                 FAKE + 0x400000, 8, 64, 1000, mode, cu, FAKE + 0x500000, 1 << 20,
                                 None)
    assert st == status, (st, ila.bilogp_last_error())


@pytest.mark.parametrize("cu", [-1, 65537, 1 << 30])
def test_forward_mode_rejects_bad_compute_unit_counts(cu):
    lib = ila.load_library()
    for mode in (B.BILOGP_SPLITS_INVARIANT, B.BILOGP_SPLITS_THROUGHPUT):
        st = lib.bilogp_forward_mode(FAKE, FAKE + 0x100000, FAKE + 0x200000, None, 0,
                                     FAKE + 0x300000, FAKE + 0x400000, 8, 64, 1000, mode, cu,
                                     FAKE + 0x500000, 1 << 20, None)
        assert st == B.BILOGP_E_INVALID_ARG, (mode, cu, st, ila.bilogp_last_error())


def test_workspace_may_not_alias_inputs_of_either_half():
    lib = ila.load_library()
    # projection only: the workspace written over hidden / target
    st = lib.bilogp_partials(FAKE, FAKE + 0x100000, FAKE + 0x200000, None, 0, 8, 64, 1000,
                             FAKE, 1 << 20, None)
    assert st == B.BILOGP_E_INVALID_ARG, ila.bilogp_last_error()
    st = lib.bilogp_partials_range(FAKE, FAKE + 0x100000, FAKE + 0x200000, None, 0, 8, 64,
                                   128256, 0, 2, FAKE + 0x1fff00, 1 << 20, None)
    assert st == B.BILOGP_E_INVALID_ARG, ila.bilogp_last_error()
    # merge only: the workspace read over the targets
    st = lib.bilogp_merge(FAKE + 0x200000, FAKE + 0x1fff00, 1 << 20, FAKE + 0x300000 + 0x100000,
                          FAKE + 0x400000 + 0x100000, 8, 1000, None)
    assert st == B.BILOGP_E_INVALID_ARG, ila.bilogp_last_error()


def test_forward_mode_workspace_is_per_mode():
    # enough for the invariant mode's 251 splits of V=128256, but the throughput
    # mode at N=8 with 1024 compute units takes 501: the size check uses the
    # mode's own split count
    lib = ila.load_library()
    need_inv = ila.bilogp_workspace_bytes(8, 128256)
    st = lib.bilogp_forward_mode(FAKE, FAKE + 0x10000000, FAKE + 0x200000, None, 0, FAKE + 0x300000,
                                 FAKE + 0x400000, 8, 64, 128256, B.BILOGP_SPLITS_THROUGHPUT, 1024,
                                 FAKE + 0x40000000, need_inv, None)
    assert st == B.BILOGP_E_WORKSPACE, (st, ila.bilogp_last_error())


def test_empty_batch_is_a_noop():
    assert _call_ex(N=0, ws=None, ws_bytes=0) == B.BILOGP_OK
    lib = ila.load_library()
    assert lib.bilogp_forward(FAKE, FAKE + 0x100000, FAKE + 0x200000, None, FAKE + 0x300000,
                              FAKE + 0x400000, 0, 64, 1000, None) == B.BILOGP_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_no_device_is_unsupported():
    # valid arguments on a host without a gfx950 device: fail closed, no fallback
    assert _call_ex() == B.BILOGP_E_UNSUPPORTED
    assert "device" in ila.bilogp_last_error()


def test_wrapper_rejects_requires_grad():
    h = torch.zeros(4, 64, dtype=torch.bfloat16, requires_grad=True)
    w = torch.zeros(100, 64, dtype=torch.bfloat16)
    t = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(RuntimeError, match="forward-only"):
        ila.forward(h, w, t)
    wb = torch.zeros(100, 64, dtype=torch.bfloat16, requires_grad=True)
    with pytest.raises(RuntimeError, match="forward-only"):
        ila.forward(h.detach(), wb, t)
    b = torch.zeros(100, requires_grad=True)
    with pytest.raises(RuntimeError, match="forward-only"):
        ila.forward(h.detach(), w, t, b)
    # under no_grad the gate lets the call through to the device check
    with torch.no_grad():
        with pytest.raises(ValueError, match="GPU"):
            ila.forward(h, w, t)


@pytest.mark.parametrize("case", ["dtype_h", "dtype_t", "shape_h", "shape_t", "bias_shape",
                                  "bias_dtype", "cpu"])
def test_wrapper_rejects_bad_inputs(case):
    h = torch.zeros(2, 3, 64, dtype=torch.bfloat16)
    w = torch.zeros(100, 64, dtype=torch.bfloat16)
    t = torch.zeros(2, 3, dtype=torch.int64)
    b = None
    exc = ValueError
    if case == "dtype_h":
        h, exc = h.float(), TypeError
    elif case == "dtype_t":
        t, exc = t.int(), TypeError
    elif case == "shape_h":
        h = torch.zeros(2, 3, 32, dtype=torch.bfloat16)
    elif case == "shape_t":
        t = torch.zeros(6, dtype=torch.int64)
    elif case == "bias_shape":
        b = torch.zeros(99)
    elif case == "bias_dtype":
        b, exc = torch.zeros(100, dtype=torch.float64), TypeError
    with pytest.raises(exc):
        ila.forward(h, w, t, b)


def _cpu_forward_args(N=4, H=16, V=40):
    return dict(hidden=torch.zeros(N, H, dtype=torch.bfloat16),
                weight=torch.zeros(V, H, dtype=torch.bfloat16),
                target=torch.zeros(N, dtype=torch.int64), bias=None,
                logp_out=torch.zeros(N), lse_out=torch.zeros(N))


_RAW_CASES = [
    ("hidden_fp32", TypeError), ("target_int32", TypeError), ("bias_bf16_plain", TypeError),
    ("bias_fp64", TypeError), ("hidden_3d", ValueError), ("hidden_noncontig", ValueError),
    ("weight_cols", ValueError), ("target_short", ValueError), ("bias_short", ValueError),
    ("logp_short", ValueError), ("lse_fp64", TypeError), ("cpu", ValueError)]


# a bf16 bias is an error only for bilogp_forward, whose bias is fp32 by signature;
# the calls with an explicit bias dtype accept it
@pytest.mark.parametrize("fn,case,exc", [
    (fn, case, exc)
    for fn in ("bilogp_forward", "bilogp_forward_ex", "bilogp_forward_mode")
    for case, exc in _RAW_CASES if case != "bias_bf16_plain" or fn == "bilogp_forward"])
def test_raw_wrappers_check_what_pointers_stand_for(fn, case, exc):
    """The C-ABI wrappers check dtypes, shapes and layout before the library
    sees bare pointers (a bf16 bias read as fp32, an int32 target or a short
    output would otherwise be read or written out of bounds)."""
    a = _cpu_forward_args()
    if case == "hidden_fp32":
        a["hidden"] = a["hidden"].float()
    elif case == "target_int32":
        a["target"] = a["target"].int()
    elif case == "bias_bf16_plain":
        a["bias"] = torch.zeros(40, dtype=torch.bfloat16)
    elif case == "bias_fp64":
        a["bias"] = torch.zeros(40, dtype=torch.float64)
    elif case == "hidden_3d":
        a["hidden"] = a["hidden"].reshape(2, 2, 16)
    elif case == "hidden_noncontig":
        a["hidden"] = torch.zeros(16, 4, dtype=torch.bfloat16).t()
    elif case == "weight_cols":
        a["weight"] = torch.zeros(40, 24, dtype=torch.bfloat16)
    elif case == "target_short":
        a["target"] = a["target"][:3]
    elif case == "bias_short":
        a["bias"] = torch.zeros(39)
    elif case == "logp_short":
        a["logp_out"] = torch.zeros(3)
    elif case == "lse_fp64":
        a["lse_out"] = a["lse_out"].double()
    args = [a["hidden"], a["weight"], a["target"], a["bias"], a["logp_out"], a["lse_out"]]
    with pytest.raises(exc):
        if fn == "bilogp_forward":
            ila.bilogp_forward(*args)
        elif fn == "bilogp_forward_ex":
            ila.bilogp_forward_ex(*args, torch.zeros(1 << 16, dtype=torch.uint8))
        else:
            ila.bilogp_forward_mode(*args, B.BILOGP_SPLITS_INVARIANT, 0,
                                    torch.zeros(1 << 16, dtype=torch.uint8))


def test_raw_wrappers_partials_range_and_merge_checks():
    a = _cpu_forward_args(V=128256)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    # splits [0, 2) of V = 128256 hold columns [0, 1024): a slice of 1000 rows
    # would be read past its end
    with pytest.raises(ValueError, match="slice"):
        ila.bilogp_partials_range(a["hidden"], torch.zeros(1000, 16, dtype=torch.bfloat16),
                                  a["target"], None, 128256, 0, 2, ws)
    with pytest.raises(ValueError, match="split range"):
        ila.bilogp_partials_range(a["hidden"], torch.zeros(1024, 16, dtype=torch.bfloat16),
                                  a["target"], None, 128256, 3, 2, ws)
    with pytest.raises(ValueError, match="shape"):
        ila.bilogp_partials_range(a["hidden"], torch.zeros(1024, 16, dtype=torch.bfloat16),
                                  a["target"], torch.zeros(1000), 128256, 0, 2, ws)
    with pytest.raises(ValueError, match="GPU"):     # right shapes, but host tensors
        ila.bilogp_partials_range(a["hidden"], torch.zeros(1024, 16, dtype=torch.bfloat16),
                                  a["target"], None, 128256, 0, 2, ws)
    with pytest.raises(TypeError):
        ila.bilogp_merge(a["target"].int(), ws, a["logp_out"], a["lse_out"], 128256)
    with pytest.raises(ValueError):
        ila.bilogp_merge(a["target"], ws, a["logp_out"][:2], a["lse_out"], 128256)
    with pytest.raises(TypeError):
        ila.bilogp_partials(a["hidden"], a["weight"], a["target"], None, ws.numpy())


def test_binding_raises_when_library_missing(tmp_path):
    saved = B._lib
    try:
        B._lib = None
        with pytest.raises(RuntimeError, match="missing"):
            B.load_library(str(tmp_path / "libbilogp.so"))
    finally:
        B._lib = saved


# ------------------------------------------------------------- det_gemm checks
def _gemm(fn="bilogp_det_gemm_fwd", x=FAKE, y=FAKE + 0x1000000, out=FAKE + 0x2000000, M=64,
          N=64, K=64, kind=0):
    return getattr(ila.load_library(), fn)(x, y, out, M, N, K, kind, None)


@pytest.mark.parametrize("fn", ["bilogp_det_gemm_fwd", "bilogp_det_gemm_da",
                                "bilogp_det_gemm_db"])
@pytest.mark.parametrize("kw,status", [
    (dict(x=None), B.BILOGP_E_INVALID_ARG),
    (dict(y=None), B.BILOGP_E_INVALID_ARG),
    (dict(out=None), B.BILOGP_E_INVALID_ARG),
    (dict(M=-1), B.BILOGP_E_INVALID_ARG),
    (dict(N=0), B.BILOGP_E_INVALID_ARG),
    (dict(K=4), B.BILOGP_E_INVALID_ARG),
    (dict(N=(1 << 20) + 8), B.BILOGP_E_INVALID_ARG),
    (dict(kind=3), B.BILOGP_E_INVALID_ARG),
    (dict(N=60), B.BILOGP_E_UNSUPPORTED),          # N % 8 != 0
    (dict(K=68 + 2), B.BILOGP_E_UNSUPPORTED),      # K % 8 != 0
    (dict(x=FAKE + 8), B.BILOGP_E_UNSUPPORTED),    # misaligned
    (dict(out=FAKE + 0x2000004), B.BILOGP_E_UNSUPPORTED),
    (dict(out=FAKE), B.BILOGP_E_INVALID_ARG),      # output aliases an operand
])
def test_det_gemm_fails_closed(fn, kw, status):
    st = _gemm(fn, **kw)
    assert st == status, (fn, kw, st, ila.bilogp_last_error())
    assert ila.bilogp_last_error() != ""


def test_det_gemm_empty_batch():
    # forward and dA with M == 0 write nothing and succeed without a device
    assert _gemm("bilogp_det_gemm_fwd", M=0) == B.BILOGP_OK
    assert _gemm("bilogp_det_gemm_da", M=0) == B.BILOGP_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_det_gemm_no_device_is_unsupported():
    assert _gemm() == B.BILOGP_E_UNSUPPORTED
    # dB with M == 0 still writes its (zero) [N, K] output: it needs the device
    assert _gemm("bilogp_det_gemm_db", M=0) == B.BILOGP_E_UNSUPPORTED


def test_det_gemm_wrappers_reject_bad_inputs():
    a = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        ila.det_gemm(a.float(), a)
    with pytest.raises(ValueError):
        ila.det_gemm(a, torch.zeros(4, 16, dtype=torch.bfloat16))      # K mismatch
    with pytest.raises(ValueError):
        ila.det_gemm(a, a)                                              # not on a GPU
    with pytest.raises(ValueError):
        ila.det_gemm_da(torch.zeros(4, 3, dtype=torch.bfloat16), a)     # N mismatch
    with pytest.raises(ValueError):
        ila.det_gemm_db(a, torch.zeros(5, 8, dtype=torch.bfloat16))     # M mismatch


# ------------------------------------------------------------- backward checks
def test_backward_workspace_bytes():
    def up(x):
        return (x + 255) // 256 * 256
    for N, V in [(1, 1000), (7, 1000), (8, 257), (4096, 128256), (1 << 21, 1000)]:
        ldz = (N + 7) // 8 * 8
        padded = (V + 255) // 256 * 256
        assert ila.bilogp_backward_workspace_bytes(N, V) == up(2 * V * ldz) + up(4 * padded)
    assert ila.bilogp_backward_workspace_bytes(0, 1000) == up(4 * 1024)
    big = (1 << 64) - 1
    assert ila.bilogp_backward_workspace_bytes(-1, 1000) == big
    assert ila.bilogp_backward_workspace_bytes((1 << 21) + 1, 1000) == big
    assert ila.bilogp_backward_workspace_bytes(8, 0) == big
    assert ila.bilogp_backward_workspace_bytes(8, (1 << 30) + 1) == big


def _call_bwd(hidden=FAKE, weight=FAKE + 0x100000, target=FAKE + 0x200000, bias=None,
              bias_dtype=0, lse=FAKE + 0x300000, glogp=FAKE + 0x310000, glse=FAKE + 0x320000,
              gh=FAKE + 0x400000, gw=FAKE + 0x1000000, gb=None, N=8, H=64, V=1000,
              ws=FAKE + 0x2000000, ws_bytes=1 << 20):
    lib = ila.load_library()
    return lib.bilogp_backward(hidden, weight, target, bias, bias_dtype, lse, glogp, glse, gh,
                               gw, gb, N, H, V, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=None), B.BILOGP_E_INVALID_ARG),
    (dict(weight=None), B.BILOGP_E_INVALID_ARG),
    (dict(target=None), B.BILOGP_E_INVALID_ARG),
    (dict(lse=None), B.BILOGP_E_INVALID_ARG),
    (dict(glogp=None), B.BILOGP_E_INVALID_ARG),
    (dict(glse=None), B.BILOGP_E_INVALID_ARG),
    (dict(gh=None), B.BILOGP_E_INVALID_ARG),
    (dict(gw=None), B.BILOGP_E_INVALID_ARG),
    (dict(N=-1), B.BILOGP_E_INVALID_ARG),
    (dict(N=(1 << 21) + 1), B.BILOGP_E_INVALID_ARG),
    (dict(H=0), B.BILOGP_E_INVALID_ARG),
    (dict(V=0), B.BILOGP_E_INVALID_ARG),
    (dict(V=(1 << 30) + 1), B.BILOGP_E_INVALID_ARG),
    (dict(bias_dtype=7, bias=FAKE + 0x600000), B.BILOGP_E_UNSUPPORTED),
    (dict(bias_dtype=2), B.BILOGP_E_INVALID_ARG),
    (dict(bias=FAKE + 0x600000), B.BILOGP_E_INVALID_ARG),
    (dict(H=60), B.BILOGP_E_UNSUPPORTED),
    (dict(hidden=FAKE + 8), B.BILOGP_E_UNSUPPORTED),
    (dict(gw=FAKE + 0x1000008), B.BILOGP_E_UNSUPPORTED),
    (dict(target=FAKE + 0x200004), B.BILOGP_E_UNSUPPORTED),
    (dict(lse=FAKE + 0x300002), B.BILOGP_E_UNSUPPORTED),
    (dict(gb=FAKE + 0x700002), B.BILOGP_E_UNSUPPORTED),
    (dict(ws=None), B.BILOGP_E_WORKSPACE),
    (dict(ws_bytes=100), B.BILOGP_E_WORKSPACE),
    (dict(ws=FAKE + 0x2000010), B.BILOGP_E_WORKSPACE),
    (dict(gh=FAKE + 0x1000000), B.BILOGP_E_INVALID_ARG),          # gradients alias
    (dict(gb=FAKE + 0x400000), B.BILOGP_E_INVALID_ARG),           # bias grad in grad_hidden
    (dict(gh=FAKE), B.BILOGP_E_INVALID_ARG),                      # aliases hidden
    (dict(gw=FAKE + 0x300000), B.BILOGP_E_INVALID_ARG),           # overlaps lse
    (dict(gw=FAKE + 0x2000000), B.BILOGP_E_INVALID_ARG),          # overlaps the workspace
])
def test_backward_fails_closed(kw, status):
    st = _call_bwd(**kw)
    assert st == status, (kw, st, ila.bilogp_last_error())
    assert ila.bilogp_last_error() != ""


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_backward_no_device_is_unsupported():
    assert _call_bwd() == B.BILOGP_E_UNSUPPORTED
    # an empty batch still writes the (zero) weight gradient: it needs the device
    assert _call_bwd(N=0, hidden=None, target=None, lse=None, glogp=None, glse=None,
                     gh=None) == B.BILOGP_E_UNSUPPORTED


def test_backward_wrapper_rejects_bad_inputs():
    h = torch.zeros(4, 16, dtype=torch.bfloat16)
    w = torch.zeros(32, 16, dtype=torch.bfloat16)
    t = torch.zeros(4, dtype=torch.int64)
    f = torch.zeros(4)
    with pytest.raises(TypeError):
        ila.backward(h.float(), w, t, None, f, f, f)
    with pytest.raises(TypeError):
        ila.backward(h, w, t, None, f.double(), f, f)
    with pytest.raises(ValueError):
        ila.backward(h, w, t[:3], None, f, f, f)
    with pytest.raises(ValueError):
        ila.backward(h, w, t, torch.zeros(31), f, f, f)
    with pytest.raises(ValueError):
        ila.backward(h, w, t, None, f, f, f)                  # not on a GPU
    with pytest.raises(ValueError):
        ila.backward_workspace_for((1 << 21) + 1, 32, "cpu")


# ------------------------------------------------------------- split-range checks
def _call_range(begin, end, N=8, V=128256, H=64, bias=None, bias_dtype=0):
    lib = ila.load_library()
    return lib.bilogp_partials_range(FAKE, FAKE + 0x100000, FAKE + 0x200000, bias, bias_dtype, N,
                                     H, V, begin, end, FAKE + 0x40000000, 1 << 24, None)


@pytest.mark.parametrize("begin,end", [(-1, 3), (3, 3), (5, 2), (0, 252), (250, 252), (0, -1)])
def test_partials_range_rejects_bad_ranges(begin, end):
    # V = 128256 has 251 splits
    assert _call_range(begin, end) == B.BILOGP_E_INVALID_ARG, ila.bilogp_last_error()
    assert _call_range(begin, end, N=0) == B.BILOGP_E_INVALID_ARG


def test_partials_range_empty_batch_and_columns():
    assert _call_range(0, 251, N=0) == B.BILOGP_OK
    assert _call_range(10, 20, N=0) == B.BILOGP_OK
    assert ila.vocab_split_columns(128256, 0, 251) == (0, 128256)
    assert ila.vocab_split_columns(128256, 7, 9) == (7 * 2 * 256, 9 * 2 * 256)
    assert ila.vocab_split_columns(128256, 250, 251) == (500 * 256, 128256)
    assert ila.vocab_split_columns(1000, 3, 4) == (768, 1000)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_partials_range_no_device_is_unsupported():
    assert _call_range(0, 8) == B.BILOGP_E_UNSUPPORTED


def test_launch_plan_follows_the_compute_units_only_in_scheduling():
    inv, tp = B.BILOGP_SPLITS_INVARIANT, B.BILOGP_SPLITS_THROUGHPUT
    V = 151936                                   # 594 tiles, 198 splits of 3
    cus = (1, 8, 32, 80, 128, 256, 304, 1024, 4096, 65536)
    for n in (1, 7, 300, 4096):
        plans = {cu: ila.bilogp_launch_plan(n, 4096, V, inv, cu) for cu in cus}
        for cu, (rows, spg, wgs) in plans.items():
            assert rows in (128, 256) and spg >= 1
            sa, st = ila.bilogp_launch_schedule(n, 4096, V, inv, cu)
            assert 0 <= sa <= st <= 198 and sa % spg == 0
            assert wgs == (-(-n // rows) * (-(-sa // spg) + st - sa)
                           + (-(-n // 128) * (198 - st) if st < 198 else 0))
        # few compute units: 256-token blocks; enough of them: 128-token blocks
        assert plans[1][0] == 256 and plans[65536][0] == 128
        assert len(set(plans.values())) >= 2
    # at the headline V (2 tiles per split) the splits per workgroup follow the count too
    hp = {cu: ila.bilogp_launch_plan(4096, 4096, 128256, inv, cu) for cu in (1, 100, 256, 1000)}
    assert len({spg for _, spg, _ in hp.values()}) >= 2, hp
    assert ila.bilogp_launch_plan(4096, 4096, 128256, inv, 256) == (256, 2, 16 * 126)
    assert ila.bilogp_launch_plan(0, 64, 1000, inv, 256) is None
    assert ila.bilogp_launch_plan(8, 64, 0, inv, 256) is None
    assert ila.bilogp_launch_plan(8, 0, 1000, inv, 256) is None
    assert ila.bilogp_launch_plan(8, 64, 1000, inv, 0) is None
    assert ila.bilogp_launch_plan(8, 64, 1000, 7, 256) is None
    for bad in ((0, 64, 1000, inv, 256), (8, 64, 0, inv, 256), (8, 0, 1000, inv, 256),
                (8, 64, 1000, inv, 0), (8, 64, 1000, 7, 256), (8, 64, 1000, inv, 65537)):
        assert ila.bilogp_launch_schedule(*bad) is None, bad
    # the sweep shape on 256 units: 12 whole rounds of single splits, 6 splits left over
    assert ila.bilogp_launch_schedule(4096, 4096, 151936, inv, 256) == (144, 192)
    # the headline shape keeps one launch
    assert ila.bilogp_launch_schedule(4096, 4096, 128256, inv, 256) == (251, 251)
    # the throughput mode's split count follows the same count
    assert ila.bilogp_launch_plan(8, 4096, 128256, tp, 256) is not None


def test_row_block_height_follows_the_stage_count():
    """128-token blocks only where 256-token blocks leave compute units idle
    AND the 128-token plan has fewer (weighted) K stages per unit: the plans
    that measured fastest on MI355X at these shapes."""
    inv = B.BILOGP_SPLITS_INVARIANT
    plan = lambda n, h, v: ila.bilogp_launch_plan(n, h, v, inv, 256)
    # medium configuration: one 256-token tile per workgroup beats two padded
    # 128-token tiles (0.0337 against 0.0396 ms)
    assert plan(512, 1024, 32000) == (256, 1, 250)
    assert plan(256, 256, 151936)[0] == 256
    # long contractions at small N: the 3-buffer 128-token pipeline wins
    assert plan(64, 4096, 128256) == (128, 1, 251)
    assert plan(256, 4096, 128256) == (128, 2, 252)
    # 256-token blocks that fill the device are always kept
    assert plan(4096, 4096, 128256) == (256, 2, 2016)
    assert plan(1024, 1024, 32000) == (256, 2, 252)


def _plan_model(N, H, V, cu):
    """The launch-plan rules as documented in bilogp_host.cpp and include/bilogp.h,
    restated: V-only splits; runs of up to 4 tiles chosen by whole rounds of one
    workgroup per compute unit (ties to the longer run); 128-token row blocks only
    when 256-token blocks leave units idle and the 128-token plan's K stages per
    unit, at 15/32 of a 256-token stage, come out fewer (stages per tile rounded up
    to 2 buffers for 256-token blocks, 3 for 128-token blocks).  With 256-token
    blocks, a split schedule: the last ts splits (2 R ts <= cu) to a 128-token
    launch, the rest in whole rounds where they fit, single splits for the last
    ceil(3 cu / R) of them per row block, where the cost in 256-token stages per
    unit (x 32: 32 per 256-token stage and per workgroup start, 19 per 128-token
    stage, 3 stages for the second launch) beats the one-launch plan's.
    Returns (rows, spg, workgroups, split_a, split_t)."""
    T = -(-V // 256)
    vps = -(-T // 256)
    S = -(-T // vps)

    def spr(R):
        cap = min(max(1, 4 // vps), S)
        best, best_len = 1, None
        for g in range(1, cap + 1):
            length = -(-(R * -(-S // g)) // cu) * g
            if best_len is None or length <= best_len:
                best, best_len = g, length
        return best

    def stages(R, kt):
        g = spr(R)
        return -(-(R * -(-S // g)) // cu) * g * vps * kt

    r256 = -(-N // 256)
    rows = 256
    if r256 * S < cu:
        k = -(-H // 64)
        c256 = stages(r256, -(-k // 2) * 2)
        c128 = stages(-(-N // 128), -(-k // 3) * 3)
        rows = 128 if c128 * 15 < c256 * 32 else 256
    R = -(-N // rows)
    g = spr(R)
    sa = st = S
    if rows == 256 and R * S > cu and R * S <= (2 ** 32 - 1) // 512:
        k = -(-H // 64)
        kt256, kt128 = -(-k // 2) * 2, -(-k // 3) * 3
        wgs = R * -(-S // g)
        best = 32 * (-(-wgs // cu) * g * vps * kt256 + -(-wgs // cu))
        cap = min(max(1, 4 // vps), S)
        b_min = -(-3 * cu // R)
        ts = 1
        while ts < S and 2 * R * ts <= cu:
            sb = S - ts
            a = max(0, sb - b_min) // cap * cap
            starts = -(-(R * (a // cap)) // cu) + -(-(R * (sb - a)) // cu) + 1
            cost = 32 * (-(-(R * sb) // cu) * vps * kt256 + starts + 3) + 19 * vps * kt128
            if cost < best:
                best, g, sa, st = cost, (cap if a > 0 else 1), a, sb
            ts += 1
    wgs = R * (-(-sa // g) + st - sa) + (-(-N // 128) * (S - st) if st < S else 0)
    return rows, g, wgs, sa, st


def test_launch_plan_matches_its_stated_rules():
    """2000 seeded (N, H, V, compute units) against the rules restated above."""
    rng = np.random.default_rng(2024)
    inv = B.BILOGP_SPLITS_INVARIANT
    for _ in range(2000):
        N = int(rng.choice([rng.integers(1, 600), rng.integers(1, 20000), rng.integers(1, 1 << 22)]))
        H = int(rng.integers(1, 8193)) * 8
        V = int(rng.choice([rng.integers(1, 5000), rng.integers(1, 300000), rng.integers(1, 1 << 30)]))
        cu = int(rng.choice([rng.integers(1, 64), 80, 256, 304, rng.integers(1, 4096)]))
        model = _plan_model(N, H, V, cu)
        assert ila.bilogp_launch_plan(N, H, V, inv, cu) == model[:3], (N, H, V, cu)
        assert ila.bilogp_launch_schedule(N, H, V, inv, cu) == model[3:], (N, H, V, cu)
