"""ctypes binding of ``libbilogp.so`` (declared in ``include/bilogp.h``).

Argument marshalling only: every step of the forward runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  If the
library is missing or cannot be loaded, every call raises; there is no other
code path.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbilogp.so")

BILOGP_OK = 0
BILOGP_E_INVALID_ARG = 1
BILOGP_E_UNSUPPORTED = 2
BILOGP_E_WORKSPACE = 3
BILOGP_E_HIP = 4

BILOGP_BIAS_NONE = 0
BILOGP_BIAS_BF16 = 1
BILOGP_BIAS_F32 = 2

BILOGP_GEMM_OUT_BF16 = 0
BILOGP_GEMM_OUT_F32 = 1
BILOGP_GEMM_OUT_F32_ACCUM = 2

BILOGP_SPLITS_INVARIANT = 0
BILOGP_SPLITS_THROUGHPUT = 1
BILOGP_MAX_THROUGHPUT_SPLITS = 1024

_STATUS_NAMES = {0: "BILOGP_OK", 1: "BILOGP_E_INVALID_ARG", 2: "BILOGP_E_UNSUPPORTED",
                 3: "BILOGP_E_WORKSPACE", 4: "BILOGP_E_HIP"}

# name -> (restype, argtypes); mirrors include/bilogp.h
_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
SIGNATURES = {
    "bilogp_abi_version": (ctypes.c_int, []),
    "bilogp_bit_contract_version": (ctypes.c_int, []),
    "bilogp_vtile_cols": (ctypes.c_int, []),
    "bilogp_max_splits": (ctypes.c_int, []),
    "bilogp_vtiles_per_split": (ctypes.c_int, [_I64]),
    "bilogp_num_vocab_splits": (ctypes.c_int, [_I64]),
    "bilogp_workspace_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "bilogp_vtiles_per_split_mode": (ctypes.c_int, [_I64, _I64, ctypes.c_int, ctypes.c_int]),
    "bilogp_num_vocab_splits_mode": (ctypes.c_int, [_I64, _I64, ctypes.c_int, ctypes.c_int]),
    "bilogp_workspace_bytes_mode": (ctypes.c_size_t, [_I64, _I64, ctypes.c_int, ctypes.c_int]),
    "bilogp_launch_plan": (ctypes.c_int, [_I64, _I64, _I64, ctypes.c_int, ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                          ctypes.POINTER(ctypes.c_int64)]),
    "bilogp_launch_schedule": (ctypes.c_int, [_I64, _I64, _I64, ctypes.c_int, ctypes.c_int,
                                              ctypes.POINTER(ctypes.c_int),
                                              ctypes.POINTER(ctypes.c_int)]),
    "bilogp_forward_mode": (ctypes.c_int, [_VP, _VP, _VP, _VP, ctypes.c_int, _VP, _VP, _I64, _I64,
                                           _I64, ctypes.c_int, ctypes.c_int, _VP,
                                           ctypes.c_size_t, _VP]),
    "bilogp_forward": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I64, _I64, _VP]),
    "bilogp_noalloc_max_workspace_bytes": (ctypes.c_size_t, []),
    "bilogp_forward_noalloc": (ctypes.c_int, [_VP, _VP, _VP, _VP, ctypes.c_int, _VP, _VP, _I64,
                                              _I64, _I64, _VP]),
    "bilogp_forward_ex": (ctypes.c_int, [_VP, _VP, _VP, _VP, ctypes.c_int, _VP, _VP, _I64, _I64,
                                         _I64, _VP, ctypes.c_size_t, _VP]),
    "bilogp_partials": (ctypes.c_int, [_VP, _VP, _VP, _VP, ctypes.c_int, _I64, _I64, _I64, _VP,
                                       ctypes.c_size_t, _VP]),
    "bilogp_merge": (ctypes.c_int, [_VP, _VP, ctypes.c_size_t, _VP, _VP, _I64, _I64, _VP]),
    "bilogp_partials_range": (ctypes.c_int, [_VP, _VP, _VP, _VP, ctypes.c_int, _I64, _I64, _I64,
                                             ctypes.c_int, ctypes.c_int, _VP, ctypes.c_size_t,
                                             _VP]),
    "bilogp_det_gemm_fwd": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I64, _I64, ctypes.c_int, _VP]),
    "bilogp_det_gemm_da": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I64, _I64, ctypes.c_int, _VP]),
    "bilogp_det_gemm_db": (ctypes.c_int, [_VP, _VP, _VP, _I64, _I64, _I64, ctypes.c_int, _VP]),
    "bilogp_backward_workspace_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "bilogp_backward": (ctypes.c_int, [_VP, _VP, _VP, _VP, ctypes.c_int, _VP, _VP, _VP, _VP, _VP,
                                       _VP, _I64, _I64, _I64, _VP, ctypes.c_size_t, _VP]),
    "bilogp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "bilogp_last_error": (ctypes.c_char_p, []),
}

_lib = None
_lock = threading.Lock()


class BilogpError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {detail}")


def load_library(path: str = LIB_PATH):
    """Load (once) and return the ctypes handle of the HIP library."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m invariant_linear_log_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _check(status: int) -> None:
    if status != BILOGP_OK:
        lib = load_library()
        raise BilogpError(status, lib.bilogp_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


# ---------------------------------------------------------------- argument checks
# The library validates sizes, alignment, aliasing and devices, but it sees
# only pointers: a tensor of the wrong dtype or shape would be read with the
# wrong element size or past its end.  Each wrapper therefore checks what the
# pointers stand for before it calls in (TypeError for a dtype, ValueError for
# a shape, layout or device).
def _tensor(t, name: str, dtypes, shape=None, ndim=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        want = " or ".join(str(d) for d in dtypes)
        raise TypeError(f"{name} must be {want}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(ws, name: str = "workspace") -> None:
    if not isinstance(ws, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(ws).__name__}")
    if not ws.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(*tensors) -> None:
    ts = [t for t in tensors if t is not None]
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {dev}")
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError(f"all tensors must be on {dev}, got one on {t.device}")


def _forward_args(hidden, weight, target, bias, bias_dtypes, V=None, w_rows=None):
    """Checks shared by the forward-style calls; returns (N, H, V)."""
    _tensor(hidden, "hidden", torch.bfloat16, ndim=2)
    N, H = hidden.shape
    _tensor(weight, "weight", torch.bfloat16, ndim=2)
    if weight.shape[1] != H:
        raise ValueError(f"weight has {weight.shape[1]} columns, hidden has H = {H}")
    if V is None:
        V = weight.shape[0]
    if w_rows is not None and weight.shape[0] != w_rows:
        raise ValueError(f"weight slice has {weight.shape[0]} rows, the split range holds "
                         f"{w_rows} vocabulary columns")
    _tensor(target, "target", torch.int64, shape=(N,))
    if bias is not None:
        _tensor(bias, "bias", bias_dtypes, shape=(weight.shape[0],))
    return N, H, V


def _outputs(N: int, *outs) -> None:
    for name, t in zip(("logp_out", "lse_out"), outs):
        _tensor(t, name, torch.float32, shape=(N,))


def _stream_handle(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------- plain queries
def bilogp_abi_version() -> int:
    return load_library().bilogp_abi_version()


def bilogp_bit_contract_version() -> int:
    return load_library().bilogp_bit_contract_version()


def bilogp_vtile_cols() -> int:
    return load_library().bilogp_vtile_cols()


def bilogp_max_splits() -> int:
    return load_library().bilogp_max_splits()


def bilogp_vtiles_per_split(V: int) -> int:
    return load_library().bilogp_vtiles_per_split(V)


def bilogp_num_vocab_splits(V: int) -> int:
    return load_library().bilogp_num_vocab_splits(V)


def bilogp_workspace_bytes(N: int, V: int) -> int:
    return load_library().bilogp_workspace_bytes(N, V)


def bilogp_vtiles_per_split_mode(N: int, V: int, mode: int, cu_count: int) -> int:
    return load_library().bilogp_vtiles_per_split_mode(N, V, mode, cu_count)


def bilogp_num_vocab_splits_mode(N: int, V: int, mode: int, cu_count: int) -> int:
    return load_library().bilogp_num_vocab_splits_mode(N, V, mode, cu_count)


def bilogp_workspace_bytes_mode(N: int, V: int, mode: int, cu_count: int) -> int:
    return load_library().bilogp_workspace_bytes_mode(N, V, mode, cu_count)


def bilogp_launch_plan(N: int, H: int, V: int, mode: int, cu_count: int):
    """(tokens per row block, splits per workgroup, workgroups) of the
    projection launch, or None for invalid arguments."""
    rows, spg, wgs = ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
    st = load_library().bilogp_launch_plan(N, H, V, mode, cu_count, ctypes.byref(rows),
                                           ctypes.byref(spg), ctypes.byref(wgs))
    return None if st != 0 else (rows.value, spg.value, wgs.value)


def bilogp_launch_schedule(N: int, H: int, V: int, mode: int, cu_count: int):
    """(split_a, split_t) of the projection's split schedule, or None for
    invalid arguments."""
    a, t = ctypes.c_int(), ctypes.c_int()
    st = load_library().bilogp_launch_schedule(N, H, V, mode, cu_count, ctypes.byref(a),
                                               ctypes.byref(t))
    return None if st != 0 else (a.value, t.value)


def bilogp_status_string(status: int) -> str:
    return load_library().bilogp_status_string(status).decode()


def bilogp_last_error() -> str:
    return load_library().bilogp_last_error().decode()


# ---------------------------------------------------------------- forward calls
def _bias_dtype(bias: Optional[torch.Tensor]) -> int:
    if bias is None:
        return BILOGP_BIAS_NONE
    if bias.dtype == torch.bfloat16:
        return BILOGP_BIAS_BF16
    if bias.dtype == torch.float32:
        return BILOGP_BIAS_F32
    raise TypeError(f"bias must be bfloat16 or float32, got {bias.dtype}")


def bilogp_forward(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                   bias: Optional[torch.Tensor], logp_out: torch.Tensor, lse_out: torch.Tensor,
                   stream=None) -> None:
    """``bilogp_forward`` on 2-D contiguous device tensors (hidden [N, H] bf16,
    weight [V, H] bf16, target [N] int64, bias [V] fp32 or None, outputs [N]
    fp32).  The library allocates its workspace stream-ordered."""
    N, H, V = _forward_args(hidden, weight, target, bias, torch.float32)
    _outputs(N, logp_out, lse_out)
    _same_device(hidden, weight, target, bias, logp_out, lse_out)
    lib = load_library()
    with torch.cuda.device(hidden.device):
        st = lib.bilogp_forward(_ptr(hidden), _ptr(weight), _ptr(target), _ptr(bias),
                                _ptr(logp_out), _ptr(lse_out), N, H, V,
                                _stream_handle(stream, hidden.device))
    _check(st)


def bilogp_forward_ex(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                      bias: Optional[torch.Tensor], logp_out: torch.Tensor,
                      lse_out: torch.Tensor, workspace: Optional[torch.Tensor],
                      stream=None) -> None:
    """``bilogp_forward_ex`` with a caller-owned workspace tensor (any dtype;
    its byte size is passed).  Allocates nothing."""
    N, H, V = _forward_args(hidden, weight, target, bias, (torch.bfloat16, torch.float32))
    _outputs(N, logp_out, lse_out)
    if workspace is not None:
        _workspace(workspace)
    _same_device(hidden, weight, target, bias, logp_out, lse_out, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    with torch.cuda.device(hidden.device):
        st = lib.bilogp_forward_ex(_ptr(hidden), _ptr(weight), _ptr(target), _ptr(bias),
                                   _bias_dtype(bias), _ptr(logp_out), _ptr(lse_out), N, H, V,
                                   _ptr(workspace), ws_bytes,
                                   _stream_handle(stream, hidden.device))
    _check(st)


def bilogp_noalloc_max_workspace_bytes() -> int:
    return load_library().bilogp_noalloc_max_workspace_bytes()


def bilogp_forward_noalloc(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                           bias: Optional[torch.Tensor], logp_out: torch.Tensor,
                           lse_out: torch.Tensor, stream=None) -> None:
    """``bilogp_forward_noalloc``: ``bilogp_forward_ex`` with the library's
    per-GPU scratch array as the workspace; allocates nothing.  Calls that
    overlap on one GPU race (they share the array)."""
    N, H, V = _forward_args(hidden, weight, target, bias, (torch.bfloat16, torch.float32))
    _outputs(N, logp_out, lse_out)
    _same_device(hidden, weight, target, bias, logp_out, lse_out)
    lib = load_library()
    with torch.cuda.device(hidden.device):
        st = lib.bilogp_forward_noalloc(_ptr(hidden), _ptr(weight), _ptr(target), _ptr(bias),
                                        _bias_dtype(bias), _ptr(logp_out), _ptr(lse_out), N, H,
                                        V, _stream_handle(stream, hidden.device))
    _check(st)


def bilogp_forward_mode(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                        bias: Optional[torch.Tensor], logp_out: torch.Tensor,
                        lse_out: torch.Tensor, mode: int, cu_count: int,
                        workspace: Optional[torch.Tensor], stream=None) -> None:
    """``bilogp_forward_mode``: ``bilogp_forward_ex`` under split policy
    ``mode`` with ``cu_count`` compute units for the throughput policy."""
    N, H, V = _forward_args(hidden, weight, target, bias, (torch.bfloat16, torch.float32))
    _outputs(N, logp_out, lse_out)
    if workspace is not None:
        _workspace(workspace)
    _same_device(hidden, weight, target, bias, logp_out, lse_out, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load_library()
    with torch.cuda.device(hidden.device):
        st = lib.bilogp_forward_mode(_ptr(hidden), _ptr(weight), _ptr(target), _ptr(bias),
                                     _bias_dtype(bias), _ptr(logp_out), _ptr(lse_out), N, H, V,
                                     mode, cu_count, _ptr(workspace), ws_bytes,
                                     _stream_handle(stream, hidden.device))
    _check(st)


def bilogp_partials(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                    bias: Optional[torch.Tensor], workspace: torch.Tensor, stream=None) -> None:
    """``bilogp_partials``: projection + per-split online softmax into the
    workspace (partials and target logits)."""
    N, H, V = _forward_args(hidden, weight, target, bias, (torch.bfloat16, torch.float32))
    _workspace(workspace)
    _same_device(hidden, weight, target, bias, workspace)
    lib = load_library()
    with torch.cuda.device(hidden.device):
        st = lib.bilogp_partials(_ptr(hidden), _ptr(weight), _ptr(target), _ptr(bias),
                                 _bias_dtype(bias), N, H, V, _ptr(workspace),
                                 workspace.numel() * workspace.element_size(),
                                 _stream_handle(stream, hidden.device))
    _check(st)


def bilogp_partials_range(hidden: torch.Tensor, weight_slice: torch.Tensor,
                          target: torch.Tensor, bias_slice: Optional[torch.Tensor], V: int,
                          split_begin: int, split_end: int, workspace: torch.Tensor,
                          stream=None) -> None:
    """``bilogp_partials_range``: partials of splits [split_begin, split_end)
    of the full vocabulary V from that range's weight (and bias) columns."""
    S = bilogp_num_vocab_splits(V)
    if S == 0:
        raise ValueError(f"V = {V} out of range")
    if not (0 <= split_begin < split_end <= S):
        raise ValueError(f"split range must satisfy 0 <= begin < end <= {S}, got "
                         f"[{split_begin}, {split_end})")
    c0, c1 = vocab_split_columns(V, split_begin, split_end)
    N, H, _ = _forward_args(hidden, weight_slice, target, bias_slice,
                            (torch.bfloat16, torch.float32), V=V, w_rows=c1 - c0)
    _workspace(workspace)
    _same_device(hidden, weight_slice, target, bias_slice, workspace)
    lib = load_library()
    with torch.cuda.device(hidden.device):
        st = lib.bilogp_partials_range(_ptr(hidden), _ptr(weight_slice), _ptr(target),
                                       _ptr(bias_slice), _bias_dtype(bias_slice), N, H, V,
                                       split_begin, split_end, _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream_handle(stream, hidden.device))
    _check(st)


def vocab_split_columns(V: int, split_begin: int, split_end: int):
    """Vocabulary columns [c0, c1) of splits [split_begin, split_end) under
    the V-only policy (the columns bilogp_partials_range's weight slice holds)."""
    lib = load_library()
    vps = lib.bilogp_vtiles_per_split(V)
    tile = lib.bilogp_vtile_cols()
    return split_begin * vps * tile, min(split_end * vps * tile, V)


def bilogp_merge(target: torch.Tensor, workspace: torch.Tensor, logp_out: torch.Tensor,
                 lse_out: torch.Tensor, V: int, stream=None) -> None:
    """``bilogp_merge``: ascending combine of the workspace partials."""
    _tensor(target, "target", torch.int64, ndim=1)
    N = target.shape[0]
    _outputs(N, logp_out, lse_out)
    _workspace(workspace)
    _same_device(target, workspace, logp_out, lse_out)
    lib = load_library()
    with torch.cuda.device(target.device):
        st = lib.bilogp_merge(_ptr(target), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _ptr(logp_out),
                              _ptr(lse_out), N, V, _stream_handle(stream, target.device))
    _check(st)


# ---------------------------------------------------------------- det_gemm
def _gemm_kind(out: torch.Tensor, accumulate: bool) -> int:
    if out.dtype == torch.bfloat16:
        if accumulate:
            raise ValueError("accumulation needs a float32 output")
        return BILOGP_GEMM_OUT_BF16
    if out.dtype == torch.float32:
        return BILOGP_GEMM_OUT_F32_ACCUM if accumulate else BILOGP_GEMM_OUT_F32
    raise TypeError(f"output must be bfloat16 or float32, got {out.dtype}")


def bilogp_det_gemm_fwd(a: torch.Tensor, b: torch.Tensor, c: torch.Tensor,
                        accumulate: bool = False, stream=None) -> None:
    """``bilogp_det_gemm_fwd``: c[M, N] (=|+=) a[M, K] . b[N, K]^T."""
    _tensor(a, "a", torch.bfloat16, ndim=2)
    M, K = a.shape
    _tensor(b, "b", torch.bfloat16, ndim=2)
    if b.shape[1] != K:
        raise ValueError(f"b has {b.shape[1]} columns, a has K = {K}")
    N = b.shape[0]
    _tensor(c, "c", (torch.bfloat16, torch.float32), shape=(M, N))
    _same_device(a, b, c)
    with torch.cuda.device(a.device):
        st = load_library().bilogp_det_gemm_fwd(_ptr(a), _ptr(b), _ptr(c), M, N, K,
                                                _gemm_kind(c, accumulate),
                                                _stream_handle(stream, a.device))
    _check(st)


def bilogp_det_gemm_da(dc: torch.Tensor, b: torch.Tensor, da: torch.Tensor,
                       accumulate: bool = False, stream=None) -> None:
    """``bilogp_det_gemm_da``: da[M, K] (=|+=) dc[M, N] . b[N, K]."""
    _tensor(dc, "dc", torch.bfloat16, ndim=2)
    M, N = dc.shape
    _tensor(b, "b", torch.bfloat16, ndim=2)
    if b.shape[0] != N:
        raise ValueError(f"b has {b.shape[0]} rows, dc has N = {N}")
    K = b.shape[1]
    _tensor(da, "da", (torch.bfloat16, torch.float32), shape=(M, K))
    _same_device(dc, b, da)
    with torch.cuda.device(dc.device):
        st = load_library().bilogp_det_gemm_da(_ptr(dc), _ptr(b), _ptr(da), M, N, K,
                                               _gemm_kind(da, accumulate),
                                               _stream_handle(stream, dc.device))
    _check(st)


def bilogp_det_gemm_db(a: torch.Tensor, dc: torch.Tensor, db: torch.Tensor,
                       accumulate: bool = False, stream=None) -> None:
    """``bilogp_det_gemm_db``: db[N, K] (=|+=) dc[M, N]^T . a[M, K]."""
    _tensor(a, "a", torch.bfloat16, ndim=2)
    M, K = a.shape
    _tensor(dc, "dc", torch.bfloat16, ndim=2)
    if dc.shape[0] != M:
        raise ValueError(f"dc has {dc.shape[0]} rows, a has M = {M}")
    N = dc.shape[1]
    _tensor(db, "db", (torch.bfloat16, torch.float32), shape=(N, K))
    _same_device(a, dc, db)
    with torch.cuda.device(a.device):
        st = load_library().bilogp_det_gemm_db(_ptr(a), _ptr(dc), _ptr(db), M, N, K,
                                               _gemm_kind(db, accumulate),
                                               _stream_handle(stream, a.device))
    _check(st)


# ---------------------------------------------------------------- backward
def bilogp_backward_workspace_bytes(N: int, V: int) -> int:
    return load_library().bilogp_backward_workspace_bytes(N, V)


def bilogp_backward(hidden: torch.Tensor, weight: torch.Tensor, target: torch.Tensor,
                    bias: Optional[torch.Tensor], lse: torch.Tensor, grad_logp: torch.Tensor,
                    grad_lse: torch.Tensor, grad_hidden: torch.Tensor,
                    grad_weight: torch.Tensor, grad_bias: Optional[torch.Tensor],
                    workspace: torch.Tensor, stream=None) -> None:
    """``bilogp_backward`` on 2-D contiguous device tensors: hidden [N, H] and
    weight [V, H] bf16, target [N] int64, bias [V] or None, lse / grad_logp /
    grad_lse [N] fp32; writes grad_hidden [N, H], grad_weight [V, H] and
    grad_bias [V] (fp32, grad_bias optional)."""
    N, H, V = _forward_args(hidden, weight, target, bias, (torch.bfloat16, torch.float32))
    for name, t in (("lse", lse), ("grad_logp", grad_logp), ("grad_lse", grad_lse)):
        _tensor(t, name, torch.float32, shape=(N,))
    _tensor(grad_hidden, "grad_hidden", torch.float32, shape=(N, H))
    _tensor(grad_weight, "grad_weight", torch.float32, shape=(V, H))
    if grad_bias is not None:
        _tensor(grad_bias, "grad_bias", torch.float32, shape=(V,))
    _workspace(workspace)
    _same_device(hidden, weight, target, bias, lse, grad_logp, grad_lse, grad_hidden,
                 grad_weight, grad_bias, workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    lib = load_library()
    with torch.cuda.device(weight.device):
        st = lib.bilogp_backward(_ptr(hidden), _ptr(weight), _ptr(target), _ptr(bias),
                                 _bias_dtype(bias), _ptr(lse), _ptr(grad_logp), _ptr(grad_lse),
                                 _ptr(grad_hidden), _ptr(grad_weight), _ptr(grad_bias), N, H, V,
                                 _ptr(workspace), ws_bytes,
                                 _stream_handle(stream, weight.device))
    _check(st)
