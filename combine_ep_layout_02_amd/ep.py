"""Python binding of libep.so (C ABI in include/ep.h), argument marshalling only.

The functions carry the C names and take torch tensors for device buffers:
each call checks dtype, device, contiguity and size, passes raw pointers and
the current HIP stream, and raises :class:`EpError` on a non-zero status.
Every step of the path runs in the library's HIP kernels; PyTorch only
provides the device memory and the stream.  If libep.so has not been built
the first call raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from functools import cached_property
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libep.so")
_lib = None

EP_BF16 = 0
EP_FP8_E4M3 = 1
EP_MXFP8_E4M3 = 2
EP_MXFP4_E2M1 = 3
EP_OK = 0
EP_MAX_EXPERTS = 2048
EP_MAX_TOPK = 64
EP_MAX_NUM_CUS = 65535

EXPORTED = ("ep_recv_rows", "ep_layout_workspace_bytes", "ep_layout", "ep_dispatch", "ep_layout_dispatch",
            "ep_dispatch_prequantized",
            "ep_combine", "ep_dispatch_backward", "ep_combine_backward", "ep_status_string", "ep_abi_version",
            "ep_last_hip_error", "ep_check_cvt_e4m3", "ep_check_cvt_bf16", "ep_check_cvt_e2m1",
            "ep_check_quant_e4m3", "ep_probe_stream")


class EpError(RuntimeError):
    def __init__(self, func: str, status: int, hip_error: int = 0):
        msg = f"{func} failed: {status_string(status)}"
        if hip_error:
            msg += f" (hipError {hip_error})"
        super().__init__(msg)
        self.status = status
        self.hip_error = hip_error


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("num_tokens", "hidden", "num_topk", "num_experts",
                                                "num_ranks", "expert_alignment", "capacity", "num_cus")]


@dataclass(frozen=True)
class EpShape:
    """ep_shape_t: T tokens of hidden H routed to k of E experts in R ranks; num_cus is the
    launch budget of dispatch / combine (0 = the whole GPU)."""
    num_tokens: int
    hidden: int
    num_topk: int
    num_experts: int
    num_ranks: int
    expert_alignment: int = 1
    capacity: int = 0
    num_cus: int = 0

    def c(self) -> _Shape:
        return _Shape(self.num_tokens, self.hidden, self.num_topk, self.num_experts, self.num_ranks,
                      self.expert_alignment, self.capacity, self.num_cus)

    @cached_property
    def c_ref(self):
        """A ctypes pointer to this shape's ep_shape_t (built once, kept alive here)."""
        self.__dict__["_c_keep"] = self.c()
        return ctypes.byref(self.__dict__["_c_keep"])

    @cached_property
    def recv_rows(self) -> int:
        return ep_recv_rows(self)

    @cached_property
    def workspace_bytes(self) -> int:
        return ep_layout_workspace_bytes(self)


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libep.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m combine_ep_layout_02_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(_LIB_PATH)
        vp, sp = ctypes.c_void_p, ctypes.POINTER(_Shape)
        st = ctypes.c_int
        L.ep_abi_version.restype = ctypes.c_int
        L.ep_last_hip_error.restype = ctypes.c_int
        L.ep_status_string.restype = ctypes.c_char_p
        L.ep_status_string.argtypes = [st]
        L.ep_recv_rows.restype = st
        L.ep_recv_rows.argtypes = [sp, ctypes.POINTER(ctypes.c_int64)]
        L.ep_layout_workspace_bytes.restype = st
        L.ep_layout_workspace_bytes.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
        L.ep_layout.restype = st
        L.ep_layout.argtypes = [sp] + [vp] * 9 + [ctypes.c_size_t, vp]
        L.ep_dispatch.restype = st
        L.ep_dispatch.argtypes = [sp, vp, vp, ctypes.c_int, vp, vp, vp]
        L.ep_layout_dispatch.restype = st
        L.ep_layout_dispatch.argtypes = [sp] + [vp] * 9 + [ctypes.c_size_t, vp, ctypes.c_int, vp, vp, vp]
        L.ep_dispatch_prequantized.restype = st
        L.ep_dispatch_prequantized.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        L.ep_combine.restype = st
        L.ep_combine.argtypes = [sp, vp, vp, vp, vp, vp]
        L.ep_dispatch_backward.restype = st
        L.ep_dispatch_backward.argtypes = [sp, vp, vp, vp, vp]
        L.ep_combine_backward.restype = st
        L.ep_combine_backward.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp]
        L.ep_check_cvt_e4m3.restype = st
        L.ep_check_cvt_e4m3.argtypes = [vp, vp, ctypes.c_int64, vp]
        L.ep_check_quant_e4m3.restype = st
        L.ep_check_quant_e4m3.argtypes = [vp, vp, vp, ctypes.c_int64, vp]
        L.ep_check_cvt_e2m1.restype = st
        L.ep_check_cvt_e2m1.argtypes = [vp, vp, ctypes.c_int64, vp]
        L.ep_check_cvt_bf16.restype = st
        L.ep_check_cvt_bf16.argtypes = [vp, vp, ctypes.c_int64, vp]
        L.ep_probe_stream.restype = st
        L.ep_probe_stream.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ep_status_string(int(status)).decode()


def ep_status_string(status: int) -> str:
    return status_string(status)


def ep_abi_version() -> int:
    return int(lib().ep_abi_version())


def _check(func: str, status: int) -> None:
    if status != EP_OK:
        raise EpError(func, status, int(lib().ep_last_hip_error()) if status == 5 else 0)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, numel: Optional[int] = None,
         optional: bool = False) -> Optional[int]:
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    if t.numel() and t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda/HIP) tensor")
    return t.data_ptr() if t.numel() else None


_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)
_BYTE_LIKE = (torch.uint8, torch.float8_e4m3fn, torch.int8)


def ep_recv_rows(shape: EpShape) -> int:
    out = ctypes.c_int64()
    _check("ep_recv_rows", lib().ep_recv_rows(ctypes.byref(shape.c()), ctypes.byref(out)))
    return out.value


def ep_layout_workspace_bytes(shape: EpShape) -> int:
    out = ctypes.c_size_t()
    _check("ep_layout_workspace_bytes", lib().ep_layout_workspace_bytes(ctypes.byref(shape.c()), ctypes.byref(out)))
    return out.value


def _layout_args(shape: EpShape, topk_idx, expert_count, expert_offset, rank_count, rank_offset, slot,
                 src_pair, diag, workspace):
    """(shape, 9 pointers, workspace bytes) of ep_layout, checked."""
    T, k, E, R = shape.num_tokens, shape.num_topk, shape.num_experts, shape.num_ranks
    rows, ws_bytes = shape.recv_rows, shape.workspace_bytes
    i32 = torch.int32
    args = (
        _ptr(topk_idx, "topk_idx", i32, T * k, optional=T == 0),
        _ptr(expert_count, "expert_count", i32, E), _ptr(expert_offset, "expert_offset", i32, E + 1),
        _ptr(rank_count, "rank_count", i32, R), _ptr(rank_offset, "rank_offset", i32, R + 1),
        _ptr(slot, "slot", i32, T * k, optional=T == 0),
        _ptr(src_pair, "src_pair", i32, rows, optional=True), _ptr(diag, "diag", i32, 2, optional=True),
        _ptr(workspace, "workspace", None, None),
    )
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < ws_bytes:
        raise ValueError(f"workspace has {nbytes} bytes, needs {ws_bytes}")
    return (shape.c_ref, *args, nbytes)


def ep_layout_dispatch(shape: EpShape, topk_idx, expert_count, expert_offset, rank_count, rank_offset, slot,
                       src_pair, diag, workspace, x, recv_dtype: int, recv_x, recv_scale=None, stream=None) -> None:
    """ep_layout then ep_dispatch; one launch for batches of at most 1024 pairs (the decode shape)."""
    largs = _layout_args(shape, topk_idx, expert_count, expert_offset, rank_count, rank_offset, slot, src_pair,
                         diag, workspace)
    dargs = _dispatch_args(shape, x, slot, recv_dtype, recv_x, recv_scale)
    _check("ep_layout_dispatch", lib().ep_layout_dispatch(*largs, *dargs[1:2], *dargs[3:], _stream(stream)))


def ep_layout(shape: EpShape, topk_idx, expert_count, expert_offset, rank_count, rank_offset, slot,
              src_pair=None, diag=None, workspace=None, stream=None) -> None:
    T, k, E, R = shape.num_tokens, shape.num_topk, shape.num_experts, shape.num_ranks
    rows = ep_recv_rows(shape)
    ws_bytes = ep_layout_workspace_bytes(shape)
    i32 = torch.int32
    args = (
        _ptr(topk_idx, "topk_idx", i32, T * k, optional=T == 0),
        _ptr(expert_count, "expert_count", i32, E), _ptr(expert_offset, "expert_offset", i32, E + 1),
        _ptr(rank_count, "rank_count", i32, R), _ptr(rank_offset, "rank_offset", i32, R + 1),
        _ptr(slot, "slot", i32, T * k, optional=T == 0),
        _ptr(src_pair, "src_pair", i32, rows, optional=True), _ptr(diag, "diag", i32, 2, optional=True),
        _ptr(workspace, "workspace", None, None),
    )
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < ws_bytes:
        raise ValueError(f"workspace has {nbytes} bytes, needs {ws_bytes}")
    _check("ep_layout", lib().ep_layout(ctypes.byref(shape.c()), *args, nbytes, _stream(stream)))


def recv_layout(shape: EpShape, recv_dtype: int):
    """(bytes per receive row, scale entries per row, scale dtype) of a dispatch format."""
    H = shape.hidden
    if recv_dtype == EP_BF16:
        return 2 * H, 0, None
    if recv_dtype == EP_FP8_E4M3:
        return H, H // 128, torch.float32
    if recv_dtype == EP_MXFP8_E4M3:
        return H, H // 32, torch.uint8
    if recv_dtype == EP_MXFP4_E2M1:
        return H // 2, H // 32, torch.uint8
    raise ValueError(f"unknown recv_dtype {recv_dtype}")


def _dispatch_args(shape: EpShape, x, slot, recv_dtype: int, recv_x, recv_scale):
    T, H, k = shape.num_tokens, shape.hidden, shape.num_topk
    rows = shape.recv_rows
    row_bytes, nsc, sdt = recv_layout(shape, recv_dtype)
    if recv_dtype == EP_BF16:
        rx, rs = _ptr(recv_x, "recv_x", _BF16_LIKE, rows * H), None
    else:
        rx = _ptr(recv_x, "recv_x", _BYTE_LIKE, rows * row_bytes)
        rs = _ptr(recv_scale, "recv_scale", sdt if sdt is torch.float32 else _BYTE_LIKE, rows * nsc)
    return (shape.c_ref, _ptr(x, "x", _BF16_LIKE, T * H, optional=T == 0),
            _ptr(slot, "slot", torch.int32, T * k, optional=T == 0), int(recv_dtype), rx, rs)


def _prequantized_args(shape: EpShape, x_q, x_scale, slot, recv_x, recv_scale):
    T, H, k = shape.num_tokens, shape.hidden, shape.num_topk
    rows = shape.recv_rows
    return (shape.c_ref, _ptr(x_q, "x_q", _BYTE_LIKE, T * H, optional=T == 0),
            _ptr(x_scale, "x_scale", torch.float32, T * (H // 128), optional=T == 0),
            _ptr(slot, "slot", torch.int32, T * k, optional=T == 0),
            _ptr(recv_x, "recv_x", _BYTE_LIKE, rows * H, optional=T == 0),
            _ptr(recv_scale, "recv_scale", torch.float32, rows * (H // 128), optional=T == 0))


def ep_dispatch(shape: EpShape, x, slot, recv_dtype: int, recv_x, recv_scale=None, stream=None) -> None:
    _check("ep_dispatch", lib().ep_dispatch(*_dispatch_args(shape, x, slot, recv_dtype, recv_x, recv_scale),
                                            _stream(stream)))


def ep_dispatch_prequantized(shape: EpShape, x_q, x_scale, slot, recv_x, recv_scale, stream=None) -> None:
    """Scatter caller-quantised E4M3 codes [T, H] and fp32 block scales [T, H/128] to every valid slot."""
    _check("ep_dispatch_prequantized", lib().ep_dispatch_prequantized(
        *_prequantized_args(shape, x_q, x_scale, slot, recv_x, recv_scale), _stream(stream)))


def ep_combine(shape: EpShape, y, slot, topk_weights, out, stream=None) -> None:
    T, H, k = shape.num_tokens, shape.hidden, shape.num_topk
    rows = ep_recv_rows(shape)
    _check("ep_combine", lib().ep_combine(
        ctypes.byref(shape.c()), _ptr(y, "y", _BF16_LIKE, rows * H, optional=T == 0),
        _ptr(slot, "slot", torch.int32, T * k, optional=T == 0),
        _ptr(topk_weights, "topk_weights", torch.float32, T * k, optional=T == 0),
        _ptr(out, "out", _BF16_LIKE, T * H, optional=T == 0), _stream(stream)))


def _dispatch_backward_args(shape: EpShape, grad_recv_x, slot, grad_x):
    T, H, k = shape.num_tokens, shape.hidden, shape.num_topk
    rows = shape.recv_rows
    return (shape.c_ref, _ptr(grad_recv_x, "grad_recv_x", _BF16_LIKE, rows * H, optional=T == 0),
            _ptr(slot, "slot", torch.int32, T * k, optional=T == 0),
            _ptr(grad_x, "grad_x", _BF16_LIKE, T * H, optional=T == 0))


def _combine_backward_args(shape: EpShape, grad_out, y, slot, topk_weights, grad_y, grad_weights):
    T, H, k = shape.num_tokens, shape.hidden, shape.num_topk
    rows = shape.recv_rows
    return (shape.c_ref, _ptr(grad_out, "grad_out", _BF16_LIKE, T * H, optional=T == 0),
            _ptr(y, "y", _BF16_LIKE, rows * H, optional=T == 0 or grad_weights is None),
            _ptr(slot, "slot", torch.int32, T * k, optional=T == 0),
            _ptr(topk_weights, "topk_weights", torch.float32, T * k, optional=T == 0),
            _ptr(grad_y, "grad_y", _BF16_LIKE, rows * H, optional=T == 0),
            _ptr(grad_weights, "grad_weights", torch.float32, T * k, optional=True))


def ep_dispatch_backward(shape: EpShape, grad_recv_x, slot, grad_x, stream=None) -> None:
    """grad_x[t] = BF16(sum over valid j of grad_recv_x[slot[t, j]]) (unit-weight combine)."""
    _check("ep_dispatch_backward",
           lib().ep_dispatch_backward(*_dispatch_backward_args(shape, grad_recv_x, slot, grad_x), _stream(stream)))


def ep_combine_backward(shape: EpShape, grad_out, y, slot, topk_weights, grad_y, grad_weights=None,
                        stream=None) -> None:
    """grad_y[slot[t, j]] = BF16(w[t, j] * grad_out[t]); grad_weights[t, j] = <grad_out[t], y[slot[t, j]]>
    (skipped, and y unused, when grad_weights is None)."""
    _check("ep_combine_backward", lib().ep_combine_backward(
        *_combine_backward_args(shape, grad_out, y, slot, topk_weights, grad_y, grad_weights), _stream(stream)))


def ep_check_cvt_e4m3(inp, out, stream=None) -> None:
    n = inp.numel()
    _check("ep_check_cvt_e4m3", lib().ep_check_cvt_e4m3(
        _ptr(inp, "in", torch.float32, n, optional=n == 0), _ptr(out, "out", _BYTE_LIKE, n, optional=n == 0),
        n, _stream(stream)))


def ep_check_quant_e4m3(x, s, out, stream=None) -> None:
    n = x.numel()
    _check("ep_check_quant_e4m3", lib().ep_check_quant_e4m3(
        _ptr(x, "x", _BF16_LIKE, n, optional=n == 0), _ptr(s, "s", torch.float32, n, optional=n == 0),
        _ptr(out, "out", _BYTE_LIKE, n, optional=n == 0), n, _stream(stream)))


def ep_probe_stream(src, dst, units: int, read_chunks: int, write_chunks: int, policy: int = 0,
                    stream=None) -> None:
    """Measurement helper: streams units * read_chunks KiB of src into units * write_chunks KiB of dst
    (policy 0..3 picks the loads' and stores' cache policy; + 4 takes the units in XCD-contiguous order)."""
    for t, name, kib in ((src, "src", read_chunks), (dst, "dst", write_chunks)):
        if t.numel() * t.element_size() < units * kib * 1024:
            raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {units * kib * 1024}")
    _check("ep_probe_stream", lib().ep_probe_stream(_ptr(src, "src", optional=units == 0),
                                                    _ptr(dst, "dst", optional=units == 0), units, read_chunks,
                                                    write_chunks, policy, _stream(stream)))


def ep_check_cvt_e2m1(inp, out, stream=None) -> None:
    n = inp.numel()
    _check("ep_check_cvt_e2m1", lib().ep_check_cvt_e2m1(
        _ptr(inp, "in", torch.float32, n, optional=n == 0), _ptr(out, "out", _BYTE_LIKE, n, optional=n == 0),
        n, _stream(stream)))


def ep_check_cvt_bf16(inp, out, stream=None) -> None:
    n = inp.numel()
    _check("ep_check_cvt_bf16", lib().ep_check_cvt_bf16(
        _ptr(inp, "in", torch.float32, n, optional=n == 0), _ptr(out, "out", _BF16_LIKE, n, optional=n == 0),
        n, _stream(stream)))


# ---------------------------------------------------------------------------
# Prepared calls: validate the arguments once, then launch with the stored
# pointers (for loops that call the same entry point on the same buffers).
# ---------------------------------------------------------------------------

class Prepared:
    """One entry point bound to fixed, already checked arguments.

    With `stream` given at prepare time the handle is resolved once and every
    call without a stream of its own launches there, which saves looking up
    torch's current stream on each call (a few microseconds per step of a
    decode loop).  Without it each call launches on torch's current stream.
    """
    __slots__ = ("name", "_fn", "_args", "_keep", "_bound")

    def __init__(self, name, fn, args, keep, stream=None):
        self.name, self._fn, self._args, self._keep = name, fn, args, keep
        self._bound = None if stream is None else _stream(stream)

    def __call__(self, stream=None) -> None:
        s = _stream(stream) if stream is not None or self._bound is None else self._bound
        status = self._fn(*self._args, s)
        if status != EP_OK:
            _check(self.name, status)


def prepare_layout(shape: EpShape, topk_idx, expert_count, expert_offset, rank_count, rank_offset, slot,
                   src_pair=None, diag=None, workspace=None, stream=None) -> Prepared:
    keep = (topk_idx, expert_count, expert_offset, rank_count, rank_offset, slot, src_pair, diag, workspace)
    return Prepared("ep_layout", lib().ep_layout, _layout_args(shape, *keep), keep, stream)


def prepare_layout_dispatch(shape: EpShape, topk_idx, expert_count, expert_offset, rank_count, rank_offset, slot,
                            src_pair, diag, workspace, x, recv_dtype: int, recv_x, recv_scale=None,
                            stream=None) -> Prepared:
    lkeep = (topk_idx, expert_count, expert_offset, rank_count, rank_offset, slot, src_pair, diag, workspace)
    largs = _layout_args(shape, *lkeep)
    dargs = _dispatch_args(shape, x, slot, recv_dtype, recv_x, recv_scale)
    return Prepared("ep_layout_dispatch", lib().ep_layout_dispatch, (*largs, dargs[1], *dargs[3:]),
                    (*lkeep, x, recv_x, recv_scale), stream)


def prepare_dispatch(shape: EpShape, x, slot, recv_dtype: int, recv_x, recv_scale=None, stream=None) -> Prepared:
    return Prepared("ep_dispatch", lib().ep_dispatch, _dispatch_args(shape, x, slot, recv_dtype, recv_x, recv_scale),
                    (x, slot, recv_x, recv_scale), stream)


def prepare_dispatch_prequantized(shape: EpShape, x_q, x_scale, slot, recv_x, recv_scale, stream=None) -> Prepared:
    return Prepared("ep_dispatch_prequantized", lib().ep_dispatch_prequantized,
                    _prequantized_args(shape, x_q, x_scale, slot, recv_x, recv_scale),
                    (x_q, x_scale, slot, recv_x, recv_scale), stream)


def prepare_combine(shape: EpShape, y, slot, topk_weights, out, stream=None) -> Prepared:
    T, H, k = shape.num_tokens, shape.hidden, shape.num_topk
    rows = shape.recv_rows
    args = (shape.c_ref, _ptr(y, "y", _BF16_LIKE, rows * H, optional=T == 0),
            _ptr(slot, "slot", torch.int32, T * k, optional=T == 0),
            _ptr(topk_weights, "topk_weights", torch.float32, T * k, optional=T == 0),
            _ptr(out, "out", _BF16_LIKE, T * H, optional=T == 0))
    return Prepared("ep_combine", lib().ep_combine, args, (y, slot, topk_weights, out), stream)


def prepare_dispatch_backward(shape: EpShape, grad_recv_x, slot, grad_x, stream=None) -> Prepared:
    return Prepared("ep_dispatch_backward", lib().ep_dispatch_backward,
                    _dispatch_backward_args(shape, grad_recv_x, slot, grad_x), (grad_recv_x, slot, grad_x), stream)


def prepare_combine_backward(shape: EpShape, grad_out, y, slot, topk_weights, grad_y, grad_weights=None,
                             stream=None) -> Prepared:
    return Prepared("ep_combine_backward", lib().ep_combine_backward,
                    _combine_backward_args(shape, grad_out, y, slot, topk_weights, grad_y, grad_weights),
                    (grad_out, y, slot, topk_weights, grad_y, grad_weights), stream)


# ---------------------------------------------------------------------------
# Convenience: allocate outputs with torch, then call the entry points above.
# ---------------------------------------------------------------------------

@dataclass
class LayoutBuffers:
    """The routing handle: ep_layout outputs (plus its workspace)."""
    shape: EpShape
    expert_count: torch.Tensor
    expert_offset: torch.Tensor
    rank_count: torch.Tensor
    rank_offset: torch.Tensor
    slot: torch.Tensor
    src_pair: torch.Tensor
    diag: torch.Tensor
    workspace: torch.Tensor

    @staticmethod
    def allocate(shape: EpShape, device="cuda") -> "LayoutBuffers":
        i32 = dict(dtype=torch.int32, device=device)
        E, R = shape.num_experts, shape.num_ranks
        ws = ep_layout_workspace_bytes(shape)
        return LayoutBuffers(
            shape, torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(R, **i32),
            torch.empty(R + 1, **i32), torch.empty((shape.num_tokens, shape.num_topk), **i32),
            torch.empty(ep_recv_rows(shape), **i32), torch.empty(2, **i32),
            torch.empty((ws + 15) // 16 * 4, **i32))

    def run(self, topk_idx: torch.Tensor, stream=None) -> "LayoutBuffers":
        ep_layout(self.shape, topk_idx, self.expert_count, self.expert_offset, self.rank_count,
                  self.rank_offset, self.slot, self.src_pair, self.diag, self.workspace, stream)
        return self

    def run_dispatch(self, topk_idx: torch.Tensor, x, recv_dtype: int, recv_x, recv_scale=None,
                     stream=None) -> "LayoutBuffers":
        """Layout and dispatch in one call (one launch for batches of at most 1024 pairs)."""
        ep_layout_dispatch(self.shape, topk_idx, self.expert_count, self.expert_offset, self.rank_count,
                           self.rank_offset, self.slot, self.src_pair, self.diag, self.workspace, x, recv_dtype,
                           recv_x, recv_scale, stream)
        return self

    def prepare_dispatch(self, topk_idx: torch.Tensor, x, recv_dtype: int, recv_x, recv_scale=None,
                         stream=None) -> Prepared:
        return prepare_layout_dispatch(self.shape, topk_idx, self.expert_count, self.expert_offset, self.rank_count,
                                       self.rank_offset, self.slot, self.src_pair, self.diag, self.workspace, x,
                                       recv_dtype, recv_x, recv_scale, stream)

    def prepare(self, topk_idx: torch.Tensor, stream=None) -> Prepared:
        return prepare_layout(self.shape, topk_idx, self.expert_count, self.expert_offset, self.rank_count,
                              self.rank_offset, self.slot, self.src_pair, self.diag, self.workspace, stream)


def alloc_recv(shape: EpShape, recv_dtype: int, device="cuda"):
    """Receive buffers of a dispatch format: (recv_x, recv_scale or None)."""
    rows, H = ep_recv_rows(shape), shape.hidden
    if recv_dtype == EP_BF16:
        return torch.empty((rows, H), dtype=torch.bfloat16, device=device), None
    row_bytes, nsc, sdt = recv_layout(shape, recv_dtype)
    return (torch.empty((rows, row_bytes), dtype=torch.uint8, device=device),
            torch.empty((rows, nsc), dtype=sdt, device=device))
