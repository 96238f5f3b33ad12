"""CPU oracle for MoE routing layout, dispatch and combine.

TEST INFRASTRUCTURE ONLY: the test-suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path (the
HIP library and its Python binding) never imports this package.

The arithmetic lives in ``oracle.c`` (plain scalar C, no shared code with
the HIP sources); this module loads it with ctypes and exposes numpy-level
wrappers.  Every function states the reading of the pages it follows in the
C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

i64 = ctypes.c_int64
vp = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        L.oracle_abi.restype = ctypes.c_int
        L.oracle_recv_rows.restype = i64
        L.oracle_recv_rows.argtypes = [i64] * 5
        L.oracle_layout.restype = ctypes.c_int
        L.oracle_layout.argtypes = [i64] * 6 + [vp] * 7 + [i64, vp]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_bf16_rne.argtypes = [ctypes.c_float]
        L.oracle_bf16_rne_array.argtypes = [vp, vp, i64]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode_array.argtypes = [vp, vp, i64]
        L.oracle_fp8_quantize_array.argtypes = [vp, vp, vp, i64]
        L.oracle_dispatch_bf16.argtypes = [i64, i64, i64, vp, vp, vp]
        L.oracle_dispatch_fp8.argtypes = [i64, i64, i64, vp, vp, vp, vp]
        L.oracle_combine.argtypes = [i64, i64, i64, vp, vp, vp, vp]
        L.oracle_dispatch_backward.argtypes = [i64, i64, i64, vp, vp, vp]
        L.oracle_combine_backward.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.oracle_dispatch_prequantized.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
        L.oracle_e2m1_decode.restype = ctypes.c_double
        L.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_encode.restype = ctypes.c_uint8
        L.oracle_e2m1_encode.argtypes = [ctypes.c_float]
        L.oracle_e2m1_encode_array.argtypes = [vp, vp, i64]
        L.oracle_mx_exponent.restype = ctypes.c_int
        L.oracle_mx_exponent.argtypes = [ctypes.c_float, ctypes.c_int]
        L.oracle_dispatch_mx.argtypes = [i64, i64, i64, ctypes.c_int, vp, vp, vp, vp]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(vp)


def _c(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def recv_rows(T: int, k: int, E: int, A: int = 1, C: int = 0) -> int:
    return int(lib().oracle_recv_rows(T, k, E, A, C))


@dataclass
class Layout:
    expert_count: np.ndarray   # int32 [E]
    expert_offset: np.ndarray  # int32 [E+1]
    rank_count: np.ndarray     # int32 [R]
    rank_offset: np.ndarray    # int32 [R+1]
    slot: np.ndarray           # int32 [T, k]
    src_pair: np.ndarray       # int32 [rows]
    diag: np.ndarray           # int32 [2]


def layout(topk_idx: np.ndarray, num_experts: int, num_ranks: int,
           expert_alignment: int = 1, capacity: int = 0) -> Layout:
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    E, R = num_experts, num_ranks
    rows = recv_rows(T, k, E, expert_alignment, capacity)
    out = Layout(np.zeros(E, np.int32), np.zeros(E + 1, np.int32), np.zeros(R, np.int32),
                 np.zeros(R + 1, np.int32), np.zeros((T, k), np.int32),
                 np.zeros(rows, np.int32), np.zeros(2, np.int32))
    rc = lib().oracle_layout(T, k, E, R, expert_alignment, capacity, _p(idx),
                             _p(out.expert_count), _p(out.expert_offset), _p(out.rank_count),
                             _p(out.rank_offset), _p(out.slot), _p(out.src_pair), rows,
                             _p(out.diag))
    if rc != 0:
        raise MemoryError("oracle_layout: allocation failed")
    return out


def bf16_rne(f: np.ndarray) -> np.ndarray:
    f = _c(np.asarray(f, dtype=np.float32), np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().oracle_bf16_rne_array(_p(f), _p(out), f.size)
    return out


def e4m3_encode(f: np.ndarray) -> np.ndarray:
    f = _c(np.asarray(f, dtype=np.float32), np.float32)
    out = np.empty(f.shape, np.uint8)
    lib().oracle_e4m3_encode_array(_p(f), _p(out), f.size)
    return out


def e4m3_decode(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([L.oracle_e4m3_decode(int(v)) for v in c.ravel()], np.float64).reshape(c.shape)


def dispatch_bf16(x: np.ndarray, slot: np.ndarray, rows: int) -> np.ndarray:
    x = _c(x, np.uint16)
    slot = _c(slot, np.int32)
    T, H = x.shape
    k = slot.shape[1]
    out = np.zeros((rows, H), np.uint16)
    lib().oracle_dispatch_bf16(T, H, k, _p(x), _p(slot), _p(out))
    return out


def dispatch_fp8(x: np.ndarray, slot: np.ndarray, rows: int, out=None):
    """FP8 dispatch; `out` = (codes [rows, H] uint8, scales [rows, H/128] fp32) to fill in place
    (rows no slot of these tokens maps to are left as they are)."""
    x = _c(x, np.uint16)
    slot = _c(slot, np.int32)
    T, H = x.shape
    k = slot.shape[1]
    assert H % 128 == 0
    if out is None:
        out = (np.zeros((rows, H), np.uint8), np.zeros((rows, H // 128), np.float32))
    q, s = out
    assert q.flags.c_contiguous and s.flags.c_contiguous and q.shape == (rows, H) and s.shape == (rows, H // 128)
    lib().oracle_dispatch_fp8(T, H, k, _p(x), _p(slot), _p(q), _p(s))
    return q, s


def combine(y: np.ndarray, slot: np.ndarray, weights: np.ndarray, out=None) -> np.ndarray:
    """Combine; `out` = a C-contiguous uint16 [T, H] array to fill in place."""
    y = _c(y, np.uint16)
    slot = _c(slot, np.int32)
    w = _c(weights, np.float32)
    T, k = slot.shape
    H = y.shape[1]
    if out is None:
        out = np.zeros((T, H), np.uint16)
    assert out.flags.c_contiguous and out.shape == (T, H) and out.dtype == np.uint16
    lib().oracle_combine(T, H, k, _p(y), _p(slot), _p(w), _p(out))
    return out


def dispatch_backward(grad_recv: np.ndarray, slot: np.ndarray) -> np.ndarray:
    """Gradient of x given the gradient of the dispatched rows (BF16 bits)."""
    g = _c(grad_recv, np.uint16)
    slot = _c(slot, np.int32)
    T, k = slot.shape
    H = g.shape[1]
    out = np.zeros((T, H), np.uint16)
    lib().oracle_dispatch_backward(T, H, k, _p(g), _p(slot), _p(out))
    return out


def combine_backward(grad_out: np.ndarray, y: np.ndarray, slot: np.ndarray, weights: np.ndarray,
                     grad_y_init: Optional[np.ndarray] = None):
    """Gradients of y (BF16 bits, [rows, H]; rows no pair maps to keep
    grad_y_init, zeros by default) and of the weights (float64 [T, k])."""
    g = _c(grad_out, np.uint16)
    y = _c(y, np.uint16)
    slot = _c(slot, np.int32)
    w = _c(weights, np.float32)
    T, k = slot.shape
    H = g.shape[1]
    gy = np.zeros(y.shape, np.uint16) if grad_y_init is None else np.array(grad_y_init, np.uint16)
    gw = np.zeros((T, k), np.float64)
    lib().oracle_combine_backward(T, H, k, _p(g), _p(y), _p(slot), _p(w), _p(gy), _p(gw))
    return gy, gw


def dispatch_prequantized(x_q: np.ndarray, x_s: np.ndarray, slot: np.ndarray, rows: int):
    """Copy the caller's E4M3 codes [T, H] and fp32 block scales [T, H/128] to every valid slot."""
    x_q = _c(x_q, np.uint8)
    x_s = _c(x_s, np.float32)
    slot = _c(slot, np.int32)
    T, H = x_q.shape
    k = slot.shape[1]
    q = np.zeros((rows, H), np.uint8)
    s = np.zeros((rows, H // 128), np.float32)
    lib().oracle_dispatch_prequantized(T, H, k, _p(x_q), _p(x_s), _p(slot), _p(q), _p(s))
    return q, s


def e2m1_encode(f) -> np.ndarray:
    f = _c(np.asarray(f, dtype=np.float32), np.float32)
    out = np.empty(f.shape, np.uint8)
    lib().oracle_e2m1_encode_array(_p(f), _p(out), f.size)
    return out


def e2m1_decode(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([L.oracle_e2m1_decode(int(v)) for v in c.ravel()], np.float64).reshape(c.shape)


def mx_exponent(amax: float, emax: int) -> int:
    return int(lib().oracle_mx_exponent(float(amax), int(emax)))


def dispatch_mx(x: np.ndarray, slot: np.ndarray, rows: int, elem_bits: int):
    """MXFP8 (elem_bits 8) or MXFP4 (4) dispatch: codes [rows, H or H/2] and E8M0 scales [rows, H/32]."""
    x = _c(x, np.uint16)
    slot = _c(slot, np.int32)
    T, H = x.shape
    k = slot.shape[1]
    assert H % 32 == 0 and elem_bits in (4, 8)
    q = np.zeros((rows, H if elem_bits == 8 else H // 2), np.uint8)
    s = np.zeros((rows, H // 32), np.uint8)
    lib().oracle_dispatch_mx(T, H, k, elem_bits, _p(x), _p(slot), _p(q), _p(s))
    return q, s


def fp8_quantize(x_bits: np.ndarray, s: np.ndarray) -> np.ndarray:
    """E4M3 code of each BF16 value x (bits) over its fp32 block scale s (FP8 dispatch's step)."""
    x = _c(x_bits, np.uint16)
    s = _c(s, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_fp8_quantize_array(_p(x), _p(s), _p(out), x.size)
    return out
