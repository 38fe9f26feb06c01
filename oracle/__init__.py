"""CPU oracle for the int4 routed-expert MoE layer (TEST INFRASTRUCTURE ONLY).

Thin ctypes wrapper over ``oracle.c``: plain scalar C with double
accumulation. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this package; the product path never does. Every function here
marshals numpy arrays and calls the C code; none of the method's arithmetic is
done in Python.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so (gcc, C99, OpenMP over output rows)."""
    src = os.path.join(_HERE, "oracle.c")
    tmp = _SO + ".tmp"
    if force or not os.path.exists(_SO):
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class Expert(ctypes.Structure):
    _fields_ = [("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p),
                ("down_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p), ("bits", ctypes.c_int32)]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_SO):
                build(force=True)
            L = ctypes.CDLL(_SO)
            vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
            L.oracle_quantize_int4.argtypes = [vp, i64, i64, i32, vp, vp]
            L.oracle_dequantize_int4.argtypes = [vp, vp, i64, i64, i32, vp]
            L.oracle_quantize_int8.argtypes = [vp, i64, i64, i32, vp, vp]
            L.oracle_dequantize_int8.argtypes = [vp, vp, i64, i64, i32, vp]
            L.oracle_router_logits.argtypes = [vp, vp, i32, i32, i32, vp]
            L.oracle_route.argtypes = [vp, vp, i32, i32, i32, vp, vp]
            L.oracle_route_topp.argtypes = [vp, vp, i32, i32, i32, f32, vp, vp]
            L.oracle_union.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
            L.oracle_expert_ffn.argtypes = [ctypes.POINTER(Expert), i32, i32, i32, vp, vp]
            L.oracle_expert_ffn_union.argtypes = [ctypes.POINTER(Expert), i32, i32, i32, vp, i32,
                                                  i32, vp, vp, vp, i32, vp]
            L.oracle_layer.argtypes = [i32, i32, i32, i32, i32, f32, f32, vp, i32, vp, vp, vp,
                                       ctypes.POINTER(Expert), ctypes.POINTER(Expert), vp, vp,
                                       vp, vp]
            L.oracle_num_threads.restype = ctypes.c_int
            L.oracle_set_num_threads.argtypes = [ctypes.c_int]
            L.oracle_set_num_threads.restype = None
            L.oracle_fp8_e4m3_value.argtypes = [ctypes.c_uint8]
            L.oracle_fp8_e4m3_value.restype = ctypes.c_double
            L.oracle_fp8_block_dequant.argtypes = [vp, vp, i64, i64, vp]
            L.oracle_convert_fp8_int4.argtypes = [vp, vp, i64, i64, i32, vp, vp]
            _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of the oracle's loops (results do not depend on it)."""
    lib().oracle_set_num_threads(int(n))


# ----------------------------------------------------------------- quantiser

def quantize_int4(w: np.ndarray, group: int = 0):
    """w f32 [rows][cols] -> (q u8 [rows][cols/2], s f32 [rows] or [rows][cols/64])."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    s = np.empty((rows,) if group == 0 else (rows, cols // group), dtype=np.float32)
    rc = lib().oracle_quantize_int4(_p(w), rows, cols, group, _p(q), _p(s))
    if rc:
        raise ValueError("oracle_quantize_int4: bad arguments")
    return q, s


def quantize_int8(w: np.ndarray, group: int = 0):
    """w f32 [rows][cols] -> (q int8 [rows][cols], s f32 [rows] or [rows][cols/64])."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols), dtype=np.int8)
    s = np.empty((rows,) if group == 0 else (rows, cols // group), dtype=np.float32)
    if lib().oracle_quantize_int8(_p(w), rows, cols, group, _p(q), _p(s)):
        raise ValueError("oracle_quantize_int8: bad arguments")
    return q, s


def dequantize_int8(q: np.ndarray, s: np.ndarray, group: int = 0) -> np.ndarray:
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    out = np.empty(q.shape, dtype=np.float64)
    lib().oracle_dequantize_int8(_p(q), _p(s), q.shape[0], q.shape[1], group, _p(out))
    return out


def dequantize_int4(q: np.ndarray, s: np.ndarray, cols: int, group: int = 0) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    out = np.empty((q.shape[0], cols), dtype=np.float64)
    lib().oracle_dequantize_int4(_p(q), _p(s), q.shape[0], cols, group, _p(out))
    return out


# ------------------------------------------------------------- FP8 converter

def fp8_e4m3_value(b: int) -> float:
    return float(lib().oracle_fp8_e4m3_value(b))


def fp8_block_dequant(w8: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """w8 u8 [rows][cols] (e4m3 codes), scale f32 [ceil(rows/128)][ceil(cols/128)] -> f32."""
    w8 = _c(w8, np.uint8)
    scale = _c(scale, np.float32)
    rows, cols = w8.shape
    out = np.empty((rows, cols), dtype=np.float32)
    if lib().oracle_fp8_block_dequant(_p(w8), _p(scale), rows, cols, _p(out)):
        raise ValueError("oracle_fp8_block_dequant: bad arguments")
    return out


def convert_fp8_int4(w8: np.ndarray, scale: np.ndarray, group: int = 0):
    w8 = _c(w8, np.uint8)
    scale = _c(scale, np.float32)
    rows, cols = w8.shape
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    s = np.empty((rows,) if group == 0 else (rows, cols // group), dtype=np.float32)
    if lib().oracle_convert_fp8_int4(_p(w8), _p(scale), rows, cols, group, _p(q), _p(s)):
        raise ValueError("oracle_convert_fp8_int4: bad arguments")
    return q, s


# -------------------------------------------------------------------- router

def router_logits(wr: np.ndarray, x: np.ndarray) -> np.ndarray:
    wr = _c(wr, np.float32)
    x = _c(x, np.float32)
    E, H = wr.shape
    T = x.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib().oracle_router_logits(_p(wr), _p(x), T, H, E, _p(out))
    return out


def route(logits: np.ndarray, bias, k: int, topp: float = 0.0):
    """(idx [T][k], w [T][k]); with 0 < topp < 1 dropped slots have idx -1, w 0."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    b = None if bias is None else _c(bias, np.float32)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    if topp == 0.0:
        rc = lib().oracle_route(_p(logits), _p(b), T, E, k, _p(idx), _p(w))
    else:
        rc = lib().oracle_route_topp(_p(logits), _p(b), T, E, k, topp, _p(idx), _p(w))
    if rc:
        raise ValueError("oracle_route: bad arguments")
    return idx, w


def union(idx: np.ndarray, E: int):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    unique = np.empty(E, dtype=np.int32)
    n_unique = np.zeros(1, dtype=np.int32)
    if lib().oracle_union(_p(idx), T, k, E, _p(counts), _p(offsets), _p(perm), _p(unique),
                          _p(n_unique)):
        raise ValueError("oracle_union: bad arguments")
    return counts, offsets, perm, unique[: int(n_unique[0])].copy()


# ------------------------------------------------------------------- experts

class QExpert:
    """Host copy of one quantised expert: keeps the arrays alive for the C struct.
    bits 4: packed nibbles; bits 8: signed bytes."""

    def __init__(self, gate_q, up_q, down_q, gate_s, up_s, down_s, bits=4):
        qt = np.int8 if bits == 8 else np.uint8
        self.bits = bits
        self.parts = [_c(gate_q, qt), _c(up_q, qt), _c(down_q, qt),
                      _c(gate_s, np.float32), _c(up_s, np.float32), _c(down_s, np.float32)]
        self.struct = Expert(*[a.ctypes.data for a in self.parts], bits)

    @classmethod
    def quantize(cls, gate, up, down, group=0, bits=4):
        qf = quantize_int8 if bits == 8 else quantize_int4
        gq, gs = qf(gate, group)
        uq, us = qf(up, group)
        dq, ds = qf(down, group)
        return cls(gq, uq, dq, gs, us, ds, bits)


def expert_ffn(ex: QExpert, x: np.ndarray, H: int, I: int, group: int = 0) -> np.ndarray:
    """x f32 [T][H] -> y f64 [T][H], one expert applied to every row."""
    x = _c(np.atleast_2d(x), np.float32)
    y = np.empty((x.shape[0], H), dtype=np.float64)
    for t in range(x.shape[0]):
        lib().oracle_expert_ffn(ctypes.byref(ex.struct), H, I, group, _p(x[t]), _p(y[t]))
    return y


def _expert_array(experts):
    arr = (Expert * max(1, len(experts)))()
    for i, e in enumerate(experts):
        arr[i] = e.struct
    return arr


def expert_ffn_union(experts, x, k, offsets, perm, unique, H, I, group=0) -> np.ndarray:
    x = _c(x, np.float32)
    T = x.shape[0]
    offsets, perm, unique = _c(offsets, np.int32), _c(perm, np.int32), _c(unique, np.int32)
    y = np.zeros((T * k, H), dtype=np.float64)
    arr = _expert_array(experts)
    if lib().oracle_expert_ffn_union(arr, H, I, group, _p(x), T, k, _p(offsets), _p(perm),
                                     _p(unique), len(unique), _p(y)):
        raise ValueError("oracle_expert_ffn_union: bad arguments")
    return y


def layer(x, experts, shared, k, group=0, routed_scale=1.0, logits=None, wr=None, bias=None,
          topp=0.0):
    """Whole layer. Returns (y f32 [T][H], y64 f64 [T][H], idx [T][k], w [T][k])."""
    x = _c(x, np.float32)
    T, H = x.shape
    E = len(experts)
    I = experts[0].parts[0].shape[0]
    lg = None if logits is None else _c(logits, np.float32)
    wrc = None if wr is None else _c(wr, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    y = np.empty((T, H), dtype=np.float32)
    y64 = np.empty((T, H), dtype=np.float64)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    arr = _expert_array(experts)
    sh = ctypes.byref(shared.struct) if shared is not None else None
    rc = lib().oracle_layer(H, I, E, k, group, routed_scale, topp, _p(x), T, _p(lg), _p(wrc), _p(b),
                            arr, sh, _p(y), _p(y64), _p(idx), _p(w))
    if rc:
        raise ValueError("oracle_layer: bad arguments")
    return y, y64, idx, w
