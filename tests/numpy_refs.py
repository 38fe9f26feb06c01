"""Independent numpy formulations used to pin the C oracle.

Each one computes the same quantity as an oracle function by a different
route (whole-array numpy operations, sorting, counting or enumeration instead
of the oracle's scalar loops), so that a slip in the oracle — a dropped term,
a wrong sign, a swapped index, a transposed operand — shows up as a mismatch.
"""
from __future__ import annotations

import itertools

import numpy as np


def unpack_nibbles(q: np.ndarray, cols: int) -> np.ndarray:
    """u8 [rows][cols/2] -> int8 [rows][cols], two's complement, even column in the low nibble."""
    q = np.asarray(q, dtype=np.uint8)
    lo = (q & 0x0F).astype(np.int16)
    hi = (q >> 4).astype(np.int16)
    out = np.empty((q.shape[0], cols), dtype=np.int16)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return ((out ^ 8) - 8).astype(np.int8)


def quantize_numpy(w: np.ndarray, group: int = 0):
    """Per-row or gs64 quantisation written with numpy's rint on float32 arrays."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    span = cols if group == 0 else group
    wg = w.reshape(rows, cols // span, span)
    m = np.abs(wg).max(axis=2)                                   # float32
    scale = (m / np.float32(7.0)).astype(np.float32)             # float32 division
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.rint(wg / scale[:, :, None])                      # float32 division, half-even
    v = np.where(scale[:, :, None] == 0, 0, v)
    v = np.clip(v, -8, 7).astype(np.int8).reshape(rows, cols)
    nib = (v.astype(np.int16) & 0x0F).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    s = scale.reshape(rows) if group == 0 else scale
    return packed, s, v


def quantize8_numpy(w: np.ndarray, group: int = 0):
    """int8: scale = max|w| / 127 in float32, numpy rint of the float32 quotient, clamp."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    span = cols if group == 0 else group
    wg = w.reshape(rows, cols // span, span)
    scale = (np.abs(wg).max(axis=2) / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.rint(wg / scale[:, :, None])
    v = np.where(scale[:, :, None] == 0, 0, v)
    q = np.clip(v, -128, 127).astype(np.int8).reshape(rows, cols)
    return q, (scale.reshape(rows) if group == 0 else scale)


def dequant8(q: np.ndarray, s: np.ndarray, group: int = 0) -> np.ndarray:
    v = np.asarray(q, dtype=np.int8).astype(np.float64)
    s = np.asarray(s, dtype=np.float64)
    if group == 0:
        return v * s.reshape(-1, 1)
    return v * np.repeat(s.reshape(v.shape[0], -1), group, axis=1)


def dequant(q: np.ndarray, s: np.ndarray, cols: int, group: int = 0) -> np.ndarray:
    v = unpack_nibbles(q, cols).astype(np.float64)
    s = np.asarray(s, dtype=np.float64)
    if group == 0:
        return v * s.reshape(-1, 1)
    return v * np.repeat(s.reshape(v.shape[0], -1), group, axis=1)


def ffn_dense(gate, up, down, x):
    """Dense f64 SwiGLU on already-dequantised matrices: y = down (silu(gate x) * up x)."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ gate.T
    u = x @ up.T
    h = g / (1.0 + np.exp(-g)) * u
    return h @ down.T


def sigmoid_f32(logits: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-logits.astype(np.float64)))).astype(np.float32)


def route_by_rank(logits, bias, k):
    """Selection by the rank definition: e is chosen iff fewer than k experts beat it,
    where e' beats e if key[e'] > key[e], or the keys are equal and e' < e."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    s = sigmoid_f32(logits)
    b = np.zeros(E, np.float32) if bias is None else np.asarray(bias, np.float32)
    key = (s + b[None, :]).astype(np.float32)
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        kt = key[t]
        beats = (kt[None, :] > kt[:, None]) | ((kt[None, :] == kt[:, None]) &
                                                 (np.arange(E)[None, :] < np.arange(E)[:, None]))
        rank = beats.sum(axis=1)                      # rank[e] = #experts beating e
        chosen = np.where(rank < k)[0]
        idx[t] = chosen[np.argsort(rank[chosen])]     # slot order = rank order
    return idx, s


def best_subset(key_row: np.ndarray, k: int):
    """Exhaustive search: among all k-subsets with the largest key sum, the one with the
    lexicographically smallest sorted index list (float64 sums of float32 keys)."""
    E = key_row.shape[0]
    best, best_sum = None, -np.inf
    for sub in itertools.combinations(range(E), k):
        s = float(np.sum(key_row[list(sub)].astype(np.float64)))
        if s > best_sum:
            best, best_sum = sub, s
    return best


def union_numpy(idx: np.ndarray, E: int):
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    unique = np.nonzero(counts)[0].astype(np.int32)
    return counts, offsets, perm, unique
