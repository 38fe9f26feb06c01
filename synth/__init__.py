"""Seeded synthetic inputs shared by the CPU oracle tests and the GPU path.

Holds no part of the layer's arithmetic: it only draws numbers (see synth.c).
The five workloads (tiny layer, batch-1 decode, MTP verify with gs64 scales,
2048-token prefill, 16-layer streaming decode) are described in
``synth.workloads``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lock = threading.Lock()
_lib = None

# Stream tags: one Philox key per kind of input.
TAG_WEIGHT = 1      # expert weights, sub0 = layer, sub1 = expert * 4 + matrix
TAG_ROUTER = 2      # router weights, sub0 = layer
TAG_BIAS = 3        # selection bias, sub0 = layer
TAG_X = 4           # activations, sub0 = layer, sub1 = token
TAG_PERM = 5        # popularity rank permutation, sub0 = layer
TAG_GUMBEL = 6      # Gumbel noise for popularity logits, sub0 = layer, sub1 = token
TAG_LOCALITY = 7    # temporal-locality routing draws, sub0 = layer, sub1 = token

MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc and OpenMP."""
    src = os.path.join(_HERE, "synth.c")
    tmp = _SO + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", tmp, src, "-lm"]
    if force or not os.path.exists(_SO):
        subprocess.check_call(cmd)
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_SO):
                build(force=True)
            L = ctypes.CDLL(_SO)
            u32, i64, i32, dbl = ctypes.c_uint32, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
            vp = ctypes.c_void_p
            L.synth_philox4x32_10.argtypes = [vp, vp, vp]
            L.synth_normal_f32.argtypes = [u32, u32, u32, u32, i64, i64, dbl, dbl, vp]
            L.synth_uniform_f64.argtypes = [u32, u32, u32, u32, i64, i64, vp]
            L.synth_permutation.argtypes = [u32, u32, u32, u32, i32, vp]
            L.synth_zipf_gumbel_logits.argtypes = [u32, u32, u32, i64, i64, i32, dbl, dbl, vp, vp]
            L.synth_locality_logits.argtypes = [u32, u32, u32, i64, i32, i32, dbl, dbl, vp,
                                                dbl, dbl, dbl, dbl, vp, vp]
            L.synth_num_threads.restype = ctypes.c_int
            _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def normal(seed, tag, sub0, sub1, n, mean=0.0, std=1.0, first=0, out=None) -> np.ndarray:
    if out is None:
        out = np.empty(n, dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size == n
    lib().synth_normal_f32(seed, tag, sub0, sub1, first, n, mean, std, _ptr(out))
    return out


def uniform(seed, tag, sub0, sub1, n, first=0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform_f64(seed, tag, sub0, sub1, first, n, _ptr(out))
    return out


def permutation(seed, tag, sub0, sub1, n) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().synth_permutation(seed, tag, sub0, sub1, n, _ptr(out))
    return out


# ---------------------------------------------------------------- layer inputs

def expert_matrix(seed, layer, expert, mat, rows, cols, std=0.02, out=None) -> np.ndarray:
    """One expert matrix, f32 [rows][cols] ~ N(0, std). gate/up are [I][H], down is [H][I]."""
    if out is None:
        out = np.empty((rows, cols), dtype=np.float32)
    normal(seed, TAG_WEIGHT, layer, expert * 4 + mat, rows * cols, 0.0, std, out=out.reshape(-1))
    return out


def expert_weights(seed, layer, expert, hidden, inter, std=0.02):
    """(gate [I][H], up [I][H], down [H][I]) f32 for one expert (expert == n_routed is the shared one)."""
    g = expert_matrix(seed, layer, expert, MAT_GATE, inter, hidden, std)
    u = expert_matrix(seed, layer, expert, MAT_UP, inter, hidden, std)
    d = expert_matrix(seed, layer, expert, MAT_DOWN, hidden, inter, std)
    return g, u, d


def fp8_block_matrix(seed, layer, expert, mat, rows, cols, std=0.02):
    """A checkpoint-style FP8 matrix: the f32 expert matrix N(0, std), one
    scale per 128 x 128 block (block max / 448, the largest e4m3 value), and
    the e4m3 codes of w / scale (torch's float8_e4m3fn rounding). Returns
    (codes u8 [rows][cols], scales f32 [ceil(rows/128)][ceil(cols/128)])."""
    import torch
    w = expert_matrix(seed, layer, expert, mat, rows, cols, std)
    br, bc = (rows + 127) // 128, (cols + 127) // 128
    pad = np.zeros((br * 128, bc * 128), np.float32)
    pad[:rows, :cols] = np.abs(w)
    amax = pad.reshape(br, 128, bc, 128).max(axis=(1, 3))
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    full = np.repeat(np.repeat(scale, 128, axis=0), 128, axis=1)[:rows, :cols]
    codes = torch.from_numpy(w / full).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.ascontiguousarray(codes), scale


def activations(seed, layer, t_first, T, hidden, std=1.0) -> np.ndarray:
    """x [T][H] f32 ~ N(0, std); token t uses stream (layer, t_first + t)."""
    x = np.empty((T, hidden), dtype=np.float32)
    for t in range(T):
        normal(seed, TAG_X, layer, t_first + t, hidden, 0.0, std, out=x[t])
    return x


def router_weights(seed, layer, n_experts, hidden, std=0.02) -> np.ndarray:
    w = np.empty((n_experts, hidden), dtype=np.float32)
    normal(seed, TAG_ROUTER, layer, 0, n_experts * hidden, 0.0, std, out=w.reshape(-1))
    return w


def bias(seed, layer, n_experts, std=0.1) -> np.ndarray:
    return normal(seed, TAG_BIAS, layer, 0, n_experts, 0.0, std)


def popularity_perm(seed, layer, n_experts) -> np.ndarray:
    """perm[e] = popularity rank (0 = most popular) of expert e in this layer."""
    return permutation(seed, TAG_PERM, layer, 0, n_experts)


def zipf_logits(seed, layer, t_first, T, n_experts, s=1.1, mix=0.0) -> np.ndarray:
    """logits [T][E]: ln p(rank(e)) + Gumbel(0,1), p = (1-mix) Zipf(s) + mix/E."""
    perm = popularity_perm(seed, layer, n_experts)
    out = np.empty((T, n_experts), dtype=np.float32)
    lib().synth_zipf_gumbel_logits(seed, TAG_GUMBEL, layer, t_first, T, n_experts, s, mix,
                                   _ptr(perm), _ptr(out))
    return out


def locality_logits(seed, layer, T, n_experts, k, keep_p=0.6, s=1.1):
    """logits [T][E] with temporal locality, and the chosen sets [T][k] in draw order."""
    perm = popularity_perm(seed, layer, n_experts)
    out = np.empty((T, n_experts), dtype=np.float32)
    chosen = np.empty((T, k), dtype=np.int32)
    lib().synth_locality_logits(seed, TAG_LOCALITY, layer, T, n_experts, k, keep_p, s,
                                _ptr(perm), 2.0, 4.0, -4.0, 1.0, _ptr(out), _ptr(chosen))
    return out, chosen


def num_threads() -> int:
    return int(lib().synth_num_threads())
