"""Python binding of libcoli_moe (one int4 routed-expert MoE layer, MI355X).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels (``csrc/``); this module turns torch tensors into device pointers and
the current torch stream into a ``hipStream_t``. The names follow the C ABI in
``include/coli_moe.h``. There is no CPU fallback: if the library is missing,
``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(HERE, "libcoli_moe.so")

COLI_OK, COLI_EINVAL, COLI_EUNSUPPORTED, COLI_EHIP, COLI_ENOMEM, COLI_EBUSY = 0, -1, -2, -3, -4, -5
PATH_AUTO, PATH_GEMV, PATH_MFMA = 0, 1, 2

EXPORTED = [
    "coli_last_error", "coli_version", "coli_expert_blob_layout", "coli_quantize_int4",
    "coli_quantize_expert", "coli_convert_fp8_int4", "coli_convert_fp8_expert",
    "coli_moe_router_logits", "coli_moe_route", "coli_moe_route_topp",
    "coli_moe_union_workspace_size", "coli_moe_union", "coli_moe_workspace_size",
    "coli_moe_expert_ffn", "coli_moe_layer_fwd", "coli_moe_layer_fwd_noalloc",
    "coli_expert_cache_create",
    "coli_expert_cache_destroy", "coli_expert_cache_ensure", "coli_expert_cache_wait",
    "coli_expert_cache_release", "coli_expert_cache_table", "coli_expert_cache_stats",
    "coli_expert_cache_reset", "coli_expert_cache_pin", "coli_expert_cache_usage",
    "coli_expert_cache_pin_hot", "coli_expert_cache_repin", "coli_expert_cache_prefetch",
    "coli_moe_lookahead", "coli_debug_fail_copies", "coli_debug_read_log",
    "coli_profile_enable", "coli_profile_clear",
    "coli_profile_summary", "coli_profile_rerun", "coli_read_probe",
]


class ColiError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"coli status {code}: {msg}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_routed", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("group", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("topp", ctypes.c_float),
                ("wbits", ctypes.c_int32)]


class CacheCfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("slots_per_layer", ctypes.c_int32), ("blob_bytes", ctypes.c_size_t),
                ("d_arena", ctypes.c_void_p), ("h_pools", ctypes.c_void_p),
                ("copy_stream", ctypes.c_void_p)]


class CacheStats(ctypes.Structure):
    _fields_ = [("hits", ctypes.c_uint64), ("misses", ctypes.c_uint64),
                ("evictions", ctypes.c_uint64), ("bytes_h2d", ctypes.c_uint64),
                ("copy_ns", ctypes.c_uint64), ("lookups", ctypes.c_uint64),
                ("pin_hits", ctypes.c_uint64), ("pin_loads", ctypes.c_uint64),
                ("prefetches", ctypes.c_uint64), ("prefetch_hits", ctypes.c_uint64),
                ("repin_swaps", ctypes.c_uint64)]


_lock = threading.Lock()
_lib = None


def lib():
    """Load libcoli_moe.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(SO_PATH):
                raise ImportError(f"{SO_PATH} is missing: run __graft_entry__.build() first")
            L = ctypes.CDLL(SO_PATH)
            vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
            f32 = ctypes.c_float
            P = ctypes.POINTER
            for name in EXPORTED:
                getattr(L, name).restype = ctypes.c_int32
            L.coli_last_error.restype = ctypes.c_char_p
            L.coli_version.restype = ctypes.c_char_p
            L.coli_expert_blob_layout.argtypes = [P(Shape), P(sz), P(sz)]
            L.coli_quantize_int4.argtypes = [vp, i64, i64, i32, vp, vp, vp]
            L.coli_quantize_expert.argtypes = [P(Shape), vp, vp, vp, vp, vp]
            L.coli_convert_fp8_int4.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp]
            L.coli_convert_fp8_expert.argtypes = [P(Shape), vp, vp, vp, vp, vp, vp, vp, vp]
            L.coli_moe_router_logits.argtypes = [vp, vp, i32, i32, i32, vp, vp]
            L.coli_moe_route.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
            L.coli_moe_route_topp.argtypes = [vp, vp, i32, i32, i32, f32, vp, vp, vp]
            L.coli_moe_union_workspace_size.argtypes = [i32, i32, i32, P(sz)]
            L.coli_moe_union.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
            L.coli_moe_workspace_size.argtypes = [P(Shape), i32, i32, P(sz)]
            L.coli_moe_expert_ffn.argtypes = [P(Shape), vp, vp, i32, vp, vp, vp, vp, vp, i32, vp,
                                              sz, vp]
            L.coli_moe_layer_fwd.argtypes = [P(Shape), vp, i32, vp, vp, vp, vp, vp, vp, i32, vp,
                                             vp, vp, i32, vp, sz, vp]
            L.coli_moe_layer_fwd_noalloc.argtypes = [P(Shape), vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                                     vp, i32, vp]
            L.coli_expert_cache_create.argtypes = [P(CacheCfg), P(vp)]
            L.coli_expert_cache_destroy.argtypes = [vp]
            L.coli_expert_cache_ensure.argtypes = [vp, i32, vp, i32, vp]
            L.coli_expert_cache_wait.argtypes = [vp, i32, vp]
            L.coli_expert_cache_release.argtypes = [vp, i32, vp]
            L.coli_expert_cache_table.argtypes = [vp, i32, P(vp)]
            L.coli_expert_cache_stats.argtypes = [vp, P(CacheStats)]
            L.coli_expert_cache_reset.argtypes = [vp]
            L.coli_expert_cache_pin.argtypes = [vp, i32, vp, i32]
            L.coli_expert_cache_usage.argtypes = [vp, vp]
            L.coli_expert_cache_pin_hot.argtypes = [vp, vp, i32]
            L.coli_expert_cache_repin.argtypes = [vp, i32, f32, f32, P(i32)]
            L.coli_expert_cache_prefetch.argtypes = [vp, i32, vp, i32, P(i32)]
            L.coli_moe_lookahead.argtypes = [P(Shape), vp, i32, vp, vp, vp, vp, i32, P(i32), vp,
                                             sz, vp]
            L.coli_debug_fail_copies.argtypes = [i32]
            L.coli_debug_read_log.argtypes = [vp, vp, i32]
            L.coli_profile_enable.argtypes = [i32]
            L.coli_profile_clear.argtypes = []
            L.coli_profile_summary.argtypes = [ctypes.c_char_p, P(i64), P(ctypes.c_double)]
            L.coli_profile_rerun.argtypes = [P(Shape), i32, vp, vp, i32, vp, sz, vp]
            L.coli_read_probe.argtypes = [vp, sz, i32, i32, i32, vp, sz, vp]
            _lib = L
    return _lib


def _check(rc: int):
    if rc != COLI_OK:
        raise ColiError(rc, lib().coli_last_error().decode(errors="replace"))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name):
    import torch
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class MoEShape:
    hidden: int
    inter: int
    n_routed: int
    n_shared: int = 1
    top_k: int = 8
    group: int = 0
    routed_scale: float = 1.0
    topp: float = 0.0
    wbits: int = 4

    def c(self) -> Shape:
        return Shape(self.hidden, self.inter, self.n_routed, self.n_shared, self.top_k, self.group,
                     self.routed_scale, self.topp, self.wbits)


def version() -> str:
    return lib().coli_version().decode()


def blob_layout(shape: MoEShape):
    """(offsets of gate_q, up_q, down_q, gate_s, up_s, down_s; blob bytes)."""
    off = (ctypes.c_size_t * 6)()
    nb = ctypes.c_size_t()
    _check(lib().coli_expert_blob_layout(ctypes.byref(shape.c()), off, ctypes.byref(nb)))
    return list(off), nb.value


def quantize_int4(w, group=0, q=None, s=None, stream=None):
    import torch
    _need(w, torch.float32, "w")
    rows, cols = w.shape
    if q is None:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=w.device)
    if s is None:
        s = torch.empty((rows,) if group == 0 else (rows, cols // 64), dtype=torch.float32,
                        device=w.device)
    _check(lib().coli_quantize_int4(_ptr(w), rows, cols, group, _ptr(q), _ptr(s), _stream(stream)))
    return q, s


def quantize_expert(shape: MoEShape, gate, up, down, blob=None, stream=None):
    import torch
    for t, n in ((gate, "gate"), (up, "up"), (down, "down")):
        _need(t, torch.float32, n)
    if blob is None:
        blob = torch.empty(blob_layout(shape)[1], dtype=torch.uint8, device=gate.device)
    _check(lib().coli_quantize_expert(ctypes.byref(shape.c()), _ptr(gate), _ptr(up), _ptr(down),
                                      _ptr(blob), _stream(stream)))
    return blob


def convert_fp8_int4(w8, scale, group=0, q=None, s=None, stream=None):
    """FP8 e4m3 codes (uint8 [rows][cols]) with block scales (f32
    [ceil(rows/128)][ceil(cols/128)]) -> (q uint8 [rows][cols/2], s f32)."""
    import torch
    _need(w8, torch.uint8, "w8")
    _need(scale, torch.float32, "scale")
    rows, cols = w8.shape
    if scale.numel() != ((rows + 127) // 128) * ((cols + 127) // 128):
        raise ValueError("scale must hold one value per 128 x 128 block")
    if q is None:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=w8.device)
    if s is None:
        shp = (rows,) if group == 0 else (rows, cols // group)
        s = torch.empty(shp, dtype=torch.float32, device=w8.device)
    _check(lib().coli_convert_fp8_int4(_ptr(w8), _ptr(scale), rows, cols, group, _ptr(q), _ptr(s),
                                       _stream(stream)))
    return q, s


def convert_fp8_expert(shape: MoEShape, gate8, gate_scale, up8, up_scale, down8, down_scale,
                       blob=None, stream=None):
    import torch
    for t, n in ((gate8, "gate8"), (up8, "up8"), (down8, "down8")):
        _need(t, torch.uint8, n)
    for t, n in ((gate_scale, "gate_scale"), (up_scale, "up_scale"), (down_scale, "down_scale")):
        _need(t, torch.float32, n)
    H, I = shape.hidden, shape.inter
    for t, sc, r, c in ((gate8, gate_scale, I, H), (up8, up_scale, I, H), (down8, down_scale, H, I)):
        if tuple(t.shape) != (r, c) or sc.numel() != ((r + 127) // 128) * ((c + 127) // 128):
            raise ValueError("FP8 matrix or scale shape does not match the layer shape")
    if blob is None:
        blob = torch.empty(blob_layout(shape)[1], dtype=torch.uint8, device=gate8.device)
    _check(lib().coli_convert_fp8_expert(ctypes.byref(shape.c()), _ptr(gate8), _ptr(gate_scale),
                                         _ptr(up8), _ptr(up_scale), _ptr(down8), _ptr(down_scale),
                                         _ptr(blob), _stream(stream)))
    return blob


def router_logits(wr, x, out=None, stream=None):
    import torch
    _need(wr, torch.float32, "wr")
    _need(x, torch.float32, "x")
    E, H = wr.shape
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check(lib().coli_moe_router_logits(_ptr(wr), _ptr(x), T, H, E, _ptr(out), _stream(stream)))
    return out


def route(logits, bias, k, idx=None, w=None, stream=None, topp=None):
    """coli_moe_route, or coli_moe_route_topp when topp is given."""
    import torch
    _need(logits, torch.float32, "logits")
    _need(bias, torch.float32, "bias")
    T, E = logits.shape
    if idx is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    if topp is None:
        _check(lib().coli_moe_route(_ptr(logits), _ptr(bias), T, E, k, _ptr(idx), _ptr(w),
                                    _stream(stream)))
    else:
        _check(lib().coli_moe_route_topp(_ptr(logits), _ptr(bias), T, E, k, float(topp), _ptr(idx),
                                         _ptr(w), _stream(stream)))
    return idx, w


def union(idx, E, stream=None):
    import torch
    _need(idx, torch.int32, "idx")
    T, k = idx.shape
    dev = idx.device
    nb = ctypes.c_size_t()
    _check(lib().coli_moe_union_workspace_size(T, k, E, ctypes.byref(nb)))
    ws = torch.empty(max(1, nb.value), dtype=torch.uint8, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(1, T * k), dtype=torch.int32, device=dev)
    unique = torch.empty(E, dtype=torch.int32, device=dev)
    n_unique = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib().coli_moe_union(_ptr(idx), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm),
                                _ptr(unique), _ptr(n_unique), _ptr(ws), nb.value, _stream(stream)))
    return counts, offsets, perm[: T * k], unique, n_unique


def workspace_size(shape: MoEShape, T: int, path: int = PATH_AUTO) -> int:
    nb = ctypes.c_size_t()
    _check(lib().coli_moe_workspace_size(ctypes.byref(shape.c()), T, path, ctypes.byref(nb)))
    return nb.value


def workspace(shape: MoEShape, T: int, path: int = PATH_AUTO, device="cuda"):
    """A workspace of the size coli_moe_workspace_size gives (no initialisation
    needed: every call writes what it reads)."""
    import torch
    return torch.empty(max(1, workspace_size(shape, T, path)), dtype=torch.uint8, device=device)


def blob_table(blobs, device="cuda"):
    """Device array of blob pointers from a list of device tensors (or ints)."""
    import torch
    ptrs = [b if isinstance(b, int) else b.data_ptr() for b in blobs]
    return torch.tensor(ptrs, dtype=torch.int64, device=device)


def expert_ffn(shape: MoEShape, table, x, offsets, perm, unique, n_unique, y_assign=None,
               path=PATH_AUTO, ws=None, stream=None):
    import torch
    _need(x, torch.float32, "x")
    T = x.shape[0]
    if y_assign is None:
        y_assign = torch.zeros((T * shape.top_k, shape.hidden), dtype=torch.float32,
                               device=x.device)
    if ws is None:
        ws = workspace(shape, T, path, x.device)
    _check(lib().coli_moe_expert_ffn(ctypes.byref(shape.c()), _ptr(table), _ptr(x), T,
                                     _ptr(offsets), _ptr(perm), _ptr(unique), _ptr(n_unique),
                                     _ptr(y_assign), path, _ptr(ws), ws.numel(), _stream(stream)))
    return y_assign


def layer_fwd(shape: MoEShape, x, table=None, shared_blob=None, logits=None, router_w=None,
              bias=None, cache=None, layer=0, y=None, idx_out=None, w_out=None, path=PATH_AUTO,
              ws=None, stream=None):
    import torch
    _need(x, torch.float32, "x")
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, shape.hidden), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(shape, T, path, x.device)
    _check(lib().coli_moe_layer_fwd(ctypes.byref(shape.c()), _ptr(x), T, _ptr(logits),
                                    _ptr(router_w), _ptr(bias), _ptr(table), _ptr(shared_blob),
                                    None if cache is None else ctypes.c_void_p(cache.handle), layer,
                                    _ptr(y), _ptr(idx_out), _ptr(w_out), path, _ptr(ws), ws.numel(),
                                    _stream(stream)))
    return y


def layer_fwd_noalloc(shape: MoEShape, x, table, shared_blob=None, logits=None, router_w=None,
                      bias=None, y=None, idx_out=None, w_out=None, path=PATH_AUTO, stream=None):
    """coli_moe_layer_fwd_noalloc: the layer on the library's static scratch
    (no workspace, no cache). `y` must be given to allocate nothing here too."""
    import torch
    _need(x, torch.float32, "x")
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, shape.hidden), dtype=torch.float32, device=x.device)
    _check(lib().coli_moe_layer_fwd_noalloc(ctypes.byref(shape.c()), _ptr(x), T, _ptr(logits),
                                            _ptr(router_w), _ptr(bias), _ptr(table),
                                            _ptr(shared_blob), _ptr(y), _ptr(idx_out), _ptr(w_out),
                                            path, _stream(stream)))
    return y


class LayerCall:
    """coli_moe_layer_fwd with every argument but x, y and idx_out fixed, for
    loops of same-shaped calls (one-token decode): the argument objects are
    built once, so each call costs little host time. Pointers are device
    addresses (ints); the caller keeps the tensors alive."""

    def __init__(self, shape: MoEShape, T, ws, table=None, shared_blob=None, logits=None,
                 router_w=None, bias=None, cache=None, layer=0, path=PATH_AUTO, stream=None):
        self._shape = shape.c()
        self._fn = lib().coli_moe_layer_fwd
        self._keep = (ws, table, shared_blob, logits, router_w, bias, cache)
        self._args = [ctypes.byref(self._shape), None, T, _ptr(logits), _ptr(router_w),
                      _ptr(bias), _ptr(table), _ptr(shared_blob),
                      None if cache is None else ctypes.c_void_p(cache.handle), layer, None, None,
                      None, path, _ptr(ws), ws.numel(), _stream(stream)]

    def __call__(self, x_ptr: int, y_ptr: int, idx_ptr: int = 0, w_ptr: int = 0):
        a = self._args
        a[1], a[10], a[11], a[12] = x_ptr, y_ptr, idx_ptr or None, w_ptr or None
        rc = self._fn(*a)
        if rc != COLI_OK:
            _check(rc)


def lookahead(shape: MoEShape, x, cache, layer, logits=None, router_w=None, bias=None, ws=None,
              stream=None) -> int:
    """coli_moe_lookahead: route x with `layer`'s router and prefetch its picks;
    returns the number of copies started."""
    import torch
    _need(x, torch.float32, "x")
    T = x.shape[0]
    if ws is None:
        ws = workspace(shape, T, PATH_AUTO, x.device)
    n = ctypes.c_int32()
    _check(lib().coli_moe_lookahead(ctypes.byref(shape.c()), _ptr(x), T, _ptr(logits),
                                    _ptr(router_w), _ptr(bias), ctypes.c_void_p(cache.handle),
                                    layer, ctypes.byref(n), _ptr(ws), ws.numel(), _stream(stream)))
    return n.value


def debug_fail_copies(n: int):
    """coli_debug_fail_copies: the next n expert-cache copies fail (COLI_EHIP)
    before anything is enqueued."""
    _check(lib().coli_debug_fail_copies(n))


def debug_read_log(count=None, records=None):
    """coli_debug_read_log: log the weight tiles the GEMV kernels stream.
    count: a zeroed 1-element int32/uint32 device tensor; records: an int32
    device tensor [capacity, 4]. No arguments: log off."""
    if count is None:
        _check(lib().coli_debug_read_log(None, None, 0))
        return
    cap = 0 if records is None else int(records.shape[0])
    _check(lib().coli_debug_read_log(_ptr(count), _ptr(records), cap))


def profile_enable(max_records: int):
    _check(lib().coli_profile_enable(max_records))


def profile_clear():
    _check(lib().coli_profile_clear())


def profile_summary(name: str):
    """(launches timed, total milliseconds) for kernel `name`."""
    n = ctypes.c_int64()
    ms = ctypes.c_double()
    _check(lib().coli_profile_summary(name.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def profile_rerun(shape: MoEShape, T: int, table, shared_blob, which: int, ws, stream=None):
    """coli_profile_rerun: one more launch of the gate/up (which=0) or down (1)
    GEMV pass of the last layer call made with `ws`."""
    _check(lib().coli_profile_rerun(ctypes.byref(shape.c()), T, _ptr(table), _ptr(shared_blob),
                                    which, _ptr(ws), ws.numel(), _stream(stream)))


def read_probe(src, pattern: int, row_bytes: int, rows_per_wg: int, sink, stream=None,
               nbytes: int = None):
    """coli_read_probe: stream `nbytes` (default all) of the uint8 tensor `src`
    in a read-only pattern (0: contiguous chunks of row_bytes per workgroup;
    1: rows of row_bytes, rows_per_wg per workgroup), one word per wave to sink."""
    n = src.numel() if nbytes is None else nbytes
    _check(lib().coli_read_probe(_ptr(src), n, pattern, row_bytes, rows_per_wg, _ptr(sink),
                                 sink.numel() * sink.element_size(), _stream(stream)))


class ExpertCache:
    """Per-layer LRU of expert blobs in an HBM arena in front of pinned host
    memory (coli_expert_cache_*). With arena and pool both None the cache only
    keeps the books (policy simulation, no GPU needed)."""

    def __init__(self, n_layers, n_experts, slots_per_layer, blob_bytes, arena=None, pools=None,
                 copy_stream=None):
        """pools: one pinned host tensor (n_experts * blob_bytes bytes) per layer, or
        one tensor holding all layers back to back."""
        ptrs = None
        if pools is not None:
            if not isinstance(pools, (list, tuple)):
                base = pools.data_ptr()
                layer_bytes = n_experts * blob_bytes
                pools_list = [base + l * layer_bytes for l in range(n_layers)]
            else:
                pools_list = [p if isinstance(p, int) else p.data_ptr() for p in pools]
            ptrs = (ctypes.c_void_p * n_layers)(*pools_list)
        self.cfg = CacheCfg(n_layers, n_experts, slots_per_layer, blob_bytes,
                            None if arena is None else arena.data_ptr(),
                            None if ptrs is None else ctypes.cast(ptrs, ctypes.c_void_p).value,
                            None if copy_stream is None else copy_stream.cuda_stream)
        self._keep = (arena, pools, copy_stream, ptrs)
        h = ctypes.c_void_p()
        _check(lib().coli_expert_cache_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self.handle = h.value
        self.n_experts = n_experts

    def close(self):
        if self.handle:
            lib().coli_expert_cache_destroy(ctypes.c_void_p(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def ensure(self, layer, ids):
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        miss = np.zeros(len(ids), dtype=np.int32)
        _check(lib().coli_expert_cache_ensure(ctypes.c_void_p(self.handle), layer,
                                              ids.ctypes.data_as(ctypes.c_void_p), len(ids),
                                              miss.ctypes.data_as(ctypes.c_void_p)))
        return miss

    def _stream_arg(self, stream):
        # a bookkeeping-only cache records no events: no stream needed
        return None if self._keep[0] is None else _stream(stream)

    def wait(self, layer, stream=None):
        _check(lib().coli_expert_cache_wait(ctypes.c_void_p(self.handle), layer,
                                            self._stream_arg(stream)))

    def release(self, layer, stream=None):
        _check(lib().coli_expert_cache_release(ctypes.c_void_p(self.handle), layer,
                                               self._stream_arg(stream)))

    def pin(self, layer, ids):
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        _check(lib().coli_expert_cache_pin(ctypes.c_void_p(self.handle), layer,
                                           ids.ctypes.data_as(ctypes.c_void_p), len(ids)))

    def usage(self):
        """Usage history, uint64 [n_layers][n_experts]."""
        import numpy as np
        out = np.zeros((self.cfg.n_layers, self.n_experts), dtype=np.uint64)
        _check(lib().coli_expert_cache_usage(ctypes.c_void_p(self.handle),
                                             out.ctypes.data_as(ctypes.c_void_p)))
        return out

    def pin_hot(self, per_layer, counts=None):
        import numpy as np
        c = None
        if counts is not None:
            c = np.ascontiguousarray(np.asarray(counts, dtype=np.uint64))
            assert c.shape == (self.cfg.n_layers, self.n_experts)
        _check(lib().coli_expert_cache_pin_hot(
            ctypes.c_void_p(self.handle), None if c is None else c.ctypes.data_as(ctypes.c_void_p),
            per_layer))

    def repin(self, max_swaps=4, hysteresis=0.25, decay=0.5) -> int:
        n = ctypes.c_int32()
        _check(lib().coli_expert_cache_repin(ctypes.c_void_p(self.handle), max_swaps, hysteresis,
                                             decay, ctypes.byref(n)))
        return n.value

    def prefetch(self, layer, ids) -> int:
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        n = ctypes.c_int32()
        _check(lib().coli_expert_cache_prefetch(ctypes.c_void_p(self.handle), layer,
                                                ids.ctypes.data_as(ctypes.c_void_p), len(ids),
                                                ctypes.byref(n)))
        return n.value

    def table_ptr(self, layer) -> int:
        p = ctypes.c_void_p()
        _check(lib().coli_expert_cache_table(ctypes.c_void_p(self.handle), layer, ctypes.byref(p)))
        return p.value

    def stats(self) -> dict:
        s = CacheStats()
        _check(lib().coli_expert_cache_stats(ctypes.c_void_p(self.handle), ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in CacheStats._fields_}

    def reset(self):
        _check(lib().coli_expert_cache_reset(ctypes.c_void_p(self.handle)))
