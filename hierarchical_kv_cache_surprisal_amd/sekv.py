"""Thin Python binding of the SeKV C ABI (include/sekv.h).

Argument marshalling only: every step of the path runs in the HIP library.
Functions keep the C names (sekv_create, sekv_build, sekv_decode_attn, ...);
device buffers are torch tensors on the context's device (PyTorch is used as
the allocator and stream source), host buffers are numpy arrays.

The library is loaded from this package directory (libsekv.so, built by
build_lib.py).  There is no fallback: if it is missing, importing works but
every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsekv.so")

SEKV_OK, SEKV_ERR_INVALID, SEKV_ERR_OOM, SEKV_ERR_HIP, SEKV_ERR_STATE = range(5)
SEKV_F32, SEKV_BF16 = 0, 1
SEKV_BASES_HOST, SEKV_BASES_DEVICE, SEKV_BASES_HOST_STAGED = 0, 1, 2
_STATUS = {0: "OK", 1: "INVALID", 2: "OOM", 3: "HIP", 4: "STATE"}

EXPORTED = ["sekv_create", "sekv_destroy", "sekv_last_error", "sekv_build", "sekv_get_spans",
            "sekv_get_bases_layout", "sekv_decode_attn", "sekv_decode_attn_budget",
            "sekv_route_scores", "sekv_zoom_fetch",
            "sekv_import_spans", "sekv_import_layout", "sekv_import_head", "sekv_export_head",
            "sekv_get_stats", "sekv_set_routing", "sekv_import_route_summary",
            "sekv_export_route_summary", "sekv_apply_rank_gates", "sekv_append_tokens", "sekv_get_window",
            "sekv_set_basis_cache", "sekv_reserve_spans", "sekv_append_surprisal", "sekv_resegment_window",
            "sekv_get_zoom_counts", "sekv_decode_attn_noalloc"]


class SekvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sekv status {_STATUS.get(status, status)}: {msg}")
        self.status = status


class sekv_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("batch", C.c_int32), ("n_ctx", C.c_int32),
                ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("d_head", C.c_int32),
                ("kv_dtype", C.c_int32), ("local_window", C.c_int32), ("basis_home", C.c_int32),
                ("device", C.c_int32)]


class sekv_stats(C.Structure):
    _fields_ = [("decode_calls", C.c_uint64), ("fetch_calls", C.c_uint64),
                ("spans_fetched", C.c_uint64), ("bytes_fetched", C.c_uint64),
                ("memcpy_calls", C.c_uint64), ("device_resident_bytes", C.c_int64),
                ("host_basis_bytes", C.c_int64), ("full_kv_bytes", C.c_int64),
                ("tokens_appended", C.c_uint64), ("cache_zoomed", C.c_uint64),
                ("cache_hits", C.c_uint64), ("cache_spans_fetched", C.c_uint64),
                ("cache_bytes_fetched", C.c_uint64)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libsekv.so and declare the C signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          f"`python -m hierarchical_kv_cache_surprisal_amd.build_lib`")
    lib = C.CDLL(path)
    P, I32, I64, U64, D = C.c_void_p, C.c_int32, C.c_int64, C.c_uint64, C.c_double
    pI32, pI64 = C.POINTER(C.c_int32), C.POINTER(C.c_int64)
    sig = {
        "sekv_create": (I32, [C.POINTER(sekv_config), C.POINTER(P)]),
        "sekv_destroy": (None, [P]),
        "sekv_last_error": (C.c_char_p, [P]),
        "sekv_build": (I32, [P, I32, P, P, P, D, pI32, I32, U64, P]),
        "sekv_get_spans": (I32, [P, I32, pI32, pI32, pI32, pI32, pI32, pI32]),
        "sekv_get_bases_layout": (I32, [P, I32, I32, I32, pI32, pI64, pI64]),
        "sekv_decode_attn": (I32, [P, I32, P, C.POINTER(C.c_float), P, P, P]),
        "sekv_decode_attn_budget": (I32, [P, I32, P, C.POINTER(C.c_float), pI32, P, P, P]),
        "sekv_decode_attn_noalloc": (I32, [P, I32, P, C.POINTER(C.c_float), P, P, P]),
        "sekv_route_scores": (I32, [P, I32, P, P, P]),
        "sekv_zoom_fetch": (I32, [P, I32, pI32, pI32, P, P]),
        "sekv_import_spans": (I32, [P, I32, I32, pI32, pI32, I32, pI32]),
        "sekv_import_layout": (I32, [P, I32, pI32]),
        "sekv_import_head": (I32, [P, I32, I32, I32, P, P, P, P, pI32, P, I64]),
        "sekv_export_head": (I32, [P, I32, I32, I32, P, P, P, P, pI32, P]),
        "sekv_get_stats": (I32, [P, C.POINTER(sekv_stats)]),
        "sekv_set_routing": (I32, [P, I32, I32, C.POINTER(C.c_float)]),
        "sekv_append_tokens": (I32, [P, I32, P, P, I32, P]),
        "sekv_set_basis_cache": (I32, [P, I64]),
        "sekv_get_window": (I32, [P, I32, I32, pI32]),
        "sekv_reserve_spans": (I32, [P, I32]),
        "sekv_append_surprisal": (I32, [P, C.POINTER(C.c_float), I32]),
        "sekv_resegment_window": (I32, [P, P]),
        "sekv_import_route_summary": (I32, [P, I32, I32, I32, P]),
        "sekv_export_route_summary": (I32, [P, I32, I32, I32, P]),
        "sekv_apply_rank_gates": (I32, [P, I32, I32, I32, C.POINTER(C.c_float), C.POINTER(C.c_float), P]),
        "sekv_get_zoom_counts": (I32, [P, I32, C.POINTER(C.c_uint64), C.POINTER(C.c_uint64), I32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int, ctx) -> None:
    if status != SEKV_OK:
        msg = load_library().sekv_last_error(ctx)
        raise SekvError(status, (msg or b"").decode())


def _i32(a) -> "C.POINTER(C.c_int32)":
    return a.ctypes.data_as(C.POINTER(C.c_int32))


def _i64(a) -> "C.POINTER(C.c_int64)":
    return a.ctypes.data_as(C.POINTER(C.c_int64))


def _dptr(t) -> Optional[int]:
    """Device pointer of a contiguous torch tensor (None for None)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _hbuf(a) -> int:
    return a.ctypes.data


# ----------------------------------------------------------------------------- C-named wrappers

def sekv_create(n_layers: int, batch: int, n_ctx: int, n_q_heads: int, n_kv_heads: int, d_head: int,
                kv_dtype: int, local_window: int, basis_home: int, device: int = 0) -> int:
    lib = load_library()
    cfg = sekv_config(n_layers, batch, n_ctx, n_q_heads, n_kv_heads, d_head, kv_dtype,
                      local_window, basis_home, device)
    out = C.c_void_p()
    _check(lib.sekv_create(C.byref(cfg), C.byref(out)), None)
    return out.value


def sekv_destroy(ctx: int) -> None:
    load_library().sekv_destroy(ctx)


def sekv_build(ctx, layer, H, K, V, alpha, rank_choices: Sequence[int], rank_seed: int, stream=None):
    ch = np.ascontiguousarray(rank_choices, dtype=np.int32)
    _check(load_library().sekv_build(ctx, layer, _dptr(H), _dptr(K), _dptr(V), float(alpha), _i32(ch),
                                      len(ch), int(rank_seed) & ((1 << 64) - 1), _stream(stream)), ctx)


def sekv_get_spans(ctx, b: int):
    lib = load_library()
    m, na, mm = C.c_int32(), C.c_int32(), C.c_int32()
    _check(lib.sekv_get_spans(ctx, b, C.byref(m), C.byref(na), C.byref(mm), None, None, None), ctx)
    ms = np.zeros(m.value, np.int32)
    mc = np.zeros(m.value, np.int32)
    an = np.zeros(na.value, np.int32)
    _check(lib.sekv_get_spans(ctx, b, None, None, None, _i32(ms), _i32(mc), _i32(an)), ctx)
    return ms, mc, an, mm.value


def sekv_get_bases_layout(ctx, layer: int, b: int, g: int, m: int):
    rank = np.zeros(m, np.int32)
    off = np.zeros(m, np.int64)
    tot = np.zeros(1, np.int64)
    _check(load_library().sekv_get_bases_layout(ctx, layer, b, g, _i32(rank), _i64(off), _i64(tot)), ctx)
    return rank, off, int(tot[0])


def sekv_decode_attn(ctx, layer: int, q, tau, out, zoom_mask=None, stream=None):
    t = np.ascontiguousarray(tau, dtype=np.float32)
    _check(load_library().sekv_decode_attn(ctx, layer, _dptr(q), t.ctypes.data_as(C.POINTER(C.c_float)),
                                           _dptr(out), _dptr(zoom_mask), _stream(stream)), ctx)


def sekv_decode_attn_budget(ctx, layer: int, q, tau, budget, out, zoom_mask=None, stream=None):
    t = np.ascontiguousarray(tau, dtype=np.float32)
    k = np.ascontiguousarray(budget, dtype=np.int32)
    _check(load_library().sekv_decode_attn_budget(ctx, layer, _dptr(q), t.ctypes.data_as(C.POINTER(C.c_float)),
                                                  _i32(k), _dptr(out), _dptr(zoom_mask), _stream(stream)), ctx)


def sekv_decode_attn_noalloc(ctx, layer: int, q, tau, out, zoom_mask=None, stream=None):
    t = np.ascontiguousarray(tau, dtype=np.float32)
    _check(load_library().sekv_decode_attn_noalloc(ctx, layer, _dptr(q), t.ctypes.data_as(C.POINTER(C.c_float)),
                                                   _dptr(out), _dptr(zoom_mask), _stream(stream)), ctx)


def sekv_route_scores(ctx, layer: int, q, scores, stream=None):
    _check(load_library().sekv_route_scores(ctx, layer, _dptr(q), _dptr(scores), _stream(stream)), ctx)


def sekv_zoom_fetch(ctx, layer: int, entries: np.ndarray, counts: np.ndarray, side=None, done=None):
    e = np.ascontiguousarray(entries, dtype=np.int32)
    c = np.ascontiguousarray(counts, dtype=np.int32)
    _check(load_library().sekv_zoom_fetch(ctx, layer, _i32(e), _i32(c), _stream(side) if side else None,
                                          done), ctx)


def sekv_import_spans(ctx, b: int, mstart, mcount, anchors):
    ms = np.ascontiguousarray(mstart, dtype=np.int32)
    mc = np.ascontiguousarray(mcount, dtype=np.int32)
    an = np.ascontiguousarray(anchors, dtype=np.int32)
    _check(load_library().sekv_import_spans(ctx, b, len(ms), _i32(ms), _i32(mc), len(an), _i32(an)), ctx)


def sekv_import_layout(ctx, layer: int, rank):
    r = np.ascontiguousarray(rank, dtype=np.int32)
    _check(load_library().sekv_import_layout(ctx, layer, _i32(r)), ctx)


def sekv_import_head(ctx, layer, b, g, kbar, vbar, KA, VA, rank, bases):
    """Host numpy arrays in the KV dtype's storage (float32, or uint16 bf16 bits)."""
    arrs = [np.ascontiguousarray(x) for x in (kbar, vbar, KA, VA, bases)]
    r = np.ascontiguousarray(rank, dtype=np.int32)
    _check(load_library().sekv_import_head(ctx, layer, b, g, *[_hbuf(x) for x in arrs[:4]], _i32(r),
                                           _hbuf(arrs[4]), arrs[4].size), ctx)


def sekv_export_head(ctx, layer, b, g, m, n_a, d, basis_elems, storage_dtype):
    kbar = np.zeros((m, d), storage_dtype)
    vbar = np.zeros((m, d), storage_dtype)
    KA = np.zeros((n_a, d), storage_dtype)
    VA = np.zeros((n_a, d), storage_dtype)
    rank = np.zeros(m, np.int32)
    bases = np.zeros(basis_elems, storage_dtype)
    _check(load_library().sekv_export_head(ctx, layer, b, g, _hbuf(kbar), _hbuf(vbar), _hbuf(KA), _hbuf(VA),
                                           _i32(rank), _hbuf(bases)), ctx)
    return kbar, vbar, KA, VA, rank, bases


def sekv_get_stats(ctx) -> dict:
    s = sekv_stats()
    _check(load_library().sekv_get_stats(ctx, C.byref(s)), ctx)
    return {f: getattr(s, f) for f, _ in sekv_stats._fields_}


def sekv_append_tokens(ctx, layer: int, K_new, V_new, stream=None):
    """K_new, V_new: device tensors [B][H_kv][n_new][d] in the KV dtype."""
    n_new = int(K_new.shape[2])
    _check(load_library().sekv_append_tokens(ctx, layer, _dptr(K_new), _dptr(V_new), n_new, _stream(stream)), ctx)


def sekv_set_basis_cache(ctx, nbytes: int):
    _check(load_library().sekv_set_basis_cache(ctx, int(nbytes)), ctx)


def sekv_get_window(ctx, layer: int, b: int) -> int:
    n = np.zeros(1, np.int32)
    _check(load_library().sekv_get_window(ctx, layer, b, _i32(n)), ctx)
    return int(n[0])


def sekv_reserve_spans(ctx, extra: int):
    _check(load_library().sekv_reserve_spans(ctx, int(extra)), ctx)


def sekv_append_surprisal(ctx, H_new):
    """H_new: host float32 [B][n_new]."""
    h = np.ascontiguousarray(H_new, dtype=np.float32)
    n_new = int(h.shape[1]) if h.ndim == 2 else 0
    _check(load_library().sekv_append_surprisal(ctx, h.ctypes.data_as(C.POINTER(C.c_float)), n_new), ctx)


def sekv_resegment_window(ctx, stream=None):
    _check(load_library().sekv_resegment_window(ctx, _stream(stream)), ctx)


def sekv_set_routing(ctx, layer: int, d_route: int, W=None):
    """W: host float32 [H_kv][d_route][d] (None with d_route = 0)."""
    if d_route == 0:
        _check(load_library().sekv_set_routing(ctx, layer, 0, None), ctx)
        return
    w = np.ascontiguousarray(W, dtype=np.float32)
    _check(load_library().sekv_set_routing(ctx, layer, d_route, w.ctypes.data_as(C.POINTER(C.c_float))), ctx)


def sekv_import_route_summary(ctx, layer: int, b: int, g: int, Kr):
    k = np.ascontiguousarray(Kr)
    _check(load_library().sekv_import_route_summary(ctx, layer, b, g, _hbuf(k)), ctx)


def sekv_export_route_summary(ctx, layer: int, b: int, g: int, m: int, d_route: int, storage_dtype):
    k = np.zeros((m, d_route), storage_dtype)
    _check(load_library().sekv_export_route_summary(ctx, layer, b, g, _hbuf(k)), ctx)
    return k


def sekv_apply_rank_gates(ctx, layer: int, b: int, g: int, gate_k=None, gate_v=None, stream=None):
    """gate_k, gate_v: host float32 [m][d] or None."""
    gk = None if gate_k is None else np.ascontiguousarray(gate_k, dtype=np.float32)
    gv = None if gate_v is None else np.ascontiguousarray(gate_v, dtype=np.float32)
    fp = C.POINTER(C.c_float)
    _check(load_library().sekv_apply_rank_gates(ctx, layer, b, g, None if gk is None else gk.ctypes.data_as(fp),
                                                None if gv is None else gv.ctypes.data_as(fp), _stream(stream)),
           ctx)


def sekv_get_zoom_counts(ctx, layer: int, n: int, reset: bool = False):
    """(counts uint64 [n] = [B * H_q], calls) of one layer."""
    counts = np.zeros(n, np.uint64)
    calls = np.zeros(1, np.uint64)
    u64 = C.POINTER(C.c_uint64)
    _check(load_library().sekv_get_zoom_counts(ctx, layer, counts.ctypes.data_as(u64), calls.ctypes.data_as(u64),
                                               1 if reset else 0), ctx)
    return counts, int(calls[0])


# ----------------------------------------------------------------------------- argument checks

def _check_tensor(t, name: str, dtype, numel: int, device: int, optional: bool = False):
    """Raise ValueError unless t is a contiguous tensor of `dtype` with exactly
    `numel` elements on cuda:`device`: the library reads and writes that many
    elements through the raw pointer."""
    import torch
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_cuda or t.device.index != device:
        raise ValueError(f"{name} must be on cuda:{device}, not {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, not {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_host(a, name: str, n: int):
    if a is None or np.asarray(a).size != n:
        raise ValueError(f"{name} must hold {n} entries")


# ----------------------------------------------------------------------------- convenience object

class Context:
    """Owns one sekv_ctx; methods forward to the C-named wrappers above."""

    def __init__(self, n_layers, batch, n_ctx, n_q_heads, n_kv_heads, d_head, kv_dtype="bf16",
                 local_window=512, basis_home="device", device=0):
        self.kv_dtype = kv_dtype
        self.d = d_head
        self.B, self.Hq, self.Hkv, self.L, self.n = batch, n_q_heads, n_kv_heads, n_layers, n_ctx
        dt = {"f32": SEKV_F32, "bf16": SEKV_BF16}[kv_dtype]
        home = {"host": SEKV_BASES_HOST, "device": SEKV_BASES_DEVICE,
                "host_staged": SEKV_BASES_HOST_STAGED}[basis_home]
        self.device = device
        self.ptr = sekv_create(n_layers, batch, n_ctx, n_q_heads, n_kv_heads, d_head, dt, local_window,
                               home, device)

    def close(self):
        if getattr(self, "ptr", None):
            sekv_destroy(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def storage_dtype(self):
        return np.float32 if self.kv_dtype == "f32" else np.uint16

    @property
    def kv_torch_dtype(self):
        import torch
        return torch.float32 if self.kv_dtype == "f32" else torch.bfloat16

    def build(self, layer, H, K, V, alpha, rank_choices, rank_seed, stream=None):
        import torch
        _check_tensor(H, "H", torch.float32, self.B * self.n, self.device)
        kv = self.B * self.Hkv * self.n * self.d
        _check_tensor(K, "K", self.kv_torch_dtype, kv, self.device)
        _check_tensor(V, "V", self.kv_torch_dtype, kv, self.device)
        sekv_build(self.ptr, layer, H, K, V, alpha, rank_choices, rank_seed, stream)

    def spans(self, b):
        return sekv_get_spans(self.ptr, b)

    def m_max(self):
        # the size query alone (no span tables copied): every decode call checks
        # the mask's size with it
        lib = load_library()
        m, na, mm = C.c_int32(), C.c_int32(), C.c_int32()
        _check(lib.sekv_get_spans(self.ptr, 0, C.byref(m), C.byref(na), C.byref(mm), None, None, None), self.ptr)
        return mm.value

    def decode_attn(self, layer, q, tau, out, zoom_mask=None, stream=None, budget=None, noalloc=False):
        import torch
        qn = self.B * self.Hq * self.d
        _check_tensor(q, "q", torch.float32, qn, self.device)
        _check_tensor(out, "out", torch.float32, qn, self.device)
        if zoom_mask is not None:
            _check_tensor(zoom_mask, "zoom_mask", torch.uint8, self.B * self.Hq * self.m_max(), self.device)
        _check_host(tau, "tau", self.Hq)
        if budget is not None:
            _check_host(budget, "budget", self.Hq)
        if noalloc:
            if budget is not None:
                raise ValueError("the entry point that allocates nothing takes no budget")
            sekv_decode_attn_noalloc(self.ptr, layer, q, tau, out, zoom_mask, stream)
        elif budget is None:
            sekv_decode_attn(self.ptr, layer, q, tau, out, zoom_mask, stream)
        else:
            sekv_decode_attn_budget(self.ptr, layer, q, tau, budget, out, zoom_mask, stream)

    def route_scores(self, layer, q, scores, stream=None):
        import torch
        _check_tensor(q, "q", torch.float32, self.B * self.Hq * self.d, self.device)
        _check_tensor(scores, "scores", torch.float32, self.B * self.Hq * self.m_max(), self.device)
        sekv_route_scores(self.ptr, layer, q, scores, stream)

    def bases_layout(self, layer, b, g):
        m = len(self.spans(b)[0])
        return sekv_get_bases_layout(self.ptr, layer, b, g, m)

    def export_head(self, layer, b, g):
        ms, _, _, _ = self.spans(b)
        _, _, tot = self.bases_layout(layer, b, g)
        return sekv_export_head(self.ptr, layer, b, g, len(ms), self.window(layer, b), self.d, tot,
                                self.storage_dtype)

    def import_spans(self, b, mstart, mcount, anchors):
        sekv_import_spans(self.ptr, b, mstart, mcount, anchors)

    def import_layout(self, layer, rank):
        r = np.ascontiguousarray(rank, dtype=np.int32)
        if r.size != self.B * self.Hkv * self.m_max():  # the library reads exactly this many
            raise ValueError(f"rank must hold B * H_kv * m_max = {self.B * self.Hkv * self.m_max()} entries")
        sekv_import_layout(self.ptr, layer, r)

    def import_head(self, layer, b, g, kbar, vbar, KA, VA, rank, bases):
        sekv_import_head(self.ptr, layer, b, g, kbar, vbar, KA, VA, rank, bases)

    def stats(self):
        return sekv_get_stats(self.ptr)

    def append_tokens(self, layer, K_new, V_new, stream=None):
        n_new = int(K_new.shape[2]) if K_new is not None and K_new.dim() == 4 else -1
        if n_new < 0:
            raise ValueError("K_new must be [B][H_kv][n_new][d]")
        kv = self.B * self.Hkv * n_new * self.d
        _check_tensor(K_new, "K_new", self.kv_torch_dtype, kv, self.device)
        _check_tensor(V_new, "V_new", self.kv_torch_dtype, kv, self.device)
        sekv_append_tokens(self.ptr, layer, K_new, V_new, stream)

    def set_basis_cache(self, nbytes):
        sekv_set_basis_cache(self.ptr, nbytes)

    def window(self, layer, b):
        return sekv_get_window(self.ptr, layer, b)

    def reserve_spans(self, extra):
        sekv_reserve_spans(self.ptr, extra)

    def append_surprisal(self, H_new):
        sekv_append_surprisal(self.ptr, H_new)

    def resegment_window(self, stream=None):
        sekv_resegment_window(self.ptr, stream)

    def set_routing(self, layer, d_route, W=None):
        sekv_set_routing(self.ptr, layer, d_route, W)

    def import_route_summary(self, layer, b, g, Kr):
        sekv_import_route_summary(self.ptr, layer, b, g, Kr)

    def export_route_summary(self, layer, b, g, d_route):
        m = len(self.spans(b)[0])
        return sekv_export_route_summary(self.ptr, layer, b, g, m, d_route, self.storage_dtype)

    def zoom_counts(self, layer, reset=False):
        """(counts [B][H_q] uint64, calls): spans zoomed per (sequence, query head) of a layer."""
        counts, calls = sekv_get_zoom_counts(self.ptr, layer, self.B * self.Hq, reset)
        return counts.reshape(self.B, self.Hq), calls

    def apply_rank_gates(self, layer, b, g, gate_k=None, gate_v=None, stream=None):
        sekv_apply_rank_gates(self.ptr, layer, b, g, gate_k, gate_v, stream)
