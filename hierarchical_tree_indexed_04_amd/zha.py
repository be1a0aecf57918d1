"""ctypes binding of ``libzha.so`` (the C ABI declared in ``include/zha.h``).

Argument marshalling only: every step runs in the HIP kernels of the library.
Torch tensors serve as device buffers and ``torch.cuda.current_stream()`` as
the stream.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzha.so")

ZHA_F32 = 0
ZHA_BF16 = 1
ZHA_KV_SPLIT = 0
ZHA_KV_CHUNKED = 1

ERRORS = {
    -1: "ZHA_ERR_NULL", -2: "ZHA_ERR_GEOM", -3: "ZHA_ERR_DTYPE", -4: "ZHA_ERR_DIM",
    -5: "ZHA_ERR_P", -6: "ZHA_ERR_ALIGN", -7: "ZHA_ERR_CAP", -8: "ZHA_ERR_LAUNCH",
    -9: "ZHA_ERR_NPOS", -10: "ZHA_ERR_LAYOUT", -11: "ZHA_ERR_ROPE", -12: "ZHA_ERR_SCRATCH",
}
ZHA_NOALLOC_SCRATCH_BYTES = 4 << 20

# Every function the header declares, with its ctypes signature.
_c_size_p = ctypes.POINTER(ctypes.c_size_t)


class Geom(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H_q", ctypes.c_int32), ("H_kv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("T", ctypes.c_int64), ("C", ctypes.c_int32),
                ("L", ctypes.c_int32), ("R", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("kv_layout", ctypes.c_int32), ("T_cap", ctypes.c_int64)]


class Rope(ctypes.Structure):
    _fields_ = [("dims", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("theta", ctypes.POINTER(ctypes.c_double))]


_GP = ctypes.POINTER(Geom)
_RP = ctypes.POINTER(Rope)
_VP = ctypes.c_void_p
_I32 = ctypes.c_int32

SIGNATURES = {
    "zha_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "zha_tree_bytes": (ctypes.c_int, [_GP, _c_size_p, _c_size_p]),
    "zha_tree_level_offset": (ctypes.c_int, [_GP, _I32, _c_size_p, _c_size_p, _c_size_p]),
    "zha_build": (ctypes.c_int, [_GP, _VP, _VP, _RP, _VP, _VP, _VP]),
    "zha_tree_update": (ctypes.c_int, [_GP, ctypes.c_int64, _VP, _VP, _RP, _VP, _VP, _VP]),
    "zha_route_scratch_bytes": (ctypes.c_int, [_GP, _I32, _I32, _c_size_p]),
    "zha_route": (ctypes.c_int, [_GP, _VP, _VP, _I32, _VP, ctypes.c_float, _VP, _VP, _I32, _VP,
                                 _VP, _VP, _VP]),
    "zha_route_frontier_capacity": (ctypes.c_int32, []),
    "zha_attn_scratch_bytes": (ctypes.c_int, [_GP, _I32, _I32, _c_size_p]),
    "zha_attn": (ctypes.c_int, [_GP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP]),
    "zha_attn_noalloc": (ctypes.c_int, [_GP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP,
                                        _VP]),
    "zha_route_attn_scratch_bytes": (ctypes.c_int, [_GP, _I32, _I32, _c_size_p]),
    "zha_route_attn": (ctypes.c_int, [_GP, _VP, _VP, _I32, _VP, ctypes.c_float, _VP, _VP, _VP,
                                      _VP, _I32, _VP, _VP, _VP, _VP, _VP]),
    "zha_dense_decode_scratch_bytes": (ctypes.c_int, [_GP, _I32, _c_size_p]),
    "zha_dense_decode": (ctypes.c_int, [_GP, _VP, _I32, _VP, _VP, _VP, _VP, _VP]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libzha.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m hierarchical_tree_indexed_04_amd.build_lib`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class ZhaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = load().zha_strerror(code).decode()
        super().__init__(f"{where}: {ERRORS.get(code, code)} ({msg})")


def _check(rc: int, where: str):
    if rc != 0:
        raise ZhaError(rc, where)


def geom(g, kv_layout: int = ZHA_KV_SPLIT, T_cap: int = 0) -> Geom:
    """zha_geom from any object with B, H_q, H_kv, d, T, C, L, R and dtype ('f32'/'bf16');
    T_cap > 0 lays the KV cache and the tree out for T_cap tokens (T of them valid)."""
    dt = g.dtype
    if isinstance(dt, str):
        dt = ZHA_BF16 if dt == "bf16" else ZHA_F32
    return Geom(g.B, g.H_q, g.H_kv, g.d, g.T, g.C, g.L, g.R, dt, kv_layout, T_cap)


def with_length(g: Geom, T: int) -> Geom:
    """The same geometry and capacity holding T tokens (the capacity is pinned
    to the current length when none was set)."""
    return Geom(g.B, g.H_q, g.H_kv, g.d, T, g.C, g.L, g.R, g.dtype, g.kv_layout,
                g.T_cap if g.T_cap else g.T)


def capacity(g: Geom) -> int:
    return g.T_cap if g.T_cap else g.T


def kv_shape(g: Geom):
    """Shape of K (and V) in the split layout, or of the KV buffer in the chunked one
    (capacity rows; the first T are the cached tokens)."""
    tc = capacity(g)
    if g.kv_layout == ZHA_KV_CHUNKED:
        return (g.B, g.H_kv, -(-tc // g.C), 2, g.C, g.d)
    return (g.B, g.H_kv, tc, g.d)


def tree_bytes(g: Geom):
    tb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().zha_tree_bytes(ctypes.byref(g), ctypes.byref(tb), ctypes.byref(sb)),
           "zha_tree_bytes")
    return tb.value, sb.value


def level_offset(g: Geom, level: int):
    k, b, s = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().zha_tree_level_offset(ctypes.byref(g), level, ctypes.byref(k), ctypes.byref(b),
                                        ctypes.byref(s)), "zha_tree_level_offset")
    return k.value, b.value, s.value


def route_scratch_bytes(g: Geom, n_pos: int, cap: int) -> int:
    n = ctypes.c_size_t()
    _check(load().zha_route_scratch_bytes(ctypes.byref(g), n_pos, cap, ctypes.byref(n)),
           "zha_route_scratch_bytes")
    return n.value


def attn_scratch_bytes(g: Geom, n_pos: int, cap: int) -> int:
    n = ctypes.c_size_t()
    _check(load().zha_attn_scratch_bytes(ctypes.byref(g), n_pos, cap, ctypes.byref(n)),
           "zha_attn_scratch_bytes")
    return n.value


def dense_scratch_bytes(g: Geom, n_pos: int) -> int:
    n = ctypes.c_size_t()
    _check(load().zha_dense_decode_scratch_bytes(ctypes.byref(g), n_pos, ctypes.byref(n)),
           "zha_dense_decode_scratch_bytes")
    return n.value


def frontier_capacity() -> int:
    return int(load().zha_route_frontier_capacity())


# ----------------------------------------------------------------------------
# Torch-facing wrappers
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _store_dtype(g: Geom):
    torch = _torch()
    return torch.bfloat16 if g.dtype == ZHA_BF16 else torch.float32


def _need(t, shape, dtype, name):
    torch = _torch()
    if not (t.is_cuda and t.is_contiguous() and t.dtype == dtype and tuple(t.shape) == tuple(shape)):
        raise ValueError(f"{name}: expected contiguous cuda {dtype} {tuple(shape)}, got "
                         f"{t.device} {t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")
    del torch


def _bytes(n, device):
    torch = _torch()
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def to_chunked(K, V, C: int):
    """Device copy of split K, V [B, H_kv, T, d] into the chunked KV buffer
    [B, H_kv, ceil(T / C), 2, C, d] (rows of the last page past T are zero)."""
    torch = _torch()
    B, H, T, d = K.shape
    n1, r = T // C, T % C
    KV = torch.zeros((B, H, -(-T // C), 2, C, d), dtype=K.dtype, device=K.device)
    if n1:
        KV[:, :, :n1, 0] = K[:, :, :n1 * C].reshape(B, H, n1, C, d)
        KV[:, :, :n1, 1] = V[:, :, :n1 * C].reshape(B, H, n1, C, d)
    if r:
        KV[:, :, n1, 0, :r] = K[:, :, n1 * C:]
        KV[:, :, n1, 1, :r] = V[:, :, n1 * C:]
    return KV


@dataclass
class Workspace:
    """Device buffers reused across calls (allocated once by the caller)."""
    tree: object = None
    build_scratch: object = None
    route_scratch: object = None
    attn_scratch: object = None
    dense_scratch: object = None


def rope(dims: int, theta):
    """zha_rope for `dims` rotated dims with angular frequencies theta (dims / 2 values);
    returns (struct, backing array): keep both alive for the call."""
    import numpy as np
    th = np.ascontiguousarray(theta, dtype=np.float64).reshape(-1)
    if th.size != dims // 2:
        raise ValueError(f"rope: {th.size} frequencies for {dims} dims")
    return Rope(dims, 0, th.ctypes.data_as(ctypes.POINTER(ctypes.c_double))), th


def _rope_ref(r):
    if r is None:
        return None
    if isinstance(r, tuple) and len(r) == 2 and isinstance(r[0], Rope):
        return ctypes.byref(r[0])
    raise TypeError("rope: pass the value returned by zha.rope(dims, theta)")


def build(g: Geom, K, qref, tree=None, scratch=None, stream=None, rope=None):
    """zha_build; returns the tree blob (uint8 tensor).  rope: zha.rope(dims, theta) or None.
    qref None: every reference query is zero."""
    torch = _torch()
    _need(K, kv_shape(g), _store_dtype(g), "K")
    if qref is not None:
        _need(qref, (g.H_kv, g.R, g.d), torch.float32, "qref")
    tb, sb = tree_bytes(g)
    if tree is None:
        tree = _bytes(tb, K.device)
    if scratch is None:
        scratch = _bytes(sb, K.device)
    _check(load().zha_build(ctypes.byref(g), _ptr(K), _ptr(qref), _rope_ref(rope), _ptr(tree),
                            _ptr(scratch), _stream(stream)), "zha_build")
    return tree


def tree_update(g: Geom, T_old: int, K, qref, tree, scratch, stream=None, rope=None):
    """zha_tree_update: extend a tree built for T_old tokens to g.T tokens in place.
    ``tree`` and ``scratch`` are the buffers of the earlier build or update; qref None: every
    reference query is zero."""
    torch = _torch()
    _need(K, kv_shape(g), _store_dtype(g), "K")
    if qref is not None:
        _need(qref, (g.H_kv, g.R, g.d), torch.float32, "qref")
    tb, sb = tree_bytes(g)
    if tree.numel() * tree.element_size() < tb or (sb and scratch.numel() * scratch.element_size() < sb):
        raise ValueError("tree_update: tree or scratch smaller than the layout needs")
    _check(load().zha_tree_update(ctypes.byref(g), int(T_old), _ptr(K), _ptr(qref),
                                  _rope_ref(rope), _ptr(tree), _ptr(scratch), _stream(stream)),
           "zha_tree_update")
    return tree


def _need_ctx(g: Geom, ctx_len, n_pos: int):
    if ctx_len is not None:
        _need(ctx_len, (g.B, n_pos), _torch().int32, "ctx_len")


def route(g: Geom, tree, Q, n_pos: int, p: float, cap: int, want_stats=True, want_gap=True,
          out=None, scratch=None, stream=None, ctx_len=None):
    """zha_route; returns (sel, cnt, stats or None, gap or None).  ctx_len: int32 [B, n_pos]
    tokens visible to each position (causal prefill: t + 1), or None for all T."""
    torch = _torch()
    _need(Q, (g.B, n_pos, g.H_q, g.d), _store_dtype(g), "Q")
    _need_ctx(g, ctx_len, n_pos)
    dev = Q.device
    if out is None:
        sel = torch.empty((g.B, n_pos, g.H_q, cap), dtype=torch.int32, device=dev)
        cnt = torch.empty((g.B, n_pos, g.H_q), dtype=torch.int32, device=dev)
        stats = (torch.empty((g.B, n_pos, g.H_q, g.L, 2), dtype=torch.int32, device=dev)
                 if want_stats else None)
        gap = (torch.empty((g.B, n_pos, g.H_q, g.L), dtype=torch.float32, device=dev)
               if want_gap else None)
    else:
        sel, cnt, stats, gap = out
    if scratch is None:
        scratch = _bytes(route_scratch_bytes(g, n_pos, cap), dev)
    _check(load().zha_route(ctypes.byref(g), _ptr(tree), _ptr(Q), n_pos, _ptr(ctx_len),
                            float(p), _ptr(sel),
                            _ptr(cnt), cap, _ptr(stats), _ptr(gap), _ptr(scratch),
                            _stream(stream)), "zha_route")
    return sel, cnt, stats, gap


def _need_kv(g: Geom, K, V):
    dt = _store_dtype(g)
    _need(K, kv_shape(g), dt, "K")
    if g.kv_layout == ZHA_KV_CHUNKED:
        if V is not None:
            raise ValueError("V: the chunked layout holds the values in K's buffer; pass None")
    else:
        _need(V, kv_shape(g), dt, "V")


def attn(g: Geom, Q, n_pos: int, K, V, sel, cnt, cap: int, O=None, scratch=None, stream=None,
         ctx_len=None):
    """zha_attn; returns O [B, n_pos, H_q, d].  Chunked layout: K is the KV buffer, V None.
    ctx_len: the same visible lengths as given to route (or None)."""
    torch = _torch()
    dt = _store_dtype(g)
    _need(Q, (g.B, n_pos, g.H_q, g.d), dt, "Q")
    _need_ctx(g, ctx_len, n_pos)
    _need_kv(g, K, V)
    _need(sel, (g.B, n_pos, g.H_q, cap), torch.int32, "sel")
    _need(cnt, (g.B, n_pos, g.H_q), torch.int32, "cnt")
    if O is None:
        O = torch.empty((g.B, n_pos, g.H_q, g.d), dtype=dt, device=Q.device)
    if scratch is None:
        scratch = _bytes(attn_scratch_bytes(g, n_pos, cap), Q.device)
    _check(load().zha_attn(ctypes.byref(g), _ptr(Q), n_pos, _ptr(ctx_len), _ptr(K), _ptr(V),
                           _ptr(sel),
                           _ptr(cnt), cap, _ptr(O), _ptr(scratch), _stream(stream)), "zha_attn")
    return O


def attn_noalloc(g: Geom, Q, n_pos: int, K, V, sel, cnt, cap: int, O=None, stream=None,
                 ctx_len=None):
    """zha_attn_noalloc: zha_attn with the library's fixed device buffer as scratch
    (O may be given, so that the call allocates nothing at all)."""
    torch = _torch()
    dt = _store_dtype(g)
    _need(Q, (g.B, n_pos, g.H_q, g.d), dt, "Q")
    _need_ctx(g, ctx_len, n_pos)
    _need_kv(g, K, V)
    _need(sel, (g.B, n_pos, g.H_q, cap), torch.int32, "sel")
    _need(cnt, (g.B, n_pos, g.H_q), torch.int32, "cnt")
    if O is None:
        O = torch.empty((g.B, n_pos, g.H_q, g.d), dtype=dt, device=Q.device)
    else:
        _need(O, (g.B, n_pos, g.H_q, g.d), dt, "O")
    _check(load().zha_attn_noalloc(ctypes.byref(g), _ptr(Q), n_pos, _ptr(ctx_len), _ptr(K),
                                   _ptr(V), _ptr(sel), _ptr(cnt), cap, _ptr(O), _stream(stream)),
           "zha_attn_noalloc")
    return O


def route_attn_scratch_bytes(g: Geom, n_pos: int, cap: int) -> int:
    n = ctypes.c_size_t()
    _check(load().zha_route_attn_scratch_bytes(ctypes.byref(g), n_pos, cap, ctypes.byref(n)),
           "zha_route_attn_scratch_bytes")
    return n.value


def route_attn(g: Geom, tree, Q, n_pos: int, p: float, K, V, cap: int, want_stats=True,
               want_gap=True, out=None, O=None, scratch=None, stream=None, ctx_len=None):
    """zha_route_attn: returns (sel, cnt, level_stats or None, gap or None, O)."""
    torch = _torch()
    dt = _store_dtype(g)
    _need(Q, (g.B, n_pos, g.H_q, g.d), dt, "Q")
    _need_ctx(g, ctx_len, n_pos)
    _need_kv(g, K, V)
    dev = Q.device
    if out is None:
        sel = torch.empty((g.B, n_pos, g.H_q, cap), dtype=torch.int32, device=dev)
        cnt = torch.empty((g.B, n_pos, g.H_q), dtype=torch.int32, device=dev)
        stats = (torch.empty((g.B, n_pos, g.H_q, g.L, 2), dtype=torch.int32, device=dev)
                 if want_stats else None)
        gap = torch.empty((g.B, n_pos, g.H_q, g.L), dtype=torch.float32, device=dev) if want_gap else None
    else:
        sel, cnt, stats, gap = out
    if O is None:
        O = torch.empty((g.B, n_pos, g.H_q, g.d), dtype=dt, device=dev)
    if scratch is None:
        scratch = _bytes(route_attn_scratch_bytes(g, n_pos, cap), dev)
    _check(load().zha_route_attn(ctypes.byref(g), _ptr(tree), _ptr(Q), n_pos, _ptr(ctx_len),
                                 ctypes.c_float(p), _ptr(K), _ptr(V), _ptr(sel), _ptr(cnt), cap,
                                 _ptr(stats), _ptr(gap), _ptr(O), _ptr(scratch), _stream(stream)),
           "zha_route_attn")
    return sel, cnt, stats, gap, O


def dense_decode(g: Geom, Q, n_pos: int, K, V, O=None, scratch=None, stream=None):
    """zha_dense_decode; returns O [B, n_pos, H_q, d].  K, V as for attn."""
    dt = _store_dtype(g)
    _need(Q, (g.B, n_pos, g.H_q, g.d), dt, "Q")
    _need_kv(g, K, V)
    torch = _torch()
    if O is None:
        O = torch.empty((g.B, n_pos, g.H_q, g.d), dtype=dt, device=Q.device)
    if scratch is None:
        scratch = _bytes(dense_scratch_bytes(g, n_pos), Q.device)
    _check(load().zha_dense_decode(ctypes.byref(g), _ptr(Q), n_pos, _ptr(K), _ptr(V), _ptr(O),
                                   _ptr(scratch), _stream(stream)), "zha_dense_decode")
    return O
