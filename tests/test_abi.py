"""The C-ABI library loads, exports every declared symbol and validates arguments (no GPU).

Only host-side paths are exercised: size queries and argument checks that
return before any launch.
"""
import ctypes
import math
import os
import re

import pytest

from hierarchical_tree_indexed_04_amd import zha as Z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zha.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zha_\w+)\s*\(", text)))


def g(**kw):
    base = dict(B=1, H_q=8, H_kv=2, d=128, T=4096, C=16, L=3, R=1, dtype=Z.ZHA_BF16)
    base.update(kw)
    return Z.Geom(**base)


def test_library_exports_every_declared_function():
    lib = Z.load()
    names = declared_functions()
    assert len(names) == 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(Z.SIGNATURES)


def test_strerror_names_every_code():
    lib = Z.load()
    for code in [0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11, -12]:
        assert lib.zha_strerror(code) not in (None, b"", b"unknown error")
    assert lib.zha_strerror(-1000) == b"unknown error"


def expected_layout(gm, es):
    tc = gm.T_cap or gm.T  # rows of capacity follow the capacity, not the length
    n = [None] + [tc // gm.C ** l for l in range(1, gm.L + 1)]
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    off, khat, bhat = 0, {}, {}
    for l in range(1, gm.L + 1):
        khat[l] = off
        off += a256(n[l] * gm.R * gm.d * es)
    for l in range(1, gm.L + 1):
        bhat[l] = off
        off += a256(n[l] * gm.R * 4)
    return khat, bhat, off


@pytest.mark.parametrize("kw", [dict(), dict(dtype=Z.ZHA_F32, R=3, T=5000), dict(C=8, L=6, T=8 ** 6 + 77),
                                dict(T=4096, T_cap=70000), dict(dtype=Z.ZHA_F32, T=5000, T_cap=5001)])
def test_tree_layout_matches_documented_rules(kw):
    gm = g(**kw)
    es = 2 if gm.dtype == Z.ZHA_BF16 else 4
    khat, bhat, stride = expected_layout(gm, es)
    tb, sb = Z.tree_bytes(gm)
    assert tb == stride * gm.B * gm.H_kv
    for l in range(1, gm.L + 1):
        assert Z.level_offset(gm, l) == (khat[l], bhat[l], stride)
    # build scratch: fp64 F and k_hat for levels 1..L-1
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    tc = gm.T_cap or gm.T
    want = sum(a256(gm.B * gm.H_kv * (tc // gm.C ** l) * gm.R * 8)
               + a256(gm.B * gm.H_kv * (tc // gm.C ** l) * gm.R * gm.d * 8)
               for l in range(1, gm.L))
    assert sb == want


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), -4), (dict(dtype=7), -3), (dict(H_q=6, H_kv=4), -2), (dict(C=1), -2),
    (dict(L=0), -2), (dict(R=17), -2), (dict(T=0), -2), (dict(B=0), -2), (dict(L=17), -2),
    (dict(kv_layout=2), -10), (dict(kv_layout=-1), -10),
    (dict(T_cap=4095), -2), (dict(T_cap=-1), -2), (dict(T_cap=1 << 31), -2),
])
def test_invalid_geometry_is_rejected(kw, code):
    gm = g(**kw)
    tb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    assert Z.load().zha_tree_bytes(ctypes.byref(gm), ctypes.byref(tb), ctypes.byref(sb)) == code


def test_null_and_argument_errors_before_any_launch():
    lib = Z.load()
    gm = g()
    buf = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation
    n = ctypes.c_size_t()
    assert lib.zha_tree_bytes(None, ctypes.byref(n), ctypes.byref(n)) == -1
    assert lib.zha_build(ctypes.byref(gm), None, buf, None, buf, buf, None) == -1
    assert lib.zha_build(ctypes.byref(gm), ctypes.c_void_p(17), buf, None, buf, buf, None) == -6
    # rope: even dims in [0, d], frequencies given, reserved field zero
    th = (ctypes.c_double * 64)()
    tp = ctypes.cast(th, ctypes.POINTER(ctypes.c_double))
    for r in (Z.Rope(3, 0, tp), Z.Rope(-2, 0, tp), Z.Rope(130, 0, tp), Z.Rope(8, 0, None),
              Z.Rope(8, 1, tp)):
        assert lib.zha_build(ctypes.byref(gm), buf, buf, ctypes.byref(r), buf, buf, None) == -11
        assert lib.zha_tree_update(ctypes.byref(gm), 0, buf, buf, ctypes.byref(r), buf, buf,
                                   None) == -11
    # a valid rope passes validation (the call then fails on the NULL keys)
    r = Z.Rope(128, 0, tp)
    assert lib.zha_build(ctypes.byref(gm), None, buf, ctypes.byref(r), buf, buf, None) == -1
    assert lib.zha_build(ctypes.byref(gm), None, buf, ctypes.byref(Z.Rope(0, 0, None)), buf,
                         buf, None) == -1
    # p outside (0, 1]
    for p in (0.0, -0.5, 1.5, math.nan):
        assert lib.zha_route(ctypes.byref(gm), buf, buf, 1, None, p, buf, buf, 4, None, None, None,
                             None) == -5
    assert lib.zha_route(ctypes.byref(gm), buf, buf, 1, None, 0.9, buf, buf, 0, None, None, None,
                         None) == -7
    assert lib.zha_route(ctypes.byref(gm), buf, buf, 0, None, 0.9, buf, buf, 4, None, None, None,
                         None) == -9
    assert lib.zha_route(ctypes.byref(gm), None, buf, 1, None, 0.9, buf, buf, 4, None, None, None,
                         None) == -1
    assert lib.zha_attn(ctypes.byref(gm), buf, 1, None, buf, buf, None, buf, 4, buf, buf, None) == -1
    assert lib.zha_attn(ctypes.byref(gm), buf, 1, None, buf, buf, buf, buf, 0, buf, buf, None) == -7
    assert lib.zha_dense_decode(ctypes.byref(gm), buf, 0, buf, buf, buf, buf, None) == -9
    assert lib.zha_dense_decode(ctypes.byref(gm), ctypes.c_void_p(24), 1, buf, buf, buf, buf,
                                None) == -6
    # tree update: the old length must lie in [0, T]; pointers as for zha_build
    for t_old in (-1, gm.T + 1):
        assert lib.zha_tree_update(ctypes.byref(gm), t_old, buf, buf, None, buf, buf, None) == -2
    assert lib.zha_tree_update(ctypes.byref(gm), 0, None, buf, None, buf, buf, None) == -1
    assert lib.zha_tree_update(ctypes.byref(gm), gm.T, buf, buf, None, buf, None, None) == -1
    assert lib.zha_tree_update(ctypes.byref(gm), 5, buf, buf, None, ctypes.c_void_p(40), buf,
                               None) == -6
    assert lib.zha_tree_level_offset(ctypes.byref(gm), 0, ctypes.byref(n), ctypes.byref(n),
                                     ctypes.byref(n)) == -2
    # KV layout: split needs V; chunked takes the KV buffer as K and rejects a V
    assert lib.zha_attn(ctypes.byref(gm), buf, 1, None, buf, None, buf, buf, 4, buf, buf, None) == -1
    assert lib.zha_dense_decode(ctypes.byref(gm), buf, 1, buf, None, buf, buf, None) == -1
    gc = g(kv_layout=Z.ZHA_KV_CHUNKED)
    assert lib.zha_attn(ctypes.byref(gc), buf, 1, None, buf, buf, buf, buf, 4, buf, buf, None) == -10
    assert lib.zha_dense_decode(ctypes.byref(gc), buf, 1, buf, buf, buf, buf, None) == -10
    assert lib.zha_attn(ctypes.byref(gc), buf, 1, None, None, None, buf, buf, 4, buf, buf, None) == -1


def test_chunked_layout_shape_and_tree_layout_are_independent():
    gs, gc = g(T=5000), g(T=5000, kv_layout=Z.ZHA_KV_CHUNKED)
    assert Z.kv_shape(gs) == (1, 2, 5000, 128)
    assert Z.kv_shape(gc) == (1, 2, 313, 2, 16, 128)  # ceil(5000 / 16) pages
    assert Z.tree_bytes(gs) == Z.tree_bytes(gc)


def test_short_contexts_have_empty_upper_levels():
    # T < C^L is valid (a decode context that has not filled the top level yet):
    # the empty levels take no bytes unless a capacity reserves them.
    for T in (1, 15, 16, 255, 4095):
        gm = g(T=T)
        tb, sb = Z.tree_bytes(gm)
        expect = expected_layout(gm, 2)[2] * gm.B * gm.H_kv
        assert tb == expect
    assert Z.tree_bytes(g(T=1))[0] == 0
    assert Z.tree_bytes(g(T=1, T_cap=4096)) == Z.tree_bytes(g(T=4096))


def test_capacity_sets_strides_and_length_sets_nothing_else():
    # Layout (tree offsets, scratch sizes, KV shape) depends on the capacity only,
    # so a cache and tree laid out once stay valid as the length grows.
    base = dict(T_cap=20000, C=16, L=3)
    sizes = {Z.tree_bytes(g(T=t, **base)) for t in (4096, 5000, 19999, 20000)}
    offs = {Z.level_offset(g(T=t, **base), 2) for t in (4096, 5000, 20000)}
    assert len(sizes) == 1 and len(offs) == 1
    assert Z.tree_bytes(g(T=20000)) == sizes.pop()
    assert Z.kv_shape(g(T=4096, T_cap=20000)) == (1, 2, 20000, 128)
    assert Z.kv_shape(g(T=4096, T_cap=20000, kv_layout=Z.ZHA_KV_CHUNKED)) == (1, 2, 1250, 2, 16, 128)
    g2 = Z.with_length(g(T=4096), 4100)
    assert (g2.T, g2.T_cap) == (4100, 4096) and Z.tree_bytes(Z.with_length(g(T=4096), 4096))
    # with_length keeps the capacity, and a length beyond it is rejected
    n = ctypes.c_size_t()
    assert Z.load().zha_tree_bytes(ctypes.byref(g2), ctypes.byref(n), ctypes.byref(n)) == -2


def test_scratch_sizes_are_consistent():
    # n_1 = 4096: every frontier fits the router's on-chip capacity
    small = g(B=8, H_q=32, H_kv=4, T=32768, C=8, L=5)
    assert Z.frontier_capacity() == 4096
    assert Z.route_scratch_bytes(small, 1, 4096) == 0
    assert Z.route_scratch_bytes(small, 16, 4096) >= (8 * 16 * 32 + 1) * 4  # many heads: re-route list
    # n_1 = 32768: frontiers of up to n_1 candidates in device memory (ids twice, scores)
    gm = g(B=8, H_q=32, H_kv=4, T=262144, C=8, L=6)
    few = Z.route_scratch_bytes(gm, 1, 32768)
    assert few >= 12 * 32768 + 256 * 4
    many = Z.route_scratch_bytes(gm, 16, 32768)
    assert many >= few + (8 * 16 * 32 + 1) * 4
    # sized for the capacity, so the same at every length up to it
    assert Z.route_scratch_bytes(g(B=8, H_q=32, H_kv=4, T=5000, T_cap=262144, C=8, L=6), 1,
                                 32768) == few
    a = Z.attn_scratch_bytes(gm, 1, 32768)
    assert a >= (256 + 32) * 4 * (gm.d + 2)  # plan + at least one partial per workgroup and head
    assert Z.dense_scratch_bytes(gm, 1) % (4 * (gm.d + 2)) == 0
    assert Z.frontier_capacity() >= 1024


def test_child_index_by_multiply_high_is_exact():
    # The router's child expansion takes a parent index floor(x / C) as the high
    # word of x * ceil(2^32 / C) (zha_route's cdiv argument); exact for every x
    # the expansion meets (x < 2^16) and every chunk size (2 <= C <= 1024).
    import numpy as np
    x = np.arange(1 << 16, dtype=np.uint64)
    for C in range(2, 1025):
        magic = np.uint64(((1 << 32) + C - 1) // C)
        assert magic < (1 << 32)
        assert np.array_equal((x * magic) >> np.uint64(32), x // np.uint64(C)), C


def test_route_rejects_frontiers_of_2_pow_24_candidates():
    # A level's cut sums one 40-bit fixed-point mass per candidate in 64 bits:
    # zha_route (and its scratch query) refuse geometries whose level 1 could
    # hold 2^24 nodes, before any launch; build and attention do not route.
    lib = Z.load()
    buf = ctypes.c_void_p(16)
    n = ctypes.c_size_t()
    for C, T, ok in ((16, (1 << 24) * 16 - 1, True), (16, (1 << 24) * 16, False),
                     (2, (1 << 25) - 1, True), (2, 1 << 25, False), (1024, (1 << 31) - 1, True)):
        gm = g(C=C, L=1, T=T, H_q=2, H_kv=1)
        rc = lib.zha_route_scratch_bytes(ctypes.byref(gm), 1, 4, ctypes.byref(n))
        assert (rc == 0) == ok, (C, T, rc)
        # p = 0 fails p validation first; a valid p reaches the frontier check
        rc = lib.zha_route(ctypes.byref(gm), buf, buf, 1, None, 0.9, buf, buf, 4, None, None, None,
                           None)
        assert rc == (-2 if not ok else rc), (C, T, rc)
        assert lib.zha_tree_bytes(ctypes.byref(gm), ctypes.byref(n), ctypes.byref(n)) == 0
    # with a capacity: the capacity, not the length, bounds the frontier
    gm = g(C=16, L=1, T=4096, T_cap=(1 << 24) * 16, H_q=2, H_kv=1)
    assert lib.zha_route_scratch_bytes(ctypes.byref(gm), 1, 4, ctypes.byref(n)) == -2


def test_failed_route_codes_are_declared():
    text = open(HEADER).read()
    assert "ZHA_ROUTE_BAD_CTX = -1" in text and "ZHA_ROUTE_SLOT_BUSY = -2" in text


def test_attn_noalloc_rejects_calls_past_its_fixed_buffer():
    # zha_attn_noalloc checks, before touching the device, that the call's
    # scratch fits ZHA_NOALLOC_SCRATCH_BYTES; a balanced call of 2048 heads at
    # d = 256 fits, the block path at the 1M block does not.
    lib = Z.load()
    buf = ctypes.c_void_p(256)  # never dereferenced: these calls fail validation
    big = g(B=1, H_q=16, H_kv=2, T=1 << 20, C=32, L=4)
    need = Z.attn_scratch_bytes(big, 2048, 32768)
    assert need > Z.ZHA_NOALLOC_SCRATCH_BYTES
    assert lib.zha_attn_noalloc(ctypes.byref(big), buf, 2048, None, buf, buf, buf, buf, 32768,
                                buf, None) == -12
    assert Z.attn_scratch_bytes(g(B=1, H_q=16, H_kv=2, d=256, T=1 << 20), 128, 64) <= \
        Z.ZHA_NOALLOC_SCRATCH_BYTES
    # the same argument checks as zha_attn, before the size check
    assert lib.zha_attn_noalloc(ctypes.byref(big), None, 2048, None, buf, buf, buf, buf, 32768,
                                buf, None) == -1
    assert lib.zha_attn_noalloc(ctypes.byref(big), buf, 0, None, buf, buf, buf, buf, 32768,
                                buf, None) == -9
