"""Decode-time tree maintenance on the GPU against the fp64 oracle.

A KV cache and its tree are laid out once for a token capacity; tokens are
appended in place and zha_tree_update summarises only the spans that completed
(paper §III-A and App. D-B2: a leaf when its chunk is full, a parent when its
last child is).  After every append the stored tree must equal the oracle's
tree of the cached prefix bit for bit, and routes and outputs at the new length
must match the oracle to the usual parity bar.  Rows past the current length
hold NaN, so a kernel that read one would show it in its outputs.
"""
import sys

import numpy as np
import pytest

import oracle as O
from hierarchical_tree_indexed_04_amd import workload as W
from zha_testutil import (TOL, Parity, attend_on, compare_head, from_device, oracle_trees,
                          to_device, tree_mismatch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    from hierarchical_tree_indexed_04_amd import zha
    zha.load()
    return zha


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def nan_bits(dtype):
    return np.uint16(0x7FC0) if dtype == W.BF16 else np.float32(np.nan)


class Cache:
    """Device KV cache of capacity Tc in either layout, filled token by token."""

    def __init__(self, Z, g, K, V, Tc, chunked):
        import torch
        self.Z, self.g, self.K, self.V, self.Tc, self.chunked = Z, g, K, V, Tc, chunked
        sdt = K.dtype
        if chunked:
            pages = -(-Tc // g.C)
            host = np.full((g.B, g.H_kv, pages, 2, g.C, g.d), nan_bits(g.dtype), sdt)
            self.KV = to_device(host, g.dtype)
            self.Kd, self.Vd = self.KV, None
        else:
            host = np.full((g.B, g.H_kv, Tc, g.d), nan_bits(g.dtype), sdt)
            self.Kd, self.Vd = to_device(host, g.dtype), to_device(host, g.dtype)
        del torch

    def append(self, t0, t1):
        """Writes the K/V rows of tokens [t0, t1) into the cache."""
        g = self.g
        k = to_device(self.K[:, :, t0:t1], g.dtype)
        v = to_device(self.V[:, :, t0:t1], g.dtype)
        if not self.chunked:
            self.Kd[:, :, t0:t1] = k
            self.Vd[:, :, t0:t1] = v
            return
        for t in range(t0, t1):
            self.KV[:, :, t // g.C, 0, t % g.C] = k[:, :, t - t0]
            self.KV[:, :, t // g.C, 1, t % g.C] = v[:, :, t - t0]


def check_length(Z, g, gm, cache, tree, qref, T, n_pos, p, steps_seed):
    """Tree (bit-exact), routes and outputs at length T against the oracle."""
    import torch
    gT = W.replace(g, T=T)
    pairs = [(b, h) for b in range(g.B) for h in range(g.H_kv)]
    trees = oracle_trees(gT, cache.K[:, :, :T], qref, pairs)
    bad_k, bad_b, total = tree_mismatch(Z, gT, tree.cpu().numpy(), trees, gm)
    assert bad_k == 0 and bad_b == 0, (T, bad_k, bad_b, total)
    Qn = W.make_query_block(gT, cache.K[:, :, :T], range(steps_seed, steps_seed + n_pos))
    Qd = to_device(Qn, g.dtype)
    cap = max(gT.n_level(1), 1)
    sel, cnt, stats, gap = Z.route(gm, tree, Qd, n_pos, p, cap)
    Od = Z.attn(gm, Qd, n_pos, cache.Kd, cache.Vd, sel, cnt, cap)
    Dd = Z.dense_decode(gm, Qd, n_pos, cache.Kd, cache.Vd)
    torch.cuda.synchronize()
    sel, cnt, stats, gap = (sel.cpu().numpy(), cnt.cpu().numpy(), stats.cpu().numpy(),
                            gap.cpu().numpy())
    Og, Dg = from_device(Od, g.dtype), from_device(Dd, g.dtype)
    par = Parity()
    dense_err = 0.0
    for (b, kvh) in pairs:
        Kf = W.to_float(cache.K[b, kvh, :T], g.dtype)
        Vf = W.to_float(cache.V[b, kvh, :T], g.dtype)
        for t in range(n_pos):
            for h in range(kvh * g.G, (kvh + 1) * g.G):
                q = W.to_float(Qn[b, t, h], g.dtype)
                r, o = O.zha_head(trees[(b, kvh)], q, Kf, Vf, p)
                compare_head(par, r, sel[b, t, h], int(cnt[b, t, h]), stats[b, t, h],
                             Og[b, t, h], o, TOL[g.dtype], (T, b, t, h), gap_row=gap[b, t, h],
                             attend_set=attend_on(q, Kf, Vf, g.C, T))
                dense_err = max(dense_err, float(np.abs(Dg[b, t, h] - O.dense(q, Kf, Vf)).max()))
    par.check()
    assert dense_err <= TOL[g.dtype], (T, dense_err)
    return par, total


# Appends per case: single tokens across chunk ends, a burst that completes a
# level-2 node, and one that completes the root level's next node.
@pytest.mark.parametrize("dtype,chunked,R", [(W.BF16, False, 4), (W.BF16, True, 1),
                                             (W.F32, False, 2)])
def test_appends_match_oracle_at_every_length(Z, dtype, chunked, R):
    import torch
    C, L = 8, 3
    T0 = C ** L + 3
    grow = [1, 1, 1, 1, 1, 4, 13, C * C - 2, 1, 1, C ** 3 - 50, 77]
    T_end = T0 + sum(grow)
    Tc = T_end + 11
    say(f"decode appends: {dtype}, {'chunked' if chunked else 'split'} KV, R={R}, "
        f"T {T0} -> {T_end}, capacity {Tc}")
    g = W.custom(f"dec{R}", 150 + R, dtype=dtype, B=2, H_q=4, H_kv=2, T=T_end, C=C, L=L,
                 p=0.9, R=R)
    K, V = W.make_kv(g)
    qref = W.make_qref(g, K)
    qd = torch.from_numpy(qref).cuda()
    cache = Cache(Z, g, K, V, Tc, chunked)
    layout = Z.ZHA_KV_CHUNKED if chunked else Z.ZHA_KV_SPLIT
    cache.append(0, T0)
    gm = Z.geom(W.replace(g, T=T0), layout, T_cap=Tc)
    tb, sb = Z.tree_bytes(gm)
    tree = torch.full((tb,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN past the valid rows
    scratch = torch.empty((max(sb, 1),), dtype=torch.uint8, device="cuda")
    Z.build(gm, cache.Kd, qd, tree, scratch)
    par, total = check_length(Z, g, gm, cache, tree, qref, T0, 2, 0.9, 0)
    T = T0
    for i, n in enumerate(grow):
        cache.append(T, T + n)
        gm = Z.with_length(gm, T + n)
        assert Z.tree_bytes(gm) == (tb, sb)
        Z.tree_update(gm, T, cache.Kd, qd, tree, scratch)
        T += n
        par, total = check_length(Z, g, gm, cache, tree, qref, T, 2, 0.9, 10 * (i + 1))
        say(f"  T={T}: tree exact over {total} values; {par.summary()}")
    assert T == T_end


def test_update_from_zero_equals_build(Z):
    # T_old = 0 summarises every node: the same tree as zha_build, in a layout
    # with spare capacity.
    import torch
    g = W.custom("dec0", 160, dtype=W.BF16, B=1, H_q=2, H_kv=1, T=16 ** 2 * 5 + 9, C=16, L=2,
                 p=0.9, R=3)
    K, V = W.make_kv(g)
    qref = W.make_qref(g, K)
    qd = torch.from_numpy(qref).cuda()
    gm = Z.geom(g, Z.ZHA_KV_SPLIT, T_cap=g.T + 300)
    cache = Cache(Z, g, K, V, g.T + 300, False)
    cache.append(0, g.T)
    tb, sb = Z.tree_bytes(gm)
    t_build = torch.zeros((tb,), dtype=torch.uint8, device="cuda")
    t_upd = torch.zeros((tb,), dtype=torch.uint8, device="cuda")
    Z.build(gm, cache.Kd, qd, t_build, torch.empty((sb,), dtype=torch.uint8, device="cuda"))
    Z.tree_update(gm, 0, cache.Kd, qd, t_upd, torch.empty((sb,), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(t_build, t_upd)
    trees = oracle_trees(g, K, qref, [(0, 0)])
    assert tree_mismatch(Z, g, t_upd.cpu().numpy(), trees, gm)[:2] == (0, 0)
    # no new token: nothing to do, nothing changes
    Z.tree_update(gm, g.T, cache.Kd, qd, t_upd, torch.empty((sb,), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(t_build, t_upd)


@pytest.mark.parametrize("dtype,chunked", [(W.BF16, False), (W.F32, True)])
def test_decode_from_one_token(Z, dtype, chunked):
    # Every length from 1 to past C^L, one token per step: no full chunk (I(q)
    # is every token), then empty upper levels, then the first top node.
    import torch
    C, L, T_end = 4, 3, 4 ** 3 + 9
    say(f"decode from one token: {dtype}, {'chunked' if chunked else 'split'} KV, T 1 -> {T_end}")
    g = W.custom("dec1", 170, dtype=dtype, B=1, H_q=4, H_kv=2, T=T_end, C=C, L=L, p=0.8, R=2)
    K, V = W.make_kv(g)
    qref = W.make_qref(g, K)
    qd = torch.from_numpy(qref).cuda()
    cache = Cache(Z, g, K, V, T_end, chunked)
    layout = Z.ZHA_KV_CHUNKED if chunked else Z.ZHA_KV_SPLIT
    cache.append(0, 1)
    gm = Z.geom(W.replace(g, T=1), layout, T_cap=T_end)
    tb, sb = Z.tree_bytes(gm)
    tree = torch.full((tb,), 0xFF, dtype=torch.uint8, device="cuda")
    scratch = torch.empty((sb,), dtype=torch.uint8, device="cuda")
    Z.build(gm, cache.Kd, qd, tree, scratch)
    check_length(Z, g, gm, cache, tree, qref, 1, 2, 0.8, 0)
    for T in range(2, T_end + 1):
        cache.append(T - 1, T)
        gm = Z.with_length(gm, T)
        Z.tree_update(gm, T - 1, cache.Kd, qd, tree, scratch)
        par, _ = check_length(Z, g, gm, cache, tree, qref, T, 2, 0.8, 7 * T)
    say(f"  {T_end} lengths exact; last: {par.summary()}")


@pytest.mark.parametrize("T,dtype", [(5, W.BF16), (8 * 3 + 2, W.BF16), (70, W.BF16), (70, W.F32)])
def test_short_context_many_heads(Z, T, dtype):
    # 4120 query heads: the router's throughput shape, and the block attention
    # path (bf16) or one workgroup per head (fp32), on a tree with empty upper
    # levels (C^L = 512 > T).
    import torch
    say(f"short context T={T} ({dtype}), 1030 positions x 4 heads")
    g = W.custom("short", 171, dtype=dtype, B=1, H_q=4, H_kv=1, T=T, C=8, L=3, p=0.9, R=1)
    K, V = W.make_kv(g)
    qref = W.make_qref(g, K)
    cache = Cache(Z, g, K, V, T, False)
    cache.append(0, T)
    gm = Z.geom(g)
    tree = Z.build(gm, cache.Kd, torch.from_numpy(qref).cuda())
    par, _ = check_length(Z, g, gm, cache, tree, qref, T, 1030, 0.9, 0)
    say(f"  {par.summary()}")
